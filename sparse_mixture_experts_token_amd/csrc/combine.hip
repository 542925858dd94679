// Stage 4 of the layer: the weighted sum over the selected experts
// ("gpt-oss-40b-64a8-init" page, section 2, Proof: FFN(h) = sum p_i E_i(h)).
// The down stage already multiplied each expert output by its weight p_i and
// stored it at the assignment's slot, so
//     out[t, :] = y[t*k + 0, :] + y[t*k + 1, :] + ... + y[t*k + k-1, :]
// summed in fp32 in slot order (= ascending expert id), rounded once.  In the
// pre-normalised block the residual-stream row x[t, :] is added to that sum
// before the rounding ("gpt-oss 20B" field guide, cutaway 04: each sublayer
// is added back to the residual stream).
// Memory bound: 4 outputs per thread, 16-byte loads.
#include "moe_internal.h"

namespace moe {
namespace {

// kSlotBatch: slot rows whose loads are in flight together (8 up to top-8;
// 24 beyond, so a decode-sized top-20 call waits for memory once per thread)
template <bool kBf16Out, int kSlotBatch>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, void* __restrict__ out, int T,
                                                      int H, int k, const void* __restrict__ residual) {
    const int h4 = H >> 2;
    const size_t n4 = (size_t)T * h4;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / h4;
        const size_t c = i % h4;
        const float4* src = reinterpret_cast<const float4*>(y) + (t * k) * h4 + c;
        // slots in batches of kSlotBatch loads issued together, added in slot order
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < k; s0 += kSlotBatch) {
            float4 v[kSlotBatch];
#pragma unroll
            for (int j = 0; j < kSlotBatch; ++j)
                if (s0 + j < k) v[j] = src[(size_t)(s0 + j) * h4];
#pragma unroll
            for (int j = 0; j < kSlotBatch; ++j) {
                if (s0 + j >= k) break;
                if (s0 + j == 0) {
                    acc = v[0];
                } else {
                    acc.x += v[j].x;
                    acc.y += v[j].y;
                    acc.z += v[j].z;
                    acc.w += v[j].w;
                }
            }
        }
        if (residual) {
            if constexpr (kBf16Out) {
                const uint2 r = reinterpret_cast<const uint2*>(residual)[i];
                acc.x += bf16_bits_to_f32(r.x & 0xffffu);
                acc.y += bf16_bits_to_f32(r.x >> 16);
                acc.z += bf16_bits_to_f32(r.y & 0xffffu);
                acc.w += bf16_bits_to_f32(r.y >> 16);
            } else {
                const float4 r = reinterpret_cast<const float4*>(residual)[i];
                acc.x += r.x;
                acc.y += r.y;
                acc.z += r.z;
                acc.w += r.w;
            }
        }
        if constexpr (kBf16Out) {
            uint2 o;
            o.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
            o.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
            reinterpret_cast<uint2*>(out)[i] = o;
        } else {
            reinterpret_cast<float4*>(out)[i] = acc;
        }
    }
}

}  // namespace

hipError_t launch_combine(int act_dtype, const float* y, void* out, int T, int H, int k, const void* residual,
                          hipStream_t stream) {
    const size_t n4 = (size_t)T * (H / 4);
    const int blocks = (int)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
    if (act_dtype == DT_BF16) {
        if (k <= 8) combine_kernel<true, 8><<<blocks, 256, 0, stream>>>(y, out, T, H, k, residual);
        else combine_kernel<true, 24><<<blocks, 256, 0, stream>>>(y, out, T, H, k, residual);
    } else {
        if (k <= 8) combine_kernel<false, 8><<<blocks, 256, 0, stream>>>(y, out, T, H, k, residual);
        else combine_kernel<false, 24><<<blocks, 256, 0, stream>>>(y, out, T, H, k, residual);
    }
    return hipGetLastError();
}

}  // namespace moe
