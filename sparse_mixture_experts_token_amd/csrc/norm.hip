// Prologue of the pre-normalised MoE sublayer: RMSNorm of the residual stream
// ("gpt-oss 20B" field guide, cutaway 04 "One decoder block": RMSNorm before
// the MoE sublayer; one gain per hidden feature, no bias, per the
// "openai/gpt-oss-20b" fixture page's parameter table):
//
//   n[t, :] = g * x[t, :] * r_t,   r_t = 1 / sqrt(mean_j x[t, j]^2 + eps)
//
// One wave per token.  The mean square is accumulated in fp32: each lane sums
// its 16-byte chunks in order, then the lanes are added by the fixed DPP
// reduction, so the result does not depend on scheduling.  A second pass over
// the row (now in L1/L2) writes the expert GEMMs' input, in the format they
// multiply in:
//   bf16 activations: n16 = (g * x) * r_t rounded once to bf16;
//   fp32 activations: n32 = (g * x) * r_t, also the fp32 router's input.
// bf16 routing must not see the rounded n16 (a last-bit difference would move
// a logit by ~1e-4): the logits are r_t * (x . (W_r * g)), x taken exactly.
// Blocks past the tokens fold the gain into the router: W_r * g, a product of
// two bf16 values, has at most 16 significant bits, so it splits exactly into
// hi = bf16(W_r * g) and lo = W_r * g - hi (at most 8 bits: a bf16 value),
// which the bf16 logit kernel multiplies by x in two MFMAs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNormWaves = 4;  // tokens per workgroup
constexpr int kFoldPerBlock = 256 * 8;

template <bool kBf16>
struct Chunk;  // one 16-byte load: 8 bf16 or 4 fp32 values
template <>
struct Chunk<true> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const void* p, size_t i, float (&v)[8]) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
            v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        }
    }
};
template <>
struct Chunk<false> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const void* p, size_t i, float (&v)[4]) {
        const float4 q = reinterpret_cast<const float4*>(p)[i];
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    }
};

template <bool kBf16>
__global__ __launch_bounds__(kNormWaves * 64) void rms_norm_kernel(const void* __restrict__ x,
                                                                    const void* __restrict__ g, float eps, int T,
                                                                    int H, float* __restrict__ n32,
                                                                    uint16_t* __restrict__ n16,
                                                                    float* __restrict__ row_scale,
                                                                    const uint16_t* __restrict__ w_router, int E,
                                                                    uint16_t* __restrict__ wr_hi,
                                                                    uint16_t* __restrict__ wr_lo) {
    using C = Chunk<kBf16>;
    constexpr int N = C::N;
    const int tblocks = (T + kNormWaves - 1) / kNormWaves;
    if ((int)blockIdx.x >= tblocks) {
        // the router with the gain folded in, as two exact bf16 parts (bf16 only)
        const uint16_t* gb = reinterpret_cast<const uint16_t*>(g);
        const size_t i0 = ((size_t)blockIdx.x - tblocks) * kFoldPerBlock;
        const size_t nw = (size_t)E * H;
        for (size_t i = i0 + threadIdx.x; i < i0 + kFoldPerBlock && i < nw; i += blockDim.x) {
            const float p = bf16_bits_to_f32(w_router[i]) * bf16_bits_to_f32(gb[i % (size_t)H]);
            const uint32_t hi = f32_to_bf16_bits(p);
            wr_hi[i] = (uint16_t)hi;
            wr_lo[i] = (uint16_t)f32_to_bf16_bits(p - bf16_bits_to_f32(hi));
        }
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kNormWaves + wave;
    if (t >= T) return;  // wave-uniform; no barriers below
    const int nc = H / N;  // chunks per row (H is a multiple of 64)
    const size_t row = (size_t)t * nc;
    float ss = 0.f;
    for (int c = lane; c < nc; c += 64) {
        float v[N];
        C::load(x, row + c, v);
#pragma unroll
        for (int j = 0; j < N; ++j) ss = fmaf(v[j], v[j], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    if constexpr (kBf16)
        if (lane == 0) row_scale[t] = r;
    for (int c = lane; c < nc; c += 64) {
        float v[N], gv[N];
        C::load(x, row + c, v);
        C::load(g, (size_t)c, gv);
        float o[N];
#pragma unroll
        for (int j = 0; j < N; ++j) o[j] = (gv[j] * v[j]) * r;
        if constexpr (!kBf16) {
            reinterpret_cast<float4*>(n32)[row + c] = make_float4(o[0], o[1], o[2], o[3]);
        } else {
            uint4 q;
            q.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
            q.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
            q.z = f32_to_bf16_bits(o[4]) | (f32_to_bf16_bits(o[5]) << 16);
            q.w = f32_to_bf16_bits(o[6]) | (f32_to_bf16_bits(o[7]) << 16);
            reinterpret_cast<uint4*>(n16)[row + c] = q;
        }
    }
}

}  // namespace

hipError_t launch_rms_norm(int act_dtype, const void* x, const void* g, float eps, int T, int H, float* n32,
                           uint16_t* n16, float* row_scale, const void* w_router, int E, uint16_t* wr_hi,
                           uint16_t* wr_lo, hipStream_t stream) {
    const int tblocks = (T + kNormWaves - 1) / kNormWaves;
    if (act_dtype == DT_BF16) {
        const int wblocks = (int)(((size_t)E * H + kFoldPerBlock - 1) / kFoldPerBlock);
        rms_norm_kernel<true><<<tblocks + wblocks, kNormWaves * 64, 0, stream>>>(
            x, g, eps, T, H, nullptr, n16, row_scale, (const uint16_t*)w_router, E, wr_hi, wr_lo);
    } else {
        rms_norm_kernel<false><<<tblocks, kNormWaves * 64, 0, stream>>>(x, g, eps, T, H, n32, nullptr, nullptr,
                                                                       nullptr, E, nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace moe
