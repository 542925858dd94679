// Stand-alone MXFP4 -> bf16 decode with the device routine the grouped GEMMs
// use while staging weight tiles (exact: every decoded value is representable
// in bf16).  One thread per 32-element group; groups are contiguous 16-byte
// runs of packed codes with one E8M0 scale byte each.
#include "moe.h"
#include "moe_internal.h"

namespace {

__global__ __launch_bounds__(256) void mxfp4_decode_kernel(const moe::u32x4* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales, int64_t groups,
                                                           moe::u32x4* __restrict__ out) {
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * blockDim.x) {
        uint32_t d[16];
        moe::decode_mxfp4_32(packed[g], scales[g], d);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[g * 4 + i] = moe::u32x4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
    }
}

}  // namespace

extern "C" int moe_mxfp4_decode(const uint8_t* packed, const uint8_t* scales, int64_t n_groups, void* out_bf16,
                                void* stream) {
    if (n_groups < 0) return MOE_ERR_SHAPE;
    if (n_groups == 0) return MOE_OK;
    if (!packed || !scales || !out_bf16) return MOE_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(out_bf16)) % 16) return MOE_ERR_ALIGN;
    const int64_t blocks64 = (n_groups + 255) / 256;
    const int blocks = (int)(blocks64 < 16384 ? blocks64 : 16384);
    mxfp4_decode_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const moe::u32x4*>(packed), scales, n_groups, reinterpret_cast<moe::u32x4*>(out_bf16));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
