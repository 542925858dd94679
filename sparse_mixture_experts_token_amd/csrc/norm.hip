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
// the row (now in L1/L2) writes
//   n32 = (g * x) * r_t in fp32 - the router's input: for bf16 x and g the
//         product g * x is exact in fp32, so the logits see the normalised
//         input to fp32 precision;
//   n16 = n32 rounded to bf16 (bf16 activations only) - the expert GEMMs'
//         input, in the format they multiply in.
// With bf16 activations the router then runs in fp32: blocks past the tokens
// widen W_r and b_r to fp32 (exact).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNormWaves = 4;  // tokens per workgroup
constexpr int kWidenPerBlock = 256 * 8;

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
                                                                    const uint16_t* __restrict__ w_router,
                                                                    const uint16_t* __restrict__ b_router, int E,
                                                                    float* __restrict__ wr32,
                                                                    float* __restrict__ br32) {
    using C = Chunk<kBf16>;
    constexpr int N = C::N;
    const int tblocks = (T + kNormWaves - 1) / kNormWaves;
    if ((int)blockIdx.x >= tblocks) {
        // widen the router to fp32 (bf16 activations only)
        const size_t i0 = ((size_t)blockIdx.x - tblocks) * kWidenPerBlock;
        const size_t nw = (size_t)E * H;
        for (size_t i = i0 + threadIdx.x; i < i0 + kWidenPerBlock && i < nw; i += blockDim.x)
            wr32[i] = bf16_bits_to_f32(w_router[i]);
        if (blockIdx.x == (unsigned)tblocks && b_router)
            for (int e = threadIdx.x; e < E; e += blockDim.x) br32[e] = bf16_bits_to_f32(b_router[e]);
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
    for (int c = lane; c < nc; c += 64) {
        float v[N], gv[N];
        C::load(x, row + c, v);
        C::load(g, (size_t)c, gv);
        float o[N];
#pragma unroll
        for (int j = 0; j < N; ++j) o[j] = (gv[j] * v[j]) * r;
        float4* d = reinterpret_cast<float4*>(n32 + (row + c) * N);
#pragma unroll
        for (int j = 0; j < N / 4; ++j) d[j] = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
        if constexpr (kBf16) {
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
                           uint16_t* n16, const void* w_router, const void* b_router, int E, float* wr32,
                           float* br32, hipStream_t stream) {
    const int tblocks = (T + kNormWaves - 1) / kNormWaves;
    if (act_dtype == DT_BF16) {
        const int wblocks = (int)(((size_t)E * H + kWidenPerBlock - 1) / kWidenPerBlock);
        rms_norm_kernel<true><<<tblocks + wblocks, kNormWaves * 64, 0, stream>>>(
            x, g, eps, T, H, n32, n16, (const uint16_t*)w_router, (const uint16_t*)b_router, E, wr32, br32);
    } else {
        rms_norm_kernel<false><<<tblocks, kNormWaves * 64, 0, stream>>>(x, g, eps, T, H, n32, nullptr, nullptr,
                                                                       nullptr, E, nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace moe
