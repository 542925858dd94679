// Gradients of the sparse MoE layer ("gpt-oss-40b-64a8-init" page: section 1,
// Train Wide, Deploy Narrow, why the expanded layers are trained; section
// 5.2, original experts frozen while the copies and the router train;
// section 2, Proof, the layer being differentiated).  With the forward's
// routing (selected experts, weights p, expert-major permutation) held fixed,
// per routed row r = (token t, expert e):
//
//   g = W_g[e] h_t, u = W_u[e] h_t, a = silu(g) u          (recomputed)
//   gy = W_d[e]^T dout_t,  dp_r = gy . a,  da = p gy
//   dg = da u silu'(g),  du = da silu(g)
//   dh_t += W_g[e]^T dg + W_u[e]^T du
//   dW_d[e] += (p dout_t) a^T,  dW_g[e] += dg h_t^T,  dW_u[e] += du h_t^T
//   ds = p (dp - sum_S p dp) per token;  dW_r += ds h^T,  db_r += ds,  dh += ds W_r
//
// Kernels, in launch order:
//   bwd_tiles   - 128-row tiles of every expert's row range (one workgroup);
//   bwd_gather  - expert-major copies of h and dout, p * dout in bf16, and
//                 the inverse permutation;
//   bwd_gemm    - one MFMA grouped GEMM for all six products (below);
//   bwd_swiglu  - per row: act, dp, dg, du (bf16 for the next products);
//   bwd_token   - per token: ds, dh = sum of its rows' input gradients +
//                 ds W_r (one rounding), ds as a dense [T, E] matrix;
//   bwd_bias    - db_r as column sums of ds.
//
// bwd_gemm: C[M, N] (=, or +=) A[M, K] B[K, N], bf16 operands, fp32
// accumulate, 128 x 128 tiles of four waves (64 x 64 each, 32x32x16 bf16
// MFMAs), 32-deep K steps double-buffered in LDS with the next step's global
// loads in flight during the current step's MFMAs.  Each operand is either
// K-contiguous (A[m][k], B[n][k]) or not (A[k][m], B[k][n]); the latter is
// transposed on its way into LDS.  Groups: by rows (an expert's rows of the
// permuted matrix against that expert's weights), by K (an expert's rows are
// the contraction: weight gradients), or one plain product.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGB = 128;    // tile rows and columns
constexpr int kGK = 32;     // K per step
constexpr int kLdsRow = 40; // halves per LDS row (32 + 8 padding)

struct BwdGemm {
    const uint16_t* A;
    const uint16_t* B;
    float* C;
    long long lda, ldb, ldc;
    long long b_gs, c_gs;  // per-expert strides of B (row groups) and C (K groups), elements
    int M, N, K;           // M: store bound (row groups: unused); K: contraction (K groups: unused)
    int Ma;                // rows of A that may be read (multiple of 8 when A is not K-contiguous)
    int mode;              // 0 row groups, 1 K groups, 2 plain
    const int32_t* offsets;
    const int32_t* tiles;   // row groups: (expert << 16) | tile within the expert
    const int32_t* ntiles;
    const uint8_t* trainable;  // K groups: experts with 0 are skipped (null: all)
    int accumulate;
};

// 16 bytes of 8 bf16 at the given element index or zeros.
__device__ __forceinline__ u32x4 ld16(const uint16_t* p, long long i, bool ok) {
    return ok ? *reinterpret_cast<const u32x4*>(p + i) : u32x4{0u, 0u, 0u, 0u};
}

// Global loads of one operand's 128 x 32 step: two 16-byte pieces per thread.
// K-contiguous (X[r][k]): piece c -> row c / 4, k 8 (c % 4).  Otherwise
// (X[k][r]): piece c -> k c / 16, rows 8 (c % 16) .. +7.
template <bool KC>
__device__ __forceinline__ void step_load(const uint16_t* X, long long ld, int r0, int rows, int k0, int K, int tid,
                                          u32x4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        if constexpr (KC) {
            const int r = c >> 2, kc = (c & 3) * 8;
            const bool ok = r0 + r < rows && k0 + kc < K;
            v[i] = ld16(X, ok ? (long long)(r0 + r) * ld + k0 + kc : 0, ok);
        } else {
            const int kr = c >> 4, rc = (c & 15) * 8;
            const bool ok = k0 + kr < K && r0 + rc < rows;
            v[i] = ld16(X, ok ? (long long)(k0 + kr) * ld + r0 + rc : 0, ok);
        }
    }
}

// The same pieces into LDS as [row][k] (k contiguous).
template <bool KC>
__device__ __forceinline__ void step_store(uint16_t* S, int tid, const u32x4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        if constexpr (KC) {
            const int r = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<u32x4*>(S + r * kLdsRow + kc) = v[i];
        } else {
            const int kr = c >> 4, rc = (c & 15) * 8;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[(rc + 2 * e) * kLdsRow + kr] = (uint16_t)(w[e] & 0xffffu);
                S[(rc + 2 * e + 1) * kLdsRow + kr] = (uint16_t)(w[e] >> 16);
            }
        }
    }
}

template <bool AK, bool BK>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm g) {
    __shared__ __align__(16) uint16_t sA[2][kGB * kLdsRow];
    __shared__ __align__(16) uint16_t sB[2][kGB * kLdsRow];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint16_t* A = g.A;
    const uint16_t* B = g.B;
    float* C = g.C;
    int m0, rowsA, Mst, K;
    const int n0 = blockIdx.y * kGB;
    if (g.mode == 0) {
        if ((int)blockIdx.x >= *g.ntiles) return;
        const int t = g.tiles[blockIdx.x];
        const int e = t >> 16, ti = t & 0xffff;
        const int r0 = g.offsets[e] + ti * kGB;
        A += (long long)r0 * g.lda;
        B += (long long)e * g.b_gs;
        C += (long long)r0 * g.ldc;
        m0 = 0;
        rowsA = min(kGB, g.offsets[e + 1] - r0);
        Mst = rowsA;
        K = g.K;
    } else if (g.mode == 1) {
        const int e = blockIdx.z;
        if (g.trainable && !g.trainable[e]) return;
        const int k0 = g.offsets[e];
        A += (long long)k0 * g.lda;
        B += (long long)k0 * g.ldb;
        C += (long long)e * g.c_gs;
        m0 = blockIdx.x * kGB;
        rowsA = g.Ma;
        Mst = g.M;
        K = g.offsets[e + 1] - k0;
    } else {
        m0 = blockIdx.x * kGB;
        rowsA = g.Ma;
        Mst = g.M;
        K = g.K;
    }
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = (K + kGK - 1) / kGK;
    u32x4 va[2], vb[2];
    if (nk > 0) {
        step_load<AK>(A, g.lda, m0, rowsA, 0, K, tid, va);
        step_load<BK>(B, g.ldb, n0, g.N, 0, K, tid, vb);
        step_store<AK>(sA[0], tid, va);
        step_store<BK>(sB[0], tid, vb);
    }
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        if (s + 1 < nk) {
            step_load<AK>(A, g.lda, m0, rowsA, (s + 1) * kGK, K, tid, va);
            step_load<BK>(B, g.ldb, n0, g.N, (s + 1) * kGK, K, tid, vb);
        }
#pragma unroll
        for (int kk = 0; kk < kGK / 16; ++kk) {
            const int ko = 16 * kk + 8 * (lane >> 5);
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][(wm * 64 + i * 32 + (lane & 31)) * kLdsRow + ko]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[cur][(wn * 64 + j * 32 + (lane & 31)) * kLdsRow + ko]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (s + 1 < nk) {
            step_store<AK>(sA[cur ^ 1], tid, va);
            step_store<BK>(sB[cur ^ 1], tid, vb);
        }
        __syncthreads();
    }
    // D[4a+b] of a 32x32 block: row 8a + 4(l/32) + b, column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int row = m0 + wm * 64 + i * 32 + 8 * a + 4 * (lane >> 5) + b;
                    if (row < Mst) {
                        float* dst = C + (long long)row * g.ldc + col;
                        const float v = acc[i][j][4 * a + b];
                        *dst = g.accumulate ? *dst + v : v;
                    }
                }
        }
}

// 128-row tiles of each expert's range: tiles[i] = (e << 16) | tile.
__global__ __launch_bounds__(64) void bwd_tiles_kernel(const int32_t* offsets, int E, int32_t* tiles,
                                                     int32_t* ntiles) {
    if (threadIdx.x != 0) return;
    int n = 0;
    for (int e = 0; e < E; ++e) {
        const int cnt = offsets[e + 1] - offsets[e];
        for (int t = 0; t * kGB < cnt; ++t) tiles[n++] = (e << 16) | t;
    }
    *ntiles = n;
}

// One wave per permuted row r (token t = src / k): Xp[r] = h[t], Dp[r] = dout[t],
// dY[r] = p dout[t] rounded once to bf16, inv[src] = r.
__global__ __launch_bounds__(256) void bwd_gather_kernel(const uint16_t* h, const uint16_t* dout,
                                                       const int32_t* perm, const float* topk_w, int R, int H, int k,
                                                       uint16_t* Xp, uint16_t* Dp, uint16_t* dY, int32_t* inv) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (r >= R) return;
    const int src = perm[r];
    const long long t = src / k;
    if (lane == 0) inv[src] = r;
    const float p = topk_w[src];
    for (int c = lane * 8; c < H; c += 64 * 8) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(h + t * H + c);
        const u32x4 d = *reinterpret_cast<const u32x4*>(dout + t * H + c);
        *reinterpret_cast<u32x4*>(Xp + (long long)r * H + c) = x;
        *reinterpret_cast<u32x4*>(Dp + (long long)r * H + c) = d;
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = f32_to_bf16_bits(p * bf16_bits_to_f32(dw[e] & 0xffffu));
            const uint32_t hi = f32_to_bf16_bits(p * bf16_bits_to_f32(dw[e] >> 16));
            o[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dY + (long long)r * H + c) = u32x4{o[0], o[1], o[2], o[3]};
    }
}

__device__ __forceinline__ float block_sum(float x, float* red) {
    x = wave_sum(x);
    x = __shfl(x, 63, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float s = 0.0f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
    return s;
}

// One workgroup per permuted row r: from g, u (recomputed) and gy = W_d^T dout,
//   a = silu(g) u,  dp = gy . a,  da = p gy,
//   dG = bf16(da u silu'(g)),  dU = bf16(da silu(g)),  ACT = bf16(a);
// dp goes to dp[src] (token-slot order).
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(const float* G, const float* U, const float* GY,
                                                       const int32_t* perm, const float* topk_w, int I,
                                                       uint16_t* dG, uint16_t* dU, uint16_t* ACT, float* dp) {
    __shared__ float red[4];
    const long long r = blockIdx.x;
    const int src = perm[r];
    const float p = topk_w[src];
    float part = 0.0f;
    for (int c = threadIdx.x * 4; c < I; c += 256 * 4) {
        const float4 g = *reinterpret_cast<const float4*>(G + r * I + c);
        const float4 u = *reinterpret_cast<const float4*>(U + r * I + c);
        const float4 gy = *reinterpret_cast<const float4*>(GY + r * I + c);
        const float gg[4] = {g.x, g.y, g.z, g.w}, uu[4] = {u.x, u.y, u.z, u.w}, yy[4] = {gy.x, gy.y, gy.z, gy.w};
        uint32_t og[2], ou[2], oa[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            uint32_t bg[2], bu[2], ba[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float z = gg[e + q];
                const float sig = 1.0f / (1.0f + __expf(-z));
                const float sl = z * sig;
                const float a = sl * uu[e + q];
                part = fmaf(yy[e + q], a, part);
                const float da = p * yy[e + q];
                bg[q] = f32_to_bf16_bits(da * uu[e + q] * (sig * (1.0f + z * (1.0f - sig))));
                bu[q] = f32_to_bf16_bits(da * sl);
                ba[q] = f32_to_bf16_bits(a);
            }
            og[e / 2] = bg[0] | (bg[1] << 16);
            ou[e / 2] = bu[0] | (bu[1] << 16);
            oa[e / 2] = ba[0] | (ba[1] << 16);
        }
        *reinterpret_cast<uint2*>(dG + r * I + c) = uint2{og[0], og[1]};
        *reinterpret_cast<uint2*>(dU + r * I + c) = uint2{ou[0], ou[1]};
        *reinterpret_cast<uint2*>(ACT + r * I + c) = uint2{oa[0], oa[1]};
    }
    const float s = block_sum(part, red);
    if (threadIdx.x == 0) dp[src] = s;
}

// One workgroup per token t:
//   ds_j = p_j (dp_j - sum_S p dp) for its k selected experts;
//   dh[t] = sum_j DA[inv[t k + j]] + sum_j ds_j W_r[idx_j]   (fp32, one rounding);
//   dsd[t, :Ep] = ds as a dense bf16 row (zeros off S), dsf[t, :E] the same in fp32.
__global__ __launch_bounds__(256) void bwd_token_kernel(const float* DA, const int32_t* inv, const int32_t* topk_idx,
                                                      const float* topk_w, const float* dp, const uint16_t* w_router,
                                                      int H, int E, int Ep, int k, uint16_t* dh, uint16_t* dsd,
                                                      float* dsf) {
    extern __shared__ float s_ds[];  // [k]
    __shared__ float red[4];
    const long long t = blockIdx.x;
    float part = 0.0f;
    for (int j = threadIdx.x; j < k; j += 256) part += topk_w[t * k + j] * dp[t * k + j];
    const float mean = block_sum(part, red);
    for (int j = threadIdx.x; j < k; j += 256) s_ds[j] = topk_w[t * k + j] * (dp[t * k + j] - mean);
    for (int e = threadIdx.x; e < Ep; e += 256) dsd[t * Ep + e] = 0;
    for (int e = threadIdx.x; e < E; e += 256) dsf[t * E + e] = 0.0f;
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += 256) {
        const int e = topk_idx[t * k + j];
        dsd[t * Ep + e] = (uint16_t)f32_to_bf16_bits(s_ds[j]);
        dsf[t * E + e] = s_ds[j];
    }
    if (!dh) return;
    for (int c = threadIdx.x; c < H; c += 256) {
        float v = 0.0f;
        for (int j = 0; j < k; ++j) {
            v += DA[(long long)inv[t * k + j] * H + c];
            v = fmaf(s_ds[j], bf16_bits_to_f32(w_router[(long long)topk_idx[t * k + j] * H + c]), v);
        }
        dh[t * H + c] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// db[e] = sum_t dsf[t, e]: one workgroup per expert.
__global__ __launch_bounds__(256) void bwd_bias_kernel(const float* dsf, int T, int E, float* db) {
    __shared__ float red[4];
    const int e = blockIdx.x;
    float part = 0.0f;
    for (int t = threadIdx.x; t < T; t += 256) part += dsf[(long long)t * E + e];
    const float s = block_sum(part, red);
    if (threadIdx.x == 0) db[e] = s;
}

template <bool AK, bool BK>
hipError_t gemm(const BwdGemm& g, int gx, int gy, int gz, hipStream_t stream) {
    if (gx <= 0 || gy <= 0 || gz <= 0) return hipSuccess;
    bwd_gemm_kernel<AK, BK><<<dim3(gx, gy, gz), 256, 0, stream>>>(g);
    return hipGetLastError();
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace

int bwd_max_tiles(int T, int k, int E) { return cdiv(T * k, kGB) + E; }

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k, R = T * k, Ep = (E + 7) & ~7;
    const int maxt = bwd_max_tiles(T, k, E);
    hipError_t e;
#define BWD_CHECK(x)                       \
    do {                                   \
        e = (x);                           \
        if (e != hipSuccess) return e;     \
    } while (0)
    bwd_tiles_kernel<<<1, 64, 0, stream>>>(a.offsets, E, a.tiles, a.ntiles);
    BWD_CHECK(hipGetLastError());
    bwd_gather_kernel<<<cdiv(R, 4), 256, 0, stream>>>(a.h, a.dout, a.perm, a.topk_w, R, H, k, a.Xp, a.Dp, a.dY,
                                                       a.inv);
    BWD_CHECK(hipGetLastError());
    // g = Xp W_g^T, u = Xp W_u^T (row groups; B = W [I, H] is K-contiguous)
    BwdGemm g{};
    g.mode = 0;
    g.offsets = a.offsets;
    g.tiles = a.tiles;
    g.ntiles = a.ntiles;
    g.A = a.Xp; g.lda = H;
    g.ldb = H; g.b_gs = (long long)I * H;
    g.ldc = I;
    g.N = I; g.K = H;
    g.B = a.w_gate; g.C = a.G;
    BWD_CHECK((gemm<true, true>(g, maxt, cdiv(I, kGB), 1, stream)));
    g.B = a.w_up; g.C = a.U;
    BWD_CHECK((gemm<true, true>(g, maxt, cdiv(I, kGB), 1, stream)));
    // gy = Dp W_d (B = W_d [H, I] is [K, N])
    g.A = a.Dp; g.B = a.w_down; g.ldb = I; g.b_gs = (long long)H * I; g.C = a.GY;
    BWD_CHECK((gemm<true, false>(g, maxt, cdiv(I, kGB), 1, stream)));
    bwd_swiglu_kernel<<<R, 256, 0, stream>>>(a.G, a.U, a.GY, a.perm, a.topk_w, I, a.dG, a.dU, a.ACT, a.dp);
    BWD_CHECK(hipGetLastError());
    if (a.dh) {
        // DA = dG W_g + dU W_u (B = W [I, H] is [K, N])
        g.A = a.dG; g.lda = I; g.B = a.w_gate; g.ldb = H; g.b_gs = (long long)I * H; g.C = a.DA; g.ldc = H;
        g.N = H; g.K = I; g.accumulate = 0;
        BWD_CHECK((gemm<true, false>(g, maxt, cdiv(H, kGB), 1, stream)));
        g.A = a.dU; g.B = a.w_up; g.accumulate = 1;
        BWD_CHECK((gemm<true, false>(g, maxt, cdiv(H, kGB), 1, stream)));
    }
    bwd_token_kernel<<<T, 256, k * sizeof(float), stream>>>(a.DA, a.inv, a.topk_idx, a.topk_w, a.dp, a.w_router, H, E,
                                                           Ep, k, a.dh, a.dsd, a.dsf);
    BWD_CHECK(hipGetLastError());
    if (a.db_router) {
        bwd_bias_kernel<<<E, 256, 0, stream>>>(a.dsf, T, E, a.db_router);
        BWD_CHECK(hipGetLastError());
    }
    if (a.dw_router) {  // dW_r = dsd^T h: A = dsd [T, Ep] as [K, M], B = h [T, H] as [K, N]
        BwdGemm r{};
        r.mode = 2;
        r.A = a.dsd; r.lda = Ep; r.Ma = Ep; r.M = E;
        r.B = a.h; r.ldb = H; r.N = H; r.K = T;
        r.C = a.dw_router; r.ldc = H;
        BWD_CHECK((gemm<false, false>(r, cdiv(E, kGB), cdiv(H, kGB), 1, stream)));
    }
    // weight gradients, K groups over each expert's rows (frozen experts skipped)
    BwdGemm w{};
    w.mode = 1;
    w.offsets = a.offsets;
    w.trainable = a.trainable;
    if (a.dw_down) {  // dW_d[e] = dY^T ACT: [H, I]
        w.A = a.dY; w.lda = H; w.Ma = H; w.M = H;
        w.B = a.ACT; w.ldb = I; w.N = I;
        w.C = a.dw_down; w.ldc = I; w.c_gs = (long long)H * I;
        BWD_CHECK((gemm<false, false>(w, cdiv(H, kGB), cdiv(I, kGB), E, stream)));
    }
    w.Ma = I; w.M = I; w.lda = I;
    w.B = a.Xp; w.ldb = H; w.N = H; w.ldc = H; w.c_gs = (long long)I * H;
    if (a.dw_gate) {  // dW_g[e] = dG^T Xp: [I, H]
        w.A = a.dG; w.C = a.dw_gate;
        BWD_CHECK((gemm<false, false>(w, cdiv(I, kGB), cdiv(H, kGB), E, stream)));
    }
    if (a.dw_up) {
        w.A = a.dU; w.C = a.dw_up;
        BWD_CHECK((gemm<false, false>(w, cdiv(I, kGB), cdiv(H, kGB), E, stream)));
    }
#undef BWD_CHECK
    return hipSuccess;
}

}  // namespace moe
