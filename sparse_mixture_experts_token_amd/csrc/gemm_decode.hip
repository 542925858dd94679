// Stages 2 and 3 for decode-sized batches (few rows per expert): the same two
// grouped products as the prefill kernels,
//
//   act[r]  = silu(W_gate[e] . x_r) * (W_up[e] . x_r)       x_r = h[perm_src[r] / k]
//   Y[a]    = p_a * (W_down[e] . act[r])                     a = perm_src[r]
//
// ("gpt-oss-40b-64a8-init" page, section 2, Proof; "gpt-oss 20B" field guide,
// cutaway 03: SwiGLU experts), organised for the case where they are bound by
// reading the experts' weights once from HBM rather than by the matrix cores.
//
// One wave computes one (row tile of at most 16 rows of one expert) x (16
// weight rows) block with 16x16x32 bf16 MFMAs: the weights are the A operand,
// streamed from HBM straight into registers (no LDS, no barriers), the
// tile's activation rows are the B operand (small, L2-resident).  Lanes of
// rows past the tile's end read at an offset beyond the buffer, which returns
// zero without touching memory.
//
// K is walked 128 at a time, as four 32-deep MFMA steps j.  For bf16 weights
// each load instruction takes the native MFMA order (lane (row l%16, quarter
// q = l/16) reads K elements 128g + 32j + 8q .. +7), so one instruction reads
// 64 contiguous bytes of each of 16 weight rows.  For MXFP4 a lane reads the
// 32 codes [128g + 32q, 128g + 32q + 32) of its row in one 16-byte load plus
// exactly one E8M0 scale, and feeds them to the four steps as elements
// 8j..8j+7; a contraction is unchanged by a permutation of K applied to both
// operands, so the activation operand is read in the same permuted order.
//
// Each wave owns two 16-row weight panels (32 weight rows), sharing every
// activation fragment between them (and between gate and up), and the down
// kernel issues the loads of two K steps before their MFMAs: together this
// keeps enough bytes in flight per CU for HBM while every work item of a
// decode-sized batch is resident at once.  Consecutive waves take consecutive
// panels of the same row tile, so a workgroup streams one contiguous weight
// region and shares the tile's activation rows in L1.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kDecWaves = 4;           // waves per workgroup (independent)
constexpr int kDecRows = 16;           // rows per tile (MFMA N)
constexpr int kPanels = 2;             // 16-row weight panels per wave
constexpr int kDecCols = 16 * kPanels; // weight rows per wave
constexpr uint32_t kOob = 0x7ffffff0u; // byte offset past every buffer used here (all < 2^30 bytes)

struct DArgs {
    const void* a_src;  // bf16 rows of length K: h (gate/up) or act (down)
    uint32_t a_bytes;
    const void* w0;     // this stage's weights, [E][N][K] (bf16) or [E][N][K/2] (MXFP4 codes)
    const void* w1;     // up weights (gate/up only)
    const uint8_t* s0;  // MXFP4 scales [E][N][K/32]
    const uint8_t* s1;
    const int32_t* perm_src;
    const float* topk_w;
    const Tile* tiles;
    const int32_t* n_tiles;
    void* out;          // act [T*k][N] bf16 (gate/up) or Y [T*k][N] f32 (down)
    int K, N, k, n_cb;  // n_cb = N / 32
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }

// Raw weight data of one 128-wide K step for this lane (decoded at use).
template <int WDT>
struct WRaw {
    u32x4 v[4];
};
template <>
struct WRaw<DT_MXFP4> {
    u32x4 q;
    uint32_t scale;
};

template <int WDT>
__device__ __forceinline__ void load_w(buf_rsrc w, buf_rsrc s, uint32_t n, uint32_t K, uint32_t g, uint32_t qd,
                                       WRaw<WDT>& o) {
    if constexpr (WDT == DT_MXFP4) {
        const uint32_t kq = g * 128 + qd * 32;
        const bool kv = kq < K;
        o.q = buf_load16(w, kv ? n * (K / 2) + kq / 2 : kOob, 0);
        o.scale = buf_load1(s, kv ? n * (K / 32) + kq / 32 : kOob, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t kk = g * 128 + 32 * j + 8 * qd;
            o.v[j] = buf_load16(w, kk < K ? (n * K + kk) * 2u : kOob, 0);
        }
    }
}

template <int WDT>
__device__ __forceinline__ void w_frags(const WRaw<WDT>& o, bf16x8 (&f)[4]) {
    if constexpr (WDT == DT_MXFP4) {
        uint32_t d[16];
        decode_mxfp4_32(o.q, o.scale, d);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f[j] = __builtin_bit_cast(bf16x8, u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]});
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __builtin_bit_cast(bf16x8, o.v[j]);
    }
}

// Activation fragments of one K step, in the K order of the weights.
template <int WDT>
__device__ __forceinline__ void load_b(buf_rsrc b, uint32_t b_base, bool has_row, uint32_t K, uint32_t g, uint32_t qd,
                                       u32x4 (&f)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t kk = WDT == DT_MXFP4 ? g * 128 + 32 * qd + 8 * j : g * 128 + 32 * j + 8 * qd;
        f[j] = buf_load16(b, (has_row && kk < K) ? b_base + kk * 2u : kOob, 0);
    }
}

template <int MODE, int WDT>
__global__ __launch_bounds__(kDecWaves * 64) void decode_gemm_kernel(DArgs a) {
    constexpr int G = MODE == 0 ? 1 : 2;  // K steps whose loads are issued together
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = blockIdx.x * kDecWaves + wave;
    const int mt = q / a.n_cb, cb = q % a.n_cb;
    if (mt >= a.n_tiles[0]) return;  // wave-uniform; this kernel has no barriers
    const Tile tile = a.tiles[mt];
    const int e = tile.expert, row0 = tile.row_start, rows = tile.rows;
    const uint32_t K = (uint32_t)a.K, N = (uint32_t)a.N;
    const int r = lane & 15;
    const uint32_t qd = (uint32_t)(lane >> 4);

    // activation operand: this lane's row, or none (reads past the buffer)
    const bool has_row = r < rows;
    uint32_t b_base = 0;
    if (has_row) {
        const int src = MODE == 0 ? a.perm_src[row0 + r] / a.k : row0 + r;
        b_base = (uint32_t)src * K * 2u;
    }
    const buf_rsrc bsrc = make_rsrc(a.a_src, a.a_bytes);

    // weight operand: rows n[p] of expert e
    uint32_t n[kPanels];
#pragma unroll
    for (int p = 0; p < kPanels; ++p) n[p] = (uint32_t)(cb * kDecCols + p * 16 + r);
    buf_rsrc w0, w1, s0, s1;
    if constexpr (WDT == DT_MXFP4) {
        const uint32_t wb = N * K / 2, sb = N * K / 32;
        w0 = make_rsrc((const unsigned char*)a.w0 + (size_t)e * wb, wb);
        s0 = make_rsrc(a.s0 + (size_t)e * sb, sb);
        w1 = MODE == 0 ? make_rsrc((const unsigned char*)a.w1 + (size_t)e * wb, wb) : w0;
        s1 = MODE == 0 ? make_rsrc(a.s1 + (size_t)e * sb, sb) : s0;
    } else {
        const uint32_t wb = N * K * 2;
        w0 = make_rsrc((const unsigned char*)a.w0 + (size_t)e * wb, wb);
        w1 = MODE == 0 ? make_rsrc((const unsigned char*)a.w1 + (size_t)e * wb, wb) : w0;
        s0 = s1 = w0;
    }

    f32x4 acc0[kPanels], acc1[kPanels];
#pragma unroll
    for (int p = 0; p < kPanels; ++p) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t ng = (K + 127) / 128;
    for (uint32_t g0 = 0; g0 < ng; g0 += G) {
        WRaw<WDT> ra[G][kPanels], ru[G][kPanels];
        u32x4 fb[G][4];
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const uint32_t g = g0 + gg;  // past the end: every offset is beyond K, so all zero
#pragma unroll
            for (int p = 0; p < kPanels; ++p) {
                load_w<WDT>(w0, s0, n[p], K, g, qd, ra[gg][p]);
                if constexpr (MODE == 0) load_w<WDT>(w1, s1, n[p], K, g, qd, ru[gg][p]);
            }
            load_b<WDT>(bsrc, b_base, has_row, K, g, qd, fb[gg]);
        }
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
#pragma unroll
            for (int p = 0; p < kPanels; ++p) {
                bf16x8 fa[4];
                w_frags<WDT>(ra[gg][p], fa);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc0[p] = mfma16(fa[j], __builtin_bit_cast(bf16x8, fb[gg][j]), acc0[p]);
                if constexpr (MODE == 0) {
                    bf16x8 fu[4];
                    w_frags<WDT>(ru[gg][p], fu);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc1[p] = mfma16(fu[j], __builtin_bit_cast(bf16x8, fb[gg][j]), acc1[p]);
                }
            }
        }
    }

    // D: lane l holds weight rows 4(l/16)+i (i = 0..3) of the panel, for row l%16 of the tile
    if (!has_row) return;
    if constexpr (MODE == 0) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (size_t)(row0 + r) * N;
#pragma unroll
        for (int p = 0; p < kPanels; ++p) {
            const uint32_t n0 = (uint32_t)(cb * kDecCols + p * 16) + 4 * qd;
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16_bits(silu_f(acc0[p][i]) * acc1[p][i]);
            *reinterpret_cast<uint2*>(orow + n0) = uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
        }
    } else {
        const int asg = a.perm_src[row0 + r];
        const float pw = a.topk_w[asg];
        float* orow = reinterpret_cast<float*>(a.out) + (size_t)asg * N;
#pragma unroll
        for (int p = 0; p < kPanels; ++p) {
            const uint32_t n0 = (uint32_t)(cb * kDecCols + p * 16) + 4 * qd;
            *reinterpret_cast<float4*>(orow + n0) =
                float4{acc0[p][0] * pw, acc0[p][1] * pw, acc0[p][2] * pw, acc0[p][3] * pw};
        }
    }
}

DArgs make_dargs(const GemmProblem& p, int mode) {
    DArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.tiles = p.tiles;
    a.n_tiles = p.n_tiles;
    a.k = p.k;
    if (mode == 0) {
        a.a_src = p.h;
        a.a_bytes = (uint32_t)((size_t)p.T * p.H * 2);
        a.w0 = p.w_gate;
        a.w1 = p.w_up;
        a.s0 = p.s_gate;
        a.s1 = p.s_up;
        a.out = p.act;
        a.K = p.H;
        a.N = p.I;
    } else {
        a.a_src = p.act;
        a.a_bytes = (uint32_t)((size_t)p.T * p.k * p.I * 2);
        a.w0 = p.w_down;
        a.s0 = p.s_down;
        a.out = p.y;
        a.K = p.I;
        a.N = p.H;
    }
    a.n_cb = a.N / kDecCols;  // N is a multiple of 64
    return a;
}

template <int MODE, int WDT>
hipError_t launch_dec(const GemmProblem& p, hipStream_t stream) {
    const DArgs a = make_dargs(p, MODE);
    const size_t waves = (size_t)p.max_tiles * a.n_cb;
    const int blocks = (int)((waves + kDecWaves - 1) / kDecWaves);
    decode_gemm_kernel<MODE, WDT><<<blocks, kDecWaves * 64, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

// Decode kernels serve bf16 activations when the average expert gets at most
// one 16-row tile and every operand buffer stays below 2^30 bytes.
bool decode_path(int act_dtype, int T, int H, int I, int E, int k) {
    if (act_dtype != DT_BF16) return false;
    const int64_t rows = (int64_t)T * k;
    if (rows > (int64_t)kDecRows * E) return false;
    const int64_t lim = int64_t(1) << 30;
    return (int64_t)T * H * 2 < lim && rows * I * 2 < lim && (int64_t)H * I * 2 < lim;
}

int decode_block_m() { return kDecRows; }

hipError_t launch_gateup_decode(const GemmProblem& p, hipStream_t stream) {
    return p.expert_dtype == DT_MXFP4 ? launch_dec<0, DT_MXFP4>(p, stream) : launch_dec<0, DT_BF16>(p, stream);
}

hipError_t launch_down_decode(const GemmProblem& p, hipStream_t stream) {
    return p.expert_dtype == DT_MXFP4 ? launch_dec<1, DT_MXFP4>(p, stream) : launch_dec<1, DT_BF16>(p, stream);
}

}  // namespace moe
