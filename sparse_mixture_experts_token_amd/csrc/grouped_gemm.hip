// Stages 2 and 3 of the layer for fp32 activations and weights (the generic
// path; bf16 activations use gemm_bf16.hip and gemm_decode.hip): the
// experts' SwiGLU networks as two grouped GEMMs over the expert-major row tiles ("gpt-oss 20B" field guide, cutaway 03:
// SwiGLU experts; "openai/gpt-oss-20b" fixture comparison: hidden_act silu).
//
//   gate/up:  act[r, :] = silu(x_r W_gate[e]^T) * (x_r W_up[e]^T)
//             x_r = h[token of row r]  (rows gathered through perm_src)
//   down:     y[a, :]   = p_a * (act[r, :] W_down[e]^T),  a = perm_src[r]
//
// Both are tiles of BM rows (one expert) x BN output columns, K swept in BK
// steps through double-buffered LDS; four waves in a 2x2 layout, each owning a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles with fp32 accumulators.  The
// gate/up kernel keeps the gate and up tiles of the same columns in one
// workgroup so the SiLU*up product is formed in registers.
//
// Weights are [out, in] row-major (K contiguous) for fp32/bf16, or MXFP4
// (packed E2M1 pairs + one E8M0 byte per 32 K-elements), decoded exactly to
// bf16 while the B tile is staged into LDS.
//
// Work order: blocks are remapped so that each XCD (8 per device, blocks
// dealt round-robin) gets a contiguous range of the tile space, and within
// that range a group of GROUP_M row tiles is swept across all column tiles
// before moving on: a group's activation rows stay in that XCD's L2 while each
// weight tile is shared by the group's row tiles.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

template <int MODE, typename TA, int WDT, int BM, int BN>
struct GemmCfg {
    static constexpr bool kF32 = sizeof(TA) == 4;           // fp32 path (fp32 MFMA)
    static constexpr int NMAT = MODE == 0 ? 2 : 1;          // gate+up or down
    static constexpr int BK = kF32 ? 32 : 64;               // 128 bytes of K per row
    static constexpr int PITCH = BK + (kF32 ? 4 : 8);       // +16 bytes per LDS row
    static constexpr int KSTEP = kF32 ? 2 : 16;             // K per 32x32 MFMA
    static constexpr int WTM = BM / 2, WTN = BN / 2;        // wave tile
    static constexpr int MB = WTM / 32, NB = WTN / 32;      // 32x32 blocks per wave
    static constexpr int A_CHUNKS = BM * 8 / kThreads;      // 16-byte chunks per thread
    static constexpr int B_ROWS = NMAT * BN;
    static constexpr int B_CHUNKS = WDT == DT_MXFP4 ? B_ROWS * 2 / kThreads : B_ROWS * 8 / kThreads;
    static constexpr size_t SMEM = (size_t)2 * (BM + B_ROWS) * PITCH * sizeof(TA);
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "chunks");
    static_assert(!(WDT == DT_MXFP4 && kF32), "MXFP4 weights need bf16 activations");
};

struct Args {
    const void* a_src;  // h (gate/up) or act (down)
    const void* w0;     // gate or down
    const void* w1;     // up
    const uint8_t* s0;
    const uint8_t* s1;
    const int32_t* perm_src;
    const float* topk_w;
    const Tile* tiles;
    const int32_t* n_tiles;
    void* out;          // act (gate/up) or y (down)
    int max_tiles, n_ntiles;
    int K, N, k, ldo;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int MODE, typename TA, int WDT, int BM, int BN>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(Args args) {
    using C = GemmCfg<MODE, TA, WDT, BM, BN>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    TA* sA = reinterpret_cast<TA*>(smem_raw);                       // [2][BM][PITCH]
    TA* sB = sA + 2 * BM * C::PITCH;                                 // [2][B_ROWS][PITCH]

    // ---- XCD-aware remap of the linear block id, then group-M swizzle ----
    const int nblocks = args.max_tiles * args.n_ntiles;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    const int q = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (q >= nblocks) return;
    const int group_span = kGroupM * args.n_ntiles;
    const int g = q / group_span;
    const int in_g = q % group_span;
    const int g_rows = min(kGroupM, args.max_tiles - g * kGroupM);
    const int mt = g * kGroupM + in_g % g_rows;
    const int nt = in_g / g_rows;
    if (mt >= args.n_tiles[0]) return;
    const Tile tile = args.tiles[mt];
    const int e = tile.expert;
    const int row0 = tile.row_start;
    const int rows = tile.rows;
    const int n0 = nt * BN;

    const int K = args.K, N = args.N;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- A row sources ----
    const TA* a_ptr[C::A_CHUNKS];
    const int a_cc = tid & 7;  // 16-byte chunk within the 128-byte K slice
#pragma unroll
    for (int j = 0; j < C::A_CHUNKS; ++j) {
        int r = (tid >> 3) + 32 * j;
        int rr = r < rows ? r : 0;
        size_t src_row;
        if constexpr (MODE == 0) {
            src_row = (size_t)(args.perm_src[row0 + rr] / args.k);
        } else {
            src_row = (size_t)(row0 + rr);
        }
        a_ptr[j] = reinterpret_cast<const TA*>(args.a_src) + src_row * K + a_cc * (16 / sizeof(TA));
    }

    // ---- B row sources ----
    constexpr int B_PER_ROW = WDT == DT_MXFP4 ? 2 : 8;  // chunks per row per K step
    const unsigned char* b_ptr[C::B_CHUNKS];
    const uint8_t* s_ptr[C::B_CHUNKS];
#pragma unroll
    for (int j = 0; j < C::B_CHUNKS; ++j) {
        int c = tid + kThreads * j;
        int br = c / B_PER_ROW;          // row in the B tile (0 .. NMAT*BN)
        int cc = c % B_PER_ROW;
        int mat = br / BN;
        int n = min(n0 + (br % BN), N - 1);
        const void* wbase = mat == 0 ? args.w0 : args.w1;
        size_t grow = (size_t)e * N + n;
        if constexpr (WDT == DT_MXFP4) {
            b_ptr[j] = reinterpret_cast<const unsigned char*>(wbase) + grow * (K / 2) + cc * 16;
            s_ptr[j] = (mat == 0 ? args.s0 : args.s1) + grow * (K / 32) + cc;
        } else if constexpr (WDT == DT_BF16) {
            b_ptr[j] = reinterpret_cast<const unsigned char*>(wbase) + (grow * K) * 2 + cc * 16;
            s_ptr[j] = nullptr;
        } else {
            b_ptr[j] = reinterpret_cast<const unsigned char*>(wbase) + (grow * K) * 4 + cc * 16;
            s_ptr[j] = nullptr;
        }
    }

    uint4 ra[C::A_CHUNKS];
    uint4 rb[C::B_CHUNKS];
    uint32_t rs[C::B_CHUNKS];

    auto load_global = [&](int k0) {
#pragma unroll
        for (int j = 0; j < C::A_CHUNKS; ++j) ra[j] = *reinterpret_cast<const uint4*>(a_ptr[j] + k0);
#pragma unroll
        for (int j = 0; j < C::B_CHUNKS; ++j) {
            if constexpr (WDT == DT_MXFP4) {
                rb[j] = *reinterpret_cast<const uint4*>(b_ptr[j] + k0 / 2);
                rs[j] = s_ptr[j][k0 / 32];
            } else {
                rb[j] = *reinterpret_cast<const uint4*>(b_ptr[j] + (size_t)k0 * sizeof(TA));
            }
        }
    };

    auto store_lds = [&](int buf) {
        TA* a = sA + buf * BM * C::PITCH;
#pragma unroll
        for (int j = 0; j < C::A_CHUNKS; ++j) {
            int r = (tid >> 3) + 32 * j;
            *reinterpret_cast<uint4*>(a + r * C::PITCH + a_cc * (16 / sizeof(TA))) = ra[j];
        }
        TA* b = sB + buf * C::B_ROWS * C::PITCH;
#pragma unroll
        for (int j = 0; j < C::B_CHUNKS; ++j) {
            int c = tid + kThreads * j;
            int br = c / B_PER_ROW;
            int cc = c % B_PER_ROW;
            if constexpr (WDT == DT_MXFP4) {
                uint32_t d[16];
                decode_mxfp4_32(rb[j], rs[j], d);
                uint4* dst = reinterpret_cast<uint4*>(b + br * C::PITCH + cc * 32);
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = uint4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
            } else {
                *reinterpret_cast<uint4*>(b + br * C::PITCH + cc * (16 / sizeof(TA))) = rb[j];
            }
        }
    };

    f32x16 acc[C::NMAT][C::MB][C::NB];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
            for (int j = 0; j < C::NB; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][i][j][v] = 0.f;

    const int nk = K / C::BK;
    load_global(0);
    store_lds(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global((kt + 1) * C::BK);
        const TA* a = sA + buf * BM * C::PITCH;
        const TA* b = sB + buf * C::B_ROWS * C::PITCH;
#pragma unroll
        for (int ks = 0; ks < C::BK / C::KSTEP; ++ks) {
            if constexpr (C::kF32) {
                float af[C::MB];
                float bfr[C::NMAT][C::NB];
                const int kk = ks * C::KSTEP + (lane >> 5);
#pragma unroll
                for (int i = 0; i < C::MB; ++i) af[i] = a[(wm * C::WTM + i * 32 + (lane & 31)) * C::PITCH + kk];
#pragma unroll
                for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                    for (int j = 0; j < C::NB; ++j)
                        bfr[m][j] = b[(m * BN + wn * C::WTN + j * 32 + (lane & 31)) * C::PITCH + kk];
#pragma unroll
                for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                    for (int i = 0; i < C::MB; ++i)
#pragma unroll
                        for (int j = 0; j < C::NB; ++j) acc[m][i][j] = mfma32(af[i], bfr[m][j], acc[m][i][j]);
            } else {
                bf16x8 af[C::MB];
                bf16x8 bfr[C::NMAT][C::NB];
                const int kk = ks * C::KSTEP + (lane >> 5) * 8;
#pragma unroll
                for (int i = 0; i < C::MB; ++i)
                    af[i] = *reinterpret_cast<const bf16x8*>(a + (wm * C::WTM + i * 32 + (lane & 31)) * C::PITCH + kk);
#pragma unroll
                for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                    for (int j = 0; j < C::NB; ++j)
                        bfr[m][j] = *reinterpret_cast<const bf16x8*>(
                            b + (m * BN + wn * C::WTN + j * 32 + (lane & 31)) * C::PITCH + kk);
#pragma unroll
                for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                    for (int i = 0; i < C::MB; ++i)
#pragma unroll
                        for (int j = 0; j < C::NB; ++j) acc[m][i][j] = mfma32(af[i], bfr[m][j], acc[m][i][j]);
            }
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < C::MB; ++i) {
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
            const int n = n0 + wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < rows && n < N) {
                    if constexpr (MODE == 0) {
                        const float val = silu_f(acc[0][i][j][v]) * acc[1][i][j][v];
                        const size_t o = (size_t)(row0 + m) * args.ldo + n;
                        if constexpr (C::kF32) {
                            reinterpret_cast<float*>(args.out)[o] = val;
                        } else {
                            reinterpret_cast<uint16_t*>(args.out)[o] = (uint16_t)f32_to_bf16_bits(val);
                        }
                    } else {
                        const int asg = args.perm_src[row0 + m];
                        const float val = acc[0][i][j][v] * args.topk_w[asg];
                        reinterpret_cast<float*>(args.out)[(size_t)asg * args.ldo + n] = val;
                    }
                }
            }
        }
    }
}

template <int MODE, typename TA, int WDT, int BM, int BN>
hipError_t launch_on(const Args& a, hipStream_t stream) {
    using C = GemmCfg<MODE, TA, WDT, BM, BN>;
    auto kern = grouped_gemm_kernel<MODE, TA, WDT, BM, BN>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::SMEM);
    if (attr != hipSuccess) return attr;
    const int nblocks = a.max_tiles * a.n_ntiles;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    kern<<<per_xcd * kXcds, kThreads, C::SMEM, stream>>>(a);
    return hipGetLastError();
}

constexpr int kBM = 128;
constexpr int kBNGateUp = 128;
constexpr int kBNDown = 128;

Args make_args(const GemmProblem& p, int mode) {
    Args a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.tiles = p.tiles;
    a.n_tiles = p.n_tiles;
    a.max_tiles = p.max_tiles;
    a.k = p.k;
    if (mode == 0) {
        a.a_src = p.h;
        a.w0 = p.w_gate;
        a.w1 = p.w_up;
        a.s0 = p.s_gate;
        a.s1 = p.s_up;
        a.out = p.act;
        a.K = p.H;
        a.N = p.I;
        a.ldo = p.I;
        a.n_ntiles = (p.I + kBNGateUp - 1) / kBNGateUp;
    } else {
        a.a_src = p.act;
        a.w0 = p.w_down;
        a.w1 = nullptr;
        a.s0 = p.s_down;
        a.s1 = nullptr;
        a.out = p.y;
        a.K = p.I;
        a.N = p.H;
        a.ldo = p.H;
        a.n_ntiles = (p.H + kBNDown - 1) / kBNDown;
    }
    return a;
}

}  // namespace


int gemm_block_m(int act_dtype, int expert_dtype, int, int, int) {
    if (act_dtype == DT_F32) return kBM;
    (void)expert_dtype;
    return bf16_block_m();
}

// fp32 activations take the generic kernel; bf16 activations the decode kernels
// (few rows per expert) or the prefill ones (gemm_bf16.hip, bf16 or MXFP4
// weights).
hipError_t launch_gateup(const GemmProblem& p, hipStream_t stream) {
    if (p.act_dtype == DT_F32) return launch_on<0, float, DT_F32, kBM, kBNGateUp>(make_args(p, 0), stream);
    if (p.decode) return launch_gateup_decode(p, stream);
    return launch_gateup_bf16w(p, stream);
}

hipError_t launch_down(const GemmProblem& p, hipStream_t stream) {
    if (p.act_dtype == DT_F32) return launch_on<1, float, DT_F32, kBM, kBNDown>(make_args(p, 1), stream);
    if (p.decode) return launch_down_decode(p, stream);
    return launch_down_bf16w(p, stream);
}

}  // namespace moe
