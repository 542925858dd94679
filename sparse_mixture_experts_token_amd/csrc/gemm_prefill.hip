// Stages 2 and 3 for bf16 activations (bf16 or MXFP4 expert weights): the
// experts' SwiGLU networks as grouped GEMMs over expert-major row tiles
// ("gpt-oss 20B" field guide, cutaway 03: SwiGLU experts, weighted sum;
// "openai/gpt-oss-20b" fixture comparison: hidden_act silu).
//
//   gate/up:  act[r, :] = silu(x_r W_gate[e]^T) * (x_r W_up[e]^T),  x_r = h[token of row r]
//   down:     y[a, :]   = p_a * (act[r, :] W_down[e]^T),            a = perm_src[r]
//
// Workgroup tile: BM = 128 rows of one expert x BN weight rows (per matrix),
// K swept in steps of 64 through two LDS stages.  The four waves split N
// (1 x 4): every wave owns all 128 rows and BN/4 columns of each matrix, as
// 16x16x32 bf16 MFMA tiles with fp32 accumulators (gate/up: 8 x 3 tiles of
// gate and of up = 192 accumulators; down: 8 x 5 tiles = 160).  BN = 192
// (gate/up) and 320 (down) divide 2880 exactly.
//
// LDS rows are 128 bytes (64 bf16 of K); the 16-byte chunk c of row r is
// stored at chunk c ^ (r & 7) ^ ((r >> 3) & 1).  Fragment reads (16 rows, one
// chunk) then hit distinct banks whether the LDS serves 8 lanes per cycle
// (rows r..r+7 take all 8 chunk slots) or 16 (rows r and r+8 differ too), and
// the staging writes (whole rows) are conflict-free as well.
//
// MXFP4 weights are decoded exactly to bf16 while being staged into LDS.
// Row tiles shorter than 128 rows run only the first 4, 2 or 1 16-row blocks
// when the rest are empty (separate branch-free loop instantiations).
//
// Block order: each XCD (blocks are dealt round-robin to 8) gets a contiguous
// range of the (row tile, column tile) space; inside it, GROUP_M row tiles are
// swept across all column tiles, so a weight tile is fetched once per group
// and the group's activation rows stay in that XCD's L2.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;
constexpr int kBK = 64;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
constexpr int kBNGateUp = 192;
constexpr int kBNDown = 320;

struct PArgs {
    const uint16_t* a_src;  // h (gate/up) or act (down), bf16
    const void* w0;         // gate or down
    const void* w1;         // up
    const uint8_t* s0;
    const uint8_t* s1;
    const int32_t* perm_src;
    const float* topk_w;
    const Tile* tiles;
    const int32_t* n_tiles;
    void* out;
    uint32_t a_bytes;       // size of the activation buffer
    int max_tiles, n_ntiles;
    int K, N, k;
};

__device__ __forceinline__ int swz(int row, int chunk) {
    return (row << 7) + (((chunk ^ row ^ (row >> 3)) & 7) << 4);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int MODE, int WDT, int BN>
struct PCfg {
    static constexpr int NMAT = MODE == 0 ? 2 : 1;
    static constexpr int WN = BN / 4;             // columns per wave per matrix
    static constexpr int NBW = WN / 16;           // 16-col blocks per wave per matrix
    static constexpr int MBW = kBM / 16;          // 16-row blocks
    static constexpr int BROWS = NMAT * BN;       // weight rows per stage
    static constexpr int A_CH = kBM * 8 / kThreads;                 // 16B chunks of A per thread
    static constexpr int PER_ROW = WDT == DT_MXFP4 ? 2 : 8;         // 16B chunks per weight row per stage
    static constexpr int M_CH_TOTAL = BN * PER_ROW;                 // chunks of one matrix per stage
    static constexpr int M_CH = (M_CH_TOTAL + kThreads - 1) / kThreads;  // per thread per matrix
    static constexpr int B_CH = NMAT * M_CH;
    static constexpr int STAGE = (kBM + BROWS) * 128;               // bytes per LDS stage
    static constexpr size_t SMEM = 2 * (size_t)STAGE;
    static_assert(BN % 64 == 0, "BN");
};

// Chunk j of a thread belongs to matrix j / M_CH (uniform across the
// workgroup, so the weight base stays scalar) and is chunk
// tid + 256 * (j % M_CH) of that matrix's stage tile.
template <class C>
__device__ __forceinline__ bool chunk_live(int tid, int j) {
    return C::M_CH_TOTAL % kThreads == 0 || tid + kThreads * (j % C::M_CH) < C::M_CH_TOTAL;
}

struct Srcs {
    buf_rsrc a;      // activations (h or act)
    buf_rsrc w[2];   // this expert's gate/up (or down) matrix
    buf_rsrc s[2];   // MXFP4 scales of those matrices
};

template <class C, int WDT>
__device__ __forceinline__ void load_stage(const Srcs& src, const uint32_t (&a_off)[C::A_CH],
                                           const uint32_t (&b_off)[C::B_CH], const uint32_t (&s_off)[C::B_CH],
                                           int k0, u32x4 (&ra)[C::A_CH], u32x4 (&rb)[C::B_CH],
                                           uint32_t (&rs)[C::B_CH]) {
#pragma unroll
    for (int j = 0; j < C::A_CH; ++j) ra[j] = buf_load16(src.a, a_off[j], (uint32_t)k0 * 2);
#pragma unroll
    for (int j = 0; j < C::B_CH; ++j) {
        const int m = j / C::M_CH;
        if constexpr (WDT == DT_MXFP4) {
            rb[j] = buf_load16(src.w[m], b_off[j], (uint32_t)k0 / 2);
            rs[j] = buf_load1(src.s[m], s_off[j], (uint32_t)k0 / 32);
        } else {
            rb[j] = buf_load16(src.w[m], b_off[j], (uint32_t)k0 * 2);
        }
    }
}

template <class C, int WDT, int BN>
__device__ __forceinline__ void store_stage(unsigned char* stage, int tid, const u32x4 (&ra)[C::A_CH],
                                            const u32x4 (&rb)[C::B_CH], const uint32_t (&rs)[C::B_CH]) {
    unsigned char* sbt = stage + kBM * 128;
#pragma unroll
    for (int j = 0; j < C::A_CH; ++j) {
        const int c = tid + kThreads * j;
        *reinterpret_cast<u32x4*>(stage + swz(c >> 3, c & 7)) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < C::B_CH; ++j) {
        if (!chunk_live<C>(tid, j)) continue;
        const int m = j / C::M_CH;
        const int c = tid + kThreads * (j % C::M_CH);
        if constexpr (WDT == DT_MXFP4) {
            const int r = m * BN + (c >> 1), gq = c & 1;
            uint32_t d[16];
            decode_mxfp4_32(rb[j], rs[j], d);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(sbt + swz(r, gq * 4 + i)) = u32x4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
        } else {
            *reinterpret_cast<u32x4*>(sbt + swz(m * BN + (c >> 3), c & 7)) = rb[j];
        }
    }
}

// Fragments of one 64-deep K step (both 32-wide halves) of this wave.
template <class C, int BN, int MB>
struct Frags {
    bf16x8 a[2][MB];
    bf16x8 b[2][C::NMAT][C::NBW];
};

template <class C, int BN, int MB>
__device__ __forceinline__ void read_frags(const unsigned char* stage, int wave, int lane, Frags<C, BN, MB>& f) {
    const unsigned char* sbt = stage + kBM * 128;
    const int fr = lane & 15;
    const int fq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int chunk = ks * 4 + fq;
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
                f.b[ks][m][j] = *reinterpret_cast<const bf16x8*>(sbt + swz(m * BN + wave * C::WN + j * 16 + fr, chunk));
#pragma unroll
        for (int i = 0; i < MB; ++i) f.a[ks][i] = *reinterpret_cast<const bf16x8*>(stage + swz(i * 16 + fr, chunk));
    }
}

template <class C, int BN, int MB>
__device__ __forceinline__ void mfma_frags(const Frags<C, BN, MB>& f, f32x4 (&acc)[C::NMAT][C::MBW][C::NBW]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) acc[m][i][j] = mfma16(f.a[ks][i], f.b[ks][m][j], acc[m][i][j]);
}

template <class C, int WDT, int BN, int MB>
__device__ __forceinline__ void main_loop(const Srcs& src, unsigned char* smem, int nk,
                                          const uint32_t (&a_off)[C::A_CH], const uint32_t (&b_off)[C::B_CH],
                                          const uint32_t (&s_off)[C::B_CH], u32x4 (&ra)[C::A_CH],
                                          u32x4 (&rb)[C::B_CH], uint32_t (&rs)[C::B_CH],
                                          f32x4 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // Order within a K step: this stage's fragment reads, then the next
        // stage's global loads, then the MFMAs (fences keep the compiler from
        // interleaving them, which made the fragment reads wait on the loads).
        Frags<C, BN, MB> f;
        read_frags<C, BN, MB>(smem + buf * C::STAGE, wave, lane, f);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) load_stage<C, WDT>(src, a_off, b_off, s_off, (kt + 1) * kBK, ra, rb, rs);
        __builtin_amdgcn_sched_barrier(0);
        mfma_frags<C, BN, MB>(f, acc);
        if (kt + 1 < nk) store_stage<C, WDT, BN>(smem + (buf ^ 1) * C::STAGE, tid, ra, rb, rs);
        __syncthreads();
    }
}

template <int MODE, int WDT, int BN>
__device__ __forceinline__ void gemm_body(const PArgs& args) {
    using C = PCfg<MODE, WDT, BN>;
    extern __shared__ __align__(16) unsigned char smem[];

    // ---- block -> (row tile, column tile) ----
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

    // ---- per-thread global sources: scalar bases + 32-bit offsets ----
    uint32_t a_off[C::A_CH];  // elements
#pragma unroll
    for (int j = 0; j < C::A_CH; ++j) {
        const int c = tid + kThreads * j;
        const int r = c >> 3;
        const int rr = r < rows ? r : 0;
        int src_row;
        if constexpr (MODE == 0) src_row = args.perm_src[row0 + rr] / args.k;
        else src_row = row0 + rr;
        a_off[j] = (uint32_t)(src_row * K + (c & 7) * 8) * 2u;
    }
    const size_t mat_elems = (size_t)N * K;
    Srcs src;
    src.a = make_rsrc(args.a_src, args.a_bytes);
    if constexpr (WDT == DT_MXFP4) {
        const uint32_t wbytes = (uint32_t)(mat_elems / 2), sbytes = (uint32_t)(mat_elems / 32);
        src.w[0] = make_rsrc((const unsigned char*)args.w0 + (size_t)e * wbytes, wbytes);
        src.w[1] = MODE == 0 ? make_rsrc((const unsigned char*)args.w1 + (size_t)e * wbytes, wbytes) : src.w[0];
        src.s[0] = make_rsrc(args.s0 + (size_t)e * sbytes, sbytes);
        src.s[1] = MODE == 0 ? make_rsrc(args.s1 + (size_t)e * sbytes, sbytes) : src.s[0];
    } else {
        const uint32_t wbytes = (uint32_t)(mat_elems * 2);
        src.w[0] = make_rsrc((const unsigned char*)args.w0 + (size_t)e * wbytes, wbytes);
        src.w[1] = MODE == 0 ? make_rsrc((const unsigned char*)args.w1 + (size_t)e * wbytes, wbytes) : src.w[0];
        src.s[0] = src.s[1] = src.w[0];
    }
    uint32_t b_off[C::B_CH];  // bytes: row start + chunk (bf16) or group (mxfp4) at k = 0
    uint32_t s_off[C::B_CH];  // mxfp4: scale index of the chunk's group at k = 0
#pragma unroll
    for (int j = 0; j < C::B_CH; ++j) {
        const int c = min(tid + kThreads * (j % C::M_CH), C::M_CH_TOTAL - 1);
        const int r = c / C::PER_ROW;
        const int cc = c % C::PER_ROW;
        const int n = min(n0 + r, N - 1);
        if constexpr (WDT == DT_MXFP4) {
            b_off[j] = (uint32_t)(n * (K / 2) + cc * 16);
            s_off[j] = (uint32_t)(n * (K / 32) + cc);
        } else {
            b_off[j] = (uint32_t)(n * K * 2 + cc * 16);
            s_off[j] = 0;
        }
    }

    u32x4 ra[C::A_CH];
    u32x4 rb[C::B_CH];
    uint32_t rs[C::B_CH];
    f32x4 acc[C::NMAT][C::MBW][C::NBW];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int i = 0; i < C::MBW; ++i)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kBK;
    load_stage<C, WDT>(src, a_off, b_off, s_off, 0, ra, rb, rs);
    store_stage<C, WDT, BN>(smem, tid, ra, rb, rs);
    __syncthreads();
    // Only the 16-row blocks that hold rows get MFMAs: 8, 4, 2 or 1 of them.
    const int live = (rows + 15) >> 4;
    if (live > 4)
        main_loop<C, WDT, BN, 8>(src, smem, nk, a_off, b_off, s_off, ra, rb, rs, acc);
    else if (live > 2)
        main_loop<C, WDT, BN, 4>(src, smem, nk, a_off, b_off, s_off, ra, rb, rs, acc);
    else if (live > 1)
        main_loop<C, WDT, BN, 2>(src, smem, nk, a_off, b_off, s_off, ra, rb, rs, acc);
    else
        main_loop<C, WDT, BN, 1>(src, smem, nk, a_off, b_off, s_off, ra, rb, rs, acc);

    const int fr = lane & 15;
    const int fq = lane >> 4;
    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < C::MBW; ++i) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = i * 16 + fq * 4 + jj;
            if (r >= rows) continue;
            if constexpr (MODE == 0) {
                uint16_t* orow = reinterpret_cast<uint16_t*>(args.out) + (size_t)(row0 + r) * N;
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int n = n0 + wave * C::WN + j * 16 + fr;
                    if (n < N) orow[n] = (uint16_t)f32_to_bf16_bits(silu_f(acc[0][i][j][jj]) * acc[1][i][j][jj]);
                }
            } else {
                const int asg = args.perm_src[row0 + r];
                const float p = args.topk_w[asg];
                float* orow = reinterpret_cast<float*>(args.out) + (size_t)asg * N;
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int n = n0 + wave * C::WN + j * 16 + fr;
                    if (n < N) orow[n] = acc[0][i][j][jj] * p;
                }
            }
        }
    }
}

template <int WDT>
__global__ __launch_bounds__(kThreads, 1) void gateup_gemm_kernel(PArgs args) {
    gemm_body<0, WDT, kBNGateUp>(args);
}

template <int WDT>
__global__ __launch_bounds__(kThreads, 1) void down_gemm_kernel(PArgs args) {
    gemm_body<1, WDT, kBNDown>(args);
}

template <typename Kern>
hipError_t launch_k(Kern kern, size_t smem, const PArgs& a, hipStream_t stream) {
    const int nblocks = a.max_tiles * a.n_ntiles;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    kern<<<per_xcd * kXcds, kThreads, smem, stream>>>(a);
    return hipGetLastError();
}

PArgs make_pargs(const GemmProblem& p, int mode, int BN) {
    PArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.tiles = p.tiles;
    a.n_tiles = p.n_tiles;
    a.max_tiles = p.max_tiles;
    a.k = p.k;
    if (mode == 0) {
        a.a_src = (const uint16_t*)p.h;
        a.a_bytes = (uint32_t)((size_t)p.T * p.H * 2);
        a.w0 = p.w_gate;
        a.w1 = p.w_up;
        a.s0 = p.s_gate;
        a.s1 = p.s_up;
        a.out = p.act;
        a.K = p.H;
        a.N = p.I;
    } else {
        a.a_src = (const uint16_t*)p.act;
        a.a_bytes = (uint32_t)((size_t)p.T * p.k * p.I * 2);
        a.w0 = p.w_down;
        a.w1 = nullptr;
        a.s0 = p.s_down;
        a.s1 = nullptr;
        a.out = p.y;
        a.K = p.I;
        a.N = p.H;
    }
    a.n_ntiles = (a.N + BN - 1) / BN;
    return a;
}

template <typename Kern>
hipError_t set_smem(Kern kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

int prefill_block_m() { return kBM; }

hipError_t launch_gateup_bf16(const GemmProblem& p, hipStream_t stream) {
    const PArgs a = make_pargs(p, 0, kBNGateUp);
    if (p.expert_dtype == DT_MXFP4) {
        constexpr size_t sm = PCfg<0, DT_MXFP4, kBNGateUp>::SMEM;
        static const hipError_t attr = set_smem(gateup_gemm_kernel<DT_MXFP4>, sm);
        if (attr != hipSuccess) return attr;
        return launch_k(gateup_gemm_kernel<DT_MXFP4>, sm, a, stream);
    }
    constexpr size_t sm = PCfg<0, DT_BF16, kBNGateUp>::SMEM;
    static const hipError_t attr = set_smem(gateup_gemm_kernel<DT_BF16>, sm);
    if (attr != hipSuccess) return attr;
    return launch_k(gateup_gemm_kernel<DT_BF16>, sm, a, stream);
}

hipError_t launch_down_bf16(const GemmProblem& p, hipStream_t stream) {
    const PArgs a = make_pargs(p, 1, kBNDown);
    if (p.expert_dtype == DT_MXFP4) {
        constexpr size_t sm = PCfg<1, DT_MXFP4, kBNDown>::SMEM;
        static const hipError_t attr = set_smem(down_gemm_kernel<DT_MXFP4>, sm);
        if (attr != hipSuccess) return attr;
        return launch_k(down_gemm_kernel<DT_MXFP4>, sm, a, stream);
    }
    constexpr size_t sm = PCfg<1, DT_BF16, kBNDown>::SMEM;
    static const hipError_t attr = set_smem(down_gemm_kernel<DT_BF16>, sm);
    if (attr != hipSuccess) return attr;
    return launch_k(down_gemm_kernel<DT_BF16>, sm, a, stream);
}

}  // namespace moe
