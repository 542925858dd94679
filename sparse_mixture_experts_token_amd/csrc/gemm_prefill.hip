// Stages 2 and 3 for bf16 activations (bf16 or MXFP4 expert weights): the
// experts' SwiGLU networks as grouped GEMMs over expert-major row tiles
// ("gpt-oss 20B" field guide, cutaway 03: SwiGLU experts, weighted sum;
// "openai/gpt-oss-20b" fixture comparison: hidden_act silu).
//
//   gate/up:  act[r, :] = silu(x_r W_gate[e]^T) * (x_r W_up[e]^T),  x_r = h[token of row r]
//   down:     y[a, :]   = p_a * (act[r, :] W_down[e]^T),            a = perm_src[r]
//
// Workgroup tile: BM = 256 rows of one expert x BN weight rows per matrix,
// four waves in a 2 x 2 layout (one per SIMD).  Wave (wm, wn) owns the 32-row
// blocks wm, wm + 2, wm + 4, wm + 6 (interleaved, so a short row tile still
// splits evenly) and columns wn*BN/2 .. (wn+1)*BN/2 of every matrix, as
// 32x32x16 bf16 MFMA tiles with fp32 accumulators held in the accumulation
// registers (gate/up: 4 x 2 tiles of gate and the matching 4 x 2 of up = 256
// accumulators, so SiLU*up is formed in registers; down: 4 x 3 = 192).
// BN = 128 (gate/up; the last column tile of 2880 is half full) and 192
// (down; 15 x 192 = 2880).  A wave computes 16 (12) MFMAs per 16-deep K half
// from 8 (7) operand fragments.
//
// K is swept 32 at a time through a ring of 3 LDS stages filled by
// buffer-to-LDS DMA loads (no staging registers).  A stage holds every operand
// fragment as one 1 KB block in fragment order: for K half s of the stage,
// lane l of the 32x32x16 MFMA reads bytes 16l..16l+15 of its block, i.e. row
// (or weight column) l mod 32 and K elements 16s + 8(l/32) .. +7.  Fragment
// reads are thus linear (conflict-free), and each DMA instruction writes one
// block linearly while its lanes fetch the matching rows from memory.
//
// Software pipeline, per stage kt: the fragments of half 1 are read while the
// MFMAs of half 0 run; then (stage kt+1 landed, one barrier) the DMA of stage
// kt+3 is issued into the slot stage kt has just released and the fragments
// of stage kt+1's half 0 are read while the MFMAs of half 1 run.  Two stages
// are in flight behind the one being computed, and the matrix cores never
// wait for an LDS round trip that could have been issued earlier.
//
// MXFP4 weights are staged packed (fragment order in 4-byte slots, 256-byte
// blocks) with the tile's scales for all of K, and decoded exactly to bf16 in
// registers as their fragments are read.
//
// A wave whose 32-row blocks are partly past the tile's end runs a loop
// instantiation for 4, 2 or 1 blocks (rows past the end are computed from a
// valid row and discarded); all take the same barriers.  Every wave issues
// the same number of DMA loads per stage (padded with loads into a scratch
// block), so one vmcnt threshold serves all of them.
//
// Block order: each XCD (blocks are dealt round-robin to 8) gets a contiguous
// range of a work list built with the routing tables: experts in order, for
// each expert its column tiles, for each column tile all the expert's row
// tiles.  An expert's row tiles then read each weight tile at about the same
// time on one XCD (one fetch from HBM, the rest from L2), and its activation
// rows stay in that XCD's L2 across the column tiles.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 256;
constexpr int kBK = 32;      // K per LDS stage
constexpr int kStages = 3;   // LDS ring depth (two stages in flight)
constexpr int kXcds = 8;
constexpr int kBNGateUp = 128;
constexpr int kBNDown = 192;

struct PArgs {
    const uint16_t* a_src;  // h (gate/up) or act (down), bf16
    const void* w0;         // gate or down
    const void* w1;         // up
    const uint8_t* s0;
    const uint8_t* s1;
    const int32_t* perm_src;
    const float* topk_w;
    const Tile* tiles;
    const int32_t* work;     // row tile * n_ntiles + column tile, expert-grouped order
    const int32_t* n_work;
    void* out;
    uint32_t a_bytes;        // size of the activation buffer
    int max_work, n_ntiles;
    int K, N, k;
};

typedef __attribute__((address_space(3))) void lds_void;

// Buffer-to-LDS DMA: lane l's `bytes` land at lds_block + bytes * l.
__device__ __forceinline__ void dma16(buf_rsrc r, unsigned char* lds_block, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(buf_rsrc r, unsigned char* lds_block, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 4, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's DMA loads of all but the last `ahead` stages issued
// have landed (each stage is DPS loads per lane).
template <int DPS>
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
    if (ahead >= 3) wait_vmcnt<3 * DPS>();
    else if (ahead == 2) wait_vmcnt<2 * DPS>();
    else if (ahead == 1) wait_vmcnt<DPS>();
    else wait_vmcnt<0>();
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without the release fence of __syncthreads(): that fence
// would wait for every DMA load in flight (they count as LDS writes).  Callers
// wait for exactly the loads they need first; the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int MODE, int WDT, int BN>
struct PCfg {
    static constexpr bool MX = WDT == DT_MXFP4;
    static constexpr int NMAT = MODE == 0 ? 2 : 1;
    static constexpr int MBW = 4;                     // 32-row blocks per wave
    static constexpr int BPM = BN / 32;               // 32-column blocks per matrix
    static constexpr int NBW = BPM / 2;               // 32-column blocks per wave per matrix
    static constexpr int A_BLK = (kBM / 32) * 2;      // activation blocks per stage (row blocks x 2 K halves)
    static constexpr int B_BLK = NMAT * BPM * 2;      // weight blocks per stage
    static constexpr int A_DMA = A_BLK / kWaves;      // issued per wave per stage
    static constexpr int B_DMA = (B_BLK + kWaves - 1) / kWaves;
    static constexpr int BBLK = MX ? 256 : 1024;      // bytes per weight block
    static constexpr int A_BYTES = A_BLK * 1024;
    static constexpr int STAGE = A_BYTES + B_BLK * BBLK;
    static constexpr int PAD_OFF = kStages * STAGE;   // scratch block for padding DMA loads
    static constexpr int PAD_BYTES = (B_BLK % kWaves) ? 1024 : 0;
    static constexpr int SCALE_OFF = PAD_OFF + PAD_BYTES;
    static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;  // per thread
    static_assert(A_BLK % kWaves == 0, "activation blocks must split evenly over the waves");
    static_assert(BPM % 2 == 0, "columns must split over two waves");
};

struct Srcs {
    buf_rsrc a;     // activations
    buf_rsrc w[2];  // this expert's matrices
    buf_rsrc s[2];  // MXFP4 scales of those matrices
};

// Weight block b = wave + 4i (over both matrices; b >= B_BLK is a padding load).
template <class C>
__device__ __forceinline__ void dma_stage(const Srcs& src, unsigned char* smem, int kt, int wave,
                                          const uint32_t (&a_voff)[C::A_DMA], const uint32_t (&b_voff)[C::B_DMA],
                                          const int (&b_mat)[C::B_DMA]) {
    unsigned char* st = smem + (kt % kStages) * C::STAGE;
    const uint32_t k0 = (uint32_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) dma16(src.a, st + (wave + kWaves * i) * 1024, a_voff[i], k0 * 2);
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i) {
        const int b = wave + kWaves * i;
        unsigned char* blk = b < C::B_BLK ? st + C::A_BYTES + b * C::BBLK : smem + C::PAD_OFF;
        const buf_rsrc r = b_mat[i] ? src.w[1] : src.w[0];
        if constexpr (C::MX) dma4(r, blk, b_voff[i], k0 / 2);
        else dma16(r, blk, b_voff[i], k0 * 2);
    }
}

// Weight operand of block (m, cb, s) for this lane.
template <class C>
__device__ __forceinline__ bf16x8 w_frag(const unsigned char* st, const unsigned char* scales, int kg, int kt,
                                         int m, int cb, int s, int lane, int BN) {
    const int blk = (m * C::BPM + cb) * 2 + s;
    if constexpr (C::MX) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(st + C::A_BYTES + blk * C::BBLK + lane * 4);
        const uint32_t scale = scales[(m * BN + cb * 32 + (lane & 31)) * kg + kt];
        u32x4 v;
        if (scale >= 2u && scale <= 252u) {
            const float sc = __uint_as_float(scale << 23);
            v = u32x4{cvt_fp4x2_bf16x2(q, sc, 0), cvt_fp4x2_bf16x2(q, sc, 1), cvt_fp4x2_bf16x2(q, sc, 2),
                      cvt_fp4x2_bf16x2(q, sc, 3)};
        } else {
            uint32_t w[4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint32_t byte = (q >> (8 * bb)) & 0xffu;
                w[bb] = e2m1_to_bf16_exact(byte & 0xfu, scale) | (e2m1_to_bf16_exact(byte >> 4, scale) << 16);
            }
            v = u32x4{w[0], w[1], w[2], w[3]};
        }
        return __builtin_bit_cast(bf16x8, v);
    } else {
        return *reinterpret_cast<const bf16x8*>(st + C::A_BYTES + blk * C::BBLK + lane * 16);
    }
}

// Operand fragments of one 16-deep K half for this wave: MB activation blocks
// (row blocks wm + 2i) and NMAT x NBW weight blocks.
template <class C, int MB>
struct Frags {
    bf16x8 a[MB];
    bf16x8 b[C::NMAT][C::NBW];
};

template <class C, int BN, int MB>
__device__ __forceinline__ void read_frags(const unsigned char* st, const unsigned char* scales, int kg, int kt, int s,
                                           int wm, int wn, int lane, Frags<C, MB>& f) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
        f.a[i] = *reinterpret_cast<const bf16x8*>(st + ((wm + 2 * i) * 2 + s) * 1024 + lane * 16);
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int j = 0; j < C::NBW; ++j) f.b[m][j] = w_frag<C>(st, scales, kg, kt, m, wn * C::NBW + j, s, lane, BN);
}

template <class C, int MB>
__device__ __forceinline__ void mma_half(const Frags<C, MB>& f, f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int j = 0; j < C::NBW; ++j)
#pragma unroll
            for (int i = 0; i < MB; ++i) acc[m][i][j] = mfma32(f.a[i], f.b[m][j], acc[m][i][j]);
}

// Stages 0 .. min(3, nk) - 1 were issued by the caller.
template <class C, int BN, int MB>
__device__ __forceinline__ void main_loop(const Srcs& src, unsigned char* smem, const unsigned char* scales, int nk,
                                          int wave, int lane, const uint32_t (&a_voff)[C::A_DMA],
                                          const uint32_t (&b_voff)[C::B_DMA], const int (&b_mat)[C::B_DMA],
                                          f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    const int wm = wave >> 1, wn = wave & 1;
    Frags<C, MB> f0, f1;
    // stage 0 landed for every thread
    wait_stages_ahead<C::DMA_PER_STAGE>(min(nk, kStages) - 1);
    bare_barrier();
    read_frags<C, BN, MB>(smem, scales, nk, 0, 0, wm, wn, lane, f0);
    for (int kt = 0; kt < nk; ++kt) {
        const unsigned char* st = smem + (kt % kStages) * C::STAGE;
        read_frags<C, BN, MB>(st, scales, nk, kt, 1, wm, wn, lane, f1);
        mma_half<C, MB>(f0, acc);
        if (kt + 1 < nk) {
            // stage kt+1 landed here and (barrier) for every thread; every wave
            // has also finished reading stage kt, whose slot the next DMA reuses
            wait_stages_ahead<C::DMA_PER_STAGE>(min(nk - 1, kt + kStages - 1) - (kt + 1));
            wait_lds_reads();
            bare_barrier();
            if (kt + kStages < nk) dma_stage<C>(src, smem, kt + kStages, wave, a_voff, b_voff, b_mat);
            read_frags<C, BN, MB>(smem + ((kt + 1) % kStages) * C::STAGE, scales, nk, kt + 1, 0, wm, wn, lane, f0);
        }
        mma_half<C, MB>(f1, acc);
    }
}

template <int MODE, int WDT, int BN>
__device__ __forceinline__ void gemm_body(const PArgs& args) {
    using C = PCfg<MODE, WDT, BN>;
    extern __shared__ __align__(16) unsigned char smem[];

    // ---- block -> work item (row tile, column tile) ----
    // Blocks are dealt round-robin to the 8 XCDs; XCD x takes the x-th of 8
    // equal contiguous ranges of the work list (sized by the actual item
    // count, not the grid's upper bound, so every XCD gets its share).
    const int n_work = args.n_work[0];
    const int per_xcd = (n_work + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int q = (blockIdx.x % kXcds) * per_xcd + slot;
    if (slot >= per_xcd || q >= n_work) return;
    const int item = args.work[q];
    const int mt = item / args.n_ntiles;
    const int nt = item % args.n_ntiles;
    const Tile tile = args.tiles[mt];
    const int e = tile.expert;
    const int row0 = tile.row_start;
    const int rows = tile.rows;
    const int n0 = nt * BN;
    const int K = args.K, N = args.N;

    const int tid = threadIdx.x;
    // the wave index as a scalar: everything derived from it (DMA block
    // addresses, weight matrix choice) stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;   // 2 x 2 waves
    const int fr = lane & 31;   // row / column within a 32-block
    const int fh = lane >> 5;   // which 8 of the 16 K elements of a half

    // ---- DMA sources (byte offsets) ----
    // activation block b = wave + 4i: row block b / 2, K half b % 2
    uint32_t a_voff[C::A_DMA];
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) {
        const int b = wave + kWaves * i;
        const int r = (b >> 1) * 32 + fr;
        const int rr = r < rows ? r : 0;
        int src_row;
        if constexpr (MODE == 0) src_row = args.perm_src[row0 + rr] / args.k;
        else src_row = row0 + rr;
        a_voff[i] = (uint32_t)(src_row * K + ((b & 1) * 2 + fh) * 8) * 2u;
    }
    const size_t mat_elems = (size_t)N * K;
    Srcs src;
    src.a = make_rsrc(args.a_src, args.a_bytes);
    if constexpr (C::MX) {
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
    // weight block b = wave + 4i over both matrices: matrix b / (2 BPM), then
    // column block (b mod 2 BPM) / 2 and K half b mod 2; padding loads repeat block 0
    uint32_t b_voff[C::B_DMA];
    int b_mat[C::B_DMA];
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i) {
        int b = wave + kWaves * i;
        if (b >= C::B_BLK) b = 0;
        b_mat[i] = b / (C::BPM * 2);
        const int bm = b % (C::BPM * 2);
        const int n = min(n0 + (bm >> 1) * 32 + fr, N - 1);
        const int kc = (bm & 1) * 2 + fh;   // 8-element K chunk within the stage
        if constexpr (C::MX) b_voff[i] = (uint32_t)(n * (K / 2) + kc * 4);
        else b_voff[i] = (uint32_t)(n * K + kc * 8) * 2u;
    }

    const int nk = K / kBK;
    // prologue: the first kStages stages in flight
#pragma unroll
    for (int s = 0; s < kStages; ++s)
        if (s < nk) dma_stage<C>(src, smem, s, wave, a_voff, b_voff, b_mat);

    // MXFP4: this tile's scales for the whole K range, [matrix][column][K/32]
    unsigned char* scales = smem + C::SCALE_OFF;
    if constexpr (C::MX) {
        const int kg = K / 32;
        const int per_mat = BN * kg;  // bytes, a multiple of 16
        for (int m = 0; m < C::NMAT; ++m)
            for (int c = tid * 16; c < per_mat; c += kThreads * 16) {
                const u32x4 v = buf_load16(src.s[m], (uint32_t)(n0 * kg + c), 0);
                *reinterpret_cast<u32x4*>(scales + m * per_mat + c) = v;
            }
        __syncthreads();
    }

    f32x16 acc[C::NMAT][C::MBW][C::NBW];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int i = 0; i < C::MBW; ++i)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][i][j][v] = 0.f;

    // This wave's live 32-row blocks: wm + 2i below ceil(rows / 32).
    const int live32 = (rows + 31) >> 5;
    const int mine = live32 > wm ? (live32 - wm + 1) / 2 : 0;
    if (mine > 2) main_loop<C, BN, 4>(src, smem, scales, nk, wave, lane, a_voff, b_voff, b_mat, acc);
    else if (mine == 2) main_loop<C, BN, 2>(src, smem, scales, nk, wave, lane, a_voff, b_voff, b_mat, acc);
    else main_loop<C, BN, 1>(src, smem, scales, nk, wave, lane, a_voff, b_voff, b_mat, acc);

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < C::MBW; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = (wm + 2 * i) * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
            if (r >= rows) continue;
            if constexpr (MODE == 0) {
                uint16_t* orow = reinterpret_cast<uint16_t*>(args.out) + (size_t)(row0 + r) * N;
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int n = n0 + (wn * C::NBW + j) * 32 + fr;
                    if (n < N) orow[n] = (uint16_t)f32_to_bf16_bits(silu_f(acc[0][i][j][v]) * acc[1][i][j][v]);
                }
            } else {
                const int asg = args.perm_src[row0 + r];
                const float p = args.topk_w[asg];
                float* orow = reinterpret_cast<float*>(args.out) + (size_t)asg * N;
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int n = n0 + (wn * C::NBW + j) * 32 + fr;
                    if (n < N) orow[n] = acc[0][i][j][v] * p;
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

template <int MODE, int WDT, int BN>
size_t smem_bytes(int K) {
    using C = PCfg<MODE, WDT, BN>;
    return (size_t)C::SCALE_OFF + (C::MX ? (size_t)C::NMAT * BN * (K / 32) : 0);
}

template <typename Kern>
hipError_t launch_k(Kern kern, size_t smem, const PArgs& a, hipStream_t stream) {
    const int per_xcd = (a.max_work + kXcds - 1) / kXcds;
    kern<<<per_xcd * kXcds, kThreads, smem, stream>>>(a);
    return hipGetLastError();
}
PArgs make_pargs(const GemmProblem& p, int mode) {
    PArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.tiles = p.tiles;
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
        a.work = p.work_gateup;
        a.n_work = p.n_work_gateup;
        a.n_ntiles = (p.I + kBNGateUp - 1) / kBNGateUp;
        a.max_work = p.max_tiles * a.n_ntiles;
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
        a.work = p.work_down;
        a.n_work = p.n_work_down;
        a.n_ntiles = (p.H + kBNDown - 1) / kBNDown;
        a.max_work = p.max_tiles * a.n_ntiles;
    }
    return a;
}

template <typename Kern>
hipError_t set_smem(Kern kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

int prefill_block_m() { return kBM; }

// Largest LDS footprint of the bf16-activation GEMMs for contraction depth K
// (the MXFP4 kernels keep the tile's scales for all of K in LDS).
size_t prefill_smem_bytes(int K, int expert_dtype) {
    if (expert_dtype == DT_MXFP4)
        return smem_bytes<0, DT_MXFP4, kBNGateUp>(K) > smem_bytes<1, DT_MXFP4, kBNDown>(K)
                   ? smem_bytes<0, DT_MXFP4, kBNGateUp>(K)
                   : smem_bytes<1, DT_MXFP4, kBNDown>(K);
    return smem_bytes<0, DT_BF16, kBNGateUp>(K) > smem_bytes<1, DT_BF16, kBNDown>(K)
               ? smem_bytes<0, DT_BF16, kBNGateUp>(K)
               : smem_bytes<1, DT_BF16, kBNDown>(K);
}

int prefill_col_tiles(int N, int mode) {
    const int bn = mode == 0 ? kBNGateUp : kBNDown;
    return (N + bn - 1) / bn;
}

constexpr size_t kMaxSmem = 160 * 1024;

hipError_t launch_gateup_bf16(const GemmProblem& p, hipStream_t stream) {
    const PArgs a = make_pargs(p, 0);
    if (p.expert_dtype == DT_MXFP4) {
        static const hipError_t attr = set_smem(gateup_gemm_kernel<DT_MXFP4>, kMaxSmem);
        if (attr != hipSuccess) return attr;
        return launch_k(gateup_gemm_kernel<DT_MXFP4>, smem_bytes<0, DT_MXFP4, kBNGateUp>(a.K), a, stream);
    }
    static const hipError_t attr = set_smem(gateup_gemm_kernel<DT_BF16>, kMaxSmem);
    if (attr != hipSuccess) return attr;
    return launch_k(gateup_gemm_kernel<DT_BF16>, smem_bytes<0, DT_BF16, kBNGateUp>(a.K), a, stream);
}

hipError_t launch_down_bf16(const GemmProblem& p, hipStream_t stream) {
    const PArgs a = make_pargs(p, 1);
    if (p.expert_dtype == DT_MXFP4) {
        static const hipError_t attr = set_smem(down_gemm_kernel<DT_MXFP4>, kMaxSmem);
        if (attr != hipSuccess) return attr;
        return launch_k(down_gemm_kernel<DT_MXFP4>, smem_bytes<1, DT_MXFP4, kBNDown>(a.K), a, stream);
    }
    static const hipError_t attr = set_smem(down_gemm_kernel<DT_BF16>, kMaxSmem);
    if (attr != hipSuccess) return attr;
    return launch_k(down_gemm_kernel<DT_BF16>, smem_bytes<1, DT_BF16, kBNDown>(a.K), a, stream);
}

}  // namespace moe
