// Stages 2 and 3 for bf16 activations and bf16 expert weights: the experts'
// SwiGLU networks as grouped GEMMs over expert-major row tiles
// ("gpt-oss 20B" field guide, cutaway 03: SwiGLU experts, weighted sum;
// "openai/gpt-oss-20b" fixture comparison: hidden_act silu).
//
//   gate/up:  act[r, :] = silu(x_r W_gate[e]^T) * (x_r W_up[e]^T),  x_r = h[token of row r]
//   down:     y[a, :]   = p_a * (act[r, :] W_down[e]^T),            a = perm_src[r]
//
// Workgroup tile: BM = 256 rows of one expert x BN = 128 weight rows per
// matrix (gate/up: 128 of gate and the same 128 of up; down: 128 of W_down),
// eight waves in a 4 x 2 layout, two per SIMD, so that one wave's MFMAs cover
// the other's LDS and DMA issue.  Wave (wm, wn) owns the 32-row groups wm and
// wm + 4 and half of the tile's weight rows of every matrix, as 32x32x16 bf16
// MFMA tiles with fp32 accumulators (gate/up: 2 x 2 of gate and 2 x 2 of up,
// so SiLU*up is formed in registers; down: 2 x 2).
//
// Operands reach LDS by buffer-to-LDS DMA.  What limits such a kernel on this
// hardware is how many cache lines one load instruction touches: 64 lanes x
// 16 bytes spread as 32 rows x 32 bytes (the MFMA fragment order) sustain
// about a quarter of the throughput of 8 rows x 128 bytes.  So K advances 64
// per stage (128 bytes = one cache line of every row), and one DMA
// instruction fills a 1 KB block with 8 whole rows: lane l writes slot l
// (row l/8, 16-byte slot l%8) and fetches into it the row's logical chunk
// (l%8) ^ (l/8) ^ (block & 1).  The same XOR applied when MFMA fragments are
// read back (lane l: row l%32 of a 32-row group = 4 blocks, K elements
// 16q + 8(l/32) .. +7 of step q) spreads every group of 16 lanes over all
// LDS banks.
//
// Software pipeline: an LDS ring of two 64 KB stages (gate/up) or three 48 KB
// stages (down).  Within a stage the fragments of K steps 2,3 are read while
// steps 0,1 compute; then, behind the one barrier per stage, the slot just
// released is refilled by DMA and steps 0,1 of the next stage are read while
// steps 2,3 compute.  sched_group_barrier spreads the DMA and LDS reads
// between the MFMAs.
//
// Block order: each XCD (blocks are dealt round-robin to 8) takes a
// contiguous range of a work list built with the routing tables: experts in
// order, for each expert its column tiles, for each column tile all the
// expert's row tiles, so the row tiles sharing a weight tile run together on
// one XCD and its L2 serves the repeats.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kWM = kWaves / 2;   // waves along the rows (2 along the weight rows)
constexpr int kBM = 256;          // rows per tile: 8 groups of 32, 2 per wave
constexpr int kBK = 64;      // K per LDS stage: 128 bytes of each row
constexpr int kXcds = 8;
constexpr int kBNGateUp = 128;
constexpr int kBNDown = 256;
constexpr int kStagesGateUp = 2;  // 64 KB stages
constexpr int kStagesDown = 2;    // 64 KB stages

struct BArgs {
    const uint16_t* a_src;  // h (gate/up) or act (down)
    const void* w0;         // gate or down, [E][N][K]
    const void* w1;         // up
    const int32_t* perm_src;
    const float* topk_w;
    const Tile* tiles;
    const int32_t* work;    // row tile * n_ntiles + column tile, expert-grouped order
    const int32_t* n_work;
    int32_t* queue;         // [8] per-XCD work counters, zero at launch
    void* out;
    uint32_t a_bytes;
    int max_work, n_ntiles;
    int K, N, k;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(buf_rsrc r, unsigned char* lds_block, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 16, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DPS>
__device__ __forceinline__ void wait_stages_ahead(int ahead) {
    if (ahead >= 2) wait_vmcnt<2 * DPS>();
    else if (ahead == 1) wait_vmcnt<DPS>();
    else wait_vmcnt<0>();
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Barrier without the release fence of __syncthreads(), which would wait for
// every DMA load in flight; the callers wait for exactly what they need.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int MODE, int BN, int S>
struct Cfg {
    static constexpr int NMAT = MODE == 0 ? 2 : 1;
    static constexpr int NST = S;                    // LDS ring depth
    static constexpr int MBW = kBM / (32 * kWM);     // 32-row groups per wave
    static constexpr int BPM = BN / 32;              // 32-row weight groups per matrix
    static constexpr int NBW = BPM / 2;              // per wave per matrix
    static constexpr int A_BLK = kBM / 8;            // 8-row DMA blocks of activations
    static constexpr int B_BLK = NMAT * BN / 8;      // of weights
    static constexpr int A_DMA = A_BLK / kWaves;     // per wave per stage
    static constexpr int B_DMA = B_BLK / kWaves;
    static constexpr int DPS = A_DMA + B_DMA;        // DMA loads per lane per stage
    static constexpr int A_BYTES = A_BLK * 1024;
    static constexpr int STAGE = A_BYTES + B_BLK * 1024;
    static constexpr int SMEM = S * STAGE;
    static_assert(A_BLK % kWaves == 0 && B_BLK % kWaves == 0, "DMA blocks must split evenly over the waves");
    static_assert(BPM % 2 == 0, "weight rows must split over two waves");
    static_assert(SMEM <= 160 * 1024, "LDS");
    static_assert(NMAT * MBW * NBW * 16 <= 256, "accumulators");
};

// Fragments of two consecutive K steps for this wave's MB row groups.
template <class C, int MB>
struct Frags2 {
    bf16x8 a[2][MB];
    bf16x8 b[2][C::NMAT][C::NBW];
};

// Fragments of K step q: lane offset within a 4-block (32-row) group.
__device__ __forceinline__ uint32_t frag_lane_off(int lane, int q) {
    const int r = lane & 31, rb = lane & 7;
    const int c = 2 * q + (lane >> 5);
    return (uint32_t)((r >> 3) * 1024 + rb * 128 + ((c ^ rb ^ ((r >> 3) & 1)) * 16));
}

// Read the fragments of steps q0, q0+1 of stage `st`.
template <class C, int BN, int MB>
__device__ __forceinline__ void read_frags2(const unsigned char* st, const uint32_t (&loff)[4], int q0, int wm, int wn,
                                            Frags2<C, MB>& f) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
            f.a[h][i] = *reinterpret_cast<const bf16x8*>(st + (wm + kWM * i) * 4096 + loff[q0 + h]);
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
                f.b[h][m][j] = *reinterpret_cast<const bf16x8*>(st + C::A_BYTES +
                                                                (m * (BN / 32) + wn * C::NBW + j) * 4096 + loff[q0 + h]);
    }
}

template <class C, int MB>
__device__ __forceinline__ void mma2(const Frags2<C, MB>& f, f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[m][i][j] = mfma32(f.a[h][i], f.b[h][m][j], acc[m][i][j]);
}

struct Srcs {
    buf_rsrc a;
    buf_rsrc w[2];
};

// Block b of a stage is filled by wave b % 4; a wave's blocks are b = wave + 4i.
template <class C>
__device__ __forceinline__ void dma_stage(const Srcs& src, unsigned char* smem, int kt, int wave,
                                          const uint32_t (&a_voff)[C::A_DMA], const uint32_t (&b_voff)[C::B_DMA],
                                          const int (&b_mat)[C::B_DMA]) {
    unsigned char* st = smem + (kt % C::NST) * C::STAGE;
    const uint32_t k0 = (uint32_t)kt * kBK * 2;  // bytes
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) dma16(src.a, st + (wave + kWaves * i) * 1024, a_voff[i], k0);
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i)
        dma16(b_mat[i] ? src.w[1] : src.w[0], st + C::A_BYTES + (wave + kWaves * i) * 1024, b_voff[i], k0);
}

// Instruction interleaving inside one scheduling region: MFMA i is preceded
// by its share of NV VMEM loads (the DMA) and ND LDS fragment reads, so the
// texture unit and LDS work in the shadow of the matrix cores instead of
// stalling the wave in a burst.
template <int I, int NV, int ND, int NM>
__device__ __forceinline__ void interleave() {
    if constexpr (I < NM) {
        constexpr int v = (I + 1) * NV / NM - I * NV / NM;
        constexpr int d = (I + 1) * ND / NM - I * ND / NM;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // VMEM read
        if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // MFMA
        interleave<I + 1, NV, ND, NM>();
    }
}

// One stage kt: steps 2,3 are read while steps 0,1 compute; then (stage kt+1
// landed, one barrier: every wave is done reading stage kt) the freed slot is
// refilled with stage kt+NST (DMA) and steps 0,1 of stage kt+1 are read while
// steps 2,3 compute.  WAIT = stages allowed in flight at the wait (-1: read
// `ahead` at run time).
template <class C, int BN, int MB, bool DMA, bool NEXT, int WAIT>
__device__ __forceinline__ void stage_iter(const Srcs& src, unsigned char* smem, int nk, int kt, int wave, int wm,
                                           int wn, const uint32_t (&loff)[4], const uint32_t (&a_voff)[C::A_DMA],
                                           const uint32_t (&b_voff)[C::B_DMA], const int (&b_mat)[C::B_DMA],
                                           Frags2<C, MB>& lo, Frags2<C, MB>& hi,
                                           f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    constexpr int NR = 2 * (MB + C::NMAT * C::NBW);  // fragment reads per two steps
    constexpr int NM = 2 * C::NMAT * C::NBW * MB;    // MFMAs per two steps
    const unsigned char* st = smem + (kt % C::NST) * C::STAGE;
    read_frags2<C, BN, MB>(st, loff, 2, wm, wn, hi);
    mma2<C, MB>(lo, acc);
    interleave<0, 0, NR, NM>();
    if constexpr (NEXT) {
        if constexpr (WAIT >= 0) wait_vmcnt<WAIT * C::DPS>();
        else wait_stages_ahead<C::DPS>(min(nk - 1, kt + C::NST - 1) - (kt + 1));
        wait_lds_reads();
        bare_barrier();
        if constexpr (DMA) dma_stage<C>(src, smem, kt + C::NST, wave, a_voff, b_voff, b_mat);
        read_frags2<C, BN, MB>(smem + ((kt + 1) % C::NST) * C::STAGE, loff, 0, wm, wn, lo);
        mma2<C, MB>(hi, acc);
        interleave<0, DMA ? C::DPS : 0, NR, NM>();
    } else {
        mma2<C, MB>(hi, acc);
    }
}

// Stages 0 .. min(NST, nk) - 1 were issued by the caller.
template <class C, int BN, int MB>
__device__ __forceinline__ void main_loop(const Srcs& src, unsigned char* smem, int nk, int wave, int lane,
                                          const uint32_t (&a_voff)[C::A_DMA], const uint32_t (&b_voff)[C::B_DMA],
                                          const int (&b_mat)[C::B_DMA], f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    const int wm = wave >> 1, wn = wave & 1;
    uint32_t loff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) loff[q] = frag_lane_off(lane, q);
    Frags2<C, MB> lo, hi;
    wait_stages_ahead<C::DPS>(min(nk, C::NST) - 1);
    bare_barrier();
    read_frags2<C, BN, MB>(smem, loff, 0, wm, wn, lo);
    int kt = 0;
    // steady state: the next stage exists and a stage NST ahead is refilled
    for (; kt + C::NST < nk; ++kt)
        stage_iter<C, BN, MB, true, true, C::NST - 2>(src, smem, nk, kt, wave, wm, wn, loff, a_voff, b_voff, b_mat,
                                                       lo, hi, acc);
    for (; kt + 1 < nk; ++kt)
        stage_iter<C, BN, MB, false, true, -1>(src, smem, nk, kt, wave, wm, wn, loff, a_voff, b_voff, b_mat, lo, hi,
                                               acc);
    stage_iter<C, BN, MB, false, false, 0>(src, smem, nk, kt, wave, wm, wn, loff, a_voff, b_voff, b_mat, lo, hi, acc);
}

// Main loop for the MB live row groups of this wave (MB = 1 .. MBW; a wave
// with none computes one group from a valid row and discards it).
template <class C, int BN, int MB>
__device__ __forceinline__ void dispatch_mb(int mine, const Srcs& src, unsigned char* smem, int nk, int wave, int lane,
                                            const uint32_t (&a_voff)[C::A_DMA], const uint32_t (&b_voff)[C::B_DMA],
                                            const int (&b_mat)[C::B_DMA], f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    if constexpr (MB == 1) {
        main_loop<C, BN, 1>(src, smem, nk, wave, lane, a_voff, b_voff, b_mat, acc);
    } else {
        if (mine >= MB) main_loop<C, BN, MB>(src, smem, nk, wave, lane, a_voff, b_voff, b_mat, acc);
        else dispatch_mb<C, BN, MB - 1>(mine, src, smem, nk, wave, lane, a_voff, b_voff, b_mat, acc);
    }
}

// One work item q: (row tile, column tile) of the work list.
template <int MODE, int BN, int S>
__device__ __forceinline__ void process_item(const BArgs& args, int q) {
    using C = Cfg<MODE, BN, S>;
    extern __shared__ __align__(16) unsigned char smem[];
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int rb = lane >> 3;                                  // row within a DMA block
    const uint32_t chunk_even = (uint32_t)((lane & 7) ^ rb);  // logical 16-byte chunk fetched (even block)

    // ---- DMA sources: byte offsets of this lane's chunk in stage 0 ----
    uint32_t a_voff[C::A_DMA];
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) {
        const int blk = wave + kWaves * i;
        const int r = blk * 8 + rb;
        const int rr = r < rows ? r : 0;
        int src_row;
        if constexpr (MODE == 0) src_row = args.perm_src[row0 + rr] / args.k;
        else src_row = row0 + rr;
        a_voff[i] = (uint32_t)src_row * (uint32_t)K * 2u + (chunk_even ^ (uint32_t)(blk & 1)) * 16u;
    }
    Srcs src;
    src.a = make_rsrc(args.a_src, args.a_bytes);
    const uint32_t wbytes = (uint32_t)((size_t)N * K * 2);
    src.w[0] = make_rsrc((const unsigned char*)args.w0 + (size_t)e * wbytes, wbytes);
    src.w[1] = MODE == 0 ? make_rsrc((const unsigned char*)args.w1 + (size_t)e * wbytes, wbytes) : src.w[0];
    uint32_t b_voff[C::B_DMA];
    int b_mat[C::B_DMA];
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i) {
        const int blk = wave + kWaves * i;
        b_mat[i] = (blk * 8) / BN;
        const int n = min(n0 + (blk * 8) % BN + rb, N - 1);
        b_voff[i] = (uint32_t)n * (uint32_t)K * 2u + (chunk_even ^ (uint32_t)(blk & 1)) * 16u;
    }

    const int nk = K / kBK;
#pragma unroll
    for (int s = 0; s < C::NST; ++s)
        if (s < nk) dma_stage<C>(src, smem, s, wave, a_voff, b_voff, b_mat);

    f32x16 acc[C::NMAT][C::MBW][C::NBW];
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int i = 0; i < C::MBW; ++i)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][i][j][v] = 0.f;

    // live 32-row groups of this wave: wm + kWM i below ceil(rows / 32)
    const int live32 = (rows + 31) >> 5;
    const int mine = live32 > wm ? (live32 - wm + kWM - 1) / kWM : 0;
    dispatch_mb<C, BN, C::MBW>(mine, src, smem, nk, wave, lane, a_voff, b_voff, b_mat, acc);

    // ---- epilogue: D[v] of a 32x32 tile is row 8(v/4) + 4(l/32) + v%4, column l%32 ----
    const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
    for (int i = 0; i < C::MBW; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = (wm + kWM * i) * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
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

// Persistent workgroups, one per CU.  Blocks are dealt round-robin to the 8
// XCDs; XCD x owns the x-th of 8 equal contiguous ranges of the work list
// (sized by the actual item count) and its workgroups take the range's items
// in order from the XCD's counter, so a workgroup that drew cheap items (the
// short last row tile of an expert) takes more of them, and the row tiles
// sharing a weight tile still run together on one XCD.
template <int MODE, int BN, int S>
__device__ __forceinline__ void gemm_body(const BArgs& args) {
    __shared__ int s_q;
    const int n_work = args.n_work[0];
    const int per_xcd = (n_work + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds;
    const int base = xcd * per_xcd;
    const int end = min(base + per_xcd, n_work);
    for (;;) {
        if (threadIdx.x == 0) s_q = base + atomicAdd(args.queue + xcd, 1);
        // s_q visible to every wave, and every wave done with the previous item's LDS
        wait_lds_reads();
        bare_barrier();
        const int q = __builtin_amdgcn_readfirstlane(s_q);
        if (q >= end) break;
        process_item<MODE, BN, S>(args, q);
    }
}

using CfgGateUp = Cfg<0, kBNGateUp, kStagesGateUp>;
using CfgDown = Cfg<1, kBNDown, kStagesDown>;
__global__ __launch_bounds__(kThreads) void gateup_bf16_kernel(BArgs args) {
    gemm_body<0, kBNGateUp, kStagesGateUp>(args);
}
__global__ __launch_bounds__(kThreads) void down_bf16_kernel(BArgs args) { gemm_body<1, kBNDown, kStagesDown>(args); }

BArgs make_args(const GemmProblem& p, int mode) {
    BArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.tiles = p.tiles;
    a.k = p.k;
    if (mode == 0) {
        a.a_src = (const uint16_t*)p.h;
        a.a_bytes = (uint32_t)((size_t)p.T * p.H * 2);
        a.w0 = p.w_gate;
        a.w1 = p.w_up;
        a.out = p.act;
        a.K = p.H;
        a.N = p.I;
        a.work = p.work_gateup;
        a.n_work = p.n_work_gateup;
        a.queue = p.queues;
        a.n_ntiles = (p.I + kBNGateUp - 1) / kBNGateUp;
    } else {
        a.a_src = (const uint16_t*)p.act;
        a.a_bytes = (uint32_t)((size_t)p.T * p.k * p.I * 2);
        a.w0 = p.w_down;
        a.w1 = p.w_down;
        a.out = p.y;
        a.K = p.I;
        a.N = p.H;
        a.work = p.work_down;
        a.n_work = p.n_work_down;
        a.queue = p.queues + kXcds;
        a.n_ntiles = (p.H + kBNDown - 1) / kBNDown;
    }
    a.max_work = p.max_tiles * a.n_ntiles;
    return a;
}

// One workgroup per CU (the LDS ring allows no more), never more than the
// work, and at least one per XCD range so that every range is drained.
int persistent_grid(int max_work) {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    const int g = max_work < cus ? max_work : cus;
    return g > kXcds ? g : kXcds;
}

template <typename Kern>
hipError_t launch(Kern kern, size_t smem, const BArgs& a, hipStream_t stream) {
    kern<<<persistent_grid(a.max_work), kThreads, smem, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

int bf16_block_m() { return kBM; }
int bf16_col_tiles(int N, int mode) { return (N + (mode == 0 ? kBNGateUp : kBNDown) - 1) / (mode == 0 ? kBNGateUp : kBNDown); }

hipError_t launch_gateup_bf16w(const GemmProblem& p, hipStream_t stream) {
    constexpr size_t smem = CfgGateUp::SMEM;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)gateup_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (attr != hipSuccess) return attr;
    return launch(gateup_bf16_kernel, smem, make_args(p, 0), stream);
}

hipError_t launch_down_bf16w(const GemmProblem& p, hipStream_t stream) {
    constexpr size_t smem = CfgDown::SMEM;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)down_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (attr != hipSuccess) return attr;
    return launch(down_bf16_kernel, smem, make_args(p, 1), stream);
}

}  // namespace moe
