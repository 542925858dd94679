// Stages 2 and 3 for bf16 activations and bf16 or MXFP4 expert weights: the
// experts' SwiGLU networks as grouped GEMMs over expert-major row tiles
// ("gpt-oss 20B" field guide, cutaway 03: SwiGLU experts, weighted sum;
// "openai/gpt-oss-20b" fixture comparison: hidden_act silu).
//
//   gate/up:  act[r, :] = silu(x_r W_gate[e]^T) * (x_r W_up[e]^T),  x_r = h[token of row r]
//   down:     y[a, :]   = p_a * (act[r, :] W_down[e]^T),            a = perm_src[r]
//
// Workgroup tile: BM = 256 rows of one expert x BN weight rows per matrix
// (gate/up: 128 of gate and the same 128 of up; down: 320 of W_down, 256 for
// MXFP4 weights), eight
// waves in a 4 x 2 layout, two per SIMD, so that one wave's MFMAs cover the
// other's LDS and DMA issue.  Wave (wm, wn) owns the 32-row groups wm and
// wm + 4 and half of the tile's weight rows of every matrix, as 32x32x16 bf16
// MFMA tiles with fp32 accumulators (gate/up: 2 x 2 of gate and 2 x 2 of up,
// so SiLU*up is formed in registers; down: 2 x 5, MXFP4 2 x 4).
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
// Software pipeline: an LDS ring of two 64 KB stages (three smaller ones for
// MXFP4 weights).  Within a stage the fragments of K steps 2,3 are read while
// steps 0,1 compute; then, behind the one barrier per stage, the slot just
// released is refilled by DMA and steps 0,1 of the next stage are read while
// steps 2,3 compute.  sched_group_barrier spreads the DMA and LDS reads
// between the MFMAs.
//
// MXFP4 weights ("gpt-oss-20b and gpt-oss-120b" explainer, "Four-bit expert
// weights"; element and scale encodings of OCP MX v1.0) travel packed: a
// stage holds each weight row's 32 bytes of codes for its 64 K in 32-row 1 KB
// blocks.  That pattern is four times slower per byte than whole-line fetches
// but carries a quarter of the bytes, and the smaller stages leave room for a
// three-stage ring beside the tile's E8M0 scales for all of K.  The stage's K
// order is permuted (the same for both operands) so that a lane's codes for
// all four steps are 16 contiguous bytes under one scale: one LDS read of
// codes and one of the scale per weight group and stage, decoded exactly to
// bf16 right before each MFMA (hardware scaled conversion for scales 2..252,
// integer path for the extremes).
//
// Block order: persistent workgroups, one per CU.  Each XCD (blocks are dealt
// round-robin to 8) drains a contiguous range of a work list built with the
// routing tables - experts in order, for each expert its column tiles, for
// each column tile all the expert's row tiles - through its own work-queue
// counter, so the row tiles sharing a weight tile run together on one XCD
// and its L2 serves the repeats.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kWM = kWaves / 2;   // waves along the rows (2 along the weight rows)
constexpr int kBM = 256;          // rows per tile: 8 groups of 32, 2 per wave
constexpr int kBK = 64;      // K per LDS stage: 128 bytes of each row
constexpr int kXcds = 8;
static_assert(kXcds == kXcdRanges, "the route scan cuts one work range per XCD");
constexpr int kBNGateUp = 128;
// Down tile width: 320 rows of W_down for bf16 weights (2880 = 9 x 320, no
// padded last tile, and 15% fewer operand bytes per FLOP than 256), 256 for
// MXFP4 (its 32-row code blocks must split evenly over the eight waves).
template <bool MXW>
constexpr int kBNDown = MXW ? 256 : 320;
constexpr int kStagesGateUp = 2;  // 64 KB stages
constexpr int kStagesDown = 2;    // 64 KB stages

struct BArgs {
    const uint16_t* a_src;  // h (gate/up) or act (down)
    const void* w0;         // gate or down, [E][N][K] bf16 or [E][N][K/2] MXFP4 codes
    const void* w1;         // up
    const uint8_t* s0;      // MXFP4 scales [E][N][K/32] of w0, w1
    const uint8_t* s1;
    const int32_t* perm_src;
    const float* topk_w;
    const float* row_p;     // routing weight of each expert-major row (down)
    const Tile* tiles;
    const int32_t* work;    // row tile * n_ntiles + column tile, expert-grouped order
    const int32_t* n_work;
    const int32_t* bounds;  // [kXcdRanges + 1]
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

// silu(g) = g / (1 + e^-g) with the hardware reciprocal (about 1 ulp) in place
// of the correctly rounded division, whose dozen instructions per element
// made the epilogue a visible part of each work item; the product is rounded
// to bf16 right after, 16 bits coarser.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// A buffer offset beyond every range used by the stores below (ranges stay
// under 2^30 bytes, so adding a row offset cannot wrap around).
constexpr uint32_t kOobStore = 0x7ffffff0u;

template <int MODE, int BN, int S, bool MXW>
struct Cfg {
    static constexpr bool MX = MXW;                  // MXFP4 weights
    static constexpr int NMAT = MODE == 0 ? 2 : 1;
    static constexpr int NST = S;                    // LDS ring depth
    static constexpr int MBW = kBM / (32 * kWM);     // 32-row groups per wave
    static constexpr int BPM = BN / 32;              // 32-row weight groups per matrix
    static constexpr int NBW = BPM / 2;              // per wave per matrix
    static constexpr int A_BLK = kBM / 8;            // 8-row DMA blocks of activations
    // weights: bf16 in 8-row blocks (128 bytes a row), MXFP4 codes in
    // 32-row blocks (the 32 bytes of codes a row holds for 64 K)
    static constexpr int B_BLK = MX ? NMAT * BN / 32 : NMAT * BN / 8;
    static constexpr int A_DMA = A_BLK / kWaves;     // per wave per stage
    static constexpr int B_DMA = B_BLK / kWaves;
    static constexpr int DPS = A_DMA + B_DMA;        // DMA loads per lane per stage
    static constexpr int A_BYTES = A_BLK * 1024;
    static constexpr int STAGE = A_BYTES + B_BLK * 1024;
    static constexpr int SMEM = S * STAGE;  // + the tile's MXFP4 scales for all of K
    static constexpr size_t smem(int K) { return (size_t)SMEM + (MX ? (size_t)NMAT * BN * (K / 32) : 0); }
    static_assert(A_BLK % kWaves == 0 && B_BLK % kWaves == 0, "DMA blocks must split evenly over the waves");
    static_assert(BPM % 2 == 0, "weight rows must split over two waves");
    static_assert(SMEM <= 160 * 1024, "LDS");
    static_assert(NMAT * MBW * NBW * 16 <= 256, "accumulators");
};

// Fragments of two consecutive K steps for this wave's MB row groups.  With
// MXFP4 weights the weight operand is held as raw codes and decoded right
// before each MFMA (holding decoded fragments would double the registers the
// read-ahead needs): per 32-row weight group, the lane's 16 bytes of codes for
// all four steps of the stage, and their one E8M0 scale.
template <class C, int MB, bool MX = C::MX>
struct Frags2 {
    bf16x8 a[2][MB];
    bf16x8 b[2][C::NMAT][C::NBW];
};
template <class C, int MB>
struct Frags2<C, MB, true> {
    bf16x8 a[2][MB];
    u32x4 codes[C::NMAT][C::NBW];
    float sc[C::NMAT][C::NBW];  // 2^(scale - 127) as the fp32 with exponent field `scale`
};

// K order inside a 64-wide stage.  A 32x32x16 MFMA step q takes, in lane half
// h = l / 32, eight consecutive K elements of the row; any assignment of the
// stage's eight 8-element chunks to (q, h) gives the same contraction as long
// as both operands use it.  bf16 weights: chunk 2q + h.  MXFP4 weights: chunk
// 4h + q, so that a lane half's four steps span one 32-element scale group and
// its codes for the whole stage are 16 contiguous bytes (one LDS read, one
// scale per stage).
template <bool MX>
__device__ __forceinline__ int stage_chunk(int q, int h) { return MX ? 4 * h + q : 2 * q + h; }

// Fragments of K step q: lane offset within a 4-block (32-row) group.
template <bool MX>
__device__ __forceinline__ uint32_t frag_lane_off(int lane, int q) {
    const int r = lane & 31, rb = lane & 7;
    const int c = stage_chunk<MX>(q, lane >> 5);
    return (uint32_t)((r >> 3) * 1024 + rb * 128 + ((c ^ rb ^ ((r >> 3) & 1)) * 16));
}

// MXFP4 codes in LDS: a 32-row weight group's 32 bytes per row (64 K) are
// 16-byte slots, row r's half h (K chunks 4h .. 4h+3) in slot
// 2r + (h ^ ((r >> 3) & 1)), which spreads every 16 lanes' 16-byte reads over
// all 64 banks.  The DMA lane that fills slot s fetches row s / 2, half
// (s & 1) ^ ((s >> 4) & 1).
__device__ __forceinline__ uint32_t mx_code_slot(int r, int h) { return (uint32_t)(2 * r + (h ^ ((r >> 3) & 1))); }

// MXFP4: 8 codes (4 bytes) and their E8M0 scale -> 8 bf16, exactly.  For
// scales 2..252 every product is a normal bf16 (or zero) and the hardware
// scaled conversion is exact; EXACT takes the integer path that also covers
// the extremes (subnormal results, overflow, the NaN scale).  `sc` is the
// scale's fp32 (exponent field = scale), from which the integer path takes
// the scale back.
template <bool EXACT>
__device__ __forceinline__ bf16x8 mx_frag(uint32_t q, float sc) {
    u32x4 v;
    if constexpr (!EXACT) {
        v = u32x4{cvt_fp4x2_bf16x2(q, sc, 0), cvt_fp4x2_bf16x2(q, sc, 1), cvt_fp4x2_bf16x2(q, sc, 2),
                  cvt_fp4x2_bf16x2(q, sc, 3)};
    } else {
        const uint32_t scale = __float_as_uint(sc) >> 23;
        uint32_t w[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint32_t byte = (q >> (8 * bb)) & 0xffu;
            w[bb] = e2m1_to_bf16_exact(byte & 0xfu, scale) | (e2m1_to_bf16_exact(byte >> 4, scale) << 16);
        }
        v = u32x4{w[0], w[1], w[2], w[3]};
    }
    return __builtin_bit_cast(bf16x8, v);
}

// Where a lane's MXFP4 operand lives: its 16-byte code slot within a 32-row
// group, and its row's scales (kg bytes per row, this stage's group 2kt + h).
struct MxLane {
    uint32_t code_off;   // 16 * mx_code_slot(l % 32, l / 32)
    uint32_t scale_row;  // (l % 32) * kg + l / 32
};

// Read the fragments of steps q0, q0+1 of stage kt (held at `st`).  MXFP4
// codes and scales are read once per stage, with steps 0, 1; steps 2, 3 take
// them from `same`, the fragments of steps 0, 1 of this stage.
template <class C, int BN, int MB>
__device__ __forceinline__ void read_frags2(const unsigned char* st, const uint32_t (&loff)[4], int q0, int wm, int wn,
                                            Frags2<C, MB>& f, const Frags2<C, MB>& same, const unsigned char* scales,
                                            int kg, int kt, MxLane mxl) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
            f.a[h][i] = *reinterpret_cast<const bf16x8*>(st + (wm + kWM * i) * 4096 + loff[q0 + h]);
        if constexpr (!C::MX) {
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int grp = m * (BN / 32) + wn * C::NBW + j;  // 32-row weight group
                    f.b[h][m][j] = *reinterpret_cast<const bf16x8*>(st + C::A_BYTES + grp * 4096 + loff[q0 + h]);
                }
        }
    }
    if constexpr (C::MX) {
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j) {
                if (q0 == 0) {
                    const int grp = m * (BN / 32) + wn * C::NBW + j;
                    f.codes[m][j] = *reinterpret_cast<const u32x4*>(st + C::A_BYTES + grp * 1024 + mxl.code_off);
                    const uint32_t raw = scales[(uint32_t)grp * 32u * (uint32_t)kg + mxl.scale_row + 2 * kt];
                    f.sc[m][j] = __uint_as_float(raw << 23);
                } else {
                    f.codes[m][j] = same.codes[m][j];
                    f.sc[m][j] = same.sc[m][j];
                }
            }
    }
}

// Steps Q0, Q0+1.  EXACT (MXFP4 only): decode on the integer path, for tiles
// with a scale outside 2..252.
template <class C, int MB, int Q0, bool EXACT>
__device__ __forceinline__ void mma2(const Frags2<C, MB>& f, f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
            for (int j = 0; j < C::NBW; ++j) {
                bf16x8 b;
                if constexpr (C::MX) b = mx_frag<EXACT>(f.codes[m][j][Q0 + h], f.sc[m][j]);
                else b = f.b[h][m][j];
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[m][i][j] = mfma32(f.a[h][i], b, acc[m][i][j]);
            }
}



struct Srcs {
    buf_rsrc a;
    buf_rsrc w[2];
    buf_rsrc s[2];  // MXFP4 scales
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
    const uint32_t kb = C::MX ? (uint32_t)kt * (kBK / 2) : k0;  // bytes of codes or bf16 per row
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i)
        dma16(b_mat[i] ? src.w[1] : src.w[0], st + C::A_BYTES + (wave + kWaves * i) * 1024, b_voff[i], kb);
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

// MXFP4 tiles: each wave's verdict on the part of the tile's scales it
// copied into LDS (nonzero: a scale of a live weight row outside 2..252, so
// the tile decodes on the integer path).  Written during the item's set-up,
// read after the main loop's first barrier.
__device__ __forceinline__ int* wave_verdicts() {
    __shared__ int s_odd[kWaves];
    return s_odd;
}

__device__ __forceinline__ bool tile_needs_exact() {
    const int* v = wave_verdicts();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any |= v[w];
    return __builtin_amdgcn_readfirstlane(any) != 0;
}

// Everything a work item's main loop needs besides the accumulators.
template <class C>
struct ItemCtx {
    Srcs src;
    uint32_t a_voff[C::A_DMA];  // this lane's DMA source offsets in stage 0
    uint32_t b_voff[C::B_DMA];
    int b_mat[C::B_DMA];
    const unsigned char* scales;  // MXFP4: the tile's scales in LDS, [NMAT*BN][kg]
    int kg;                       // K / 32
    MxLane mxl;
};

// One stage kt: steps 2,3 are read while steps 0,1 compute; then (stage kt+1
// landed, one barrier: every wave is done reading stage kt) the freed slot is
// refilled with stage kt+NST (DMA) and steps 0,1 of stage kt+1 are read while
// steps 2,3 compute.  WAIT = stages allowed in flight at the wait (-1: read
// `ahead` at run time).
template <class C, int BN, int MB, bool EXACT, bool DMA, bool NEXT, int WAIT>
__device__ __forceinline__ void stage_iter(const ItemCtx<C>& x, unsigned char* smem, int nk, int kt, int wave, int wm,
                                           int wn, const uint32_t (&loff)[4], Frags2<C, MB>& lo, Frags2<C, MB>& hi,
                                           f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    // fragment reads per two steps (MXFP4: the weight codes once per stage, with the first half)
    constexpr int NR = 2 * MB + (C::MX ? 0 : 2 * C::NMAT * C::NBW);
    constexpr int NR0 = NR + (C::MX ? 2 * C::NMAT * C::NBW : 0);
    constexpr int NM = 2 * C::NMAT * C::NBW * MB;    // MFMAs per two steps
    const unsigned char* st = smem + (kt % C::NST) * C::STAGE;
    read_frags2<C, BN, MB>(st, loff, 2, wm, wn, hi, lo, x.scales, x.kg, kt, x.mxl);
    mma2<C, MB, 0, EXACT>(lo, acc);
    interleave<0, 0, NR, NM>();
    if constexpr (NEXT) {
        if constexpr (WAIT >= 0) wait_vmcnt<WAIT * C::DPS>();
        else wait_stages_ahead<C::DPS>(min(nk - 1, kt + C::NST - 1) - (kt + 1));
        wait_lds_reads();
        bare_barrier();
        if constexpr (DMA) dma_stage<C>(x.src, smem, kt + C::NST, wave, x.a_voff, x.b_voff, x.b_mat);
        read_frags2<C, BN, MB>(smem + ((kt + 1) % C::NST) * C::STAGE, loff, 0, wm, wn, lo, lo, x.scales, x.kg,
                               kt + 1, x.mxl);
        mma2<C, MB, 2, EXACT>(hi, acc);
        interleave<0, DMA ? C::DPS : 0, NR0, NM>();
    } else {
        mma2<C, MB, 2, EXACT>(hi, acc);
    }
}

template <class C, int BN, int MB, bool EXACT>
__device__ __forceinline__ void main_loop_body(const ItemCtx<C>& x, unsigned char* smem, int nk, int wave, int wm,
                                               int wn, const uint32_t (&loff)[4], Frags2<C, MB>& lo,
                                               Frags2<C, MB>& hi, f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    int kt = 0;
    // steady state: the next stage exists and a stage NST ahead is refilled
    for (; kt + C::NST < nk; ++kt)
        stage_iter<C, BN, MB, EXACT, true, true, C::NST - 2>(x, smem, nk, kt, wave, wm, wn, loff, lo, hi, acc);
    for (; kt + 1 < nk; ++kt)
        stage_iter<C, BN, MB, EXACT, false, true, -1>(x, smem, nk, kt, wave, wm, wn, loff, lo, hi, acc);
    stage_iter<C, BN, MB, EXACT, false, false, 0>(x, smem, nk, kt, wave, wm, wn, loff, lo, hi, acc);
}

// Stages 0 .. min(NST, nk) - 1 were issued by the caller.
template <class C, int BN, int MB>
__device__ __forceinline__ void main_loop(const ItemCtx<C>& x, unsigned char* smem, int nk, int wave, int lane,
                                          f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    const int wm = wave >> 1, wn = wave & 1;
    uint32_t loff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) loff[q] = frag_lane_off<C::MX>(lane, q);
    Frags2<C, MB> lo, hi;
    wait_stages_ahead<C::DPS>(min(nk, C::NST) - 1);
    wait_lds_reads();  // MXFP4: this wave's scale writes
    bare_barrier();
    read_frags2<C, BN, MB>(smem, loff, 0, wm, wn, lo, lo, x.scales, x.kg, 0, x.mxl);
    if constexpr (C::MX) {
        // the waves' verdicts on the tile's scales, written before the barrier above
        if (tile_needs_exact()) main_loop_body<C, BN, MB, true>(x, smem, nk, wave, wm, wn, loff, lo, hi, acc);
        else main_loop_body<C, BN, MB, false>(x, smem, nk, wave, wm, wn, loff, lo, hi, acc);
    } else {
        main_loop_body<C, BN, MB, false>(x, smem, nk, wave, wm, wn, loff, lo, hi, acc);
    }
}

// A wave with no live row group (the short last tile of an expert) still
// fills its share of every stage and meets every barrier of main_loop (one
// before the loop, one per stage that has a successor), but reads and
// multiplies nothing, which leaves its SIMD to the wave it shares it with.
template <class C>
__device__ __forceinline__ void dma_only_loop(const ItemCtx<C>& x, unsigned char* smem, int nk, int wave) {
    wait_stages_ahead<C::DPS>(min(nk, C::NST) - 1);
    wait_lds_reads();  // MXFP4: this wave's scale writes
    bare_barrier();
    int kt = 0;
    for (; kt + C::NST < nk; ++kt) {
        wait_vmcnt<(C::NST - 2) * C::DPS>();
        bare_barrier();
        dma_stage<C>(x.src, smem, kt + C::NST, wave, x.a_voff, x.b_voff, x.b_mat);
    }
    for (; kt + 1 < nk; ++kt) {
        wait_stages_ahead<C::DPS>(min(nk - 1, kt + C::NST - 1) - (kt + 1));
        bare_barrier();
    }
}

// Main loop for the MB live row groups of this wave (MB = 1 .. MBW), or the
// DMA-only loop for a wave with none.
template <class C, int BN, int MB>
__device__ __forceinline__ void dispatch_mb(int mine, const ItemCtx<C>& x, unsigned char* smem, int nk, int wave,
                                            int lane, f32x16 (&acc)[C::NMAT][C::MBW][C::NBW]) {
    if constexpr (MB == 1) {
        if (mine >= 1) main_loop<C, BN, 1>(x, smem, nk, wave, lane, acc);
        else dma_only_loop<C>(x, smem, nk, wave);
    } else {
        if (mine >= MB) main_loop<C, BN, MB>(x, smem, nk, wave, lane, acc);
        else dispatch_mb<C, BN, MB - 1>(mine, x, smem, nk, wave, lane, acc);
    }
}

// One work item q: (row tile, column tile) of the work list.
template <int MODE, int BN, int S, bool MXW>
__device__ __forceinline__ void process_item(const BArgs& args, int q) {
    using C = Cfg<MODE, BN, S, MXW>;
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
    const int rb = lane >> 3;                                  // row within an 8-row DMA block
    const uint32_t chunk_even = (uint32_t)((lane & 7) ^ rb);  // logical 16-byte chunk fetched (even block)

    ItemCtx<C> x;
    x.kg = K / 32;
    x.scales = smem + C::SMEM;
    x.mxl.code_off = 16u * mx_code_slot(lane & 31, lane >> 5);
    x.mxl.scale_row = (uint32_t)((lane & 31) * x.kg + (lane >> 5));
    // ---- DMA sources: byte offsets of this lane's chunk in stage 0 ----
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i) {
        const int blk = wave + kWaves * i;
        const int r = blk * 8 + rb;
        const int rr = r < rows ? r : 0;
        int src_row;
        if constexpr (MODE == 0) src_row = args.perm_src[row0 + rr] / args.k;
        else src_row = row0 + rr;
        x.a_voff[i] = (uint32_t)src_row * (uint32_t)K * 2u + (chunk_even ^ (uint32_t)(blk & 1)) * 16u;
    }
    x.src.a = make_rsrc(args.a_src, args.a_bytes);
    if constexpr (C::MX) {
        const uint32_t wb = (uint32_t)((size_t)N * K / 2), sb = (uint32_t)((size_t)N * K / 32);
        x.src.w[0] = make_rsrc((const unsigned char*)args.w0 + (size_t)e * wb, wb);
        x.src.w[1] = MODE == 0 ? make_rsrc((const unsigned char*)args.w1 + (size_t)e * wb, wb) : x.src.w[0];
        x.src.s[0] = make_rsrc(args.s0 + (size_t)e * sb, sb);
        x.src.s[1] = MODE == 0 ? make_rsrc(args.s1 + (size_t)e * sb, sb) : x.src.s[0];
        // 32-row blocks of codes: lane l fills slot l, i.e. row l/2, half (l%2) ^ ((l/16)%2) of the stage's 32 bytes
#pragma unroll
        for (int i = 0; i < C::B_DMA; ++i) {
            const int blk = wave + kWaves * i;
            x.b_mat[i] = (blk * 32) / BN;
            const int n = min(n0 + (blk * 32) % BN + (lane >> 1), N - 1);
            x.b_voff[i] = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)((lane & 1) ^ ((lane >> 4) & 1)) * 16u;
        }
        // the tile's scales for all of K: [matrix][BN rows][kg], rows past N
        // read as zero; the bytes of live rows are checked on the way
        const int per_mat = BN * x.kg;  // bytes, a multiple of 16
        const int live = min(BN, N - n0) * x.kg;
        unsigned char* sc = smem + C::SMEM;
        uint32_t odd = 0;
        for (int m = 0; m < C::NMAT; ++m)
            for (int c = tid * 16; c < per_mat; c += kThreads * 16) {
                const u32x4 v = buf_load16(x.src.s[m], (uint32_t)(n0 * x.kg + c), 0);
                *reinterpret_cast<u32x4*>(sc + m * per_mat + c) = v;
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    const uint32_t raw = (v[b >> 2] >> (8 * (b & 3))) & 0xffu;
                    odd |= (uint32_t)(c + b < live) & (uint32_t)(raw - 2u > 250u);
                }
            }
        const uint64_t ballot = __builtin_amdgcn_ballot_w64(odd != 0);
        if (lane == 0) wave_verdicts()[wave] = ballot != 0;
    } else {
        const uint32_t wbytes = (uint32_t)((size_t)N * K * 2);
        x.src.w[0] = make_rsrc((const unsigned char*)args.w0 + (size_t)e * wbytes, wbytes);
        x.src.w[1] = MODE == 0 ? make_rsrc((const unsigned char*)args.w1 + (size_t)e * wbytes, wbytes) : x.src.w[0];
        x.src.s[0] = x.src.s[1] = x.src.w[0];
#pragma unroll
        for (int i = 0; i < C::B_DMA; ++i) {
            const int blk = wave + kWaves * i;
            x.b_mat[i] = (blk * 8) / BN;
            const int n = min(n0 + (blk * 8) % BN + rb, N - 1);
            x.b_voff[i] = (uint32_t)n * (uint32_t)K * 2u + (chunk_even ^ (uint32_t)(blk & 1)) * 16u;
        }
    }

    const int nk = K / kBK;
#pragma unroll
    for (int s = 0; s < C::NST; ++s)
        if (s < nk) dma_stage<C>(x.src, smem, s, wave, x.a_voff, x.b_voff, x.b_mat);

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
    dispatch_mb<C, BN, C::MBW>(mine, x, smem, nk, wave, lane, acc);

    // ---- epilogue: D[v] of a 32x32 tile is row 8(v/4) + 4(l/32) + v%4, column l%32 ----
    const int fr = lane & 31, fh = lane >> 5;
    if constexpr (MODE == 0) {
        // act = bf16(silu(g) u), stored as column pairs: lanes l and l^1 hold
        // columns c and c+1 (c even) of the same rows, so one exchange per
        // pair of rows v, v+1 gives the even lane row v and the odd lane row
        // v+1 of both columns, one 4-byte store each.  The stores go through a
        // buffer that spans the tile's rows of act: rows past the tile lie
        // beyond it, columns past N get an offset beyond it, and the hardware
        // drops both, so the loop has no branches.
        const int odd = lane & 1;
        const uint32_t N2 = (uint32_t)N * 2u;
        const buf_rsrc ob =
            make_rsrc(reinterpret_cast<const uint16_t*>(args.out) + (size_t)row0 * N, (uint32_t)rows * N2);
#pragma unroll
        for (int j = 0; j < C::NBW; ++j) {
            const int n = n0 + (wn * C::NBW + j) * 32 + (fr & ~1);  // N is even: n < N covers n + 1
            const uint32_t cb = n < N ? (uint32_t)(wm * 32 + 4 * fh + odd) * N2 + (uint32_t)n * 2u : kOobStore;
#pragma unroll
            for (int i = 0; i < C::MBW; ++i) {
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float a0 = silu_fast(acc[0][i][j][v]) * acc[1][i][j][v];
                    const float a1 = silu_fast(acc[0][i][j][v + 1]) * acc[1][i][j][v + 1];
                    const float got = dpp_f<kDppXor1>(odd ? a0 : a1);
                    const uint32_t w = pack_bf16x2(odd ? got : a0, odd ? a1 : got);
                    const uint32_t ro = (uint32_t)(kWM * i * 32 + 8 * (v >> 2) + (v & 3)) * N2;
                    __builtin_amdgcn_raw_buffer_store_b32(w, ob, cb + ro, 0, 0);
                }
            }
        }
    } else {
        // Each row's assignment and routing weight, fetched once per tile (two
        // independent loads per row: the weight is stored per row beside the
        // permutation) into the LDS ring, idle once every wave has read its
        // last fragments; the stores below then wait on no load.  The next
        // item's DMA into the ring follows the barrier of the work loop.
        int2* rtab = reinterpret_cast<int2*>(smem);
        wait_lds_reads();
        bare_barrier();
        if (tid < rows) {  // rows <= kBM <= kThreads
            const int asg = args.perm_src[row0 + tid];
            const float pw = args.row_p[row0 + tid];
            rtab[tid] = make_int2(asg, __float_as_int(pw));
        }
        wait_lds_reads();
        bare_barrier();
        // One address per row: the NBW stores of a row are 128 bytes apart
        // (immediate offsets), and a tile that lies wholly inside N (every
        // tile when BN divides N) needs no column test.
        const int nb = n0 + wn * C::NBW * 32 + fr;  // this lane's first column
        const bool full = n0 + BN <= N;             // the same for the whole workgroup
#pragma unroll
        for (int i = 0; i < C::MBW; ++i) {
            int2 ap[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = (wm + kWM * i) * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                ap[v] = rtab[max(min(r, rows - 1), 0)];
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = (wm + kWM * i) * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                if (r >= rows) continue;
                const float p = __int_as_float(ap[v].y);
                float* orow = reinterpret_cast<float*>(args.out) + (size_t)ap[v].x * N + nb;
                if (full) {
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j) orow[j * 32] = acc[0][i][j][v] * p;
                } else {
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j)
                        if (nb + j * 32 < N) orow[j * 32] = acc[0][i][j][v] * p;
                }
            }
        }
    }
}

// Persistent workgroups, one per CU.  Blocks are dealt round-robin to the 8
// XCDs; XCD x owns the x-th of 8 contiguous ranges of the work list, cut by
// the route scan so that their estimated costs are equal (a short row tile
// costs less than a full one), and its workgroups take the range's items
// in order from the XCD's counter, so a workgroup that drew cheap items (the
// short last row tile of an expert) takes more of them, and the row tiles
// sharing a weight tile still run together on one XCD.
template <int MODE, int BN, int S, bool MXW>
__device__ __forceinline__ void gemm_body(const BArgs& args) {
    __shared__ int s_q;
    const int n_work = args.n_work[0];
    const int xcd = blockIdx.x % kXcds;
    const int base = min(max(args.bounds[xcd], 0), n_work);
    const int end = min(max(args.bounds[xcd + 1], base), n_work);
    for (;;) {
        if (threadIdx.x == 0) s_q = base + atomicAdd(args.queue + xcd, 1);
        // s_q visible to every wave, and every wave done with the previous item's LDS
        wait_lds_reads();
        bare_barrier();
        const int q = __builtin_amdgcn_readfirstlane(s_q);
        if (q >= end) break;
        process_item<MODE, BN, S, MXW>(args, q);
    }
}

// MXFP4 weights: a quarter of the bytes per stage, so three stages fit beside
// the tile's scales.
template <bool MXW>
using CfgGateUp = Cfg<0, kBNGateUp, MXW ? 3 : kStagesGateUp, MXW>;
template <bool MXW>
using CfgDown = Cfg<1, kBNDown<MXW>, MXW ? 3 : kStagesDown, MXW>;

template <bool MXW>
__global__ __launch_bounds__(kThreads) void gateup_bf16_kernel(BArgs args) {
    gemm_body<0, kBNGateUp, CfgGateUp<MXW>::NST, MXW>(args);
}
template <bool MXW>
__global__ __launch_bounds__(kThreads) void down_bf16_kernel(BArgs args) {
    gemm_body<1, kBNDown<MXW>, CfgDown<MXW>::NST, MXW>(args);
}

BArgs make_args(const GemmProblem& p, int mode) {
    BArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.row_p = p.row_p;
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
        a.bounds = p.bounds_gateup;
        a.queue = p.queues;
        a.n_ntiles = (p.I + kBNGateUp - 1) / kBNGateUp;
    } else {
        a.a_src = (const uint16_t*)p.act;
        a.a_bytes = (uint32_t)((size_t)p.T * p.k * p.I * 2);
        a.w0 = p.w_down;
        a.w1 = p.w_down;
        a.s0 = p.s_down;
        a.s1 = p.s_down;
        a.out = p.y;
        a.K = p.I;
        a.N = p.H;
        a.work = p.work_down;
        a.n_work = p.n_work_down;
        a.bounds = p.bounds_down;
        a.queue = p.queues + kXcds;
        a.n_ntiles = bf16_col_tiles(p.H, 1, p.expert_dtype);
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
int bf16_col_tiles(int N, int mode, int expert_dtype) {
    const int bn = mode == 0 ? kBNGateUp : expert_dtype == DT_MXFP4 ? kBNDown<true> : kBNDown<false>;
    return (N + bn - 1) / bn;
}

// Dynamic LDS a workgroup may use: 160 KB less room for the static work-item slot.
constexpr size_t kMaxLds = 160 * 1024 - 1024;

// Largest contraction depth the MXFP4 kernels take (the tile's scales for all
// of K sit in LDS beside the ring), a multiple of 64.
int mxfp4_max_k() {
    const size_t fixed = CfgGateUp<true>::SMEM > CfgDown<true>::SMEM ? CfgGateUp<true>::SMEM : CfgDown<true>::SMEM;
    const size_t rows = 2 * kBNGateUp > kBNDown<true> ? 2 * kBNGateUp : kBNDown<true>;
    return (int)((kMaxLds - fixed) / rows * 32) / 64 * 64;
}

template <auto Kern>
hipError_t launch_mode(size_t smem, const BArgs& a, hipStream_t stream) {
    const hipError_t attr = set_max_dynamic_lds<Kern>((int)kMaxLds);
    if (attr != hipSuccess) return attr;
    return launch(Kern, smem, a, stream);
}

hipError_t launch_gateup_bf16w(const GemmProblem& p, hipStream_t stream) {
    const BArgs a = make_args(p, 0);
    if ((size_t)kBM * (size_t)a.N * 2u >= ((size_t)1 << 30)) return hipErrorInvalidValue;  // epilogue buffer range
    if (p.expert_dtype == DT_MXFP4) return launch_mode<gateup_bf16_kernel<true>>(CfgGateUp<true>::smem(a.K), a, stream);
    return launch_mode<gateup_bf16_kernel<false>>(CfgGateUp<false>::smem(a.K), a, stream);
}

hipError_t launch_down_bf16w(const GemmProblem& p, hipStream_t stream) {
    const BArgs a = make_args(p, 1);
    if (p.expert_dtype == DT_MXFP4) return launch_mode<down_bf16_kernel<true>>(CfgDown<true>::smem(a.K), a, stream);
    return launch_mode<down_bf16_kernel<false>>(CfgDown<false>::smem(a.K), a, stream);
}

}  // namespace moe
