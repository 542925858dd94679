// The layer for decode-sized batches (few rows per expert), organised for the
// case where it is bound by reading the experts' weights once from HBM rather
// than by the matrix cores.  The two grouped products are those of the
// prefill kernels,
//
//   act[r]  = silu(W_gate[e] . x_r) * (W_up[e] . x_r)       x_r = h[perm_src[r] / k]
//   Y[a]    = p_a * (W_down[e] . act[r])                     a = perm_src[r]
//
// ("gpt-oss-40b-64a8-init" page, section 2, Proof; "gpt-oss 20B" field guide,
// cutaway 03: SwiGLU experts).
//
// Products.  One wave computes one (row tile of at most 16 rows of one expert)
// x (up to 32 weight rows) block with 16x16x32 bf16 MFMAs: the weights are
// the A operand, streamed from HBM straight into registers (no LDS, no
// barriers), the tile's activation rows are the B operand (small,
// L2-resident).  Lanes of rows past the tile's end, and weight rows past the
// end of a block, read at an offset beyond the buffer, which returns zero
// without touching memory.
//
// K is walked 128 at a time, as four 32-deep MFMA steps j.  For bf16 weights
// each load instruction takes the native MFMA order (lane (row l%16, quarter
// q = l/16) reads K elements 128g + 32j + 8q .. +7), so one instruction reads
// 64 contiguous bytes of each of 16 weight rows; at this size every
// per-instruction row segment from 64 to 256 bytes streams at the same rate.
// For MXFP4 a lane takes the 32 codes [128g + 32q, 128g + 32q + 32) of its
// row (16 bytes) and their one E8M0 scale, and feeds them to the four steps
// as elements 8j..8j+7; a contraction is unchanged by a permutation of K
// applied to both operands, so the activation operand is read in the same
// permuted order.  The MXFP4 block kernels copy the codes into LDS a whole
// 128-byte line per weight row at a time (see decode_pass_lds) and keep the
// block's scales in LDS for the whole contraction.  All loads of a K step
// are issued before its MFMAs (scheduling barriers keep the compiler from
// interleaving them, which would leave only a few loads in flight); the
// block kernels keep the next step's loads in flight while multiplying.
//
// Work split.  bf16 gate/up runs with one workgroup per CU: the (tile, weight
// row) pairs are split into equal contiguous ranges, one per workgroup, and
// each range into equal sub-ranges, one per wave, with boundaries on
// multiples of four rows; a wave walks its sub-range in passes of at most 32
// rows.  Down (64-row blocks) and MXFP4 gate/up (32-row blocks) run one block
// per wave, in one-wave workgroups (measured faster for these).
//
// Fused routing.  When the batch and the router are small (T <= 64, E <= 64)
// a small kernel writes partial router logits (K split into slices), and
// every gate/up workgroup then completes the routing of the batch itself -
// logits, top-k, softmax over the selected set, the stable expert-major order
// and the tile list - in its LDS; workgroup 0 also writes it out for the down
// product and the caller.  Redundant, but a few microseconds of work on data
// in L2 instead of the router's and the route scan's dependent launches.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kDecRows = 16;           // rows per tile (MFMA N)
constexpr int kPanels = 2;             // 16-row weight panels per pass
constexpr int kDecCols = 16 * kPanels; // weight rows per pass
constexpr int kRowAlign = 4;           // range boundaries: whole 8-/16-byte output stores
constexpr int kGuWaves = 12;           // gate/up: waves per workgroup, one workgroup per CU
constexpr int kBlkWaves = 1;           // one-block-per-wave kernels: waves per workgroup (independent)
constexpr int kMinLds = 96 * 1024;     // LDS per gate/up workgroup: room for no second one on the CU
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
    const float* row_p;  // routing weight of each expert-major row (down)
    const Tile* tiles;
    const int32_t* n_tiles;
    void* out;          // act [T*k][N] bf16 (gate/up) or Y [T*k][N] f32 (down)
    int K, N, k, max_tiles;
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }

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

// The loads of one 128-wide K step, in flat register arrays (weights of
// panel p: wq[4p..4p+3] for bf16, wq[p] + ws[p] for MXFP4; up weights in
// uq / us; activations in b).
template <int MODE, int WDT, int NP>
struct Batch {
    static constexpr int NQ = WDT == DT_MXFP4 ? NP : 4 * NP;
    u32x4 wq[NQ];
    u32x4 uq[MODE == 0 ? NQ : 1];
    uint32_t ws[NP];
    uint32_t us[NP];
    u32x4 b[4];
};

template <int MODE, int WDT, int NP>
__device__ __forceinline__ void issue(Batch<MODE, WDT, NP>& x, buf_rsrc w0, buf_rsrc w1, buf_rsrc s0, buf_rsrc s1,
                                      buf_rsrc bsrc, const uint32_t (&n)[NP], const bool (&nv)[NP],
                                      uint32_t b_base, bool has_row, uint32_t K, uint32_t g, uint32_t qd) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if constexpr (WDT == DT_MXFP4) {
            const uint32_t kq = g * 128 + qd * 32;
            const bool kv = nv[p] && kq < K;
            const uint32_t co = kv ? n[p] * (K / 2) + kq / 2 : kOob, so = kv ? n[p] * (K / 32) + kq / 32 : kOob;
            x.wq[p] = buf_load16(w0, co, 0);
            x.ws[p] = buf_load1(s0, so, 0);
            if constexpr (MODE == 0) {
                x.uq[p] = buf_load16(w1, co, 0);
                x.us[p] = buf_load1(s1, so, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t kk = g * 128 + 32 * j + 8 * qd;
                const uint32_t o = (nv[p] && kk < K) ? (n[p] * K + kk) * 2u : kOob;
                x.wq[4 * p + j] = buf_load16(w0, o, 0);
                if constexpr (MODE == 0) x.uq[4 * p + j] = buf_load16(w1, o, 0);
            }
        }
    }
    load_b<WDT>(bsrc, b_base, has_row, K, g, qd, x.b);
}

template <int PATH, int NQ>
__device__ __forceinline__ void frags(const u32x4 (&q)[NQ], uint32_t scale, int p, bf16x8 (&f)[4]) {
    uint32_t d[16];
    decode_mxfp4_32<PATH>(q[p], scale, d);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        f[j] = __builtin_bit_cast(bf16x8, u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]});
}

template <int MODE, int WDT, int NP, int PATH>
__device__ __forceinline__ void compute_mx(const Batch<MODE, WDT, NP>& x, f32x4 (&acc0)[NP], f32x4 (&acc1)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        bf16x8 fa[4];
        frags<PATH>(x.wq, x.ws[p], p, fa);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc0[p] = mfma16(fa[j], __builtin_bit_cast(bf16x8, x.b[j]), acc0[p]);
        if constexpr (MODE == 0) {
            bf16x8 fu[4];
            frags<PATH>(x.uq, x.us[p], p, fu);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc1[p] = mfma16(fu[j], __builtin_bit_cast(bf16x8, x.b[j]), acc1[p]);
        }
    }
}

// UNIFORM (MXFP4): one decode path per wave and K step (else per lane, which
// costs fewer registers).
template <int MODE, int WDT, int NP, bool UNIFORM = false>
__device__ __forceinline__ void compute(const Batch<MODE, WDT, NP>& x, f32x4 (&acc0)[NP], f32x4 (&acc1)[NP]) {
    if constexpr (WDT != DT_MXFP4) {
        // each 16-byte register straight into its MFMA (no fragment copies,
        // which would keep the batch in scratch memory)
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 bj = __builtin_bit_cast(bf16x8, x.b[j]);
                acc0[p] = mfma16(__builtin_bit_cast(bf16x8, x.wq[4 * p + j]), bj, acc0[p]);
                if constexpr (MODE == 0) acc1[p] = mfma16(__builtin_bit_cast(bf16x8, x.uq[4 * p + j]), bj, acc1[p]);
            }
    } else if constexpr (!UNIFORM) {
        compute_mx<MODE, WDT, NP, 0>(x, acc0, acc1);
    } else {
        // one decision per wave and K step: the hardware decode unless a lane
        // holds a scale outside 2..252
        uint32_t odd = 0;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            odd |= (uint32_t)(x.ws[p] - 2u > 250u);
            if constexpr (MODE == 0) odd |= (uint32_t)(x.us[p] - 2u > 250u);
        }
        if (__builtin_amdgcn_ballot_w64(odd != 0) != 0) compute_mx<MODE, WDT, NP, 2>(x, acc0, acc1);
        else compute_mx<MODE, WDT, NP, 1>(x, acc0, acc1);
    }
}

// MXFP4 scales of one block, staged in LDS: the 16 rows of a panel keep their
// K/32 scale bytes contiguous in memory, so a few 4-byte-per-lane loads copy a
// panel's scales for the whole contraction straight into LDS (no registers),
// instead of one 1-byte load per K step (whose per-instruction cost dominated
// the decode kernels).  Layout: [panel][matrix] segments of nj 256-byte lines,
// nj = ceil(16 K/32 / 256), row r of a panel at byte r K/32 of its segment; a
// lane's dword past the panel's bytes lands in its own segment's padding.
typedef __attribute__((address_space(3))) void lds_void;
constexpr uint32_t kScaleMaxKg = 160;  // largest K/32 staged (MXFP4 layers: K <= 4992)

__host__ __device__ constexpr uint32_t scale_lines(uint32_t KG) { return (16 * KG + 255) / 256; }

template <int NP, int NMAT>
__device__ __forceinline__ void scales_dma(buf_rsrc s0, buf_rsrc s1, uint32_t c0, uint32_t KG, uint8_t* sl,
                                           int lane) {
    const uint32_t nj = scale_lines(KG);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint32_t base = (c0 + 16 * p) * KG;  // rows past N read past the buffer: 0
            uint8_t* seg = sl + (p * NMAT + m) * nj * 256;
            for (uint32_t j = 0; j < nj; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(m ? s1 : s0, (lds_void*)(seg + j * 256), 4,
                                                         base + j * 256 + (uint32_t)lane * 4, 0, 0, 0);
        }
}

// Scales of K step g for this lane from the LDS copy (127, i.e. one, past K
// or past the block, where the codes read as zeros: a NaN scale must not
// meet them, and a scale in 2..252 keeps the step on the hardware decode).
template <int MODE, int WDT, int NP>
__device__ __forceinline__ void scales_fetch(Batch<MODE, WDT, NP>& x, const uint8_t* sl, const bool (&nv)[NP],
                                             uint32_t KG, uint32_t g, int r, uint32_t qd) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    const uint32_t grp = 4 * g + qd, seg = scale_lines(KG) * 256;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const bool kv = nv[p] && grp < KG;
        const uint32_t o = (uint32_t)(p * NMAT) * seg + (uint32_t)r * KG + grp;
        x.ws[p] = kv ? sl[o] : 127u;
        if constexpr (MODE == 0) x.us[p] = kv ? sl[o + seg] : 127u;
    }
}

// Epilogue of a block.  D: lane l holds weight rows 4(l/16)+i (i = 0..3) of
// the panel, for row l%16 of the tile; c0 and c1 are multiples of four, so
// those four rows are all present or all absent.
template <int MODE, int NP>
__device__ __forceinline__ void store_block(const DArgs& a, const f32x4 (&acc0)[NP], const f32x4 (&acc1)[NP],
                                            int row0, int r, uint32_t qd, bool has_row, uint32_t c0, uint32_t c1,
                                            int asg, float pw) {
    const uint32_t N = (uint32_t)a.N;
    if (!has_row) return;
    if constexpr (MODE == 0) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (size_t)(row0 + r) * N;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const uint32_t n0 = c0 + (uint32_t)(p * 16) + 4 * qd;
            if (n0 >= c1) continue;
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16_bits(silu_f(acc0[p][i]) * acc1[p][i]);
            *reinterpret_cast<uint2*>(orow + n0) = uint2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
        }
    } else {
        float* orow = reinterpret_cast<float*>(a.out) + (size_t)asg * N;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const uint32_t n0 = c0 + (uint32_t)(p * 16) + 4 * qd;
            if (n0 >= c1) continue;
            *reinterpret_cast<float4*>(orow + n0) =
                float4{acc0[p][0] * pw, acc0[p][1] * pw, acc0[p][2] * pw, acc0[p][3] * pw};
        }
    }
}

// One block: weight rows [c0, c1) (c1 - c0 <= 16 NP, both multiples of four)
// of the expert of `tile` against the tile's activation rows; perm holds the
// assignment of every expert-major row (global memory or LDS).  DEPTH = K
// steps of loads in flight (1 or 2).
template <int MODE, int WDT, int DEPTH, int NP = kPanels>
__device__ __forceinline__ void decode_pass(const DArgs& a, const Tile tile, const int32_t* perm, uint32_t c0,
                                            uint32_t c1, int lane) {
    const int e = tile.expert, row0 = tile.row_start, rows = tile.rows;
    const uint32_t K = (uint32_t)a.K, N = (uint32_t)a.N;
    const int r = lane & 15;
    const uint32_t qd = (uint32_t)(lane >> 4);

    // activation operand: this lane's row, or none (reads past the buffer)
    const bool has_row = r < rows;
    uint32_t b_base = 0;
    if (has_row) {
        const int src = MODE == 0 ? perm[row0 + r] / a.k : row0 + r;
        b_base = (uint32_t)src * K * 2u;
    }
    const buf_rsrc bsrc = make_rsrc(a.a_src, a.a_bytes);

    // weight operand: rows n[p] of expert e, present while below c1
    uint32_t n[NP];
    bool nv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        n[p] = c0 + (uint32_t)(p * 16 + r);
        nv[p] = n[p] < c1;
    }
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

    f32x4 acc0[NP], acc1[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Steps past the end read beyond K: zeros, no memory traffic.
    const uint32_t ng = (K + 127) / 128;
    Batch<MODE, WDT, NP> x0, x1;
    if constexpr (DEPTH == 1) {
        for (uint32_t g = 0; g < ng; ++g) {
            issue<MODE, WDT, NP>(x0, w0, w1, s0, s1, bsrc, n, nv, b_base, has_row, K, g, qd);
            __builtin_amdgcn_sched_barrier(0);
            compute<MODE, WDT, NP>(x0, acc0, acc1);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        issue<MODE, WDT, NP>(x0, w0, w1, s0, s1, bsrc, n, nv, b_base, has_row, K, 0, qd);
        for (uint32_t g = 0; g < ng; g += 2) {
            issue<MODE, WDT, NP>(x1, w0, w1, s0, s1, bsrc, n, nv, b_base, has_row, K, g + 1, qd);
            __builtin_amdgcn_sched_barrier(0);
            compute<MODE, WDT, NP>(x0, acc0, acc1);
            __builtin_amdgcn_sched_barrier(0);
            issue<MODE, WDT, NP>(x0, w0, w1, s0, s1, bsrc, n, nv, b_base, has_row, K, g + 2, qd);
            __builtin_amdgcn_sched_barrier(0);
            compute<MODE, WDT, NP>(x1, acc0, acc1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // down: the row's assignment and routing weight, two independent loads
    // (loading them before the K loop measured slower here)
    int asg = 0;
    float pw = 0.f;
    if (MODE == 1 && has_row) {
        asg = perm[row0 + r];
        pw = a.row_p[row0 + r];
    }
    store_block<MODE, NP>(a, acc0, acc1, row0, r, qd, has_row, c0, c1, asg, pw);
}

// MXFP4 codes through LDS.  A super-step is 256 K: 128 bytes of every weight
// row of the block.  A row's codes start anywhere on the 128-byte line grid
// (row n at byte n K/2 of its expert), so the copies follow the grid, not the
// rows: line j of a row is the j-th 128-byte memory line from the one holding
// its first code, and super-step s reads lines s and s + 1.  Every request
// the L1 sends on is then a whole line; copying the rows' own 128-byte
// spans, which straddle two lines, made twice the requests and ran about 10%
// slower.  The block's 16 NP NMAT row lines (L = 16 (p NMAT + m) + r for
// panel p, matrix m, row r of the panel) take 2 NP NMAT DMA instructions of
// 16 bytes per lane, 8 lanes per line; a lane copies only the 16-byte units
// inside its row (the rest read as zero, without memory traffic).  Position
// u of line L in LDS holds unit u ^ ((r >> 1) & 7) of the memory line: a K
// step reads 16 B at 16 rows of a panel with few bank conflicts.  A ring of
// three slots holds lines s and s + 1 while line s + 2 is copied.  Step h
// (0, 1) of super-step s is K step g = 2 s + h, with the K order of the
// register path (lane quarter qd takes the codes of K [256 s + 32 c, + 32),
// c = 4 h + qd).  Smaller blocks (16-row gate/up, 32-row down) measured
// slower.
constexpr int kMxRing = 3;  // ring slots (lines) for the codes
// bytes of one ring slot: a line of each of the block's 16 NP NMAT rows
template <int NP, int NMAT>
constexpr uint32_t ring_slot() { return 16u * NP * NMAT * 128u; }

template <int NP, int NMAT>
__device__ __forceinline__ void line_dma(buf_rsrc w0, buf_rsrc w1, const uint32_t (&row_base)[2 * NP * NMAT],
                                         const int32_t (&rel)[2 * NP * NMAT], uint32_t half_k, uint32_t j,
                                         unsigned char* slot) {
#pragma unroll
    for (int i = 0; i < 2 * NP * NMAT; ++i) {
        const int m = (i / 2) % NMAT;
        const uint32_t t = 128u * j + (uint32_t)rel[i];  // byte of the unit within its row (unsigned: < 0 is large)
        const uint32_t o = t < half_k ? row_base[i] + t : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(m ? w1 : w0, (lds_void*)(slot + i * 1024), 16, o, 0, 0, 0);
    }
}

template <int MODE, int NP>
__device__ __forceinline__ void decode_pass_lds(const DArgs& a, const Tile tile, const int32_t* perm, uint32_t c0,
                                                uint32_t c1, int lane, unsigned char* lds) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    constexpr int D = kMxRing;
    const int e = tile.expert, row0 = tile.row_start, rows = tile.rows;
    const uint32_t K = (uint32_t)a.K, N = (uint32_t)a.N, half_k = K / 2;
    const int r = lane & 15;
    const uint32_t qd = (uint32_t)(lane >> 4);

    const bool has_row = r < rows;
    uint32_t b_base = 0;
    int asg = 0;     // down: this lane's row's assignment and routing weight, loaded
    float pw = 0.f;  // now (two independent loads) for the stores at the end
    if (has_row) {
        const int src = MODE == 0 ? perm[row0 + r] / a.k : row0 + r;
        b_base = (uint32_t)src * K * 2u;
        if constexpr (MODE == 1) {
            asg = perm[row0 + r];
            pw = a.row_p[row0 + r];
        }
    }
    const buf_rsrc bsrc = make_rsrc(a.a_src, a.a_bytes);
    bool nv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) nv[p] = c0 + (uint32_t)(p * 16 + r) < c1;

    const uint32_t wb = N * half_k, sb = N * K / 32;
    const unsigned char* wp0 = (const unsigned char*)a.w0 + (size_t)e * wb;
    const unsigned char* wp1 = MODE == 0 ? (const unsigned char*)a.w1 + (size_t)e * wb : wp0;
    const buf_rsrc w0 = make_rsrc(wp0, wb);
    const buf_rsrc s0 = make_rsrc(a.s0 + (size_t)e * sb, sb);
    const buf_rsrc w1 = MODE == 0 ? make_rsrc(wp1, wb) : w0;
    const buf_rsrc s1 = MODE == 0 ? make_rsrc(a.s1 + (size_t)e * sb, sb) : s0;
    // byte of the line grid where each matrix's expert block starts
    const uint32_t grid0 = (uint32_t)reinterpret_cast<uintptr_t>(wp0) & 127u;
    const uint32_t grid1 = (uint32_t)reinterpret_cast<uintptr_t>(wp1) & 127u;

    // DMA side: instruction i = 2 (p NMAT + m) + hh; lane l copies position
    // l % 8 of the line of row 8 hh + l / 8 of panel p, matrix m
    uint32_t row_base[2 * NP * NMAT];
    int32_t rel[2 * NP * NMAT];
    {
        const uint32_t pos = (uint32_t)(lane & 7);
#pragma unroll
        for (int i = 0; i < 2 * NP * NMAT; ++i) {
            const int pm = i / 2, p = pm / NMAT, m = pm % NMAT;
            const uint32_t rr = (uint32_t)(lane >> 3) + 8u * (uint32_t)(i & 1);
            const uint32_t n = c0 + 16u * (uint32_t)p + rr;
            const uint32_t off = ((m ? grid1 : grid0) + n * half_k) & 127u;  // first code's byte in its line
            const uint32_t u = pos ^ ((rr >> 1) & 7u);
            row_base[i] = n < c1 ? n * half_k : kOob;
            rel[i] = (int32_t)(16u * u) - (int32_t)off;
        }
    }
    // read side: the line position of this lane's rows' first codes, in 16-byte units
    uint32_t rd_o[NP * NMAT];
#pragma unroll
    for (int pm = 0; pm < NP * NMAT; ++pm) {
        const uint32_t n = c0 + 16u * (uint32_t)(pm / NMAT) + (uint32_t)r;
        rd_o[pm] = ((((pm % NMAT) ? grid1 : grid0) + n * half_k) & 127u) >> 4;
    }
    const uint32_t rd_row = (uint32_t)r * 128u, rd_sw = ((uint32_t)r >> 1) & 7u;
    unsigned char* ring = lds;
    constexpr uint32_t kSlot = ring_slot<NP, NMAT>();
    uint8_t* sl = lds + D * kSlot;

    f32x4 acc0[NP], acc1[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t KG = K / 32, ns = (K + 255) / 256;
    u32x4 bq[2][2][4];  // activations of super-steps s and s+1 (two K steps each)

    // issue order: scales, line 0, line 1, activations B_0; super-step s
    // issues line s + 2, then B_{s+1}, after which lines s, s + 1 and B_s
    // are all but the last loads issued
    scales_dma<NP, NMAT>(s0, s1, c0, KG, sl, lane);
    line_dma<NP, NMAT>(w0, w1, row_base, rel, half_k, 0, ring);
    line_dma<NP, NMAT>(w0, w1, row_base, rel, half_k, 1, ring + kSlot);
    load_b<DT_MXFP4>(bsrc, b_base, has_row, K, 0, qd, bq[0][0]);
    load_b<DT_MXFP4>(bsrc, b_base, has_row, K, 1, qd, bq[0][1]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    uint32_t slot_s = 0;  // ring slot of line s
    auto step = [&](uint32_t s, int cur) {
        const uint32_t slot_s1 = slot_s == D - 1 ? 0 : slot_s + 1, slot_s2 = slot_s1 == D - 1 ? 0 : slot_s1 + 1;
        line_dma<NP, NMAT>(w0, w1, row_base, rel, half_k, s + 2, ring + slot_s2 * kSlot);
        load_b<DT_MXFP4>(bsrc, b_base, has_row, K, 2 * (s + 1), qd, bq[cur ^ 1][0]);
        load_b<DT_MXFP4>(bsrc, b_base, has_row, K, 2 * (s + 1) + 1, qd, bq[cur ^ 1][1]);
        // the last 2 NP NMAT + 8 loads issued: line s + 2 and B_{s+1}
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NP * NMAT + 8) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* line0 = ring + slot_s * kSlot + rd_row;
        const unsigned char* line1 = ring + slot_s1 * kSlot + rd_row;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t g = 2 * s + (uint32_t)h;  // past K: codes and activations read as zeros, the scale as one
            Batch<MODE, DT_MXFP4, NP> x;
#pragma unroll
            for (int pm = 0; pm < NP * NMAT; ++pm) {
                const uint32_t q = rd_o[pm] + 4u * (uint32_t)h + qd;  // unit from the start of line s
                const unsigned char* src = (q & 8u) ? line1 : line0;
                const u32x4 v = *reinterpret_cast<const u32x4*>(src + pm * 2048 + (((q & 7u) ^ rd_sw) << 4));
                if (pm % NMAT == 0) x.wq[pm / NMAT] = v;
                else x.uq[pm / NMAT] = v;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) x.b[j] = bq[cur][h][j];
            scales_fetch<MODE, DT_MXFP4, NP>(x, sl, nv, KG, g, r, qd);
            compute<MODE, DT_MXFP4, NP, true>(x, acc0, acc1);
        }
        slot_s = slot_s1;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // pairs of super-steps (the activation registers alternate); an odd count
    // ends with a super-step past K, all zeros
    for (uint32_t s = 0; s < ns; s += 2) {
        step(s, 0);
        step(s + 1, 1);
    }
    // the copies still in flight read past the rows (zeros, no memory traffic)
    // but write this wave's LDS: let them land before the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_block<MODE, NP>(a, acc0, acc1, row0, r, qd, has_row, c0, c1, asg, pw);
}

// This wave's equal share of the (tile, weight row) pairs, tile-major, in
// units of kRowAlign rows: workgroups take equal contiguous ranges and their
// W waves equal sub-ranges.
template <int MODE, int WDT, int DEPTH, int W>
__device__ __forceinline__ void balanced_share(const DArgs& a, const Tile* tiles, const int32_t* perm, int ntl,
                                               int wave, int lane) {
    const int64_t upt = a.N / kRowAlign;  // units per tile
    const int64_t units = (int64_t)ntl * upt;
    const int64_t g = gridDim.x, b = blockIdx.x;
    const int64_t b_lo = units * b / g, b_hi = units * (b + 1) / g;
    const int64_t w_lo = b_lo + (b_hi - b_lo) * wave / W;
    const int64_t w_hi = b_lo + (b_hi - b_lo) * (wave + 1) / W;
    for (int64_t u = w_lo; u < w_hi;) {
        const int mt = (int)(u / upt);
        const int64_t s_lo = u - mt * upt;
        const int64_t s_hi = min(upt, s_lo + (w_hi - u));
        const uint32_t r_hi = (uint32_t)(s_hi * kRowAlign);
        const Tile tile = tiles[mt];
        for (uint32_t c = (uint32_t)(s_lo * kRowAlign); c < r_hi; c += kDecCols)
            decode_pass<MODE, WDT, DEPTH>(a, tile, perm, c, min(r_hi, c + (uint32_t)kDecCols), lane);
        u += s_hi - s_lo;
    }
}

// Balanced ranges over the tile list written by the route scan.
template <int MODE, int WDT, int DEPTH>
__global__ __launch_bounds__(kGuWaves * 64) void decode_balanced_kernel(DArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int ntl = min(a.n_tiles[0], a.max_tiles);
    balanced_share<MODE, WDT, DEPTH, kGuWaves>(a, a.tiles, a.perm_src, ntl, wave, lane);
}

// One block of 16 NP weight rows per wave: wave q takes block q % nb of tile
// q / nb, nb = ceil(N / (16 NP)).
template <int MODE, int WDT, int DEPTH, int NP>
__global__ __launch_bounds__(kBlkWaves * 64) void decode_block_kernel(DArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int ntl = min(a.n_tiles[0], a.max_tiles);
    constexpr uint32_t kRows = 16 * NP;
    const int ncb = (int)(((uint32_t)a.N + kRows - 1) / kRows);
    const int q = blockIdx.x * kBlkWaves + wave;
    const int mt = q / ncb, cb = q - mt * ncb;
    if (mt >= ntl) return;  // wave-uniform; this kernel has no barriers
    const uint32_t c0 = (uint32_t)cb * kRows;
    decode_pass<MODE, WDT, DEPTH, NP>(a, a.tiles[mt], a.perm_src, c0, min((uint32_t)a.N, c0 + kRows), lane);
}

// MXFP4, codes through LDS: one block per one-wave workgroup (the same split
// of blocks); the LDS (D ring slots and the scales) caps the waves per CU.
template <int MODE, int NP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1))) void decode_block_mxl_kernel(DArgs a) {
    const int lane = threadIdx.x & 63;
    const int ntl = min(a.n_tiles[0], a.max_tiles);
    constexpr uint32_t kRows = 16 * NP;
    const int ncb = (int)(((uint32_t)a.N + kRows - 1) / kRows);
    const int q = blockIdx.x;
    const int mt = q / ncb, cb = q - mt * ncb;
    if (mt >= ntl) return;
    const uint32_t c0 = (uint32_t)cb * kRows;
    extern __shared__ __align__(16) unsigned char dsm[];
    decode_pass_lds<MODE, NP>(a, a.tiles[mt], a.perm_src, c0, min((uint32_t)a.N, c0 + kRows), lane, dsm);
}

// ------------------------------------------------ fused routing + gate/up --
//
//   s_t,i = W_r[i] . h_t + b_r[i]          fp32, from bf16 MFMA tiles
//   S_t   = the k largest s_t,i            ties (and NaN, which ranks last) to the lower index
//   p_t,i = exp(s_t,i - max S_t) / sum_{j in S_t} exp(s_t,j - max S_t)
//
// ("gpt-oss-40b-64a8-init" page, section 2, Proof.)  The logits kernel splits
// the K range into kLogitSlices interleaved slices and writes one partial sum
// per (slice, token, expert) from a 16x16 MFMA tile per wave; the fused
// kernel adds the slices in slice order and then the bias, so every expert
// column goes through exactly the same operations (identical router rows give
// identical logits).
//
// Top-k by rank: each logit gets a 64-bit order key - its value mapped to an
// order-preserving unsigned integer (NaN lowest, -0 as +0) above the
// complement of its expert index - so "a beats b" (larger value, ties to the
// lower index) is one integer comparison, and the lane of expert e is
// selected when fewer than k keys exceed its own.  The expert-major order is
// a stable counting sort by token: with T <= 64 each expert keeps the set of
// its tokens as a 64-bit mask, and a row's place among the expert's rows is
// the number of earlier tokens in that mask.

constexpr int kFMaxT = 64;        // tokens (one bit each in a 64-bit mask)
constexpr int kFMaxE = 64;        // experts (one per lane in top-k)
constexpr int kLogitSteps = 12;   // 32-wide K steps per batch of loads in the logits kernel
constexpr int kFLogitsPerThread = (kFMaxT * kFMaxE + kGuWaves * 64 - 1) / (kGuWaves * 64);

// Partial logits: block (tile, ks) computes token tile tile / ET x expert
// tile tile % ET over the K steps s = ks (mod kLogitSlices).
// kLo (the pre-normalised block): the router matrix comes as two bf16 parts
// wr + wr_lo (together exactly W_r * g, the norm gain folded into the router),
// both multiplied into the same accumulator, and each token's sums are scaled
// by its 1/rms, row_scale[t].
template <bool kLo>
__global__ __launch_bounds__(64) void decode_logits_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* __restrict__ wr,
                                                           const uint16_t* __restrict__ wr_lo,
                                                           const float* __restrict__ row_scale, int T, int E, int H,
                                                           float* __restrict__ part) {
    constexpr int kSteps = kLo ? kLogitSteps / 2 : kLogitSteps;  // loads per batch: same registers
    const int lane = threadIdx.x;
    const int ET = (E + 15) / 16;
    const int ks = blockIdx.y, tt = blockIdx.x / ET, et = blockIdx.x - (blockIdx.x / ET) * ET;
    const int r = lane & 15, koff = (lane >> 4) * 8;
    const uint16_t* hrow = h + (size_t)min(tt * 16 + r, T - 1) * H;
    const size_t woff = (size_t)min(et * 16 + r, E - 1) * H;
    const int nsteps = H / 32;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = ks; s0 < nsteps; s0 += kLogitSlices * kSteps) {
        bf16x8 av[kSteps], bv[kSteps], cv[kLo ? kSteps : 1];
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int s = s0 + q * kLogitSlices;
            const int kk = (s < nsteps ? s : ks) * 32 + koff;  // past the end: a valid step, discarded
            av[q] = *reinterpret_cast<const bf16x8*>(hrow + kk);
            bv[q] = *reinterpret_cast<const bf16x8*>(wr + woff + kk);
            if constexpr (kLo) cv[q] = *reinterpret_cast<const bf16x8*>(wr_lo + woff + kk);
        }
        __builtin_amdgcn_sched_barrier(0);  // the whole batch of loads ahead of the MFMAs
#pragma unroll
        for (int q = 0; q < kSteps; ++q)
            if (s0 + q * kLogitSlices < nsteps) {
                acc = mfma16(av[q], bv[q], acc);
                if constexpr (kLo) acc = mfma16(av[q], cv[q], acc);
            }
    }
    // D[j]: token 4(l/16)+j of the token tile, expert l%16 of the expert tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = tt * 16 + (lane >> 4) * 4 + j, e = et * 16 + r;
        if (t < T && e < E) {
            float v = acc[j];
            if constexpr (kLo) v *= row_scale[t];
            part[((size_t)ks * T + t) * E + e] = v;
        }
    }
}

struct FArgs {
    DArgs g;            // the gate/up product (tiles and perm_src are taken from LDS)
    const float* part;  // partial logits [kLogitSlices][T][E]
    const uint16_t* br; // router bias [E] bf16, or null
    int T, E;
    float* logits;      // [T][E] or null
    int32_t* topk_idx;  // [T*k]
    float* topk_w;      // [T*k]
    int32_t* offsets;   // [E+1]
    int32_t* perm_src;  // [T*k]
    int32_t* inv;       // [T*k]
    float* row_p;       // [T*k]
    Tile* tiles;        // [max_tiles]
    int32_t* n_tiles;   // [1]
};

// LDS layout of the fused kernel (byte offsets), identical on host and device.
struct FLayout {
    uint32_t sl, key, mask, off, toff, ti, tw, perm, tiles, total;
};
__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }
__host__ __device__ inline FLayout flayout(int T, int k, int max_tiles) {
    FLayout L{};
    uint32_t o = 0;
    L.sl = o;    o += align16((uint32_t)T * kFMaxE * 4);  // logits [T][64]
    L.key = o;   o += align16((uint32_t)T * kFMaxE * 8);  // order keys [T][64], 0 past E
    L.mask = o;  o += align16(kFMaxE * 8);                // tokens of each expert
    L.off = o;   o += align16((kFMaxE + 1) * 4);
    L.toff = o;  o += align16((kFMaxE + 1) * 4);
    L.ti = o;    o += align16((uint32_t)T * k * 4);       // selected expert of each assignment
    L.tw = o;    o += align16((uint32_t)T * k * 4);       // its routing weight
    L.perm = o;  o += align16((uint32_t)T * k * 4);       // assignment of each expert-major row
    L.tiles = o; o += align16((uint32_t)max_tiles * sizeof(Tile));
    L.total = o;
    return L;
}

template <int WDT>
__global__ __launch_bounds__(kGuWaves * 64) void decode_route_gateup_kernel(FArgs f) {
    extern __shared__ __align__(16) unsigned char smem[];
    const DArgs& a = f.g;
    const int T = f.T, E = f.E, k = a.k;
    const FLayout L = flayout(T, k, a.max_tiles);
    float* sl = reinterpret_cast<float*>(smem + L.sl);
    unsigned long long* skey = reinterpret_cast<unsigned long long*>(smem + L.key);
    unsigned long long* emask = reinterpret_cast<unsigned long long*>(smem + L.mask);
    int32_t* off = reinterpret_cast<int32_t*>(smem + L.off);
    int32_t* toff = reinterpret_cast<int32_t*>(smem + L.toff);
    int32_t* ti = reinterpret_cast<int32_t*>(smem + L.ti);
    float* tw = reinterpret_cast<float*>(smem + L.tw);
    int32_t* perm = reinterpret_cast<int32_t*>(smem + L.perm);
    Tile* tl = reinterpret_cast<Tile*>(smem + L.tiles);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool writer = blockIdx.x == 0;

    // 1. logits = slices added in slice order, then the bias; their order keys.
    //    A thread owns logits tid, tid + 768, ... (at most kFLogitsPerThread)
    //    and issues all their loads before summing: one round trip to L2.
    if (tid < kFMaxE) emask[tid] = 0ull;
    for (int i = tid; i < T * kFMaxE; i += kGuWaves * 64)
        if (i % kFMaxE >= E) skey[i] = 0ull;  // past E: below every key
    {
        // an element past T*E reads element 0, and without a bias the bias
        // reads are taken from the partial sums and dropped: no branch around
        // the loads (a branch per element made the compiler wait for each
        // group in turn)
        float pv[kFLogitsPerThread][kLogitSlices], bv[kFLogitsPerThread];
        const bool has_br = f.br != nullptr;
        const uint16_t* brp = has_br ? f.br : reinterpret_cast<const uint16_t*>(f.part);
#pragma unroll
        for (int j = 0; j < kFLogitsPerThread; ++j) {
            const int i = tid + j * kGuWaves * 64;
            const bool in = i < T * E;
            const int t = in ? i / E : 0, e = in ? i - t * E : 0;
#pragma unroll
            for (int ks = 0; ks < kLogitSlices; ++ks) pv[j][ks] = f.part[((size_t)ks * T + t) * E + e];
            bv[j] = bf16_bits_to_f32(brp[e]);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above goes out before the first sum
#pragma unroll
        for (int j = 0; j < kFLogitsPerThread; ++j) bv[j] = has_br ? bv[j] : 0.f;
#pragma unroll
        for (int j = 0; j < kFLogitsPerThread; ++j) {
            const int i = tid + j * kGuWaves * 64;
            if (i >= T * E) continue;
            const int t = i / E, e = i - t * E;
            float v = 0.f;
#pragma unroll
            for (int ks = 0; ks < kLogitSlices; ++ks) v += pv[j][ks];
            v += bv[j];
            sl[t * kFMaxE + e] = v;
            skey[t * kFMaxE + e] = order_key(v, e);
            if (writer && f.logits) f.logits[(size_t)t * E + e] = v;
        }
    }
    __syncthreads();

    // 2. top-k by rank + softmax over the selected set: with E <= 32 a wave
    //    takes two tokens at once (lanes 0..31 and 32..63), else one
    if (E <= 32) {
        const int half = lane >> 5, le = lane & 31;
        for (int tp = 2 * wave; tp < T; tp += 2 * kGuWaves) {
            const int t = tp + half;
            const bool tv = t < T;  // an odd last pair has no second token
            const int trow = tv ? t : tp;
            const bool ok = tv & (le < E);
            const unsigned long long mine = skey[trow * kFMaxE + le];
            const float v = sl[trow * kFMaxE + le];
            const int rank = rank_of<16>(reinterpret_cast<const u32x4*>(skey + trow * kFMaxE), mine);
            const bool chosen = ok & (rank < k);
            const uint64_t top = __ballot(ok & (rank == 0));
            const uint32_t top0 = (uint32_t)top, top1 = (uint32_t)(top >> 32);
            const float m0 = lane_f(v, top0 ? (int)__builtin_ctz(top0) : 0);
            const float m1 = lane_f(v, top1 ? 32 + (int)__builtin_ctz(top1) : 32);
            const float z = chosen ? expf(v - (half ? m1 : m0)) : 0.f;
            // 16-lane row sums (DPP), then rows 0+1 and rows 2+3: the same
            // order as the one-token sum, whose rows 2 and 3 hold zeros here
            float x = z;
            x += dpp_f<kDppXor1>(x);
            x += dpp_f<kDppXor2>(x);
            x += dpp_f<kDppHalfMirror>(x);
            x += dpp_f<kDppMirror>(x);
            const float zs = half ? lane_f(x, 32) + lane_f(x, 48) : lane_f(x, 0) + lane_f(x, 16);
            const uint64_t bal = __ballot(chosen);
            const uint32_t balh = half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
            const uint32_t lt = le == 0 ? 0u : (~0u >> (32 - le));
            const int pos = __popc(balh & lt);  // ascending expert order
            if (chosen) {
                ti[t * k + pos] = le;
                tw[t * k + pos] = z / zs;
                atomicOr(&emask[le], 1ull << t);
                if (writer) {
                    f.topk_idx[(size_t)t * k + pos] = le;
                    f.topk_w[(size_t)t * k + pos] = z / zs;
                }
            }
        }
    } else {
        for (int t = wave; t < T; t += kGuWaves) {
            const bool ok = lane < E;
            const unsigned long long mine = skey[t * kFMaxE + lane];
            const float v = sl[t * kFMaxE + lane];
            const int rank = rank_of<32>(reinterpret_cast<const u32x4*>(skey + t * kFMaxE), mine);
            const bool chosen = ok & (rank < k);
            const uint64_t top = __ballot(ok & (rank == 0));
            const float smax = lane_f(v, (int)__builtin_ctzll(top));
            const float z = chosen ? expf(v - smax) : 0.f;
            const float zs = wave_sum(z);
            const uint64_t bal = __ballot(chosen);
            const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const int pos = __popcll(bal & lt);  // ascending expert order
            if (chosen) {
                ti[t * k + pos] = lane;
                tw[t * k + pos] = z / zs;
                atomicOr(&emask[lane], 1ull << t);
                if (writer) {
                    f.topk_idx[(size_t)t * k + pos] = lane;
                    f.topk_w[(size_t)t * k + pos] = z / zs;
                }
            }
        }
    }
    __syncthreads();

    // 3. counts, offsets and the tile list (wave 0), then every row's place
    if (wave == 0) {
        const int c = lane < E ? __popcll(emask[lane]) : 0;
        const int nt = (c + kDecRows - 1) / kDecRows;
        int xs = c, xt = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int ys = __shfl_up(xs, d, 64), yt = __shfl_up(xt, d, 64);
            if (lane >= d) {
                xs += ys;
                xt += yt;
            }
        }
        const int o = xs - c, base = xt - nt;
        if (lane < E) {
            off[lane] = o;
            toff[lane] = base;
            for (int j = 0; j < nt; ++j) {
                Tile x;
                x.expert = lane;
                x.row_start = o + j * kDecRows;
                x.rows = min(kDecRows, c - j * kDecRows);
                x.pad = 0;
                tl[base + j] = x;
                if (writer) f.tiles[base + j] = x;
            }
            if (writer) f.offsets[lane] = o;
        }
        if (lane == 63) {
            off[E] = xs;
            toff[E] = xt;
            if (writer) {
                f.offsets[E] = xs;
                f.n_tiles[0] = xt;
            }
        }
    }
    __syncthreads();
    for (int as = tid; as < T * k; as += kGuWaves * 64) {
        const int t = as / k, e = ti[as];
        const int row = off[e] + __popcll(emask[e] & ((1ull << t) - 1ull));
        perm[row] = as;
        if (writer) {
            f.perm_src[row] = as;
            f.inv[as] = row;
            f.row_p[row] = tw[as];
        }
    }
    __syncthreads();

    // 4. gate/up: this workgroup's share of the tiles
    balanced_share<0, WDT, WDT == DT_MXFP4 ? 2 : 1, kGuWaves>(a, tl, perm, min(toff[E], a.max_tiles), wave, lane);
}

DArgs make_dargs(const GemmProblem& p, int mode) {
    DArgs a{};
    a.perm_src = p.perm_src;
    a.topk_w = p.topk_w;
    a.row_p = p.row_p;
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
    a.max_tiles = p.max_tiles;  // N is a multiple of kRowAlign and of kDecCols (of 64)
    return a;
}

int cu_count() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

constexpr int kMaxLds = 160 * 1024;

template <auto Kern>
hipError_t allow_lds() {
    return set_max_dynamic_lds<Kern>(kMaxLds - 1024);
}

template <int MODE, int WDT, int DEPTH, int NP>
hipError_t launch_blocks(const GemmProblem& p, hipStream_t stream) {
    const DArgs a = make_dargs(p, MODE);
    const size_t ncb = ((size_t)a.N + 16 * NP - 1) / (16 * NP);
    const int blocks = (int)(((size_t)p.max_tiles * ncb + kBlkWaves - 1) / kBlkWaves);
    if constexpr (WDT == DT_MXFP4) {
        // LDS: the codes' ring, then the block's scales, [panel][matrix][16][K/32] bytes
        static_assert(kBlkWaves == 1, "one block per workgroup");
        if ((uint32_t)a.K / 32 > kScaleMaxKg) return hipErrorInvalidValue;  // beyond the MXFP4 K limit
        constexpr int NMAT = MODE == 0 ? 2 : 1;
        const size_t smem = kMxRing * ring_slot<NP, NMAT>() + (size_t)NP * NMAT * scale_lines(a.K / 32) * 256;
        decode_block_mxl_kernel<MODE, NP><<<blocks, 64, smem, stream>>>(a);
    } else {
        decode_block_kernel<MODE, WDT, DEPTH, NP><<<blocks, kBlkWaves * 64, 0, stream>>>(a);
    }
    return hipGetLastError();
}

constexpr int kDnPanels = 4;  // down: 16-row weight panels per wave (a tile's activation loads shared by 64 rows)

// bf16 gate/up: balanced ranges, one K step in flight.  MXFP4 gate/up moves
// a quarter of the bytes per K step, so it keeps two steps in flight and one
// block per wave (many more waves in flight than one workgroup per CU holds).
template <int WDT>
hipError_t launch_gu(const GemmProblem& p, hipStream_t stream) {
    if constexpr (WDT == DT_MXFP4) {
        return launch_blocks<0, WDT, 2, kPanels>(p, stream);
    } else {
        const DArgs a = make_dargs(p, 0);
        auto kern = decode_balanced_kernel<0, WDT, 1>;
        const hipError_t attr = allow_lds<decode_balanced_kernel<0, WDT, 1>>();
        if (attr != hipSuccess) return attr;
        kern<<<cu_count(), kGuWaves * 64, kMinLds, stream>>>(a);
        return hipGetLastError();
    }
}

template <int WDT>
hipError_t launch_dn(const GemmProblem& p, hipStream_t stream) {
    return launch_blocks<1, WDT, 2, kDnPanels>(p, stream);
}

template <int WDT>
hipError_t launch_fused(const GemmProblem& p, const FusedRouting& r, hipStream_t stream) {
    FArgs f{};
    f.g = make_dargs(p, 0);
    f.part = r.part;
    f.br = reinterpret_cast<const uint16_t*>(r.b_router);
    f.T = p.T;
    f.E = p.E;
    f.logits = r.logits;
    f.topk_idx = r.topk_idx;
    f.topk_w = r.topk_w;
    f.offsets = r.offsets;
    f.perm_src = r.perm_src;
    f.inv = r.inv;
    f.row_p = r.row_p;
    f.tiles = r.tiles;
    f.n_tiles = r.n_tiles;
    const FLayout L = flayout(p.T, p.k, p.max_tiles);
    const uint32_t smem = L.total > (uint32_t)kMinLds ? L.total : (uint32_t)kMinLds;
    if (smem > (uint32_t)(kMaxLds - 1024)) return hipErrorInvalidValue;
    auto kern = decode_route_gateup_kernel<WDT>;
    const hipError_t attr = allow_lds<decode_route_gateup_kernel<WDT>>();
    if (attr != hipSuccess) return attr;
    kern<<<cu_count(), kGuWaves * 64, smem, stream>>>(f);
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

// The fused routing + gate/up kernel serves decode problems with a small
// batch and router (its LDS holds the logits, the selection and the order).
bool decode_fused(int act_dtype, int T, int H, int I, int E, int k) {
    if (!decode_path(act_dtype, T, H, I, E, k)) return false;
    if (T < 1 || T > kFMaxT || E > kFMaxE) return false;
    const int max_tiles = (T * k + kDecRows - 1) / kDecRows + E;
    return flayout(T, k, max_tiles).total <= (uint32_t)(kMaxLds - 1024);
}

size_t decode_logit_part_bytes(int T, int E) { return (size_t)kLogitSlices * T * E * 4; }

hipError_t launch_decode_logits(const void* h, const void* w_router, const void* w_router_lo,
                                const float* row_scale, int T, int H, int E, float* part, hipStream_t stream) {
    const dim3 grid(((T + 15) / 16) * ((E + 15) / 16), kLogitSlices);
    if (w_router_lo)
        decode_logits_kernel<true><<<grid, 64, 0, stream>>>(
            reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(w_router),
            reinterpret_cast<const uint16_t*>(w_router_lo), row_scale, T, E, H, part);
    else
        decode_logits_kernel<false><<<grid, 64, 0, stream>>>(reinterpret_cast<const uint16_t*>(h),
                                                             reinterpret_cast<const uint16_t*>(w_router), nullptr,
                                                             nullptr, T, E, H, part);
    return hipGetLastError();
}

int decode_block_m() { return kDecRows; }

hipError_t launch_gateup_decode(const GemmProblem& p, hipStream_t stream) {
    return p.expert_dtype == DT_MXFP4 ? launch_gu<DT_MXFP4>(p, stream) : launch_gu<DT_BF16>(p, stream);
}

hipError_t launch_route_gateup_decode(const GemmProblem& p, const FusedRouting& r, hipStream_t stream) {
    return p.expert_dtype == DT_MXFP4 ? launch_fused<DT_MXFP4>(p, r, stream) : launch_fused<DT_BF16>(p, r, stream);
}

hipError_t launch_down_decode(const GemmProblem& p, hipStream_t stream) {
    return p.expert_dtype == DT_MXFP4 ? launch_dn<DT_MXFP4>(p, stream) : launch_dn<DT_BF16>(p, stream);
}

}  // namespace moe
