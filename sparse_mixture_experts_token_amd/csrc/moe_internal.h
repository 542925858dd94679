// Internal declarations shared by the HIP translation units of libmoe.
// gfx950 (CDNA4) only: wave64, MFMA bf16/f32, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ----------------------------------------------------------------- types --

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// Native 4 x u32 vector.  Arrays of HIP's uint4 (a struct wrapping a union)
// are left in scratch memory by the compiler; arrays of this type are kept in
// registers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_MXFP4 = 2 };

// Router/top-k tile: tokens per workgroup.
constexpr int kRouterTokens = 16;
// Small batches (T <= 64, bf16): the router logits are first written as
// partial sums over this many interleaved K slices by launch_decode_logits.
constexpr int kLogitSlices = 8;

// One row-tile of one expert in the expert-major order (built on the device).
struct Tile {
    int32_t expert;
    int32_t row_start;  // first row (expert-major order)
    int32_t rows;       // valid rows, 1..BM
    int32_t pad;
};

// ------------------------------------------------------------ buffer loads --
// Raw buffer loads: a 128-bit descriptor (base, size in bytes) in scalar
// registers plus a 32-bit per-lane byte offset and a scalar byte offset.  No
// 64-bit per-lane address arithmetic, and reads at or beyond `bytes` return 0.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufDword3 = 0x00020000;  // gfx9-family raw buffer: no format conversion

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufDword3);
}
__device__ __forceinline__ u32x4 buf_load16(buf_rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load1(buf_rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// ------------------------------------------------------ bf16 conversions --

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats to a bf16 pair (lo in the low half), round to nearest, ties to
// even, by the hardware conversion (NaN stays NaN).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_hw v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ------------------------------------------------------------ MXFP4 -> bf16 --
// Exact decode of one E2M1 code with an E8M0 scale into bf16 bits, in integer
// arithmetic.  Magnitude code c = (e, m) with e = c>>1, m = c&1 is
// 2^(e-1) (1 + m/2) for e > 0 and m/2 for e = 0, so the scaled value
// 2^(scale-127) * E2M1(c) has bf16 exponent field  e + scale - 1  (e > 0) or
// scale - 1 (c = 1, significand 1.0) and mantissa top bit m.  Fields <= 0 give
// bf16 subnormals (exact: at most a 2-bit shift of a 2-bit significand),
// fields >= 255 overflow to infinity; scale 255 is NaN.
__device__ __forceinline__ uint32_t e2m1_to_bf16_exact(uint32_t code, uint32_t scale) {
    const uint32_t sign = (code & 8u) << 12;
    const uint32_t mag = code & 7u;
    if (scale == 255u) return 0x7fc0u | sign;
    if (mag == 0u) return sign;
    const int e = (int)(mag >> 1);
    const uint32_t mbit = mag >= 2u ? ((mag & 1u) << 6) : 0u;
    const int field = (mag >= 2u ? e : 0) + (int)scale - 1;
    if (field >= 255) return 0x7f80u | sign;
    if (field >= 1) return sign | ((uint32_t)field << 7) | mbit;
    return sign | ((0x80u | mbit) >> (1 - field));  // subnormal, field in {-1, 0}
}

// Decode 32 MXFP4 elements (16 packed bytes, element 2j in the low nibble of
// byte j) sharing one E8M0 scale into 32 bf16 (two per output word, element
// 2j in the low half).  Scales 2..252 use the hardware scaled FP4->BF16
// conversion (the product is a power-of-two scaling of a 2-bit significand,
// so it is exact); the other scales take the exact integer path.
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16x2(uint32_t w, float sc, int byte) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    bf16x2 v;
    switch (byte) {  // the byte selector must be an immediate
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3); break;
    }
    return __builtin_bit_cast(uint32_t, v);
}

// 32 codes (16 bytes) and their E8M0 scale -> 32 bf16 (16 words), exactly.
// PATH 1: the hardware scaled conversion, for scales 2..252 only (every
// product is then a normal bf16 or zero); PATH 2: the integer path, any
// scale; PATH 0: chosen per lane.  Callers that know a whole wave's scales
// take PATH 1 or 2 and branch once for the wave.
template <int PATH = 0>
__device__ __forceinline__ void decode_mxfp4_32(const u32x4& q, uint32_t scale, uint32_t out[16]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    if (PATH == 1 || (PATH == 0 && scale >= 2u && scale <= 252u)) {
        const float sc = __uint_as_float(scale << 23);  // 2^(scale-127), a normal float
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) out[i * 4 + b] = cvt_fp4x2_bf16x2(w[i], sc, b);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t byte = (w[i] >> (8 * b)) & 0xffu;
                out[i * 4 + b] = e2m1_to_bf16_exact(byte & 0xfu, scale) | (e2m1_to_bf16_exact(byte >> 4, scale) << 16);
            }
    }
}

// ------------------------------------------------------- cross-lane helpers --
// Moves within 16-lane rows (DPP): no LDS round trip.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within 16

__device__ __forceinline__ float lane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Wave-wide sum in a fixed order; the result is the same in every lane (each
// step adds a pair of lanes that both end with the same value).
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<kDppMirror>(x);
    return ((lane_f(x, 0) + lane_f(x, 16)) + lane_f(x, 32)) + lane_f(x, 48);
}

// -------------------------------------------------------------- top-k order --
// 64-bit key of logit v of expert e: the value mapped to an order-preserving
// unsigned integer (NaN lowest, -0 as +0) above the complement of the index,
// so "key a > key b" is "a has the larger value, or the same value and the
// lower index" - the selection order of the top-k (ties to the lower index).
__device__ __forceinline__ unsigned long long order_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    u = (v != v) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
    return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)e);
}

// Number of the 2 NC keys at krow (LDS) that exceed `mine`.  All reads are
// issued before the first compare (a data-dependent exit between them would
// make every read wait out its own latency).
template <int NC>
__device__ __forceinline__ int rank_of(const u32x4* krow, unsigned long long mine) {
    u32x4 q[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c] = krow[c];
    int rank = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const unsigned long long k0 = ((unsigned long long)q[c].y << 32) | q[c].x;
        const unsigned long long k1 = ((unsigned long long)q[c].w << 32) | q[c].z;
        rank += (k0 > mine ? 1 : 0) + (k1 > mine ? 1 : 0);
    }
    return rank;
}

// ------------------------------------------------------------- MFMA wrappers --
// 32x32x16 bf16: lane l holds A[l%32][8(l/32)+0..7], B[8(l/32)+0..7][l%32];
// D[4i+j] is row 8i+4(l/32)+j, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x2 f32: lane l holds A[l%32][l/32], B[l/32][l%32]; same D layout.
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16: lane l holds A[l%16][8(l/16)+0..7], B[8(l/16)+0..7][l%16];
// D[j] is row 4(l/16)+j, column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 f32: lane l holds A[l%16][l/16], B[l/16][l%16]; same D layout.
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// -------------------------------------------------------------- launchers --
// All launchers enqueue on `stream` and return hipGetLastError().

// Stage 0: router logits + top-k + selected softmax + per-tile counts/ranks.
// With part non-null the logits are the slice sums of part [kLogitSlices][T][E]
// (launch_decode_logits) plus the bias, instead of being computed from h.
// Raise one kernel's dynamic LDS limit, once per process.  The static lives
// in the instantiation for that kernel (not for its type: kernels with one
// signature share a type), so every kernel gets its own call.
template <auto Kern>
hipError_t set_max_dynamic_lds(int bytes) {
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return attr;
}

hipError_t launch_router(int act_dtype, const void* h, const void* w_router, const void* b_router,
                         int T, int H, int E, int k, float* logits_opt, int32_t* topk_idx,
                         float* topk_w, int32_t* blk_counts /*[E][nblk]*/, int32_t* local_rank,
                         const float* part, hipStream_t stream);

// Stage 1: scan + stable permutation + tile list + GEMM work lists.
// A work list enumerates (row tile, column tile) pairs as
// tile * n_col_tiles + col_tile, grouped by expert: for each expert, for each
// column tile, that expert's row tiles.
struct WorkList {
    int32_t* items;    // [max_tiles * n_col_tiles]
    int32_t* count;    // [1]
    int n_col_tiles;
    int32_t* bounds;   // [kXcdRanges + 1]: item ranges of equal estimated cost, one per XCD
};
constexpr int kXcdRanges = 8;
// Estimated cost of a (row tile, column tile) item: a fixed part (the weight
// panel's DMA, which a short tile pays in full) plus one per live 32-row
// group; per work list (gate/up, down).
constexpr int kItemFixedCost[2] = {5, 5};
// zero[0 .. n_zero-1] is cleared (the GEMMs' work-queue counters).
hipError_t launch_route_scan(int T, int E, int k, int BM, const int32_t* topk_idx,
                             int32_t* blk_counts /*in: counts, out: bases*/,
                             const int32_t* local_rank, int32_t* offsets /*[E+1]*/,
                             int32_t* perm_src, int32_t* inv, const float* topk_w, float* row_p,
                             Tile* tiles, int32_t* n_tiles,
                             int max_tiles, WorkList w0, WorkList w1, int32_t* zero, int n_zero,
                             hipStream_t stream);

// Stages 2 and 3: grouped GEMMs over the tile list.
struct GemmProblem {
    int T, H, I, E, k;
    int act_dtype, expert_dtype;
    const void* h;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const uint8_t* s_gate;
    const uint8_t* s_up;
    const uint8_t* s_down;
    const int32_t* perm_src;
    const float* topk_w;
    const float* row_p;  // [T*k] topk_w[perm_src[r]] per expert-major row r (written with perm_src)
    const Tile* tiles;
    const int32_t* n_tiles;
    int max_tiles;
    const int32_t* work_gateup;
    const int32_t* n_work_gateup;
    const int32_t* work_down;
    const int32_t* n_work_down;
    const int32_t* bounds_gateup;  // [kXcdRanges + 1] item range of each XCD
    const int32_t* bounds_down;
    void* act;  // [T*k, I] act_dtype (expert-major rows)
    float* y;   // [T*k, H] fp32, indexed by assignment t*k+slot
    bool decode;  // use the skinny (decode) kernels; tiles are decode_block_m() rows
    int32_t* queues;  // [16] work-queue counters (gate/up 0..7, down 8..15), zeroed by the route scan
};
constexpr int kNumQueues = 16;
int gemm_block_m(int act_dtype, int expert_dtype, int T, int k, int E);
// bf16-weight prefill kernels (gemm_bf16.hip)
int bf16_block_m();
int bf16_col_tiles(int N, int mode, int expert_dtype);  // column tiles of the gate/up (0) or down (1) work list
hipError_t launch_gateup_bf16w(const GemmProblem& p, hipStream_t stream);
hipError_t launch_down_bf16w(const GemmProblem& p, hipStream_t stream);
// Decode-sized problems (bf16 activations, on average at most one 16-row tile
// per expert) take the weight-streaming kernels of gemm_decode.hip.
bool decode_path(int act_dtype, int T, int H, int I, int E, int k);
int decode_block_m();
hipError_t launch_gateup_decode(const GemmProblem& p, hipStream_t stream);
hipError_t launch_down_decode(const GemmProblem& p, hipStream_t stream);
// Small decode problems (decode_fused true) run stages 0-2 as two kernels:
// partial router logits (launch_decode_logits), then one kernel in which
// every workgroup completes the routing of the batch, workgroup 0 writes it
// to these buffers (the same contents the router and the route scan
// produce), and the gate/up product follows.
struct FusedRouting {
    const float* part;  // partial logits, decode_logit_part_bytes()
    const void* b_router;
    float* logits;  // optional
    int32_t* topk_idx;
    float* topk_w;
    int32_t* offsets;
    int32_t* perm_src;
    int32_t* inv;
    float* row_p;
    Tile* tiles;
    int32_t* n_tiles;
};
bool decode_fused(int act_dtype, int T, int H, int I, int E, int k);
size_t decode_logit_part_bytes(int T, int E);
// With w_router_lo non-null (the pre-normalised block) the router is the sum
// of two bf16 matrices w_router + w_router_lo and every token's sums are
// scaled by row_scale[t].
hipError_t launch_decode_logits(const void* h, const void* w_router, const void* w_router_lo,
                                const float* row_scale, int T, int H, int E, float* part, hipStream_t stream);
hipError_t launch_route_gateup_decode(const GemmProblem& p, const FusedRouting& r, hipStream_t stream);
int mxfp4_max_k();                   // largest H or I the MXFP4 kernels take
hipError_t launch_gateup(const GemmProblem& p, hipStream_t stream);
hipError_t launch_down(const GemmProblem& p, hipStream_t stream);

// Stage 4: out[t] = sum_slot y[t*k+slot] (fp32, slot order) [+ residual[t]],
// rounded to act dtype.  residual (act dtype, [T, H]) may be null.
hipError_t launch_combine(int act_dtype, const float* y, void* out, int T, int H, int k, const void* residual,
                          hipStream_t stream);

// Gradients of the layer (backward.hip).  bf16 activations and expert
// weights; the routing is the forward's.  Buffers G, U, GY, DA fp32 and Xp,
// Dp, dY, dG, dU, ACT bf16 are [T k, H or I] workspace regions; dsd [T, Ep]
// bf16 (Ep = E rounded up to 8), dsf [T, E] fp32; tiles [bwd_max_tiles].
struct BwdArgs {
    int T, H, I, E, k;
    const uint16_t *h, *dout, *w_router, *w_gate, *w_up, *w_down;
    const int32_t *topk_idx, *offsets, *perm;
    const float* topk_w;
    const uint8_t* trainable;
    uint16_t* dh;
    float *dw_router, *db_router, *dw_gate, *dw_up, *dw_down;
    int32_t *inv, *tiles, *ntiles;
    uint16_t *Xp, *Dp, *dY, *dG, *dU, *ACT, *dsd;
    float *G, *U, *GY, *DA, *dp, *dsf;
};
int bwd_max_tiles(int T, int k, int E);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

// Decode attention with learned sinks (attn_sink.hip).  Shapes: Hq a multiple
// of Hkv with at most 8 query heads per key/value head, D a multiple of 8 up
// to 64, Tk >= 1, window >= 0 (0: all keys).
// The keys are split into chunks over workgroups; the workspace holds each
// chunk's partial state (attn_workspace_bytes).
bool attn_sink_shape_ok(int B, int Hq, int Hkv, int Tk, int D, int window);
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Tk, int D, int window);
hipError_t launch_attn_sink_decode(const void* q, const void* k, const void* v, const void* sinks,
                                   const int32_t* lens, void* out, void* workspace, int B, int Hq, int Hkv, int Tk,
                                   int D, int window, float scale, hipStream_t stream);

// Block prologue, r_t = 1 / sqrt(mean(x[t]^2) + eps) in fp32.  bf16
// activations: row_scale[t] = r_t, n16 = bf16(g * x * r_t) [T, H], and the
// router with the gain folded in, split exactly into two bf16 parts
// wr_hi + wr_lo = W_r * g [E, H].  fp32 activations: n32 = g * x * r_t.
hipError_t launch_rms_norm(int act_dtype, const void* x, const void* g, float eps, int T, int H, float* n32,
                           uint16_t* n16, float* row_scale, const void* w_router, int E, uint16_t* wr_hi,
                           uint16_t* wr_lo, hipStream_t stream);

}  // namespace moe
