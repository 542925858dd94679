// Decode attention with learned sinks: the newest token of every sequence
// attends to its key/value cache ("gpt-oss-20b and gpt-oss-120b" explainer,
// "Two attention savings, and a sink"; "gpt-oss 20B" field guide, cutaway 05:
// every query head has a sink logit that joins the softmax normalisation and
// carries no value; query heads share key/value heads in groups):
//
//   s_j = scale * q_h . k_j,   out_h = sum_j exp(s_j) v_j / (exp(sink_h) + sum_j exp(s_j))
//
// over the visible keys j (all of the sequence's, or its last `window`).
//
// Two kernels.  attn_partial_kernel: one workgroup per (sequence, key/value
// head, chunk of the visible keys), so that short batches still fill the
// chip; the group's G query heads share every key and value load.  The chunk
// is cut into 64-key tiles dealt round-robin to four waves.  Per tile, all 24
// loads of a lane are issued first, then:
//   scores - S^T = K Q^T on 16x16x32 bf16 MFMAs, 16 keys per product: the
//            key rows are the A rows, read from HBM straight into operand
//            layout; the G query heads are the B columns (zero-padded to 16).
//            Lane (col, grp) = (l % 16, l / 16) ends up holding the scores of
//            head col for the 16 keys 16blk + 4grp + j;
//   softmax - running max m and sum l of head col (streaming softmax),
//            reduced over the 4 lanes that share the head;
//   values  - O^T += V^T P^T on 16x16x4 fp32 MFMAs, one 4-key step per
//            (blk, j): a lane's own fp32 weight is its B element, and its A
//            element is feature 4col + mb of the step's key row, so one
//            8-byte load per step feeds the four 16-feature blocks mb.
//            Nothing is transposed and the weights stay in fp32.
// The four waves are merged and the chunk's (m, l, sum p v) written to the
// workspace.  attn_merge_kernel: per (sequence, query head), the chunks are
// combined with the sink as the starting state (m = sink, l = 1, nothing in
// the sum), so it joins the normalisation and adds no value.  Softmax and
// sums in fp32, out rounded once.  Memory bound: every visible key and value
// row is read once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAWaves = 4;
constexpr int kAMaxG = 8;   // query heads per key/value head
constexpr int kAMaxD = 64;  // head dimension
constexpr int kATile = 64;  // keys per wave tile
constexpr int kAWorkgroupsTarget = 1024;
constexpr float kNegInf = -__builtin_inff();

struct AttnArgs {
    const uint16_t* q;      // [B, Hq, D]
    const uint16_t* k;      // [B, Hkv, Tk, D]
    const uint16_t* v;      // [B, Hkv, Tk, D]
    const uint16_t* sinks;  // [Hq]
    const int32_t* lens;    // [B] or null (all Tk)
    uint16_t* out;          // [B, Hq, D]
    float* pm;              // partial max   [B, Hq, nchunk]
    float* pl;              // partial sum   [B, Hq, nchunk]
    float* pacc;            // partial p v   [B, Hq, nchunk, D]
    int B, Hq, Hkv, Tk, D, window, nchunk, chunk;
    float scale;
};

__device__ __forceinline__ void unpack8(const uint4 w, float (&f)[8]) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_bits_to_f32(ww[e] & 0xffffu);
        f[2 * e + 1] = bf16_bits_to_f32(ww[e] >> 16);
    }
}

// Visible keys of sequence b: [lo, n).
__device__ __forceinline__ void visible(const AttnArgs& a, int b, int& lo, int& n) {
    n = a.lens ? a.lens[b] : a.Tk;
    n = n < 0 ? 0 : (n > a.Tk ? a.Tk : n);
    lo = (a.window > 0 && n > a.window) ? n - a.window : 0;
}

// G query heads share each key/value head (G <= 8); one instantiation per G.
template <int G>
__global__ __launch_bounds__(kAWaves * 64) void attn_partial_kernel(AttnArgs a) {
    __shared__ float s_m[kAWaves][16], s_l[kAWaves][16];
    __shared__ float s_acc[kAWaves][16][kAMaxD];  // [wave][head][feature]
    const int c = blockIdx.x % a.nchunk;
    const int bg = blockIdx.x / a.nchunk;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int D = a.D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;  // head column; key / feature row group
    int lo, n;
    visible(a, b, lo, n);
    const int kb = lo + c * a.chunk;
    const int ke = min(n, kb + a.chunk);
    const size_t kv0 = ((size_t)b * a.Hkv + g) * a.Tk;

    // Scores are S^T = K Q^T (16x16x32 bf16): A = key rows (row = key, K =
    // features 8grp + 32ks ..+7), B = Q^T (column = head col, zero for col >= G).
    bf16x8 qb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int f = 32 * ks + 8 * grp;
        qb[ks] = bf16x8{};
        if (col < G && f < D)
            qb[ks] = *reinterpret_cast<const bf16x8*>(a.q + ((size_t)b * a.Hq + g * G + col) * D + f);
    }
    const bool ks1 = D > 32;  // uniform
    const int fk0 = 8 * grp < D ? 8 * grp : 0, fk1 = 32 + 8 * grp < D ? 32 + 8 * grp : 0;
    const bool klive0 = 8 * grp < D, klive1 = 32 + 8 * grp < D;
    // Values: lane reads features 4col..4col+3 of a row (one per 16-feature block mb).
    const bool vlive = 4 * col < D;
    const int fv = vlive ? 4 * col : 0;

    // Running max and sum of head col (equal in the 4 lanes col + 16 grp);
    // acc[mb][j] = O^T[feature 4(4grp + j) + mb][head col].
    float m = kNegInf, l = 0.0f;
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t0 = kb + wave * kATile; t0 < ke; t0 += kAWaves * kATile) {  // wave-uniform
        // Key t0 + 16blk + col as an A row; value row t0 + 16blk + 4grp + j.
        // Rows past the chunk read key t0 (visible) and get weight 0.
        bf16x8 kr[4][2];
        uint2 vr[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int j = t0 + 16 * blk + col;
            const uint16_t* row = a.k + (kv0 + (j < ke ? j : t0)) * D;
            kr[blk][0] = *reinterpret_cast<const bf16x8*>(row + fk0);
            kr[blk][1] = ks1 ? *reinterpret_cast<const bf16x8*>(row + fk1) : bf16x8{};
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = t0 + 16 * blk + 4 * grp + jj;
                vr[blk][jj] = *reinterpret_cast<const uint2*>(a.v + (kv0 + (j < ke ? j : t0)) * D + fv);
            }
        // s[blk][jj]: score of head col and key t0 + 16blk + 4grp + jj
        float s[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
            d = mfma16(klive0 ? kr[blk][0] : bf16x8{}, qb[0], d);
            if (ks1) d = mfma16(klive1 ? kr[blk][1] : bf16x8{}, qb[1], d);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                s[blk][jj] = t0 + 16 * blk + 4 * grp + jj < ke ? d[jj] * a.scale : kNegInf;
        }
        // streaming softmax of head col over the tile's 64 keys (16 here x 4 lanes)
        float mx = s[0][0];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, s[blk][jj]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx);  // finite: key t0 is in lane col's registers
        const float corr = __expf(m - mn);
        float sum = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float p = s[blk][jj] == kNegInf ? 0.0f : __expf(s[blk][jj] - mn);
                s[blk][jj] = p;
                sum += p;
            }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        l = l * corr + sum;
        m = mn;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][e] *= corr;
        // O^T += V^T P^T, 16x16x4 fp32, one K step per (blk, jj): lane (col, grp)
        // gives V[key 16blk + 4grp + jj][feature 4col + mb] (A) and its own
        // weight P[head col][that key] (B).
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint2 w = vlive ? vr[blk][jj] : uint2{0u, 0u};
                const float vf[4] = {bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                                     bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16)};
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16(vf[mb], s[blk][jj], acc[mb]);
            }
    }
    if (grp == 0) {
        s_m[wave][col] = m;
        s_l[wave][col] = l;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_acc[wave][col][4 * (4 * grp + e) + mb] = acc[mb][e];
    __syncthreads();
    if (wave != 0) return;
    for (int h = 0; h < G; ++h) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kAWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.0f, A = 0.0f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kAWaves; ++w) {
                const float f = s_m[w][h] == kNegInf ? 0.0f : __expf(s_m[w][h] - M);
                L = fmaf(s_l[w][h], f, L);
                if (lane < D) A = fmaf(s_acc[w][h][lane], f, A);
            }
        }
        const size_t row = ((size_t)b * a.Hq + g * G + h) * a.nchunk + c;
        if (lane == 0) {
            a.pm[row] = M;
            a.pl[row] = L;
        }
        if (lane < D) a.pacc[row * D + lane] = A;
    }
}

// One wave per (sequence, query head): the chunks and the sink.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + wave;
    if (bh >= a.B * a.Hq) return;  // wave-uniform
    const int h = bh % a.Hq;
    const size_t r0 = (size_t)bh * a.nchunk;
    const float sink = bf16_bits_to_f32(a.sinks[h]);
    float M = sink;
    for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, a.pm[r0 + c]);
    float L = 0.0f, O = 0.0f;
    if (M != kNegInf) {
        L = __expf(sink - M);
        for (int c = 0; c < a.nchunk; ++c) {
            const float mc = a.pm[r0 + c];
            const float f = mc == kNegInf ? 0.0f : __expf(mc - M);
            L = fmaf(a.pl[r0 + c], f, L);
            if (lane < a.D) O = fmaf(a.pacc[(r0 + c) * a.D + lane], f, O);
        }
    }
    if (lane < a.D) a.out[(size_t)bh * a.D + lane] = (uint16_t)f32_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
}

// Chunks per (sequence, key/value head): enough workgroups to fill the chip,
// at least one tile per wave each.
void attn_split(int B, int Hkv, int Tk, int window, int& nchunk, int& chunk) {
    const int keys = window > 0 && window < Tk ? window : Tk;
    const int tiles = (keys + kATile - 1) / kATile;
    const long long bg = (long long)B * Hkv;
    const int want = bg > 0 ? (int)((kAWorkgroupsTarget + bg - 1) / bg) : 1;
    const int cap = (tiles + kAWaves - 1) / kAWaves;
    nchunk = want < 1 ? 1 : (want > cap ? cap : want);
    const int tiles_per = (tiles + nchunk - 1) / nchunk;
    chunk = tiles_per * kATile;
    nchunk = (keys + chunk - 1) / chunk;
}

}  // namespace

bool attn_sink_shape_ok(int B, int Hq, int Hkv, int Tk, int D, int window) {
    if (B < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || Hq / Hkv > kAMaxG) return false;
    if (D < 8 || D > kAMaxD || D % 8 != 0 || Tk < 1 || window < 0) return false;
    int nc, ch;
    attn_split(B, Hkv, Tk, window, nc, ch);
    return (long long)B * Hkv * nc < ((long long)1 << 31) && (long long)B * Hq < ((long long)1 << 31) - 4;
}

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Tk, int D, int window) {
    int nc, ch;
    attn_split(B, Hkv, Tk, window, nc, ch);
    const size_t rows = (size_t)B * Hq * nc;
    return rows * 2 * 4 + rows * D * 4 + 256;
}

hipError_t launch_attn_sink_decode(const void* q, const void* k, const void* v, const void* sinks,
                                   const int32_t* lens, void* out, void* workspace, int B, int Hq, int Hkv, int Tk,
                                   int D, int window, float scale, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    int nc, ch;
    attn_split(B, Hkv, Tk, window, nc, ch);
    const size_t rows = (size_t)B * Hq * nc;
    float* pm = reinterpret_cast<float*>(workspace);
    AttnArgs a{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)sinks, lens,
               (uint16_t*)out, pm, pm + rows, pm + 2 * rows, B, Hq, Hkv, Tk, D, window, nc, ch, scale};
    const dim3 grid(B * Hkv * nc), block(kAWaves * 64);
    switch (Hq / Hkv) {
    case 1: attn_partial_kernel<1><<<grid, block, 0, stream>>>(a); break;
    case 2: attn_partial_kernel<2><<<grid, block, 0, stream>>>(a); break;
    case 3: attn_partial_kernel<3><<<grid, block, 0, stream>>>(a); break;
    case 4: attn_partial_kernel<4><<<grid, block, 0, stream>>>(a); break;
    case 5: attn_partial_kernel<5><<<grid, block, 0, stream>>>(a); break;
    case 6: attn_partial_kernel<6><<<grid, block, 0, stream>>>(a); break;
    case 7: attn_partial_kernel<7><<<grid, block, 0, stream>>>(a); break;
    default: attn_partial_kernel<8><<<grid, block, 0, stream>>>(a); break;
    }
    attn_merge_kernel<<<(B * Hq + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
