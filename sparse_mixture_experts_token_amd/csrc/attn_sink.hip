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
// chip; the group's query heads share every key and value load.  The chunk
// is cut into 64-key tiles dealt round-robin to four waves.  Per tile:
//   scores - lane (kq, dc) = (l / 8, l % 8) reads 16 bytes (features
//            8dc..8dc+7) of key 8r + kq in round r, so one load instruction
//            covers 8 whole 128-byte key rows; the partial dot products are
//            summed over the 8 lanes of a key by DPP moves;
//   softmax - lane = key: a running max m and sum l per head (streaming
//            softmax); the wave's accumulator is rescaled when m grows;
//   values  - the same (kq, dc) layout reads the value rows and adds
//            p * v into per-lane sums of 8 features, reduced over kq at the end.
// The four waves are merged and the chunk's (m, l, sum p v) written to the
// workspace.  attn_merge_kernel: per (sequence, query head), the chunks are
// combined with the sink as the starting state (m = sink, l = 1, nothing in
// the sum), so it joins the normalisation and adds no value.  All in fp32,
// out rounded once.  Memory bound: every visible key and value row is read
// once.
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Sum over the 8 lanes of a key group (lanes 8i .. 8i+7), result in all 8.
__device__ __forceinline__ float sum8(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    return x;
}

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

__global__ __launch_bounds__(kAWaves * 64) void attn_partial_kernel(AttnArgs a) {
    __shared__ float s_q[kAMaxG][kAMaxD];
    __shared__ float s_s[kAWaves][kAMaxG][kATile];  // this tile's scores, then weights
    __shared__ float s_m[kAWaves][kAMaxG], s_l[kAWaves][kAMaxG];
    __shared__ float s_acc[kAWaves][kAMaxG][kAMaxD];
    const int c = blockIdx.x % a.nchunk;
    const int bg = blockIdx.x / a.nchunk;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int G = a.Hq / a.Hkv, D = a.D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kq = lane >> 3, dc = lane & 7;
    const bool dlive = 8 * dc < D;
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
        const int h = i / D, d = i - (i / D) * D;
        s_q[h][d] = bf16_bits_to_f32(a.q[((size_t)b * a.Hq + g * G + h) * D + d]) * a.scale;
    }
    __syncthreads();
    int lo, n;
    visible(a, b, lo, n);
    const int kb = lo + c * a.chunk;
    const int ke = min(n, kb + a.chunk);
    const size_t kv0 = ((size_t)b * a.Hkv + g) * a.Tk;

    float m[kAMaxG], l[kAMaxG], acc[kAMaxG][8];
#pragma unroll
    for (int h = 0; h < kAMaxG; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    }
    for (int t0 = kb + wave * kATile; t0 < ke; t0 += kAWaves * kATile) {  // wave-uniform
        // scores: 8 keys per round, 8 lanes per key.  Every lane reads inside
        // the cache (key t0 is visible, feature chunk 0 exists); lanes past the
        // chunk or the head dimension discard what they read.  (Issuing all of
        // a tile's loads at once needs ~160 registers, and the lower occupancy
        // costs more than the overlap gains.)
#pragma unroll 2
        for (int r = 0; r < kATile / 8; ++r) {
            const int j = t0 + 8 * r + kq;
            const bool valid = j < ke;
            const uint4 w = *reinterpret_cast<const uint4*>(a.k + (kv0 + (valid ? j : t0)) * D + 8 * (dlive ? dc : 0));
            float kf[8];
            unpack8((valid && dlive) ? w : uint4{0u, 0u, 0u, 0u}, kf);
#pragma unroll
            for (int h = 0; h < kAMaxG; ++h) {
                if (h >= G) break;  // uniform
                float part = 0.0f;
                if (dlive) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) part = fmaf(s_q[h][8 * dc + e], kf[e], part);
                }
                part = sum8(part);
                if (dc == 0) s_s[wave][h][8 * r + kq] = valid ? part : kNegInf;
            }
        }
        __builtin_amdgcn_wave_barrier();
        // softmax: lane = key of the tile
#pragma unroll
        for (int h = 0; h < kAMaxG; ++h) {
            if (h >= G) break;
            const float s = s_s[wave][h][lane];
            const float mn = fmaxf(m[h], wave_max(s));  // finite: key t0 is visible
            const float corr = __expf(m[h] - mn);
            const float p = s == kNegInf ? 0.0f : __expf(s - mn);
            l[h] = l[h] * corr + wave_sum(p);
            m[h] = mn;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= corr;
            s_s[wave][h][lane] = p;
        }
        __builtin_amdgcn_wave_barrier();
        // values: the same 8-lanes-per-key layout
#pragma unroll 2
        for (int r = 0; r < kATile / 8; ++r) {
            const int j = t0 + 8 * r + kq;
            const bool valid = j < ke;
            const uint4 w = *reinterpret_cast<const uint4*>(a.v + (kv0 + (valid ? j : t0)) * D + 8 * (dlive ? dc : 0));
            float vf[8];
            unpack8((valid && dlive) ? w : uint4{0u, 0u, 0u, 0u}, vf);
#pragma unroll
            for (int h = 0; h < kAMaxG; ++h) {
                if (h >= G) break;
                const float p = s_s[wave][h][8 * r + kq];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // weights read before the next tile's scores
    }
    // sum the per-lane values over the 8 key lanes kq (lanes dc, dc+8, ..., dc+56)
#pragma unroll
    for (int h = 0; h < kAMaxG; ++h) {
        if (h >= G) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[h][e];
            x += __shfl_xor(x, 8, 64);
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[h][e] = x;
        }
        if (lane == 0) {
            s_m[wave][h] = m[h];
            s_l[wave][h] = l[h];
        }
        if (kq == 0 && dlive) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * dc + e] = acc[h][e];
        }
    }
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
    attn_partial_kernel<<<B * Hkv * nc, kAWaves * 64, 0, stream>>>(a);
    attn_merge_kernel<<<(B * Hq + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace moe
