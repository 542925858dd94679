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
// is cut into 64-key tiles dealt round-robin to four waves.  Per tile, all 16
// loads of a lane are issued first, then:
//   scores - a 16x16x32 bf16 MFMA per 16 keys and 32 features: the G query
//            heads are the A rows (padded to 16 with zeros), the key rows
//            the B columns, read from HBM straight into operand layout;
//   softmax - running max m and sum l per head (streaming softmax), reduced
//            over the 16 lanes that hold a head's keys; the weights go to
//            LDS as [key][head], with the factor that rescales the sums;
//   values  - lane (kq, dc) = (l / 8, l % 8) holds 16 bytes (features
//            8dc..8dc+7) of value row 8r + kq, so one load covers 8 whole
//            128-byte rows; p * v is added into per-lane fp32 sums, reduced
//            over kq at the end.  (The MFMA would need the value tile
//            transposed, key-major per feature; on the vector unit it is
//            about 600 instructions per tile, under the time of its loads.)
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
    __shared__ __align__(16) float s_p[kAWaves][kATile][8];  // this tile's weights, [key][head]
    __shared__ __align__(16) float s_corr[kAWaves][8];       // this tile's rescale factor per head
    __shared__ float s_m[kAWaves][G], s_l[kAWaves][G];
    __shared__ float s_acc[kAWaves][G][kAMaxD];
    const int c = blockIdx.x % a.nchunk;
    const int bg = blockIdx.x / a.nchunk;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int D = a.D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;  // MFMA column (key) and row group (heads 4grp..4grp+3)
    const int kq = lane >> 3, dc = lane & 7;     // value layout: key 8r+kq, features 8dc..8dc+7
    const bool dlive = 8 * dc < D;
    int lo, n;
    visible(a, b, lo, n);
    const int kb = lo + c * a.chunk;
    const int ke = min(n, kb + a.chunk);
    const size_t kv0 = ((size_t)b * a.Hkv + g) * a.Tk;

    // Q as the MFMA A operand: row = head (rows G..15 zero), K = features;
    // K step ks covers features 32ks..32ks+31, lane's 8 at 32ks + 8grp.
    bf16x8 qa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int f = 32 * ks + 8 * grp;
        qa[ks] = bf16x8{};
        if (col < G && f < D)
            qa[ks] = *reinterpret_cast<const bf16x8*>(a.q + ((size_t)b * a.Hq + g * G + col) * D + f);
    }
    const bool ks1 = D > 32;  // uniform
    const int fk0 = 8 * grp < D ? 8 * grp : 0, fk1 = 32 + 8 * grp < D ? 32 + 8 * grp : 0;
    const bool klive0 = 8 * grp < D, klive1 = 32 + 8 * grp < D;
    const int fv = 8 * (dlive ? dc : 0);

    float m[4], l[4], acc[G][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = kNegInf;
        l[j] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

    for (int t0 = kb + wave * kATile; t0 < ke; t0 += kAWaves * kATile) {  // wave-uniform
        // key rows as the B operand (column = key t0 + 16blk + col) and value
        // rows in the value layout, all issued before any is used.  Rows past
        // the chunk read key t0 (visible) and are masked below.
        bf16x8 kr[4][2];
        uint4 vr[8];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int j = t0 + 16 * blk + col;
            const uint16_t* row = a.k + (kv0 + (j < ke ? j : t0)) * D;
            kr[blk][0] = *reinterpret_cast<const bf16x8*>(row + fk0);
            kr[blk][1] = ks1 ? *reinterpret_cast<const bf16x8*>(row + fk1) : bf16x8{};
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int j = t0 + 8 * r + kq;
            vr[r] = *reinterpret_cast<const uint4*>(a.v + (kv0 + (j < ke ? j : t0)) * D + fv);
        }
        // scores: D[j] of block blk = q[head 4grp+j] . k[key t0+16blk+col]
        float s[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
            d = mfma16(qa[0], klive0 ? kr[blk][0] : bf16x8{}, d);
            if (ks1) d = mfma16(qa[1], klive1 ? kr[blk][1] : bf16x8{}, d);
            const bool valid = t0 + 16 * blk + col < ke;
#pragma unroll
            for (int j = 0; j < 4; ++j) s[blk][j] = valid ? d[j] * a.scale : kNegInf;
        }
        // streaming softmax per head over the tile's 64 keys (16 lanes x 4 blocks)
        float corr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float mx = fmaxf(fmaxf(s[0][j], s[1][j]), fmaxf(s[2][j], s[3][j]));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float mn = fmaxf(m[j], mx);  // finite: key t0 is in every 16-lane group
            corr[j] = __expf(m[j] - mn);
            float sum = 0.0f;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const float p = s[blk][j] == kNegInf ? 0.0f : __expf(s[blk][j] - mn);
                s[blk][j] = p;
                sum += p;
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
            l[j] = l[j] * corr[j] + sum;
            m[j] = mn;
        }
        if (lane < 32) {  // heads 0..7; rows 8..15 are padding
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
                *reinterpret_cast<float4*>(&s_p[wave][16 * blk + col][4 * grp]) =
                    float4{s[blk][0], s[blk][1], s[blk][2], s[blk][3]};
            if (col == 0) *reinterpret_cast<float4*>(&s_corr[wave][4 * grp]) = float4{corr[0], corr[1], corr[2], corr[3]};
        }
        __builtin_amdgcn_wave_barrier();
        // weighted values: acc[h][e] (features 8dc+e, keys kq mod 8) on VALU
        {
            const float4 c0 = *reinterpret_cast<const float4*>(&s_corr[wave][0]);
            const float4 c1 = *reinterpret_cast<const float4*>(&s_corr[wave][4]);
            const float cr[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= cr[h];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float vf[8];
            unpack8(dlive ? vr[r] : uint4{0u, 0u, 0u, 0u}, vf);  // invalid keys have p = 0
            const float4 p0 = *reinterpret_cast<const float4*>(&s_p[wave][8 * r + kq][0]);
            const float4 p1 = *reinterpret_cast<const float4*>(&s_p[wave][8 * r + kq][4]);
            const float pr[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
        }
        __builtin_amdgcn_wave_barrier();  // weights read before the next tile writes them
    }
    // sum the per-lane values over the 8 key lanes kq (lanes dc, dc+8, ..., dc+56)
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[h][e];
            x += __shfl_xor(x, 8, 64);
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[h][e] = x;
        }
        if (kq == 0 && dlive) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * dc + e] = acc[h][e];
        }
    }
    if (lane < 32 && col == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (4 * grp + j < G) {
                s_m[wave][4 * grp + j] = m[j];
                s_l[wave][4 * grp + j] = l[j];
            }
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
