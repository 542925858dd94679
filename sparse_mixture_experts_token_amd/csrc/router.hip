// Stage 0 of the layer: router logits, top-k selection and softmax over the
// selected set, for a tile of 16 tokens per workgroup.
//
//   s_i = W_r[i] . h_t + b_r[i]                 ("gpt-oss-40b-64a8-init" page,
//   S_t = k largest s_i (lower index on ties)    section 2, Proof)
//   p_i = exp(s_i - max_S) / sum_{j in S_t} exp(s_j - max_S)
//
// Logits use 16x16 MFMA tiles (tokens x experts) with fp32 accumulation.  The
// K range (hidden) is split over the four waves by interleaved 32-wide steps
// and the four partial sums are added in a fixed order, so every expert column
// goes through exactly the same sequence of operations: two identical router
// rows (silent copies) give bitwise-identical logits.
//
// Besides topk_idx / topk_w the kernel writes, for the stable expert-major
// permutation built by the next stage:
//   blk_counts[e][tile] = number of this tile's tokens routed to e
//   local_rank[t*k+slot] = number of earlier tokens of the same tile routed to
//                          the same expert
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BT = kRouterTokens;  // tokens per workgroup
constexpr int NW = 4;              // waves per workgroup
constexpr int CB = 4;              // 16-wide expert column blocks per pass

struct RouterSmem {
    // layout offsets (bytes) for a given padded expert count
    static __host__ __device__ size_t logits_off() { return 0; }
    static __host__ __device__ size_t part_off(int Ep) { return (size_t)BT * Ep * 4; }
    static __host__ __device__ size_t selpos_off(int Ep) { return part_off(Ep) + (size_t)NW * BT * CB * 16 * 4; }
    static __host__ __device__ size_t bytes(int Ep) { return selpos_off(Ep) + (size_t)BT * Ep * 2; }
};

template <typename TA>
__device__ __forceinline__ float load_scalar(const TA* p, size_t i);
template <>
__device__ __forceinline__ float load_scalar<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_scalar<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

constexpr int kNone = 0x7fffffff;

// Wave-wide arg-max of (value, index): larger value wins, then lower index.
// A lane without a candidate holds index kNone; any candidate beats it, so a
// candidate is always found while one exists (even for NaN or -inf logits).
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        float ov = __shfl_xor(v, d, 64);
        int oi = __shfl_xor(idx, d, 64);
        bool take = oi != kNone && (idx == kNone || ov > v || (ov == v && oi < idx));
        v = take ? ov : v;
        idx = take ? oi : idx;
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

template <typename TA>
__global__ __launch_bounds__(256) void router_kernel(const TA* __restrict__ h, const TA* __restrict__ wr,
                                                     const TA* __restrict__ br, int T, int H, int E, int k,
                                                     float* __restrict__ logits_opt, int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w, int32_t* __restrict__ blk_counts,
                                                     int32_t* __restrict__ local_rank) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int Ep = (E + 63) & ~63;  // padded so every lane owns Ep/64 columns
    float* s_lds = reinterpret_cast<float*>(smem + RouterSmem::logits_off());
    float* part = reinterpret_cast<float*>(smem + RouterSmem::part_off(Ep));
    uint16_t* selpos = reinterpret_cast<uint16_t*>(smem + RouterSmem::selpos_off(Ep));

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int t0 = blockIdx.x * BT;
    const int nblk = gridDim.x;

    for (int i = tid; i < BT * Ep; i += 256) selpos[i] = 0;

    // ---------------------------------------------------------- logits --
    constexpr bool kBf16 = sizeof(TA) == 2;
    constexpr int KSTEP = kBf16 ? 32 : 4;  // K per 16x16 MFMA
    const int nsteps = H / KSTEP;
    const int arow = min(t0 + (lane & 15), T - 1);
    const TA* hrow = h + (size_t)arow * H;
    const int ncb = (E + 15) >> 4;

    for (int cb0 = 0; cb0 < ncb; cb0 += CB) {
        f32x4 acc[CB];
        const TA* wrow[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            int e = min((cb0 + c) * 16 + (lane & 15), E - 1);
            wrow[c] = wr + (size_t)e * H;
        }
        if constexpr (kBf16) {
            const int koff = (lane >> 4) * 8;
#pragma unroll 2
            for (int s = wave; s < nsteps; s += NW) {
                const int kk = s * KSTEP + koff;
                bf16x8 a = *reinterpret_cast<const bf16x8*>(hrow + kk);
                bf16x8 b[CB];
#pragma unroll
                for (int c = 0; c < CB; ++c) b[c] = *reinterpret_cast<const bf16x8*>(wrow[c] + kk);
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    if (cb0 + c < ncb) acc[c] = mfma16(a, b[c], acc[c]);
            }
        } else {
            const int koff = lane >> 4;
#pragma unroll 4
            for (int s = wave; s < nsteps; s += NW) {
                const int kk = s * KSTEP + koff;
                float a = hrow[kk];
                float b[CB];
#pragma unroll
                for (int c = 0; c < CB; ++c) b[c] = wrow[c][kk];
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    if (cb0 + c < ncb) acc[c] = mfma16(a, b[c], acc[c]);
            }
        }
        // partial sums of this wave: part[wave][row][c*16 + col]
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int row = (lane >> 4) * 4 + j;
                part[((wave * BT) + row) * (CB * 16) + c * 16 + (lane & 15)] = acc[c][j];
            }
        __syncthreads();
        // fixed-order reduction over the waves, then the bias
        for (int i = tid; i < BT * CB * 16; i += 256) {
            int row = i / (CB * 16);
            int col = i % (CB * 16);
            int e = cb0 * 16 + col;
            if (e < E) {
                float v = part[(0 * BT + row) * (CB * 16) + col];
                v += part[(1 * BT + row) * (CB * 16) + col];
                v += part[(2 * BT + row) * (CB * 16) + col];
                v += part[(3 * BT + row) * (CB * 16) + col];
                if (br) v += load_scalar(br, e);
                s_lds[row * Ep + e] = v;
            }
        }
        __syncthreads();
    }

    // -------------------------------------------- top-k + selected softmax --
    constexpr int NV = 16;  // up to 1024 experts: lane owns e = lane + 64 i
    const int nv = Ep >> 6;
    for (int tt = wave; tt < BT; tt += NW) {
        const int t = t0 + tt;
        if (t >= T) break;  // wave-uniform
        float v[NV], orig[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int e = lane + 64 * i;
            float x = (i < nv && e < E) ? s_lds[tt * Ep + e] : -INFINITY;
            v[i] = x;
            orig[i] = x;
        }
        if (logits_opt) {
            for (int i = 0; i < nv; ++i) {
                int e = lane + 64 * i;
                if (e < E) logits_opt[(size_t)t * E + e] = orig[i];
            }
        }
        uint32_t selmask = 0;
        float smax = 0.f;
        for (int r = 0; r < k; ++r) {
            float bv = -INFINITY;
            int bi = kNone;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                int e = lane + 64 * i;
                bool live = i < nv && e < E && !((selmask >> i) & 1u);
                bool take = live && (bi == kNone || v[i] > bv);  // ascending e: ties keep the lower index
                bv = take ? v[i] : bv;
                bi = take ? e : bi;
            }
            wave_argmax(bv, bi);
            if (r == 0) smax = bv;
            if (bi < E && (bi & 63) == lane) selmask |= 1u << (bi >> 6);
        }
        // softmax over the selected set, summed in a fixed order
        float z[NV];
        float zs = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            z[i] = ((selmask >> i) & 1u) ? expf(orig[i] - smax) : 0.f;
            zs += z[i];
        }
        const float denom = wave_sum(zs);
        // position in ascending expert order
        int before = 0;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int i = 0; i < nv; ++i) {
            const bool sel = (selmask >> i) & 1u;
            const uint64_t bal = __ballot(sel);
            if (sel) {
                const int pos = before + __popcll(bal & lt);
                const int e = lane + 64 * i;
                topk_idx[(size_t)t * k + pos] = e;
                topk_w[(size_t)t * k + pos] = z[i] / denom;
                selpos[tt * Ep + e] = (uint16_t)(pos + 1);
            }
            before += __popcll(bal);
        }
    }
    __syncthreads();

    // ---------------------------------- per-tile counts and local ranks --
    const int tcount = min(BT, T - t0);
    for (int e = tid; e < E; e += 256) {
        int running = 0;
        for (int tt = 0; tt < tcount; ++tt) {
            int sp = selpos[tt * Ep + e];
            if (sp) local_rank[(size_t)(t0 + tt) * k + (sp - 1)] = running++;
        }
        blk_counts[(size_t)e * nblk + blockIdx.x] = running;
    }
}

}  // namespace

hipError_t launch_router(int act_dtype, const void* h, const void* w_router, const void* b_router, int T, int H,
                         int E, int k, float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* blk_counts,
                         int32_t* local_rank, hipStream_t stream) {
    const int nblk = (T + BT - 1) / BT;
    const int Ep = (E + 63) & ~63;
    const size_t smem = RouterSmem::bytes(Ep);
    if (act_dtype == DT_BF16) {
        (void)hipFuncSetAttribute((const void*)router_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)smem);
        router_kernel<uint16_t><<<nblk, 256, smem, stream>>>(
            (const uint16_t*)h, (const uint16_t*)w_router, (const uint16_t*)b_router, T, H, E, k, logits_opt, topk_idx,
            topk_w, blk_counts, local_rank);
    } else {
        (void)hipFuncSetAttribute((const void*)router_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)smem);
        router_kernel<float><<<nblk, 256, smem, stream>>>((const float*)h, (const float*)w_router,
                                                          (const float*)b_router, T, H, E, k, logits_opt, topk_idx,
                                                          topk_w, blk_counts, local_rank);
    }
    return hipGetLastError();
}

size_t router_smem_bytes(int E) { return RouterSmem::bytes((E + 63) & ~63); }

}  // namespace moe
