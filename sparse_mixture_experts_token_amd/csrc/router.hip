// Stage 0 of the layer: router logits, top-k selection and softmax over the
// selected set, for a tile of 16 tokens per workgroup.
//
//   s_i = W_r[i] . h_t + b_r[i]                 ("gpt-oss-40b-64a8-init" page,
//   S_t = k largest s_i (lower index on ties)    section 2, Proof)
//   p_i = exp(s_i - max_S) / sum_{j in S_t} exp(s_j - max_S)
//
// Logits use 16x16 MFMA tiles (tokens x experts) with fp32 accumulation.  The
// K range (hidden) is split over the sixteen waves by interleaved 32-wide
// steps (so a wave needs about one batch of loads for H = 2880) and the
// sixteen partial sums are added in a fixed order, so every expert column goes
// through exactly the same sequence of operations: two identical router rows
// (silent copies) give bitwise-identical logits.  Top-k then takes one token
// per wave: up to 64 experts by rank (an expert is chosen when fewer than k
// order keys beat its own), beyond that by finding the k-th largest key one
// bit at a time with wave ballots (32 rounds, whatever k is).
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
constexpr int NW = 16;             // waves per workgroup
constexpr int kThreads = NW * 64;
constexpr int kCBMax = 4;          // 16-wide expert column blocks per pass (at most)
constexpr int kPartPer = 4;        // partial-logit elements per thread per round of loads

struct RouterSmem {
    // layout offsets (bytes) for a given padded expert count
    static __host__ __device__ size_t logits_off() { return 0; }
    static __host__ __device__ size_t part_off(int Ep) { return (size_t)BT * Ep * 4; }
    static __host__ __device__ size_t part_bytes() { return (size_t)NW * BT * kCBMax * 16 * 4; }
    // selection positions [BT][Ep] u16 reuse the partial-sum region once the logits are done
    static __host__ __device__ size_t selpos_off(int Ep) { return part_off(Ep); }
    // the bias [Ep] f32
    static __host__ __device__ size_t bias_off(int Ep) {
        const size_t sel = (size_t)BT * Ep * 2;
        return part_off(Ep) + (sel > part_bytes() ? sel : part_bytes());
    }
    // order keys [BT][64] u64 (one expert per lane only)
    static __host__ __device__ size_t key_off(int Ep) { return bias_off(Ep) + (size_t)Ep * 4; }
    static __host__ __device__ size_t bytes(int Ep) { return key_off(Ep) + (Ep == 64 ? (size_t)BT * 64 * 8 : 0); }
};

template <typename TA>
__device__ __forceinline__ float load_scalar(const TA* p, size_t i);
template <>
__device__ __forceinline__ float load_scalar<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_scalar<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

__device__ __forceinline__ uint32_t umax_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// One pass over K for CB 16-wide expert column blocks starting at cb0.
// Each wave takes the 32-wide K steps wave, wave + 4, ...; the loads of P
// consecutive steps are issued together before their MFMAs so that a wave
// waits for memory once per P steps.  Steps past the end load a valid address
// and contribute zero; columns past E read row E-1 and are discarded later.
template <typename TA, int CB>
__device__ __forceinline__ void logits_pass(const TA* __restrict__ hrow, const TA* __restrict__ wr, int H, int E,
                                            int cb0, int wave, int lane, f32x4 (&acc)[CB]) {
    constexpr bool kBf16 = sizeof(TA) == 2;
    constexpr int KSTEP = kBf16 ? 32 : 4;  // K per 16x16 MFMA
    constexpr int P = kBf16 ? (CB == 4 ? 3 : 6) : 8;  // steps per batch of loads (register budget)
    const int nsteps = H / KSTEP;
    const TA* wrow[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int e = min((cb0 + c) * 16 + (lane & 15), E - 1);
        wrow[c] = wr + (size_t)e * H;
    }
    if constexpr (kBf16) {
        const int koff = (lane >> 4) * 8;
        for (int s0 = wave; s0 < nsteps; s0 += NW * P) {
            bf16x8 a[P], b[P][CB];
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const int s = s0 + NW * q;
                const int kk = (s < nsteps ? s : s0) * KSTEP + koff;
                a[q] = *reinterpret_cast<const bf16x8*>(hrow + kk);
#pragma unroll
                for (int c = 0; c < CB; ++c) b[q][c] = *reinterpret_cast<const bf16x8*>(wrow[c] + kk);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of the MFMAs
#pragma unroll
            for (int q = 0; q < P; ++q) {
                if (s0 + NW * q >= nsteps) a[q] = bf16x8{};
#pragma unroll
                for (int c = 0; c < CB; ++c) acc[c] = mfma16(a[q], b[q][c], acc[c]);
            }
        }
    } else {
        const int koff = lane >> 4;
        for (int s0 = wave; s0 < nsteps; s0 += NW * P) {
            float a[P], b[P][CB];
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const int s = s0 + NW * q;
                const int kk = (s < nsteps ? s : s0) * KSTEP + koff;
                a[q] = hrow[kk];
#pragma unroll
                for (int c = 0; c < CB; ++c) b[q][c] = wrow[c][kk];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < P; ++q) {
                if (s0 + NW * q >= nsteps) a[q] = 0.f;
#pragma unroll
                for (int c = 0; c < CB; ++c) acc[c] = mfma16(a[q], b[q][c], acc[c]);
            }
        }
    }
}

template <typename TA, int CB, int NV>
__global__ __launch_bounds__(kThreads) void router_kernel(const TA* __restrict__ h, const TA* __restrict__ wr,
                                                     const TA* __restrict__ br, int T, int H, int E, int k,
                                                     float* __restrict__ logits_opt, int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w, int32_t* __restrict__ blk_counts,
                                                     int32_t* __restrict__ local_rank, const float* __restrict__ lpart) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int Ep = (E + 63) & ~63;  // padded so every lane owns Ep/64 columns
    float* s_lds = reinterpret_cast<float*>(smem + RouterSmem::logits_off());
    float* part = reinterpret_cast<float*>(smem + RouterSmem::part_off(Ep));
    uint16_t* selpos = reinterpret_cast<uint16_t*>(smem + RouterSmem::selpos_off(Ep));
    float* s_bias = reinterpret_cast<float*>(smem + RouterSmem::bias_off(Ep));
    unsigned long long* skey = reinterpret_cast<unsigned long long*>(smem + RouterSmem::key_off(Ep));

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int t0 = blockIdx.x * BT;
    const int nblk = gridDim.x;

    // the bias is read once, ahead of the logits loads, and parked in LDS with
    // the first partial sums (its latency hides behind theirs); the bf16
    // variant for 33..64 experts has no register to spare for it and reads it
    // in the reduction instead
    constexpr bool kBiasEarly = !(sizeof(TA) == 2 && CB == 4 && NV == 1);
    const float bias_r = (kBiasEarly && br && tid < E) ? load_scalar(br, tid) : 0.f;

    // ---------------------------------------------------------- logits --
    const int arow = min(t0 + (lane & 15), T - 1);
    const TA* hrow = h + (size_t)arow * H;
    const int ncb = (E + 15) >> 4;

    if (lpart) {
        // the slice sums written by the small-batch logits kernel, in slice
        // order, then the bias (parked in LDS first); the loads of kPartPer
        // elements are issued together
        for (int e = tid; e < E; e += kThreads) s_bias[e] = br ? load_scalar(br, e) : 0.f;
        __syncthreads();
        for (int i0 = tid; i0 < BT * E; i0 += kThreads * kPartPer) {
            float pv[kPartPer][kLogitSlices];
#pragma unroll
            for (int j = 0; j < kPartPer; ++j) {
                const int i = i0 + j * kThreads;
                const int row = i / E, e = i - row * E, t = t0 + row;
                const bool ok = i < BT * E && t < T;
                // an absent element reads element 0 (no branch around the loads:
                // all of them go out before the first is used)
                const size_t o = ok ? (size_t)t * E + e : 0;
#pragma unroll
                for (int ks = 0; ks < kLogitSlices; ++ks) pv[j][ks] = lpart[(size_t)ks * T * E + o];
            }
#pragma unroll
            for (int j = 0; j < kPartPer; ++j) {
                const int i = i0 + j * kThreads;
                const int row = i / E, e = i - row * E, t = t0 + row;
                if (i < BT * E && t < T) {
                    float v = 0.f;
#pragma unroll
                    for (int ks = 0; ks < kLogitSlices; ++ks) v += pv[j][ks];
                    s_lds[row * Ep + e] = br ? v + s_bias[e] : v;
                }
            }
        }
        __syncthreads();
    } else
    for (int cb0 = 0; cb0 < ncb; cb0 += CB) {
        f32x4 acc[CB];
        logits_pass<TA, CB>(hrow, wr, H, E, cb0, wave, lane, acc);
        // partial sums of this wave: part[wave][row][c*16 + col]
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int row = (lane >> 4) * 4 + j;
                part[((wave * BT) + row) * (kCBMax * 16) + c * 16 + (lane & 15)] = acc[c][j];
            }
        if (kBiasEarly && cb0 == 0 && tid < E) s_bias[tid] = bias_r;
        __syncthreads();
        // fixed-order reduction over the waves, then the bias
        for (int i = tid; i < BT * CB * 16; i += kThreads) {
            int row = i / (CB * 16);
            int col = i % (CB * 16);
            int e = cb0 * 16 + col;
            if (e < E) {
                float v = part[row * (kCBMax * 16) + col];
#pragma unroll
                for (int w = 1; w < NW; ++w) v += part[(w * BT + row) * (kCBMax * 16) + col];
                if constexpr (kBiasEarly)
                    v += s_bias[e];
                else if (br)
                    v += load_scalar(br, e);
                s_lds[row * Ep + e] = v;
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < BT * Ep; i += kThreads) selpos[i] = 0;
    __syncthreads();

    // -------------------------------------------- top-k + selected softmax --
    if constexpr (NV == 1) {
        // one expert per lane: selection by rank.  Every logit gets its order
        // key once (value, then lower index; 0 past E); expert e is chosen when
        // fewer than k keys exceed its own.  Positions are in ascending
        // expert order.
        for (int i = tid; i < BT * 64; i += kThreads) {
            const int e = i & 63;
            skey[i] = (e < E && t0 + (i >> 6) < T) ? order_key(s_lds[i], e) : 0ull;
        }
        __syncthreads();
        for (int tt = wave; tt < BT; tt += NW) {
            const int t = t0 + tt;
            if (t >= T) break;  // wave-uniform
            const bool ok = lane < E;
            const float v = ok ? s_lds[tt * Ep + lane] : 0.f;
            const unsigned long long mine = skey[tt * 64 + lane];
            const u32x4* krow = reinterpret_cast<const u32x4*>(skey + tt * 64);
            int rank = rank_of<16>(krow, mine);             // experts 0..31
            if (E > 32) rank += rank_of<16>(krow + 16, mine);  // 32..63 (two batches fit the registers)
            if (logits_opt && ok) logits_opt[(size_t)t * E + lane] = v;
            const bool chosen = ok & (rank < k);
            const uint64_t top = __ballot(ok & (rank == 0));
            const float smax = lane_f(v, (int)__builtin_ctzll(top));
            const float z = chosen ? expf(v - smax) : 0.f;
            const float denom = wave_sum(z);
            const uint64_t bal = __ballot(chosen);
            const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const int pos = __popcll(bal & lt);
            if (chosen) {
                topk_idx[(size_t)t * k + pos] = lane;
                topk_w[(size_t)t * k + pos] = z / denom;
                selpos[tt * Ep + lane] = (uint16_t)(pos + 1);
            }
        }
    } else
    // Lane owns experts e = lane + 64 i, i < NV (NV = padded E / 64).  The
    // k-th largest value key is found one bit at a time from the top: a
    // candidate stays when at least k keys reach it, a count that takes NV
    // ballots.  The experts above that key are selected, and of those equal
    // to it the lowest indices, as many as are still missing.  Steps are wave
    // uniform and independent of k.
    for (int tt = wave; tt < BT; tt += NW) {
        const int t = t0 + tt;
        if (t >= T) break;  // wave-uniform
        float orig[NV];
        uint32_t key[NV];   // value key, 0 for an absent expert (and for NaN)
        bool live[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + 64 * i;
            live[i] = e < E;
            orig[i] = live[i] ? s_lds[tt * Ep + e] : 0.f;
            key[i] = live[i] ? (uint32_t)(order_key(orig[i], e) >> 32) : 0u;
        }
        if (logits_opt) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (live[i]) logits_opt[(size_t)t * E + lane + 64 * i] = orig[i];
        }
        // largest tau with at least k keys >= tau (candidates are >= 1, so
        // absent experts never count; tau = 0 leaves only NaN logits to tie)
        uint32_t tau = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = tau | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(key[i] >= cand));
            tau = cnt >= k ? cand : tau;
        }
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int above = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) above += __popcll(__ballot(live[i] && key[i] > tau));
        const int need = k - above;  // >= 1 ties at tau, taken in ascending expert order
        uint32_t selmask = 0, kmax = 0;
        int ties_before = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool tie = live[i] && key[i] == tau;
            const uint64_t tm = __ballot(tie);
            const bool sel = (live[i] && key[i] > tau) || (tie && ties_before + __popcll(tm & lt) < need);
            selmask |= sel ? (1u << i) : 0u;
            kmax = (sel && key[i] > kmax) ? key[i] : kmax;
            ties_before += __popcll(tm);
        }
        // the largest selected value (the top-1), from its key
        kmax = umax_u32(kmax, (uint32_t)dpp_i<kDppXor1>((int)kmax));
        kmax = umax_u32(kmax, (uint32_t)dpp_i<kDppXor2>((int)kmax));
        kmax = umax_u32(kmax, (uint32_t)dpp_i<kDppHalfMirror>((int)kmax));
        kmax = umax_u32(kmax, (uint32_t)dpp_i<kDppMirror>((int)kmax));
        kmax = umax_u32(umax_u32((uint32_t)__builtin_amdgcn_readlane((int)kmax, 0),
                                 (uint32_t)__builtin_amdgcn_readlane((int)kmax, 16)),
                        umax_u32((uint32_t)__builtin_amdgcn_readlane((int)kmax, 32),
                                 (uint32_t)__builtin_amdgcn_readlane((int)kmax, 48)));
        const float smax = __uint_as_float((kmax & 0x80000000u) ? (kmax & 0x7fffffffu) : ~kmax);
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
#pragma unroll
        for (int i = 0; i < NV; ++i) {
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
    for (int e = tid; e < E; e += kThreads) {
        int running = 0;
        for (int tt = 0; tt < tcount; ++tt) {
            int sp = selpos[tt * Ep + e];
            if (sp) local_rank[(size_t)(t0 + tt) * k + (sp - 1)] = running++;
        }
        blk_counts[(size_t)e * nblk + blockIdx.x] = running;
    }
}

template <typename TA, int CB, int NV>
hipError_t launch_k(const void* h, const void* w_router, const void* b_router, int T, int H, int E, int k,
                    float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* blk_counts, int32_t* local_rank,
                    const float* part, hipStream_t stream) {
    const int nblk = (T + BT - 1) / BT;
    const size_t smem = RouterSmem::bytes((E + 63) & ~63);
    auto kern = router_kernel<TA, CB, NV>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)RouterSmem::bytes(1024));
    if (attr != hipSuccess) return attr;
    kern<<<nblk, kThreads, smem, stream>>>((const TA*)h, (const TA*)w_router, (const TA*)b_router, T, H, E, k, logits_opt,
                                      topk_idx, topk_w, blk_counts, local_rank, part);
    return hipGetLastError();
}

// Instantiation by expert count: CB column blocks per logits pass, NV experts per lane in top-k.
template <typename TA>
hipError_t launch_t(const void* h, const void* w_router, const void* b_router, int T, int H, int E, int k,
                    float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* blk_counts, int32_t* local_rank,
                    const float* part, hipStream_t stream) {
#define MOE_ROUTER_LAUNCH(CB, NV)                                                                                  \
    return launch_k<TA, CB, NV>(h, w_router, b_router, T, H, E, k, logits_opt, topk_idx, topk_w, blk_counts, \
                                local_rank, part, stream)
    if (E <= 16) MOE_ROUTER_LAUNCH(1, 1);
    if (E <= 32) MOE_ROUTER_LAUNCH(2, 1);
    if (E <= 64) MOE_ROUTER_LAUNCH(4, 1);
    if (E <= 128) MOE_ROUTER_LAUNCH(4, 2);
    if (E <= 256) MOE_ROUTER_LAUNCH(4, 4);
    MOE_ROUTER_LAUNCH(4, 16);
#undef MOE_ROUTER_LAUNCH
}

}  // namespace

hipError_t launch_router(int act_dtype, const void* h, const void* w_router, const void* b_router, int T, int H,
                         int E, int k, float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* blk_counts,
                         int32_t* local_rank, const float* part, hipStream_t stream) {
    if (act_dtype == DT_BF16)
        return launch_t<uint16_t>(h, w_router, b_router, T, H, E, k, logits_opt, topk_idx, topk_w, blk_counts,
                                  local_rank, part, stream);
    return launch_t<float>(h, w_router, b_router, T, H, E, k, logits_opt, topk_idx, topk_w, blk_counts, local_rank,
                           part, stream);
}

size_t router_smem_bytes(int E) { return RouterSmem::bytes((E + 63) & ~63); }

}  // namespace moe
