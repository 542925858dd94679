// Stage 1 of the layer: from the per-token selected sets to the expert-major
// order in which the experts' rows are processed.
//
//   counts[e]   number of (token, slot) assignments to expert e
//   offsets     exclusive prefix sum of counts, offsets[E] = T*k
//   perm_src[r] the assignment t*k+slot at row r; rows of one expert are
//               ordered by token (a stable counting sort: no atomics, so the
//               result is unique and run-to-run identical)
//   inv[a]      the row of assignment a
//   row_p[r]    topk_w[perm_src[r]], the routing weight of row r (so that the
//               down product's epilogue needs no dependent load)
//   tiles       the (expert, first row, rows) tiles of at most BM rows that the
//               grouped GEMMs walk; experts without tokens get no tile.
//   work lists  the order in which the GEMM workgroups take (row tile, column
//               tile) pairs: expert by expert, for each column tile all of the
//               expert's row tiles.
//
// One workgroup of 1024 threads.  Input: the per-token-tile expert counts and
// the within-tile ranks written by the router stage.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBaseLds = 16384;  // ints of scanned bases kept in LDS (64 KB)
constexpr int kPer = 4;           // elements per lane per round of loads (per-expert scans)
constexpr int kScatterPer = 16;   // assignments per thread per round of loads (scatter)
constexpr int kCopyPer = 8;       // counts per thread per round of loads (copy into LDS)
constexpr int kShortRow = 8;      // rows of at most this many token blocks: one thread per expert

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(int T, int E, int k, int BM,
                                                          const int32_t* __restrict__ topk_idx,
                                                          int32_t* __restrict__ blk,  // [E][nblk]
                                                          const int32_t* __restrict__ local_rank,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                                          int32_t* __restrict__ inv, const float* __restrict__ topk_w,
                                                          float* __restrict__ row_p, Tile* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles, int max_tiles, WorkList w0,
                                                          WorkList w1, int32_t* __restrict__ zero, int n_zero,
                                                          bool scatter_outside) {
    __shared__ int32_t totals[1024];
    // the scanned per-block bases, kept here when they fit (E * nblk <= kBaseLds)
    __shared__ int32_t base_lds[kBaseLds];
    __shared__ int32_t offs[1025];
    __shared__ int32_t toff[1025];
    __shared__ int32_t wsum[16];
    __shared__ int32_t wtile[16];
    __shared__ int32_t csum[2][16];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int nblk = (T + kRouterTokens - 1) / kRouterTokens;
    if (tid < n_zero) zero[tid] = 0;

    // 1. per expert: exclusive scan of its tile counts (in place) and its total.
    //    A lane owns kPer consecutive blocks, so a row of up to 64 * kPer
    //    counts is read in one round of loads; longer rows take more rounds.
    //    When the counts fit in LDS they are first copied there by all
    //    threads in a few rounds of independent loads (one wave walking its
    //    experts through global memory would wait out one load latency per
    //    expert), and the scans read LDS.
    const bool in_lds = E * nblk <= kBaseLds;
    if (in_lds) {
        const int n = E * nblk;
        for (int i0 = tid; i0 < n; i0 += 1024 * kCopyPer) {
            int v[kCopyPer];
#pragma unroll
            for (int j = 0; j < kCopyPer; ++j) {
                const int i = i0 + j * 1024;
                v[j] = i < n ? blk[i] : 0;
            }
#pragma unroll
            for (int j = 0; j < kCopyPer; ++j) {
                const int i = i0 + j * 1024;
                if (i < n) base_lds[i] = v[j];
            }
        }
        __syncthreads();
    }
    if (in_lds && nblk <= kShortRow) {
        // short rows (few token blocks): one thread per expert
        for (int e = tid; e < E; e += 1024) {
            int running = 0;
            for (int b = 0; b < nblk; ++b) {
                const int c = base_lds[e * nblk + b];
                base_lds[e * nblk + b] = running;
                blk[(size_t)e * nblk + b] = running;
                running += c;
            }
            totals[e] = running;
        }
    } else
    for (int e = wave; e < E; e += 16) {
        int running = 0;
        int32_t* row = blk + (size_t)e * nblk;
        for (int b0 = 0; b0 < nblk; b0 += 64 * kPer) {
            int c[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = b0 + lane * kPer + j;
                c[j] = i < nblk ? (in_lds ? base_lds[e * nblk + i] : row[i]) : 0;
            }
            int sum = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) sum += c[j];
            const int x = wave_incl_scan(sum, lane);
            int pre = running + x - sum;  // exclusive prefix of this lane's first block
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = b0 + lane * kPer + j;
                if (i < nblk) {
                    row[i] = pre;
                    if (in_lds) base_lds[e * nblk + i] = pre;
                }
                pre += c[j];
            }
            running += __shfl(x, 63, 64);
        }
        if (lane == 0) totals[e] = running;
    }
    __syncthreads();

    // 2. exclusive scans over experts: row offsets and tile offsets
    const int cnt = tid < E ? totals[tid] : 0;
    const int nt = tid < E ? (cnt + BM - 1) / BM : 0;
    int xs = wave_incl_scan(cnt, lane);
    int xt = wave_incl_scan(nt, lane);
    if (lane == 63) {
        wsum[wave] = xs;
        wtile[wave] = xt;
    }
    __syncthreads();
    int bs = 0, bt = 0;
    for (int w = 0; w < wave; ++w) {
        bs += wsum[w];
        bt += wtile[w];
    }
    if (tid < E) {
        offs[tid] = bs + xs - cnt;
        toff[tid] = bt + xt - nt;
    }
    if (tid == E - 1) {
        offs[E] = bs + xs;
        toff[E] = bt + xt;
    }
    __syncthreads();

    // 3. outputs: offsets and the tile list
    if (tid < E) offsets[tid] = offs[tid];
    if (tid == 0) {
        offsets[E] = offs[E];
        n_tiles[0] = toff[E];
    }
    if (tid < E) {
        const int base = toff[tid];
        for (int j = 0; j < nt && base + j < max_tiles; ++j) {
            Tile tl;
            tl.expert = tid;
            tl.row_start = offs[tid] + j * BM;
            tl.rows = min(BM, cnt - j * BM);
            tl.pad = 0;
            tiles[base + j] = tl;
        }
        // work lists: this expert's (column tile, row tile) pairs, row tiles fastest
        for (int l = 0; l < 2; ++l) {
            const WorkList& w = l ? w1 : w0;
            if (!w.items) continue;
            const int nc = w.n_col_tiles;
            int32_t* dst = w.items + (size_t)base * nc;
            for (int c = 0; c < nc; ++c)
                for (int j = 0; j < nt; ++j) dst[c * nt + j] = (base + j) * nc + c;
        }
    }
    if (tid == 0) {
        if (w0.count) w0.count[0] = toff[E] * w0.n_col_tiles;
        if (w1.count) w1.count[0] = toff[E] * w1.n_col_tiles;
    }

    // 3b. each work list cut into kXcdRanges contiguous ranges of equal
    //     estimated cost.  Expert e's items cost nc * se (se: one column of its
    //     tiles); the experts' cost intervals, from a block scan, partition
    //     [0, total), and the expert whose interval holds x * total / 8 finds
    //     the first of its items that starts at or past that cost, then
    //     moves the cut to the nearer end of that column tile's row tiles.
    {
        int groups = 0;  // live 32-row groups over this expert's tiles
        for (int j = 0; j < nt; ++j) groups += (min(BM, cnt - j * BM) + 31) / 32;
        int se[2], ce[2], xc[2];
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            se[l] = kItemFixedCost[l] * nt + groups;
            ce[l] = (l ? w1.n_col_tiles : w0.n_col_tiles) * se[l];
            xc[l] = wave_incl_scan(ce[l], lane);
            if (lane == 63) csum[l][wave] = xc[l];
        }
        __syncthreads();
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            const WorkList& w = l ? w1 : w0;
            if (!w.items || !w.bounds) continue;  // uniform
            const int nc = w.n_col_tiles;
            int bc = 0, tot = 0;
            for (int ww = 0; ww < 16; ++ww) {
                if (ww < wave) bc += csum[l][ww];
                tot += csum[l][ww];
            }
            const int pe = bc + xc[l] - ce[l];
            if (tid == 0) {
                w.bounds[0] = 0;
                w.bounds[kXcdRanges] = toff[E] * nc;
                if (tot == 0)
                    for (int x = 1; x < kXcdRanges; ++x) w.bounds[x] = 0;
            }
            if (ce[l] > 0) {
                for (int x = 1; x < kXcdRanges; ++x) {
                    const long long target = (long long)tot * x / kXcdRanges;
                    if (target < pe || target >= (long long)pe + ce[l]) continue;
                    const int rem0 = (int)(target - pe);
                    const int c = rem0 / se[l];
                    const int rem = rem0 - c * se[l];
                    int j = 0, acc = 0;
                    while (acc < rem) {
                        acc += kItemFixedCost[l] + (min(BM, cnt - j * BM) + 31) / 32;
                        ++j;
                    }
                    // snap to the nearer end of column tile c's row tiles, so
                    // that one XCD runs all of them and its L2 serves the
                    // weight panel's repeats
                    w.bounds[x] = toff[tid] * nc + (2 * j <= nt ? c : c + 1) * nt;
                }
            }
        }
    }

    // 4. stable scatter: row = offsets[e] + (earlier tiles' count) + rank in tile.
    //    Loads of kScatterPer assignments are issued together.  Large
    //    batches scatter in their own launch over many CUs instead (one CU's
    //    loads in flight would take a few dozen round trips).
    if (scatter_outside) return;
    const int total = T * k;
    for (int a0 = 0; a0 < total; a0 += 1024 * kScatterPer) {
        int e[kScatterPer], lr[kScatterPer];
        float tw[kScatterPer];
#pragma unroll
        for (int j = 0; j < kScatterPer; ++j) {
            const int a = a0 + j * 1024 + tid;
            e[j] = a < total ? topk_idx[a] : 0;
            lr[j] = a < total ? local_rank[a] : 0;
            tw[j] = a < total ? topk_w[a] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kScatterPer; ++j) {
            const int a = a0 + j * 1024 + tid;
            if (a < total) {
                const int b = (a / k) / kRouterTokens;
                const size_t bi = (size_t)e[j] * nblk + b;
                const int r = offs[e[j]] + (in_lds ? base_lds[bi] : blk[bi]) + lr[j];
                perm_src[r] = a;
                inv[a] = r;
                row_p[r] = tw[j];
            }
        }
    }
}

// Step 4 of the route scan for large batches, one assignment per thread:
// the same row formula, with the per-block bases from global memory.
__global__ __launch_bounds__(256) void route_scatter_kernel(int total, int k, int nblk,
                                                            const int32_t* __restrict__ topk_idx,
                                                            const int32_t* __restrict__ bases,
                                                            const int32_t* __restrict__ local_rank,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm_src, int32_t* __restrict__ inv,
                                                            const float* __restrict__ topk_w,
                                                            float* __restrict__ row_p) {
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= total) return;
    const int e = topk_idx[a];
    const int b = (a / k) / kRouterTokens;
    const int r = offsets[e] + bases[(size_t)e * nblk + b] + local_rank[a];
    perm_src[r] = a;
    inv[a] = r;
    row_p[r] = topk_w[a];
}

// Batches of more assignments than this scatter in their own launch.
constexpr int kScatterInKernelMax = 4096;

}  // namespace

hipError_t launch_route_scan(int T, int E, int k, int BM, const int32_t* topk_idx, int32_t* blk_counts,
                             const int32_t* local_rank, int32_t* offsets, int32_t* perm_src, int32_t* inv,
                             const float* topk_w, float* row_p, Tile* tiles, int32_t* n_tiles, int max_tiles,
                             WorkList w0, WorkList w1, int32_t* zero, int n_zero, hipStream_t stream) {
    const int total = T * k;
    const bool outside = total > kScatterInKernelMax;
    route_scan_kernel<<<1, 1024, 0, stream>>>(T, E, k, BM, topk_idx, blk_counts, local_rank, offsets, perm_src, inv,
                                              topk_w, row_p, tiles, n_tiles, max_tiles, w0, w1, zero, n_zero,
                                              outside);
    if (outside) {
        const int nblk = (T + kRouterTokens - 1) / kRouterTokens;
        route_scatter_kernel<<<(total + 255) / 256, 256, 0, stream>>>(total, k, nblk, topk_idx, blk_counts,
                                                                      local_rank, offsets, perm_src, inv, topk_w,
                                                                      row_p);
    }
    return hipGetLastError();
}

}  // namespace moe
