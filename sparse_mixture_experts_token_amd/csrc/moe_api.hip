// C interface of the sparse MoE layer (declared in include/moe.h): argument
// checks, workspace layout, stage launches on the caller's stream, the
// pre-normalised block entry point, the silent expansion and the per-stage
// timing hooks.
#include <mutex>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

// Scratch of moe_forward_noalloc: the workspace regions of one call, in a
// static array that each device holds from the code object's load on.  Host
// code never uses this name as an address (it is only a host-side stand-in);
// kernels get the device address from hipGetSymbolAddress below.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::Tile;

// Per-device address of `scratch`, looked up once per device with that device
// current (each device holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(hipStream_t stream, char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return MOE_ERR_HIP;
    }
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<char*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

int check_problem(const moe_problem* p) {
    if (!p) return MOE_ERR_NULL;
    if (p->T < 0 || p->H <= 0 || p->I <= 0 || p->E < 1 || p->E > 1024 || p->k < 1 || p->k > p->E)
        return MOE_ERR_SHAPE;
    if (p->H % 64 != 0 || p->I % 64 != 0) return MOE_ERR_SHAPE;
    const int64_t big = (int64_t)p->T * p->k * (p->H > p->I ? p->H : p->I);
    if (big >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
    if ((int64_t)p->H * p->I >= (int64_t(1) << 29)) return MOE_ERR_SHAPE;
    // MXFP4: a GEMM tile keeps its scales for the whole contraction in LDS
    if (p->expert_dtype == MOE_MXFP4 && (p->H > moe::mxfp4_max_k() || p->I > moe::mxfp4_max_k())) return MOE_ERR_SHAPE;
    const bool ok = (p->act_dtype == MOE_F32 && p->expert_dtype == MOE_F32) ||
                    (p->act_dtype == MOE_BF16 && (p->expert_dtype == MOE_BF16 || p->expert_dtype == MOE_MXFP4));
    if (!ok) return MOE_ERR_DTYPE;
    return MOE_OK;
}

// Workspace regions, in order.
struct Layout {
    size_t topk_idx, topk_w, blk, rank, offsets, perm, inv, rowp, tiles, ntiles, queues, work0, work1, part, act, y,
        total;
    int nblk, max_tiles, BM, nc0, nc1;
    bool decode;
    bool fused;  // routing computed inside the gate/up kernel (small decode problems)
    bool plogits;  // router logits from the partial-logits kernel (small bf16 batches)
    bool lists;  // prefill work lists are built
};

// router_dt: the router's input format (-1: the activation format).  The
// partial-logits kernel and the fused decode routing take bf16 input only;
// all_plogits: partial logits at every T (the block's folded router).
Layout layout(const moe_problem* p, int router_dt = -1, bool all_plogits = false) {
    Layout L{};
    const int rdt = router_dt < 0 ? p->act_dtype : router_dt;
    const size_t tk = (size_t)p->T * p->k;
    L.decode = moe::decode_path(p->act_dtype, p->T, p->H, p->I, p->E, p->k);
    L.fused = rdt == MOE_BF16 && moe::decode_fused(p->act_dtype, p->T, p->H, p->I, p->E, p->k);
    L.plogits = rdt == MOE_BF16 && (p->T <= 64 || all_plogits);
    L.BM = L.decode ? moe::decode_block_m() : moe::gemm_block_m(p->act_dtype, p->expert_dtype, p->T, p->k, p->E);
    L.nblk = (p->T + moe::kRouterTokens - 1) / moe::kRouterTokens;
    L.max_tiles = (int)((tk + L.BM - 1) / L.BM) + p->E;
    size_t o = 0;
    L.topk_idx = o; o = align_up(o + tk * 4);
    L.topk_w = o;   o = align_up(o + tk * 4);
    L.blk = o;      o = align_up(o + (size_t)p->E * L.nblk * 4);
    L.rank = o;     o = align_up(o + tk * 4);
    L.offsets = o;  o = align_up(o + ((size_t)p->E + 1) * 4);
    L.perm = o;     o = align_up(o + tk * 4);
    L.inv = o;      o = align_up(o + tk * 4);
    L.rowp = o;     o = align_up(o + tk * 4);
    L.tiles = o;    o = align_up(o + (size_t)L.max_tiles * sizeof(Tile));
    L.ntiles = o;   o = align_up(o + 256);  // tile count, the two work-list counts, then at ints 16 and 32
                                            // the two lists' XCD range bounds
    L.queues = o;   o = align_up(o + moe::kNumQueues * 4);
    // column tiles of the prefill work lists (the decode kernels need none)
    // (only the bf16-activation prefill kernels walk work lists)
    L.lists = !L.decode && p->act_dtype == MOE_BF16;
    L.nc0 = L.lists ? moe::bf16_col_tiles(p->I, 0, p->expert_dtype) : 0;
    L.nc1 = L.lists ? moe::bf16_col_tiles(p->H, 1, p->expert_dtype) : 0;
    L.work0 = o;    o = align_up(o + (size_t)L.max_tiles * L.nc0 * 4);
    L.work1 = o;    o = align_up(o + (size_t)L.max_tiles * L.nc1 * 4);
    L.part = o;     o = align_up(o + (L.plogits ? moe::decode_logit_part_bytes(p->T, p->E) : 0));
    L.act = o;      o = align_up(o + tk * p->I * act_bytes(p->act_dtype));
    L.y = o;        o = align_up(o + tk * p->H * 4);
    L.total = o;
    return L;
}

// The block entry point's workspace: the layer's, then for bf16 activations
// the GEMMs' bf16 input, each token's 1/rms and the router with the gain
// folded in (two bf16 parts); for fp32 activations the fp32 normalised input
// (the router's and the GEMMs').
struct BlockLayout {
    Layout L;
    size_t n32, n16, rs, whi, wlo, total;
};

BlockLayout block_layout(const moe_problem* p) {
    BlockLayout B{};
    const bool bf = p->act_dtype == MOE_BF16;
    B.L = bf ? layout(p, MOE_BF16, true) : layout(p, MOE_F32);
    const size_t th = (size_t)p->T * p->H, eh = (size_t)p->E * p->H;
    size_t o = B.L.total;
    B.n32 = o; o = align_up(o + (bf ? 0 : th * 4));
    B.n16 = o; o = align_up(o + (bf ? th * 2 : 0));
    B.rs = o;  o = align_up(o + (bf ? (size_t)p->T * 4 : 0));
    B.whi = o; o = align_up(o + (bf ? eh * 2 : 0));
    B.wlo = o; o = align_up(o + (bf ? eh * 2 : 0));
    B.total = o;
    return B;
}

constexpr bool kBackwardDisabled = true;

// Backward workspace regions (bf16 activations and weights).
struct BwdLayout {
    size_t inv, tiles, ntiles, Xp, Dp, dY, G, U, GY, dG, dU, ACT, DA, dp, dsd, dsf, total;
};
BwdLayout bwd_layout(const moe_problem* p) {
    BwdLayout B{};
    const size_t R = (size_t)p->T * p->k, H = p->H, I = p->I, Ep = (p->E + 7) & ~7;
    size_t o = 0;
    B.inv = o;    o = align_up(o + R * 4);
    B.tiles = o;  o = align_up(o + (size_t)moe::bwd_max_tiles(p->T, p->k, p->E) * 4);
    B.ntiles = o; o = align_up(o + 4);
    B.Xp = o;     o = align_up(o + R * H * 2);
    B.Dp = o;     o = align_up(o + R * H * 2);
    B.dY = o;     o = align_up(o + R * H * 2);
    B.G = o;      o = align_up(o + R * I * 4);
    B.U = o;      o = align_up(o + R * I * 4);
    B.GY = o;     o = align_up(o + R * I * 4);
    B.dG = o;     o = align_up(o + R * I * 2);
    B.dU = o;     o = align_up(o + R * I * 2);
    B.ACT = o;    o = align_up(o + R * I * 2);
    B.DA = o;     o = align_up(o + R * H * 4);
    B.dp = o;     o = align_up(o + R * 4);
    B.dsd = o;    o = align_up(o + (size_t)p->T * Ep * 2);
    B.dsf = o;    o = align_up(o + (size_t)p->T * p->E * 4);
    B.total = o;
    return B;
}

// ------------------------------------------------------------ profiling --
struct Profiler {
    std::mutex mu;
    bool armed = false;
    int max_calls = 0;
    int used = 0;
    uint32_t mask = 0;           // stage boundaries recorded (bit i: the event before stage i)
    std::vector<hipEvent_t> ev;  // max_calls x (MOE_NUM_STAGES + 1)
};
Profiler& prof() {
    static Profiler p;
    return p;
}

// Returns the event row for this call (and the boundaries to record), or
// nullptr when not recording.
hipEvent_t* prof_slot(uint32_t* mask) {
    Profiler& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    if (!P.armed || P.used >= P.max_calls) return nullptr;
    *mask = P.mask;
    return &P.ev[(size_t)(P.used++) * (MOE_NUM_STAGES + 1)];
}

// Checks shared by the forward entry points (h is the layer input).  T = 0
// sets *noop: nothing to do, outputs untouched.
int check_call(const moe_problem* p, const moe_weights* w, const void* h, const void* out,
               const moe_routing* routing, const void* workspace, bool* noop) {
    *noop = false;
    int st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!w) return MOE_ERR_NULL;
    if (p->T == 0) {
        *noop = true;
        return MOE_OK;
    }
    if (!h || !out || !workspace || !w->w_router || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL;
    if (p->expert_dtype == MOE_MXFP4 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_NULL;
    for (const void* q : {h, (const void*)out, (const void*)workspace, w->w_router, w->w_gate, w->w_up, w->w_down})
        if (!aligned(q, 16)) return MOE_ERR_ALIGN;
    if (w->b_router && !aligned(w->b_router, act_bytes(p->act_dtype))) return MOE_ERR_ALIGN;
    if (routing) {
        for (const void* q : {(const void*)routing->logits, (const void*)routing->topk_idx,
                              (const void*)routing->topk_w, (const void*)routing->expert_offsets,
                              (const void*)routing->perm_src})
            if (q && !aligned(q, 4)) return MOE_ERR_ALIGN;
    }
    return MOE_OK;
}

// Inputs of one pass through the stages besides the problem, the expert
// weights and the outputs.
struct PassIn {
    int router_dt;         // format of router_h, w_router and b_router
    const void* router_h;  // the router's input [T, H]
    const void* w_router;
    const void* w_router_lo;  // bf16 router as two parts (partial logits only), or null
    const float* row_scale;   // per-token scale of the partial logits, or null
    const void* b_router;     // may be null
    const void* gemm_h;    // the expert GEMMs' input [T, H] (act dtype)
    const void* residual;  // added in the combine (act dtype) or null
    // pre-norm prologue (norm_g null: none), writing n32 / n16 / wr32 / br32
    const void* norm_g;
    float eps;
    const void* x;
    float* n32;
    uint16_t* n16;
    float* rs;
    uint16_t* whi;
    uint16_t* wlo;
};

int run_pass(const moe_problem* p, const moe_weights* w, const PassIn& in, void* out, const moe_routing* routing,
             char* ws, const Layout& L, hipStream_t stream) {
    int32_t* topk_idx = (routing && routing->topk_idx) ? routing->topk_idx : (int32_t*)(ws + L.topk_idx);
    float* topk_w = (routing && routing->topk_w) ? routing->topk_w : (float*)(ws + L.topk_w);
    int32_t* offsets = (routing && routing->expert_offsets) ? routing->expert_offsets : (int32_t*)(ws + L.offsets);
    int32_t* perm = (routing && routing->perm_src) ? routing->perm_src : (int32_t*)(ws + L.perm);
    float* logits = routing ? routing->logits : nullptr;
    int32_t* blk = (int32_t*)(ws + L.blk);
    int32_t* rank = (int32_t*)(ws + L.rank);
    int32_t* inv = (int32_t*)(ws + L.inv);
    float* row_p = (float*)(ws + L.rowp);
    Tile* tiles = (Tile*)(ws + L.tiles);
    int32_t* ntiles = (int32_t*)(ws + L.ntiles);
    void* act = ws + L.act;
    float* y = (float*)(ws + L.y);

    uint32_t ev_mask = 0;
    hipEvent_t* ev = prof_slot(&ev_mask);
    auto mark = [&](int i) {
        if (ev && ((ev_mask >> i) & 1u)) (void)hipEventRecord(ev[i], stream);
    };

    hipError_t e = hipSuccess;
    moe::WorkList wl0{L.lists ? (int32_t*)(ws + L.work0) : nullptr, ntiles + 1, L.nc0, ntiles + 16};
    moe::WorkList wl1{L.lists ? (int32_t*)(ws + L.work1) : nullptr, ntiles + 2, L.nc1, ntiles + 32};
    int32_t* queues = (int32_t*)(ws + L.queues);
    float* part = (float*)(ws + L.part);
    mark(0);
    if (in.norm_g) {
        e = moe::launch_rms_norm(p->act_dtype, in.x, in.norm_g, in.eps, p->T, p->H, in.n32, in.n16, in.rs,
                                 w->w_router, p->E, in.whi, in.wlo, stream);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (L.plogits) {
        e = moe::launch_decode_logits(in.router_h, in.w_router, in.w_router_lo, in.row_scale, p->T, p->H, p->E,
                                      part, stream);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (!L.fused) {
        e = moe::launch_router(in.router_dt, in.router_h, in.w_router, in.b_router, p->T, p->H, p->E, p->k, logits,
                               topk_idx, topk_w, blk, rank, L.plogits ? part : nullptr, stream);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    mark(1);
    if (!L.fused) {
        e = moe::launch_route_scan(p->T, p->E, p->k, L.BM, topk_idx, blk, rank, offsets, perm, inv, topk_w, row_p,
                                   tiles, ntiles, L.max_tiles, wl0, wl1, queues, moe::kNumQueues, stream);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    mark(2);

    moe::GemmProblem g{};
    g.T = p->T; g.H = p->H; g.I = p->I; g.E = p->E; g.k = p->k;
    g.act_dtype = p->act_dtype;
    g.expert_dtype = p->expert_dtype;
    g.h = in.gemm_h;
    g.w_gate = w->w_gate; g.w_up = w->w_up; g.w_down = w->w_down;
    g.s_gate = w->s_gate; g.s_up = w->s_up; g.s_down = w->s_down;
    g.perm_src = perm;
    g.topk_w = topk_w;
    g.row_p = row_p;
    g.tiles = tiles;
    g.n_tiles = ntiles;
    g.max_tiles = L.max_tiles;
    g.work_gateup = wl0.items;
    g.n_work_gateup = wl0.count;
    g.work_down = wl1.items;
    g.n_work_down = wl1.count;
    g.bounds_gateup = wl0.bounds;
    g.bounds_down = wl1.bounds;
    g.act = act;
    g.y = y;
    g.decode = L.decode;
    g.queues = queues;
    if (L.fused) {
        const moe::FusedRouting fr{part, in.b_router, logits, topk_idx, topk_w, offsets, perm, inv, row_p, tiles, ntiles};
        e = moe::launch_route_gateup_decode(g, fr, stream);
    } else {
        e = moe::launch_gateup(g, stream);
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(3);
    e = moe::launch_down(g, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(4);
    e = moe::launch_combine(p->act_dtype, y, out, p->T, p->H, p->k, in.residual, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    mark(5);
    return MOE_OK;
}
}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return layout(p).total;
}

const char* moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "required pointer is NULL";
        case MOE_ERR_SHAPE: return "unsupported sizes (need 0<=T, 1<=k<=E<=1024, H and I positive multiples of 64, T*k*max(H,I) < 2^31, M>=1)";
        case MOE_ERR_DTYPE: return "unsupported dtype pair (need F32/F32, BF16/BF16 or BF16/MXFP4)";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
        case MOE_ERR_ALIGN: return "pointer not aligned (16 bytes for tensors and workspace, 4 for routing outputs and bias)";
        case MOE_ERR_HIP: return "HIP runtime error at enqueue";
        case MOE_ERR_STATE: return "profiling calls out of order";
        case MOE_ERR_DISABLED: return "entry point switched off in this build (moe_backward: GPU fault under investigation)";
        case MOE_ERR_SCRATCH: return "problem needs more workspace than moe_forward_noalloc's static scratch (MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

const char* moe_stage_name(int s) {
    static const char* names[MOE_NUM_STAGES] = {"router_topk_softmax", "route_scan_permute", "gateup_swiglu_gemm",
                                                "down_weighted_gemm", "combine"};
    return (s >= 0 && s < MOE_NUM_STAGES) ? names[s] : "unknown";
}

int moe_forward(const moe_problem* p, const moe_weights* w, const void* h, void* out, const moe_routing* routing,
                void* workspace, size_t workspace_bytes, void* stream_v) {
    bool noop = false;
    const int st = check_call(p, w, h, out, routing, workspace, &noop);
    if (st != MOE_OK || noop) return st;
    const Layout L = layout(p);
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    PassIn in{};
    in.router_dt = p->act_dtype;
    in.router_h = h;
    in.w_router = w->w_router;
    in.b_router = w->b_router;
    in.gemm_h = h;
    return run_pass(p, w, in, out, routing, reinterpret_cast<char*>(workspace), L,
                    reinterpret_cast<hipStream_t>(stream_v));
}

int moe_forward_noalloc(const moe_problem* p, const moe_weights* w, const void* h, void* out,
                        const moe_routing* routing, void* stream_v) {
    bool noop = false;
    // the static scratch is 256-byte aligned: pass any aligned non-null stand-in to the shared checks
    int st = check_call(p, w, h, out, routing, reinterpret_cast<const void*>(kAlign), &noop);
    if (st != MOE_OK || noop) return st;
    const Layout L = layout(p);
    if (L.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    char* ws = nullptr;
    st = scratch_of_current_device(stream, &ws);
    if (st != MOE_OK) return st;
    PassIn in{};
    in.router_dt = p->act_dtype;
    in.router_h = h;
    in.w_router = w->w_router;
    in.b_router = w->b_router;
    in.gemm_h = h;
    return run_pass(p, w, in, out, routing, ws, L, stream);
}

size_t moe_block_workspace_bytes(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return block_layout(p).total;
}

int moe_block_forward(const moe_problem* p, const moe_weights* w, const void* norm_weight, float eps, const void* x,
                      void* out, const moe_routing* routing, void* workspace, size_t workspace_bytes,
                      void* stream_v) {
    bool noop = false;
    const int st = check_call(p, w, x, out, routing, workspace, &noop);
    if (st != MOE_OK || noop) return st;
    if (!norm_weight) return MOE_ERR_NULL;
    if (!aligned(norm_weight, 16)) return MOE_ERR_ALIGN;
    if (!(eps >= 0.0f) || eps > 1e30f) return MOE_ERR_SHAPE;  // also rejects NaN and inf
    const BlockLayout B = block_layout(p);
    if (workspace_bytes < B.total) return MOE_ERR_WORKSPACE;
    char* ws = reinterpret_cast<char*>(workspace);
    const bool bf = p->act_dtype == MOE_BF16;
    PassIn in{};
    in.norm_g = norm_weight;
    in.eps = eps;
    in.x = x;
    in.residual = x;
    in.b_router = w->b_router;
    if (bf) {
        // logits r_t * (x . (W_r * g)) from x itself and the folded router
        in.n16 = (uint16_t*)(ws + B.n16);
        in.rs = (float*)(ws + B.rs);
        in.whi = (uint16_t*)(ws + B.whi);
        in.wlo = (uint16_t*)(ws + B.wlo);
        in.router_dt = MOE_BF16;
        in.router_h = x;
        in.w_router = in.whi;
        in.w_router_lo = in.wlo;
        in.row_scale = in.rs;
        in.gemm_h = in.n16;
    } else {
        // the fp32 router on the fp32 normalised input
        in.n32 = (float*)(ws + B.n32);
        in.router_dt = MOE_F32;
        in.router_h = in.n32;
        in.w_router = w->w_router;
        in.gemm_h = in.n32;
    }
    return run_pass(p, w, in, out, routing, ws, B.L, reinterpret_cast<hipStream_t>(stream_v));
}

size_t moe_backward_workspace_bytes(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return bwd_layout(p).total;
}

int moe_backward(const moe_problem* p, const moe_weights* w, const void* h, const void* d_out,
                 const moe_routing* routing, const uint8_t* trainable, void* d_h, const moe_grads* grads,
                 void* workspace, size_t workspace_bytes, void* stream_v) {
    const int st = check_problem(p);
    if (st != MOE_OK) return st;
    if (p->act_dtype != MOE_BF16 || p->expert_dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (!w) return MOE_ERR_NULL;
    if (p->T == 0) return MOE_OK;
    if (!h || !d_out || !routing || !workspace || !w->w_router || !w->w_gate || !w->w_up || !w->w_down)
        return MOE_ERR_NULL;
    if (!routing->topk_idx || !routing->topk_w || !routing->expert_offsets || !routing->perm_src)
        return MOE_ERR_NULL;
    for (const void* q : {h, d_out, (const void*)workspace, w->w_router, w->w_gate, w->w_up, w->w_down})
        if (!aligned(q, 16)) return MOE_ERR_ALIGN;
    if (d_h && !aligned(d_h, 16)) return MOE_ERR_ALIGN;
    for (const void* q : {(const void*)routing->topk_idx, (const void*)routing->topk_w,
                          (const void*)routing->expert_offsets, (const void*)routing->perm_src})
        if (!aligned(q, 4)) return MOE_ERR_ALIGN;
    moe_grads none{};
    const moe_grads& g = grads ? *grads : none;
    for (const void* q : {(const void*)g.d_w_router, (const void*)g.d_b_router, (const void*)g.d_w_gate,
                          (const void*)g.d_w_up, (const void*)g.d_w_down})
        if (q && !aligned(q, 4)) return MOE_ERR_ALIGN;
    const BwdLayout L = bwd_layout(p);
    if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    // Switched off: the first GPU run of the backward kernels ended in a
    // memory fault whose cause is not found yet; nothing is enqueued.
    if (kBackwardDisabled) return MOE_ERR_DISABLED;
    char* ws = reinterpret_cast<char*>(workspace);
    moe::BwdArgs a{};
    a.T = p->T; a.H = p->H; a.I = p->I; a.E = p->E; a.k = p->k;
    a.h = (const uint16_t*)h; a.dout = (const uint16_t*)d_out;
    a.w_router = (const uint16_t*)w->w_router; a.w_gate = (const uint16_t*)w->w_gate;
    a.w_up = (const uint16_t*)w->w_up; a.w_down = (const uint16_t*)w->w_down;
    a.topk_idx = routing->topk_idx; a.offsets = routing->expert_offsets; a.perm = routing->perm_src;
    a.topk_w = routing->topk_w;
    a.trainable = trainable;
    a.dh = (uint16_t*)d_h;
    a.dw_router = g.d_w_router; a.db_router = g.d_b_router;
    a.dw_gate = g.d_w_gate; a.dw_up = g.d_w_up; a.dw_down = g.d_w_down;
    a.inv = (int32_t*)(ws + L.inv); a.tiles = (int32_t*)(ws + L.tiles); a.ntiles = (int32_t*)(ws + L.ntiles);
    a.Xp = (uint16_t*)(ws + L.Xp); a.Dp = (uint16_t*)(ws + L.Dp); a.dY = (uint16_t*)(ws + L.dY);
    a.dG = (uint16_t*)(ws + L.dG); a.dU = (uint16_t*)(ws + L.dU); a.ACT = (uint16_t*)(ws + L.ACT);
    a.dsd = (uint16_t*)(ws + L.dsd);
    a.G = (float*)(ws + L.G); a.U = (float*)(ws + L.U); a.GY = (float*)(ws + L.GY); a.DA = (float*)(ws + L.DA);
    a.dp = (float*)(ws + L.dp); a.dsf = (float*)(ws + L.dsf);
    const hipError_t e = moe::launch_backward(a, reinterpret_cast<hipStream_t>(stream_v));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_attn_workspace_bytes(const moe_attn_problem* p) {
    if (!p || !moe::attn_sink_shape_ok(p->B, p->Hq, p->Hkv, p->Tk, p->D, p->window)) return 0;
    return moe::attn_workspace_bytes(p->B, p->Hq, p->Hkv, p->Tk, p->D, p->window);
}

int moe_attn_sink_decode(const moe_attn_problem* p, const void* q, const void* k_cache, const void* v_cache,
                         const void* sinks, const int32_t* lens, void* out, void* workspace, size_t workspace_bytes,
                         void* stream_v) {
    if (!p) return MOE_ERR_NULL;
    if (!moe::attn_sink_shape_ok(p->B, p->Hq, p->Hkv, p->Tk, p->D, p->window)) return MOE_ERR_SHAPE;
    if (!(p->scale == p->scale) || p->scale > 3.0e38f || p->scale < -3.0e38f) return MOE_ERR_SHAPE;
    if (p->B == 0) return MOE_OK;
    if (!q || !k_cache || !v_cache || !sinks || !out || !workspace) return MOE_ERR_NULL;
    for (const void* t : {q, k_cache, v_cache, (const void*)out, (const void*)workspace})
        if (!aligned(t, 16)) return MOE_ERR_ALIGN;
    if (!aligned(sinks, 2) || (lens && !aligned(lens, 4))) return MOE_ERR_ALIGN;
    if (workspace_bytes < moe::attn_workspace_bytes(p->B, p->Hq, p->Hkv, p->Tk, p->D, p->window))
        return MOE_ERR_WORKSPACE;
    const hipError_t e = moe::launch_attn_sink_decode(q, k_cache, v_cache, sinks, lens, out, workspace, p->B, p->Hq,
                                                      p->Hkv, p->Tk, p->D, p->window, p->scale,
                                                      reinterpret_cast<hipStream_t>(stream_v));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_expand_copies(const moe_problem* base, const moe_weights* src, const int32_t* copy_of, int32_t E_new,
                      const moe_weights* dst, void* stream_v) {
    if (!base || !src || !dst || !copy_of) return MOE_ERR_NULL;
    moe_problem q = *base;
    q.T = 0;
    int st = check_problem(&q);
    if (st != MOE_OK) return st;
    if (E_new < 1 || E_new > 1024) return MOE_ERR_SHAPE;
    for (int j = 0; j < E_new; ++j)
        if (copy_of[j] < 0 || copy_of[j] >= base->E) return MOE_ERR_SHAPE;
    const bool mx = base->expert_dtype == MOE_MXFP4;
    const size_t H = base->H, I = base->I;
    const size_t ab = act_bytes(base->act_dtype);
    const size_t eb = base->expert_dtype == MOE_F32 ? 4 : 2;

    struct T_ {
        const void* s;
        void* d;
        size_t row_bytes;
        bool required;
    };
    std::vector<T_> list = {
        {src->w_router, (void*)dst->w_router, H * ab, true},
        {src->b_router, (void*)dst->b_router, ab, false},
        {src->w_gate, (void*)dst->w_gate, mx ? I * H / 2 : I * H * eb, true},
        {src->w_up, (void*)dst->w_up, mx ? I * H / 2 : I * H * eb, true},
        {src->w_down, (void*)dst->w_down, mx ? H * I / 2 : H * I * eb, true},
    };
    if (mx) {
        list.push_back({src->s_gate, (void*)dst->s_gate, I * H / 32, true});
        list.push_back({src->s_up, (void*)dst->s_up, I * H / 32, true});
        list.push_back({src->s_down, (void*)dst->s_down, H * I / 32, true});
    }
    for (const T_& t : list) {
        if (t.required && (!t.s || !t.d)) return MOE_ERR_NULL;
        if (!t.required && ((t.s == nullptr) != (t.d == nullptr))) return MOE_ERR_NULL;
    }
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    for (const T_& t : list) {
        if (!t.s) continue;
        // runs j0 .. j0+n-1 that copy consecutive originals: one device copy each
        for (int j0 = 0; j0 < E_new;) {
            int n = 1;
            while (j0 + n < E_new && copy_of[j0 + n] == copy_of[j0] + n) ++n;
            if (hipMemcpyAsync(static_cast<char*>(t.d) + (size_t)j0 * t.row_bytes,
                               static_cast<const char*>(t.s) + (size_t)copy_of[j0] * t.row_bytes,
                               (size_t)n * t.row_bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
                return MOE_ERR_HIP;
            j0 += n;
        }
    }
    return MOE_OK;
}

int moe_expand_silent(const moe_problem* base, const moe_weights* src, int32_t M, const moe_weights* dst,
                      void* stream_v) {
    if (!base || !src || !dst) return MOE_ERR_NULL;
    if (M < 1 || base->E < 1 || (int64_t)M * base->E > 1024) return MOE_ERR_SHAPE;
    std::vector<int32_t> copy_of((size_t)M * base->E);
    for (size_t j = 0; j < copy_of.size(); ++j) copy_of[j] = (int32_t)(j % (size_t)base->E);
    return moe_expand_copies(base, src, copy_of.data(), (int32_t)copy_of.size(), dst, stream_v);
}

int moe_profile_begin(int32_t max_calls) { return moe_profile_begin_mask(max_calls, MOE_PROFILE_ALL); }

int moe_profile_begin_mask(int32_t max_calls, uint32_t boundary_mask) {
    if (max_calls < 1 || (boundary_mask & ~(uint32_t)MOE_PROFILE_ALL) != 0 || boundary_mask == 0) return MOE_ERR_SHAPE;
    Profiler& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    if (P.armed) return MOE_ERR_STATE;
    P.ev.assign((size_t)max_calls * (MOE_NUM_STAGES + 1), nullptr);
    for (auto& e : P.ev)
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto& x : P.ev)
                if (x) (void)hipEventDestroy(x);
            P.ev.clear();
            return MOE_ERR_HIP;
        }
    P.max_calls = max_calls;
    P.used = 0;
    P.mask = boundary_mask;
    P.armed = true;
    return MOE_OK;
}

int moe_profile_end(float stage_ms[MOE_NUM_STAGES], int32_t* calls_recorded) {
    Profiler& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    if (!P.armed) return MOE_ERR_STATE;
    int rc = MOE_OK;
    float sums[MOE_NUM_STAGES] = {0};
    int last = MOE_NUM_STAGES;  // the last boundary recorded
    while (last > 0 && !((P.mask >> last) & 1u)) --last;
    for (int c = 0; c < P.used; ++c) {
        hipEvent_t* row = &P.ev[(size_t)c * (MOE_NUM_STAGES + 1)];
        if (hipEventSynchronize(row[last]) != hipSuccess) rc = MOE_ERR_HIP;
        for (int s = 0; s < MOE_NUM_STAGES; ++s) {
            if (!((P.mask >> s) & 1u) || !((P.mask >> (s + 1)) & 1u)) continue;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, row[s], row[s + 1]) != hipSuccess) rc = MOE_ERR_HIP;
            sums[s] += ms;
        }
    }
    if (stage_ms)
        for (int s = 0; s < MOE_NUM_STAGES; ++s) stage_ms[s] = sums[s];
    if (calls_recorded) *calls_recorded = P.used;
    for (auto& e : P.ev) (void)hipEventDestroy(e);
    P.ev.clear();
    P.armed = false;
    P.used = 0;
    P.max_calls = 0;
    P.mask = 0;
    return rc;
}

}  // extern "C"
