/*
 * moe.h — C interface of the MI355X (gfx950) sparse mixture-of-experts
 * feed-forward layer, forward pass.
 *
 * The layer (from the "gpt-oss-40b-64a8-init" LLM-surgery page, section 2
 * "Mathematical Foundation: Silent Init", Proof; and the "gpt-oss 20B" field
 * guide, cutaway 03 "Sparse Mixture of Experts"), for every token t with
 * input row h_t:
 *
 *   s_i   = W_r[i] . h_t + b_r[i]                       router logits, all E experts
 *   S_t   = the k largest s_i                            ties: lower expert index wins
 *   p_i   = exp(s_i) / sum_{j in S_t} exp(s_j)           softmax over the selected set only
 *   E_i(x)= W_down[i] (silu(W_gate[i] x) * (W_up[i] x))  SwiGLU expert, silu(z) = z/(1+e^-z)
 *   out_t = sum_{i in S_t} p_i E_i(h_t)
 *
 * and the "silent init" expansion of the same page (section 2, Principle and
 * Proof; section 5.2 for the index convention): every expert and router row is
 * repeated M times (E' = M E) and k' = M k, which leaves out_t unchanged.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP device memory of the current
 *    device), contiguous, row-major, at least 16-byte aligned.  The caller owns
 *    every buffer; the library never allocates or frees device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it and the call returns after enqueue; results are
 *    visible after the caller synchronises the stream.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Argument errors are
 *    detected before anything is enqueued and leave every output untouched.
 *    No C++ exception crosses this interface.
 *  - Calls are independent: concurrent calls are safe when their workspaces
 *    and outputs do not overlap.
 */
#ifndef SMOE_MOE_H
#define SMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.
 *  MOE_F32   IEEE binary32.
 *  MOE_BF16  bfloat16 (the high 16 bits of a binary32).
 *  MOE_MXFP4 OCP Microscaling FP4 (expert weights only): E2M1 elements packed
 *            two per byte — element 2j in the LOW nibble of byte j, element
 *            2j+1 in the high nibble — and one E8M0 scale byte (value
 *            2^(x-127)) per group of 32 consecutive elements along the input
 *            dimension.  Decoded value = E2M1(code) * 2^(scale-127).  This is
 *            the format the "gpt-oss-20b and gpt-oss-120b" explainer describes
 *            ("Four-bit expert weights": groups share a scale, 4.25 bits per
 *            parameter, decoded exactly). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype;

enum {
    MOE_OK            = 0,
    MOE_ERR_NULL      = -1, /* a required pointer is NULL                        */
    MOE_ERR_SHAPE     = -2, /* sizes outside the supported range (see below)    */
    MOE_ERR_DTYPE     = -3, /* unsupported (act_dtype, expert_dtype) pair        */
    MOE_ERR_WORKSPACE = -4, /* workspace smaller than moe_workspace_bytes()      */
    MOE_ERR_ALIGN     = -5, /* a pointer is not 16-byte aligned                  */
    MOE_ERR_HIP       = -6, /* the HIP runtime reported an error at enqueue      */
    MOE_ERR_STATE     = -7, /* profiling calls out of order                      */
    MOE_ERR_DISABLED  = -8, /* entry point switched off in this build (see it)   */
    MOE_ERR_SCRATCH   = -9  /* problem larger than moe_forward_noalloc's scratch */
};

/* Problem sizes; field names follow the model configs on the pages
 * ("openai/gpt-oss-20b" fixture comparison page, Config changes table;
 * "gpt-oss-220a20b" page, Model Details):
 *   T  tokens (rows of h)             H  hidden_size
 *   I  intermediate_size              E  num_local_experts
 *   k  num_experts_per_tok
 * Supported: T >= 0 (T = 0 is a no-op), 1 <= k <= E <= 1024, H and I positive
 * multiples of 64, T*k*max(H,I) < 2^31, H*I < 2^29; with MXFP4 experts also
 * H, I <= 4992 (a GEMM tile keeps its scales for the whole contraction on chip).
 * Supported dtype pairs (act_dtype, expert_dtype): (F32, F32), (BF16, BF16),
 * (BF16, MXFP4).  act_dtype is the format of h, out, w_router and b_router. */
typedef struct {
    int32_t T, H, I, E, k;
    int32_t act_dtype;    /* moe_dtype */
    int32_t expert_dtype; /* moe_dtype */
} moe_problem;

/* Layer parameters (device pointers).  Every matrix is [out, in] row-major,
 * one per expert, experts stacked along the leading dimension:
 *   w_router [E, H]   act_dtype          b_router [E] act_dtype (NULL = zeros)
 *   w_gate   [E, I, H]                   w_up     [E, I, H]
 *   w_down   [E, H, I]
 * For MXFP4 the three expert tensors are uint8 [E, out, in/2] and the scales
 * are uint8 s_gate, s_up [E, I, H/32] and s_down [E, H, I/32]; the scale
 * pointers are ignored for other formats. */
typedef struct {
    const void *w_router;
    const void *b_router;
    const void *w_gate;
    const void *w_up;
    const void *w_down;
    const uint8_t *s_gate;
    const uint8_t *s_up;
    const uint8_t *s_down;
} moe_weights;

/* Optional routing outputs (device pointers, each may be NULL).
 *   logits         float [T, E]  s_t,i in fp32
 *   topk_idx       int32 [T, k]  S_t in ascending expert id
 *   topk_w         float [T, k]  p_i in the same order (fp32)
 *   expert_offsets int32 [E+1]   exclusive prefix sum of per-expert counts;
 *                                expert_offsets[E] = T*k
 *   perm_src       int32 [T*k]   row r of the expert-major order -> assignment
 *                                t*k+slot; rows of one expert are ordered by t
 */
typedef struct {
    float   *logits;
    int32_t *topk_idx;
    float   *topk_w;
    int32_t *expert_offsets;
    int32_t *perm_src;
} moe_routing;

/* Bytes of device workspace moe_forward needs for problem *p (0 if *p is
 * invalid).  The workspace holds the routing tables, the expert-major
 * intermediate activations [T*k, I] and the weighted expert outputs [T*k, H]
 * in fp32. */
size_t moe_workspace_bytes(const moe_problem *p);

/* Forward pass of the layer: out[T, H] (act_dtype) from h[T, H] (act_dtype).
 * Arithmetic: router logits, softmax and all accumulation in fp32; the
 * intermediate silu(gate)*up activation is stored in act_dtype (rounded to
 * nearest-even for bf16); the k weighted expert outputs of a token are summed
 * in fp32 in ascending expert-id order and rounded once to act_dtype.
 * Deterministic: identical inputs give bitwise-identical outputs.
 * `routing` may be NULL.  `workspace` must hold moe_workspace_bytes(p) bytes
 * (16-byte aligned) and must not be used by anything else until the stream
 * has passed this call.
 * Every kernel runs on `stream`.
 * Errors: MOE_ERR_NULL (p, w, w_router, w_gate, w_up, w_down, h, out or
 * workspace NULL while T > 0; MXFP4 scales NULL), MOE_ERR_SHAPE, MOE_ERR_DTYPE,
 * MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP. */
int moe_forward(const moe_problem *p, const moe_weights *w, const void *h, void *out,
                const moe_routing *routing, void *workspace, size_t workspace_bytes,
                void *stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, arithmetic, results and errors as moe_forward, without the
 * workspace: its regions live in one static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library runs
 * on holds from its first call until the process ends.  A problem whose
 * moe_workspace_bytes() exceeds that (e.g. T = 4096 prefill of the
 * gpt-oss-20b layer) gets MOE_ERR_SCRATCH and nothing is enqueued; decode
 * batches and short prefill chunks fit (the gpt-oss-20b layer up to T of
 * about 900).  The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.  Every call on one GPU shares that GPU's array,
 * and the array keeps the previous call's contents (the kernels clear what
 * must start at zero themselves), so calls that overlap on one GPU (two
 * streams, or two threads) race and must be serialised by the caller.
 * `stream` must belong to the current device (else MOE_ERR_HIP). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_problem *p, const moe_weights *w, const void *h, void *out,
                        const moe_routing *routing, void *stream);

/* The pre-normalised MoE sublayer of a decoder block with its residual add
 * ("gpt-oss 20B" field guide, cutaway 04 "One decoder block": RMSNorm before
 * the MoE sublayer, whose output is added back to the residual stream; the
 * "openai/gpt-oss-20b" fixture page's parameter table: one gain per hidden
 * feature, no bias):
 *     out = x + MoE(n),   n = norm_weight * x / sqrt(mean(x^2) + eps)
 * per token, mean over the H features.  x, out and norm_weight [H] are in
 * act_dtype; MoE is the layer of moe_forward with weights *w.
 * Arithmetic: the mean square and the scale in fp32.  Routing follows the
 * normalised input to fp32 precision, not a rounded copy: the logits are
 * scale * (x . (W_r * norm_weight)) + b_r with x taken exactly (bf16: the
 * folded router split exactly into two bf16 parts; fp32: the fp32 router on
 * the fp32 normalised input).  With bf16 activations the expert GEMMs take n
 * rounded once to bf16.  The residual is added in fp32 to the sum of the
 * expert outputs before the single rounding of out.
 * Deterministic.  `workspace` must hold moe_block_workspace_bytes(p) bytes;
 * out must not overlap x.  `routing` as in moe_forward (logits are those of
 * the normalised input).  Profiling stage 0 includes the normalisation.
 * Errors: as moe_forward (x in the place of h), plus MOE_ERR_NULL for
 * norm_weight, MOE_ERR_ALIGN for norm_weight not 16-byte aligned and
 * MOE_ERR_SHAPE for eps negative, NaN or infinite. */
size_t moe_block_workspace_bytes(const moe_problem *p);
int moe_block_forward(const moe_problem *p, const moe_weights *w, const void *norm_weight, float eps,
                      const void *x, void *out, const moe_routing *routing, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Decode attention with learned sinks ("gpt-oss-20b and gpt-oss-120b"
 * explainer, "Two attention savings, and a sink"; "gpt-oss 20B" field guide,
 * cutaway 05): the newest token of each of B sequences attends to its
 * key/value cache.  For query head h (key/value head g = h / (Hq/Hkv)):
 *     s_j = scale * q[b,h] . k[b,g,j]
 *     out[b,h] = sum_j exp(s_j) v[b,g,j] / (exp(sinks[h]) + sum_j exp(s_j))
 * over the visible keys j: 0 <= j < len_b, and with window > 0 only the last
 * `window` of them (len_b - window <= j, the newest key included).  The sink
 * joins the normalisation and contributes no value.
 * Layouts (bf16, row-major, 16-byte aligned): q [B, Hq, D], k_cache and
 * v_cache [B, Hkv, Tk, D], out [B, Hq, D]; sinks [Hq] bf16; lens [B] int32
 * device array (NULL: every sequence has Tk keys; values are clamped to
 * 0..Tk, and a sequence with no visible keys gives 0).  Scores, softmax and
 * sums in fp32, out rounded once.  Supported: Hq a multiple of Hkv with
 * Hq/Hkv <= 8, D a multiple of 8 up to 64, Tk >= 1, window >= 0, B >= 0
 * (B = 0 is a no-op).  The keys of a sequence are split over workgroups;
 * `workspace` (16-byte aligned, moe_attn_workspace_bytes(p) bytes, caller
 * owned, not to be touched until the stream has passed this call) holds the
 * partial results.  moe_attn_workspace_bytes returns 0 for invalid sizes.
 * Errors: MOE_ERR_NULL (p, q, k_cache, v_cache, sinks, out or workspace NULL
 * while B > 0), MOE_ERR_SHAPE (unsupported sizes, scale not finite),
 * MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP. */
typedef struct {
    int32_t B, Hq, Hkv, Tk, D, window;
    float scale;
} moe_attn_problem;
size_t moe_attn_workspace_bytes(const moe_attn_problem *p);
int moe_attn_sink_decode(const moe_attn_problem *p, const void *q, const void *k_cache, const void *v_cache,
                         const void *sinks, const int32_t *lens, void *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Gradients of the layer for fine-tuning ("gpt-oss-40b-64a8-init" page:
 * section 1, Train Wide, Deploy Narrow; section 5.2, selective gradient
 * control: original experts frozen while the copies train, the router
 * trainable throughout).  For an upstream gradient dout [T, H] of out, with
 * the routing of the moe_forward call that produced out held fixed (the
 * top-k selection passes no gradient; the selected softmax does):
 *   d_h [T, H]          input gradient, act dtype, rounded once (NULL: skip)
 *   grads->d_w_router   [E, H] fp32, grads->d_b_router [E] fp32
 *   grads->d_w_gate, d_w_up [E, I, H] fp32, grads->d_w_down [E, H, I] fp32
 * Every gradient pointer may be NULL (not computed).  Outputs are written,
 * not accumulated.  trainable [E] uint8 device array (NULL: all): experts
 * with 0 get no expert-matrix gradients (their slices are not written); the
 * router and d_h are the same either way.  routing must hold the four
 * arrays moe_forward returned for this h (topk_idx, topk_w, expert_offsets,
 * perm_src; logits unused).  Supported: act_dtype and expert_dtype MOE_BF16
 * (else MOE_ERR_DTYPE), the sizes moe_forward takes.  Products in bf16 on
 * the matrix cores with fp32 accumulation; g, u are recomputed, and
 * d(gate), d(up), act, p*dout are rounded to bf16 before the products that
 * take them.  workspace: moe_backward_workspace_bytes(p) bytes, 16-byte
 * aligned, not to be touched until the stream has passed the call.  T = 0
 * writes nothing.  Errors: MOE_ERR_NULL (p, w, h, dout, routing or one of its
 * four arrays, workspace, a weight NULL while T > 0), MOE_ERR_SHAPE,
 * MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN (16 bytes for tensors and
 * workspace, 4 for routing arrays and gradients), MOE_ERR_HIP.
 * SWITCHED OFF: the first GPU run of these kernels ended in a memory fault
 * whose cause has not been found (the kernels' index arithmetic checks out
 * against the buffers on the CPU).  Until it is, every call with T > 0 that
 * passes the argument checks returns MOE_ERR_DISABLED and enqueues nothing. */
typedef struct {
    float *d_w_router, *d_b_router, *d_w_gate, *d_w_up, *d_w_down;
} moe_grads;
size_t moe_backward_workspace_bytes(const moe_problem *p);
int moe_backward(const moe_problem *p, const moe_weights *w, const void *h, const void *d_out,
                 const moe_routing *routing, const uint8_t *trainable, void *d_h, const moe_grads *grads,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Silent expansion ("gpt-oss-40b-64a8-init" page, section 2 Principle/Proof,
 * section 5.2): for every per-expert tensor of *src (w_router, b_router,
 * w_gate, w_up, w_down and, for MXFP4, the three scale tensors) write
 * dst row j = src row (j mod E), j = 0 .. M*E-1, so the original experts keep
 * indices 0..E-1 and their copies follow.  `base` describes the unexpanded
 * layer (its T is ignored); the caller runs the expanded layer with
 * E' = M*E and k' = M*k.  Every dst tensor is caller-allocated with M*E rows
 * and must not overlap its source.  M >= 1 (M = 1 is a plain copy).
 * b_router may be NULL in both src and dst (then nothing is written for it).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (M < 1, M*E > 1024, invalid base),
 * MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_HIP. */
int moe_expand_silent(const moe_problem *base, const moe_weights *src, int32_t M,
                      const moe_weights *dst, void *stream);

/* Expansion by an explicit copy map, for expansions that do not repeat every
 * expert the same number of times (the "gpt-oss-220a20b" page, Model Details:
 * 248 expert rows made of 128 base rows and 120 added rows): for every
 * per-expert tensor of *src (as in moe_expand_silent) write dst row j =
 * src row copy_of[j], j = 0 .. E_new-1.  copy_of is a HOST array of E_new
 * int32 original expert ids in 0 .. base->E-1; each new row starts as an
 * exact copy of its original, router row and bias included, so copies of one
 * original get bitwise-equal logits and exact ties between them go to the
 * lower expanded id.  The caller runs the expanded layer with E' = E_new and
 * its chosen k'.  moe_expand_silent(M) is copy_of[j] = j mod E.  Runs of rows
 * that copy consecutive originals go out as one device copy each.
 * Errors: MOE_ERR_NULL (base, src, dst, copy_of, or a required tensor),
 * MOE_ERR_SHAPE (E_new outside 1..1024, an id outside 0..E-1, invalid base),
 * MOE_ERR_DTYPE, MOE_ERR_HIP. */
int moe_expand_copies(const moe_problem *base, const moe_weights *src, const int32_t *copy_of, int32_t E_new,
                      const moe_weights *dst, void *stream);

/* Decode MXFP4 weights to bf16 with the same device routine the forward pass
 * uses when it stages weight tiles.  `packed` holds n_groups runs of 16 bytes
 * (32 E2M1 codes, element 2j in the low nibble of byte j), `scales` one E8M0
 * byte per run, `out_bf16` receives n_groups*32 bf16 values.  A whole matrix
 * [N, K] in the layout of moe_weights is n_groups = N*K/32.  The decode is
 * exact (every E2M1 value times a power of two in range is a bf16 value;
 * results beyond the bf16 range become +-inf, scale 255 gives NaN).  Meant for
 * inspecting and checking stored weights.
 * Errors: MOE_ERR_SHAPE (n_groups < 0), MOE_ERR_NULL, MOE_ERR_ALIGN (packed or
 * out_bf16 not 16-byte aligned), MOE_ERR_HIP. */
int moe_mxfp4_decode(const uint8_t *packed, const uint8_t *scales, int64_t n_groups, void *out_bf16,
                     void *stream);

/* Static description of a status code. */
const char *moe_status_string(int status);

/* ---- measurement hooks -------------------------------------------------
 * Per-stage device timing with HIP events, for benchmarks and profiles.
 * moe_profile_begin(n) arms recording for the next n moe_forward calls made
 * from any thread (events are recorded on each call's own stream before and
 * after every stage); moe_profile_end() waits for those events and returns,
 * per stage, the summed elapsed milliseconds and the number of calls
 * recorded.  Stages: 0 router + top-k + softmax, 1 routing scan/permute,
 * 2 gate/up grouped GEMM with SiLU*up, 3 down grouped GEMM with weighting,
 * 4 combine.  Errors: MOE_ERR_STATE (begin while armed, end while not armed),
 * MOE_ERR_SHAPE (n < 1), MOE_ERR_HIP. */
#define MOE_NUM_STAGES 5
int moe_profile_begin(int32_t max_calls);
/* Same, recording only the stage boundaries in boundary_mask: bit i is the
 * event before stage i, bit MOE_NUM_STAGES the one after the last stage
 * (MOE_PROFILE_ALL = every boundary).  Each event costs a few microseconds
 * of device time, so a timed loop can record just the stages it reports.  A
 * stage whose two boundaries are not both recorded reads 0 in
 * moe_profile_end.  Errors as moe_profile_begin; MOE_ERR_SHAPE also for an
 * empty mask or bits beyond MOE_NUM_STAGES. */
#define MOE_PROFILE_ALL ((1u << (MOE_NUM_STAGES + 1)) - 1u)
int moe_profile_begin_mask(int32_t max_calls, uint32_t boundary_mask);
int moe_profile_end(float stage_ms[MOE_NUM_STAGES], int32_t *calls_recorded);
const char *moe_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_MOE_H */
