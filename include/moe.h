/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward.
 *
 * The layer (pages cited by title):
 *   1. moe_route   -- a DeepSeek-V3-style sigmoid router: every token keeps k
 *      of E experts ("25GB 内存跑 744B GLM-5.2 模型" page, section 三.1).  The
 *      per-expert bias steers selection only, DeepSeek-V3's balancing
 *      without an auxiliary loss, and routing, selection and scaling must be
 *      reproduced exactly (same page, section 四.3).
 *   2. moe_permute -- batch union: assignments that hit the same expert are
 *      grouped so the expert's weights are read once for all of them (same
 *      page, section 三.4; gathering the active experts into one batched
 *      product: "企业官网建设流程全解析" page, Colibri walk-through, section 3.3).
 *   3. moe_forward -- the routed SwiGLU experts and the always-on shared
 *      expert, weights quantised per output channel with a scale and a zero
 *      point (walk-through page, section 3.4); the shared expert belongs to
 *      the dense, resident part of the model (GLM-5.2 page, section 二).
 *   4. moe_combine -- y = shared + sum_j w_j * expert_j(x).
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller; only the
 *     moe_shape / moe_qffn structs are read on the host, during the call.
 *     The library allocates no memory and keeps no global mutable state,
 *     except moe_forward_static's static scratch array (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting for it.  Results are valid once
 *     the stream has reached that point.  Counts, offsets and the unique-
 *     expert list stay on the device; no call copies them to the host.
 *   - `ws` is a caller-owned device workspace of at least
 *     moe_workspace_size(shape) bytes, 256-byte aligned.  Calls that share a
 *     workspace must be ordered (same stream); concurrent calls need their
 *     own workspaces.  Workspace contents need no initialisation.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code.  All arguments
 *     are validated before anything is enqueued, so a failed call leaves
 *     every output untouched.  moe_last_error() gives a message for the
 *     calling thread's last failure.
 *   - Pointer arguments must be 16-byte aligned (MOE_EALIGN otherwise).
 *   - T = 0 (an empty batch) is valid.  The calls check the rest of their
 *     arguments and return MOE_OK; pointers to T-sized arrays may then be
 *     NULL.  moe_permute still writes its E-sized outputs (zero counts and
 *     offsets, uniq all -1, n_uniq 0); the other calls enqueue nothing.
 *
 * Shapes and layouts
 *   T tokens, d hidden size, E routed experts, k experts per token,
 *   I routed intermediate size, I_shared shared intermediate size (0 = none),
 *   A = T*k assignments (a = t*k + j is token t's j-th choice).
 *   x        [T][d] fp32 (MOE_ACT_F32) or bf16 (MOE_ACT_BF16), row-major.
 *   W_r      [d][E] fp32;  bias [E] fp32.
 *   Quantised matrices are row-major [out][in], one scale and zero point per
 *   output row; dequantised weight = scale * (q - zp):
 *     wbits 8: q int8, zp int8;
 *     wbits 4: q unsigned 0..15, two per byte, the even input index in the
 *              low nibble; zp fp32.
 *   moe_qffn for n experts: q_gate, q_up [n][I][in_bytes],
 *   q_down [n][d][I*wbits/8], s_* fp32 and z_* as above, [n][out].
 *   Limits: 1 <= k <= min(E, 32), E <= 1024, T*k < 2^31;
 *   d and I (and I_shared) multiples of 32 for int4 and of 16 for int8, and
 *   below MOE_MAX_DIM (the decode kernels sum up to a whole row of int8
 *   weight x 8-bit activation-digit products in int32: 2^17 x 2^14 < 2^31).
 *   Every buffer a kernel reads or writes through a 32-bit offset stays below
 *   2^31 bytes: x (T*d*4 or T*d*2), one expert matrix (I*d*wbits/8), the
 *   router's partial sums, and the forward path's intermediate h (decode
 *   path: T*k*I*4 and T*I_shared*4 bytes; matrix-core path: T*k*I*2).  A
 *   shape past these limits is rejected with MOE_EUNSUPPORTED before anything
 *   is enqueued, never computed with wrapped offsets.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* bad shape, NULL required pointer, unknown enum */
#define MOE_EUNSUPPORTED (-2) /* dtype or bit width not implemented */
#define MOE_EWORKSPACE (-3)   /* workspace missing or smaller than moe_workspace_size() */
#define MOE_EALIGN (-4)       /* pointer not 16-byte (workspace: 256-byte) aligned */
#define MOE_EDEVICE (-5)      /* kernel launch failed */

#define MOE_MAX_DIM 131072 /* d, I and I_shared must be below this */

#define MOE_ACT_F32 0
#define MOE_ACT_BF16 1

/* moe_forward expert-FFN implementation */
#define MOE_PATH_AUTO 0 /* choose from T, k and E */
#define MOE_PATH_GEMV 1 /* bandwidth-bound dequant-GEMV (decode) */
#define MOE_PATH_GEMM 2 /* MFMA grouped GEMM (prefill) */
/* MOE_PATH_AUTO runs the decode kernels up to this T and the matrix-core path above it where that path applies
 * (measured crossover: the decode kernels, taking each expert's tokens in passes of at most 16, are faster at
 * T = 40 on the mid and 256-expert layers; at T = 48 the mid layer's matrix-core path is 3 % faster). */
#define MOE_AUTO_DECODE_MAX_T 40

/*
 * Batch-shape-invariant mode.  Quantised integer kernels may round differently
 * for different batch shapes, so a token verified inside a batch (speculative
 * drafts, batched prefill) need not match the single-token path byte for
 * byte; strict reproducibility fixes the kernels and their paths ("25GB 内存跑
 * 744B GLM-5.2 模型" page, section 六).  With this flag every result for a token
 * (topk_idx, topk_w, gap, its y_perm rows, y_shared and y) is bit-identical
 * whatever the batch it sits in and its position there:
 *   - moe_route sums each token's logits in one order fixed by (d, E) alone;
 *   - moe_forward with MOE_PATH_AUTO runs the decode kernels at every T, with
 *     the K split of each pass fixed by (d, I, I_shared, E, k, wbits) alone
 *     (MOE_PATH_GEMM stays on the matrix-core path, whose rows are
 *     independent of each other too, and gives its own, different bits);
 *   - moe_combine is per token already.
 * Cost: the decode split is the one chosen for T = 1, so T <= 40 runs as fast
 * or a little slower; above T = 16 the decode kernels take each expert's tokens
 * in passes of at most 16 and stream its weights again per pass, so at large T
 * they are far slower than the matrix-core path.
 */
#define MOE_FLAG_BATCH_INVARIANT 1

/*
 * Router variants (moe_route).  The default is the sigmoid router above.  The
 * untitled Colibri deep-dive page (lshu.cn) gates 8 experts with a softmax over
 * the logits, taken against the largest logit, and keeps the top 2 (its section
 * 3.2), and gives a Mixtral-style gate a capacity factor of 1.2 (its section
 * 6.2); the walk-through page names expert choice and soft routing as router
 * logics that reuse the rest of the engine (its section 6).  As read here:
 *   MOE_ROUTER_SIGMOID_BIAS  sigmoid scores, bias for selection (see moe_route).
 *   MOE_ROUTER_SOFTMAX       the k largest logits z (softmax keeps their order),
 *       equal ones by lower id; topk_w[t][j] = lambda * exp(z_j - z_max) /
 *       sum over the selected of exp(z_j' - z_max), i.e. the softmax probability
 *       renormalised over the selected; gap in logit units; bias is not used
 *       (may be NULL).  Soft routing is this gate with k = E.
 *   MOE_ROUTER_EXPERT_CHOICE  p[t][e] = softmax over the experts of token t;
 *       every expert takes the C = min(T, ceil(capacity_factor * T / E)) tokens
 *       of largest p (equal p by lower token).  Requires k = E (one slot per
 *       expert): topk_idx[t][e] = e and topk_w[t][e] = lambda * p[t][e] when
 *       expert e took token t, else -1 and 0; gap (optional) then has E entries:
 *       p of expert e's C-th token minus p of its (C+1)-th (+inf when C = T).
 * capacity_factor (top-k routers; 0 = none): every expert keeps at most
 *   C = ceil(capacity_factor * T * k / E) of its assignments, all tokens' first
 *   choices before any second choice and tokens in order within a choice; the
 *   others become empty slots (id -1; their weights are kept, not
 *   renormalised).  Empty slots take no place in moe_permute and add nothing in
 *   moe_combine.
 */
#define MOE_ROUTER_SIGMOID_BIAS 0
#define MOE_ROUTER_SOFTMAX 1
#define MOE_ROUTER_EXPERT_CHOICE 2

typedef struct moe_shape {
    int32_t T, d, E, k, I, I_shared;
    float routed_scale;    /* lambda: the normalised combine weights are multiplied by it */
    int32_t act_dtype;     /* MOE_ACT_F32 | MOE_ACT_BF16 */
    int32_t wbits;         /* 8 | 4 */
    int32_t path;          /* MOE_PATH_* (moe_forward only) */
    int32_t flags;         /* 0 or MOE_FLAG_BATCH_INVARIANT */
    int32_t router;        /* MOE_ROUTER_* (moe_route only) */
    float capacity_factor; /* see MOE_ROUTER_*; 0 = no capacity limit for the top-k routers */
} moe_shape;

typedef struct moe_qffn {
    const void *q_gate, *q_up, *q_down;
    const float *s_gate, *s_up, *s_down;
    const void *z_gate, *z_up, *z_down;
} moe_qffn;

/*
 * Bytes of workspace that every call below needs for this shape (host only, no device work); 0 for a shape
 * that check fails.  The workspace is the per-request arena of the Colibri walk-through page
 * ("企业官网建设流程全解析", section 3.2): sized once from the shape, carved by the calls, never freed between
 * them, and owned by one request at a time (calls sharing it must be ordered on one stream).
 */
MOE_API size_t moe_workspace_size(const moe_shape *shape);

/*
 * Router ("25GB 内存跑 744B GLM-5.2 模型" page, sections 三.1 and 四.3).
 *   z[t][e]   = sum_i x[t][i] * W_r[i][e]            (fp64 accumulation)
 *   s[t][e]   = 1 / (1 + exp(-z[t][e]))              (fp64)
 *   sel[t][e] = s[t][e] + bias[e]                    (selection score, fp64)
 *   topk_idx[t][0..k): the k experts of largest sel, in descending sel,
 *                      equal scores ordered by lower expert id;
 *   topk_w[t][j] = routed_scale * s[t][idx_j] / sum_j' s[t][idx_j']  (fp32);
 *   gap[t]    = sel of the k-th choice minus sel of the (k+1)-th, fp64
 *               (+inf when k == E); optional (NULL).  Tokens with a gap
 *               below 1e-6 are the near ties a caller may want to log.
 * Outputs: topk_idx [T][k] int32, topk_w [T][k] fp32, gap [T] fp64 or NULL.
 */
MOE_API int moe_route(const moe_shape *shape, const void *x, const float *W_r, const float *bias, int32_t *topk_idx,
              float *topk_w, double *gap, void *ws, size_t ws_bytes, void *stream);

/*
 * Batch union (GLM-5.2 page, section 三.4): a stable counting sort of the A
 * assignments by expert.
 *   counts[e]      assignments routed to e                      [E]
 *   offsets[e]     exclusive prefix sum of counts               [E+1]
 *   perm[p]        assignment a = t*k + j at sorted position p  [A]
 *                  (ascending a within an expert)
 *   inv[a]         sorted position of assignment a              [A]
 *   uniq[0..n)     experts with counts > 0, ascending; -1 after [E]
 *   n_uniq[0]      number of unique experts                     [1]
 * Integer work, bit-exact and independent of scheduling.
 * Empty slots: entries equal to -1 (capacity drops, expert choice) are not
 * counted, get no place in perm and have inv = -1.
 * Invalid ids: other entries outside [0, E) are treated the same way and
 * also set n_uniq to -1 (an error flag for the caller).  counts/offsets/uniq then describe the valid assignments only;
 * moe_forward applies every expert listed in uniq (the non-negative prefix)
 * and moe_combine leaves out the dropped choices, so y[t] is the shared term
 * plus the token's valid choices.
 */
MOE_API int moe_permute(const moe_shape *shape, const int32_t *topk_idx, int32_t *counts, int32_t *offsets, int32_t *perm,
                int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route followed by moe_permute, with the same arguments, outputs and
 * checks as the two calls.  For a single token (T = 1, the top-k routers
 * without capacity) the permutation runs inside the selection's launch: the
 * workgroup that selects the token's experts then sorts the assignments, so
 * the permutation costs no launch of its own.  The outputs have the same bits as
 * the two calls'.
 */
MOE_API int moe_route_permute(const moe_shape *shape, const void *x, const float *W_r, const float *bias,
                              int32_t *topk_idx, float *topk_w, double *gap, int32_t *counts, int32_t *offsets,
                              int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * Routed and shared SwiGLU experts (walk-through page, section 3.4):
 *   g = s_g * ((q_g - z_g) . x),  u = s_u * ((q_u - z_u) . x),
 *   h = silu(g) * u,  out = s_d * ((q_d - z_d) . h),  silu(v) = v / (1 + exp(-v)).
 * Each unique expert e (uniq/n_uniq/offsets/perm from moe_permute) is applied
 * to the tokens t = perm[p] / k of its rows p in [offsets[e], offsets[e+1]),
 * reading its weights once for all of them; results go to y_perm[p] (fp32,
 * [A][d]).  The shared expert (shared != NULL, shape->I_shared > 0) is
 * applied to every token; its output goes to y_shared [T][d] fp32.
 * Accumulation is fp32; between the two products the matrix-core path
 * keeps h as fp16 plus its residual in fp6 (e2m3) under one power-of-two
 * scale per row and 32 channels.  The matrix-core path takes x as fp16
 * under one power-of-two scale per token (its largest magnitude put into
 * [2^14, 2^15)), exact for every bf16 value above 2^-29 of the row's
 * largest, so no range of activations overflows fp16; fp32 activations as
 * two fp16 values hi + lo (about 22 significant bits), every weight step
 * multiplied with both.  The decode path
 * takes each token's K part as 24-bit fixed point under one power-of-two
 * scale.  `routed` describes E experts, `shared` one.
 *
 * diag (optional, NULL = none; 4-byte alignment suffices): MOE_DIAG_COUNT
 * uint32 device counters that the call adds to (the caller zeroes them;
 * they never fail the call):
 *   diag[MOE_DIAG_H_FP16_NONFINITE]  values of h, over every row and channel
 *       of this call, that are not finite in the fp16 plane of the
 *       matrix-core path; such values make the outputs they enter
 *       non-finite.  That path stores h of each row under a power-of-two
 *       scale taken from a bound on |h| (x's L1 norm times the expert's
 *       largest |scale| x |q - zp| for gate and for up), so finite inputs
 *       whose h is finite in fp32 never count here.  The decode path keeps h
 *       in fp32 and adds nothing.
 * Near ties of the selection are reported by moe_route's gap output.
 */
#define MOE_DIAG_H_FP16_NONFINITE 0
#define MOE_DIAG_COUNT 1

MOE_API int moe_forward(const moe_shape *shape, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                float *y_perm, float *y_shared, uint32_t *diag, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward for callers that cannot allocate memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same
 * computation, arguments and results, with no workspace argument.  Its
 * scratch memory is a static device array of MOE_STATIC_SCRATCH_BYTES that
 * the library holds on every device it runs on until the process ends (the
 * array's address on a device is looked up on the first call there).
 *   - A shape whose forward needs more scratch than that (moe_forward's part
 *     of moe_workspace_size: the decode path's h, or the matrix-core path's
 *     fp16 x and h planes) fails with MOE_EWORKSPACE before anything is
 *     enqueued.  Decode batches and prefill chunks of a few hundred tokens
 *     fit; the 256-expert top-8 layer at T = 8192 does not.
 *   - No call allocates or frees memory; nothing in the scratch needs to
 *     start at zero (the kernels clear what they count with).
 *   - Every call on one GPU shares that GPU's array and leaves the last call's
 *     contents in it: calls that overlap on one GPU (different streams, or
 *     different host threads) race and give wrong results.  Order them.
 */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)

MOE_API int moe_forward_static(const moe_shape *shape, const void *x, const moe_qffn *routed,
                               const moe_qffn *shared, const int32_t *offsets, const int32_t *perm,
                               const int32_t *uniq, const int32_t *n_uniq, float *y_perm, float *y_shared,
                               uint32_t *diag, void *stream);

/*
 * Weighted combine.  The layer output adds, to the always-on shared expert
 * (dense part of the model: GLM-5.2 page, section 二), each routed expert's
 * output scaled by its router weight (GLM-5.2 page, section 四.3: the
 * routing's scaling semantics, lambda times the normalised selected scores):
 *   y[t] = y_shared[t] + sum_{j=0}^{k-1} topk_w[t][j] * y_perm[inv[t*k + j]]
 * summed in this order in fp32 (y_shared NULL = no shared term; choices with
 * inv = -1, dropped by moe_permute for an invalid id, are left out).
 * Output y [T][d] fp32.
 */
MOE_API int moe_combine(const moe_shape *shape, const float *y_perm, const float *y_shared, const int32_t *inv,
                const float *topk_w, float *y, void *stream);

/*
 * The whole layer in one call: moe_route_permute, moe_forward and
 * moe_combine on the same arguments, with the same checks, writing the same
 * outputs with the same bits (every intermediate output included).  For a
 * single token on the decode path with a top-k router and no capacity, the
 * selection and the sort of the chosen experts (GLM-5.2 page, sections 三.1
 * and 三.4) run inside the forward's first launch: every workgroup of that
 * launch selects the token's experts from the router's partial sums for
 * itself, so neither needs a launch of its own.  Otherwise the call runs the
 * three calls' kernels in turn.  ws: moe_workspace_size(shape) bytes.
 */
MOE_API int moe_layer(const moe_shape *shape, const void *x, const float *W_r, const float *bias,
                      const moe_qffn *routed, const moe_qffn *shared, int32_t *topk_idx, float *topk_w,
                      double *gap, int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *uniq,
                      int32_t *n_uniq, float *y_perm, float *y_shared, float *y, uint32_t *diag, void *ws,
                      size_t ws_bytes, void *stream);

/* Message describing the calling thread's last failed call ("" if none). */
MOE_API const char *moe_last_error(void);

/* ABI version: increases when an entry point is added or removed, or a signature or a layout changes
 * (4: moe_layer). */
MOE_API int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
