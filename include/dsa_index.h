/*
 * dsa_index.h -- C ABI of the sparse-attention indexer's top-K key selection on MI355X (gfx950).
 *
 * The GLM-5.2 page ("github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！") has the engine run the model's
 * lightning indexer and keep, per layer, the top 2048 causal keys for the attention (section 三.3): a light
 * indexer scores the history's keys first, then the top-k entries go to the real attention (section 四.4, on
 * DeepSeek Sparse Attention).  The pages give no formula.  Read here with the DSA indexer's published form and
 * integer operands, so that the selection is reproducible bit for bit:
 *
 *   I[t][s] = kscale[s] * sum_{h=0}^{H-1} w[t][h] * max(0, sum_i q[t][h][i] * k[s][i])
 *
 * with the dot products exact (int8 operands, integer sum), the head sum a chain of fused multiply-adds in
 * head order from 0 and then one product by kscale[s], all in fp64.  Query t sits at position pos0 + t and sees
 * the keys s <= pos0 + t (s < S).  top[t] lists the K visible keys of largest score (equal scores by lower
 * position) by ascending position, padded with -1 when fewer than K keys are visible.
 *
 * Conventions are those of moe.h: device pointers owned by the caller, work enqueued on `stream` (a
 * hipStream_t) without waiting, MOE_OK or a negative MOE_E* code (moe_last_error() gives the message), every
 * argument checked before anything is enqueued, pointers 16-byte aligned and the workspace 256-byte aligned.
 */
#ifndef DSA_INDEX_H
#define DSA_INDEX_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_index_shape {
    int32_t T;    /* queries (>= 0) */
    int32_t S;    /* cached keys (>= 0) */
    int32_t H;    /* indexer heads: 16, 32, 48 or 64 */
    int32_t D;    /* head dimension: 64, 128, 192 or 256 */
    int32_t K;    /* keys kept per query (>= 1; 2048 for GLM-5.2) */
    int32_t pos0; /* position of query 0 (>= 0): query t sees keys s <= pos0 + t */
} dsa_index_shape;

/* Workspace bytes for this shape (T * S fp64 scores, then two fp64 per query and block of 64 keys: the score
 * range of each scoring workgroup); 0 for a shape that fails the checks. */
MOE_API size_t dsa_index_workspace_size(const dsa_index_shape *shape);

/*
 * q      [T][H][D] int8      the indexer queries
 * w      [T][H]    fp32      the head weights of each query (any sign)
 * k      [S][D]    int8      the cached indexer keys
 * kscale [S]       fp32      per-key scale, >= 0 (the selection assumes it does not reverse the order of a
 *                            key's scores across heads; a negative scale is not checked and gives the scores
 *                            of the formula all the same)
 * top    [T][K]    int32     output: positions, ascending, -1 past the visible count
 * gap    [T]       fp64      output (optional, NULL = none): score of the K-th kept key minus that of the
 *                            (K+1)-th in the order above (+inf when every visible key is kept); a gap below a
 *                            tolerance marks a near tie
 * Limits: S * D and T * H * D below 2^31 bytes.
 */
MOE_API int dsa_index_topk(const dsa_index_shape *shape, const int8_t *q, const float *w, const int8_t *k,
                           const float *kscale, int32_t *top, double *gap, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEX_H */
