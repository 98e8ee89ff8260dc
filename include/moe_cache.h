/*
 * moe_cache.h -- C ABI of the expert residency tier on MI355X (gfx950): a per-layer cache of expert slots in
 * HBM over a host tier that holds every expert of the layer, for models whose experts do not all fit in HBM.
 *
 * What the pages describe (cited by title):
 *   - the expert cache's unit is a slot holding one expert's complete weights; the default number of slots is
 *     four times the experts a token activates; eviction is a weighted LRU: each slot keeps a last-use time and
 *     a hit count, and slots with few hits and an old last use go first (pwwt.cn Colibri write-up, section 3.1);
 *   - one LRU expert cache per layer, with the next experts read ahead while the current ones compute ("github
 *     一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！" page, section 三.5);
 *   - batch union: the positions of a batch that hit one expert share one read of it (same page, 三.4);
 *   - hot experts can be pinned in the faster tier (same page, 五).
 *
 * Readings where the pages are silent:
 *   - one step is one layer call; its requests are the layer's batch union U (moe_permute's uniq list);
 *   - a resident expert of U is a hit: its slot's hit count + 1, last use = the step number (steps count
 *     from 1, per layer);
 *   - the missing experts of U, in ascending id, take the evictable slots in the order: empty slots (lower slot
 *     first), then fewest hits, then oldest last use, then lower expert id (MOE_CACHE_LRU: the same without the
 *     hits); a slot that holds an expert of U, and a pinned slot, is not evictable;
 *   - a loaded slot starts with hit count 1 and last use = the step: counts are per residence;
 *   - pinned experts fill slots 0 .. pinned-1 and never leave;
 *   - the read-ahead is the copy of a step's missing experts on a second stream while the step's resident
 *     experts (and the shared expert) compute; the predicted next-layer read-ahead is not provided.
 *
 * A step, per layer (streams: C compute, X copy; events order them):
 *   C: moe_route, moe_permute, moe_cache_plan      -> hit list, miss list; record event P
 *   X: wait P; moe_cache_fetch(miss list)          -> the missed experts land in their slots; record event F
 *   C: moe_forward_cached(hit list, with y_shared) -> resident experts and the shared expert
 *   C: wait F; moe_forward_cached(miss list, y_shared = NULL)
 *   C: moe_combine
 * Nothing goes to the host: the lists and their counts stay in device memory and every kernel reads them
 * there.  A step's plan must not start before the previous step's fetch and forwards of the same layer are
 * done (the stream order above gives that).
 *
 * Conventions are those of moe.h (device pointers owned by the caller unless stated, work enqueued on
 * `stream` without waiting, MOE_OK or a negative MOE_E* code, arguments checked before anything is enqueued,
 * 16-byte aligned pointers).  The library allocates nothing: the caller allocates the state
 * (moe_cache_state_size bytes, device memory), the slots (a moe_qffn of `slots` experts in device memory) and
 * the host tier (a moe_qffn of E experts in pinned host memory from hipHostMalloc, or in device memory).
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_CACHE_WEIGHTED_LRU 0
#define MOE_CACHE_LRU 1

typedef struct {
    int32_t E;       /* routed experts of the layer (as in moe_shape) */
    int32_t slots;   /* HBM slots, 1 <= slots <= E */
    int32_t pinned;  /* pinned experts, held in slots 0 .. pinned-1 (0 <= pinned < slots) */
    int32_t policy;  /* MOE_CACHE_WEIGHTED_LRU or MOE_CACHE_LRU */
} moe_cache_shape;

/* Bytes of a layer's cache state (device memory, any contents before moe_cache_init); 0 for a bad shape. */
MOE_API size_t moe_cache_state_size(const moe_cache_shape *cache);

/*
 * Empties the cache and places the pinned experts: pinned_ids (HOST array of cache->pinned distinct ids in
 * [0, E)) go to slots 0 .. pinned-1.  Writes them as the miss list (miss [E], -1 past n_miss; n_miss [1] =
 * pinned) so that one moe_cache_fetch loads them.  Returns once pinned_ids has been read (it waits for
 * `stream`).
 */
MOE_API int moe_cache_init(const moe_cache_shape *cache, const int32_t *pinned_ids, void *state, int32_t *miss,
                           int32_t *n_miss, void *stream);

/*
 * One step of the cache for the experts uniq[0 .. n_uniq) (moe_permute's outputs for this layer call; with
 * n_uniq = -1 the non-negative prefix of uniq).  Writes the hits and the misses, each in ascending expert id
 * with -1 past its count (hit, miss: [E]; n_hit, n_miss: [1]), and updates the state: the misses now own their
 * slots (their weights arrive with moe_cache_fetch).  T and k are the layer call's tokens and experts per token:
 * the call is refused (MOE_EINVAL) unless slots - pinned >= min(E, T*k), so that every step's misses find a
 * slot.  Misses that still find none (n_uniq above T*k) are left out of both lists and counted in the state's
 * unplaced count.
 */
MOE_API int moe_cache_plan(const moe_cache_shape *cache, int32_t T, int32_t k, const int32_t *uniq,
                           const int32_t *n_uniq, void *state, int32_t *hit, int32_t *n_hit, int32_t *miss,
                           int32_t *n_miss, void *stream);

/*
 * Copies the weights of the experts miss[0 .. n_miss) (entries outside [0, E) skipped) from the host tier
 * (moe_qffn of E experts: HOST pointers into pinned memory from hipHostMalloc, or device pointers) to their
 * slots in `slots` (moe_qffn of cache->slots experts, device memory), all nine matrices and per-row vectors of
 * each.  layer gives d, I and wbits (the sizes of one expert's tensors).  The copy is a kernel on `stream` that
 * reads host memory over the host link: no host synchronisation, and the list stays on the device.  A host-tier
 * pointer that the runtime does not know as pinned host or device memory is refused (MOE_EINVAL).
 */
MOE_API int moe_cache_fetch(const moe_shape *layer, const moe_cache_shape *cache, const moe_qffn *host_tier,
                            const moe_qffn *slots, const void *state, const int32_t *miss, const int32_t *n_miss,
                            void *stream);

/*
 * moe_forward with the routed weights read from the cache's slots: expert e's weights are slot
 * slot_of(e) of `slots` (cache->slots experts).  list / n_list take the place of uniq / n_uniq (a hit or miss
 * list of moe_cache_plan, -1 past the count; it must hold at least min(E, T*k) entries).  An expert of the list
 * that is not resident is skipped (its y_perm rows are left unwritten).  y_shared = NULL leaves the shared
 * expert out of this call (its weights are still required when I_shared > 0); the launch configuration is the
 * layer shape's either way, so that each row's result has the same bits as moe_forward's.  Workspace as
 * moe_forward.
 */
MOE_API int moe_forward_cached(const moe_shape *layer, const moe_cache_shape *cache, const void *x,
                               const moe_qffn *slots, const void *state, const moe_qffn *shared,
                               const int32_t *offsets, const int32_t *perm, const int32_t *list,
                               const int32_t *n_list, float *y_perm, float *y_shared, uint32_t *diag, void *ws,
                               size_t ws_bytes, void *stream);

/*
 * Reads the state back (waits for `stream`): out[0] steps, out[1] hits, out[2] misses (experts copied, the
 * initial pinned ones excluded), out[3] evictions of a resident expert, out[4] misses left without a slot;
 * slot_expert (HOST, [slots] or NULL) receives each slot's expert (-1 empty).
 */
MOE_API int moe_cache_stats(const moe_cache_shape *cache, const void *state, int64_t out[5], int32_t *slot_expert,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CACHE_H */
