// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Weights of n quantised SwiGLU experts, stacked per matrix (see include/moe.h).
struct QW {
    const uint8_t *qg, *qu, *qd;
    const float *sg, *su, *sd;
    const void *zg, *zu, *zd;
};

// Everything the expert-FFN kernels read or write.
struct FfnParams {
    const void *x;
    int T, d, k, E, A;
    int I, Is;  // routed and shared intermediate sizes (Is = 0: no shared expert)
    int wbits, act;
    QW routed, shared;
    const int32_t *offsets, *perm, *uniq, *n_uniq;
    // routed weight row of expert e: wslot[e] (an expert cache's slot map) or e itself (wslot = nullptr); rows
    // outside [0, n_wrows) mark an expert whose weights are not resident, and its rows are left unwritten
    const int32_t *wslot;
    int n_wrows;
    int n_routed_slots;  // min(E, A): grid slots reserved for routed experts
    bool invariant;      // batch-invariant mode: decode K split fixed by the layer's shape alone
    float *y_perm, *y_sh;
    uint32_t *diag;      // optional counters (nullptr = none): [0] h values not finite in fp16
    // Routing inside the decode gate/up launch (one token, top-k routers without capacity; the decode path
    // only).  part = nullptr: the routing tables are read from offsets, perm, uniq and n_uniq.  Otherwise
    // every workgroup selects the token's experts from the router's split partial sums part[nsplit][1][E]
    // and sorts them for itself, and workgroup 0 writes the routing outputs below (offsets, uniq and n_uniq
    // are the buffers the down launch then reads).
    struct Route {
        const double *part;
        int nsplit, mode;  // mode 0 sigmoid + bias, 1 softmax gate
        const float *bias;
        float lambda;
        int32_t *idx;
        float *w;
        double *gap;  // optional
        int32_t *counts, *offsets, *perm, *inv, *uniq, *n_uniq;
    } route;
    // The combine inside the decode down launch (one token): y = y_sh + sum_j comb_w[j] y_perm[comb_inv[j]],
    // written to comb_y (nullptr: no combine here).
    const int32_t *comb_inv;
    const float *comb_w;
    float *comb_y;
};

// Routed weight row of expert e (wave-uniform e), or -1 when that row is outside the weights.
__device__ __forceinline__ int weight_row(const FfnParams &P, int e) {
    const int w = P.wslot ? __builtin_amdgcn_readfirstlane(P.wslot[e]) : e;
    return (unsigned)w < (unsigned)P.n_wrows ? w : -1;
}

// router.hip
// nullptr when the router kernels take the shape, else why not (a buffer beyond 32-bit descriptor offsets)
// inv: the batch-invariant mode (each token's sums in an order fixed by d and E alone)
// router: 0 sigmoid + bias, 1 softmax gate, 2 expert choice; C: capacity (0 = none for the top-k routers; the
// tokens per expert for expert choice)
const char *router_unsupported(int T, int d, int E, int act, bool inv);
size_t router_workspace_bytes(int T, int d, int E, bool inv, int k, int router, bool capacity);
// The permutation's outputs, for the router's fused form.
struct PermOut {
    int32_t *counts, *offsets, *perm, *inv, *uniq, *n_uniq;
};
// true when the selection's launch also takes the permutation (given PermOut): T = 1, top-k routers without
// capacity
bool router_fused(int T, int E, bool inv, int router, int C);
// The logits kernel alone: split partial sums part[nsplit][T][E] of x . W_r in fp64 (the select kernel's input);
// returns nsplit through *nsplit.
hipError_t launch_router_logits(int act, const void *x, const float *Wr, int T, int d, int E, bool inv, double *part,
                                int *nsplit, hipStream_t stream);
size_t router_partials_bytes(int T, int d, int E, bool inv);
// po: also sort the assignments, inside the selection's launch when router_fused (nullptr: no permutation)
hipError_t launch_router(int act, const void *x, const float *Wr, const float *bias, int T, int d, int E, int k,
                         float lambda, int32_t *idx, float *w, double *gap, void *ws, bool inv, int router, int C,
                         hipStream_t stream, const PermOut *po);

// permute.hip
size_t permute_lds_bytes(int E);
size_t permute_workspace_bytes(int A, int E);  // the multi-block path's histograms (0 below its threshold)
hipError_t launch_permute(const int32_t *idx, int A, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                          int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, hipStream_t stream);

// ffn_decode.hip: decode path, int8 MFMA with exact integer accumulation (h kept in fp32 in the workspace)
const char *decode_unsupported(const FfnParams &P);  // nullptr when the decode kernels take the shape
size_t decode_workspace_bytes(const FfnParams &P);
// true when the decode launches can route a single token inside the gate/up launch (FfnParams::route)
bool decode_routes(const FfnParams &P);
// true when the decode down launch can also combine (FfnParams::comb_y; one token, its slots' rows in LDS)
bool decode_combines(const FfnParams &P);
hipError_t launch_ffn_decode(const FfnParams &P, void *ws, hipStream_t stream);

// ffn_gemm.hip: MFMA grouped-GEMM path (d and I multiples of 64; fp32 activations as fp16 hi + lo)
bool gemm_supported(const FfnParams &P);
size_t gemm_workspace_bytes(const FfnParams &P);
hipError_t launch_ffn_gemm(const FfnParams &P, void *ws, hipStream_t stream);

// cache.hip: expert residency (slots in HBM over a host tier)
size_t cache_state_bytes(int E, int S);
const int32_t *cache_slot_map(const void *state, int E, int S);  // expert -> slot, in the state
hipError_t launch_cache_init(void *state, int E, int S, int P, int32_t *miss, int32_t *n_miss, hipStream_t stream);
hipError_t launch_cache_plan(void *state, int E, int S, int P, int policy, const int32_t *uniq, const int32_t *n_uniq,
                             int32_t *hit, int32_t *n_hit, int32_t *miss, int32_t *n_miss, hipStream_t stream);
// src: device view of the host tier (E experts); dst: the slots; bytes: per-expert bytes of the nine tensors
hipError_t launch_cache_fetch(const QW &src, const QW &dst, const long bytes[9], const int32_t *miss,
                              const int32_t *n_miss, const void *state, int E, int S, int workgroups,
                              hipStream_t stream);

// dsa_index.hip: sparse-attention indexer scores and top-K causal keys
size_t index_workspace_bytes(int T, int S);
const char *index_unsupported(int T, int S, int H, int D);
hipError_t launch_index_topk(const int8_t *q, const float *w, const int8_t *k, const float *kscale, int T, int S,
                             int H, int D, int K, int pos0, int32_t *top, double *gap, void *ws, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const float *y_perm, const float *y_shared, const int32_t *inv, const float *w, int T,
                          int d, int k, float *y, hipStream_t stream);

}  // namespace moe
