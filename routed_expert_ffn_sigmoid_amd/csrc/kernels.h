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
    int n_routed_slots;  // min(E, A): grid slots reserved for routed experts
    bool invariant;      // batch-invariant mode: decode K split fixed by the layer's shape alone
    float *y_perm, *y_sh;
    uint32_t *diag;      // optional counters (nullptr = none): [0] h values not finite in fp16
};

// router.hip
// nullptr when the router kernels take the shape, else why not (a buffer beyond 32-bit descriptor offsets)
// inv: the batch-invariant mode (each token's sums in an order fixed by d and E alone)
// router: 0 sigmoid + bias, 1 softmax gate, 2 expert choice; C: capacity (0 = none for the top-k routers; the
// tokens per expert for expert choice)
const char *router_unsupported(int T, int d, int E, int act, bool inv);
size_t router_workspace_bytes(int T, int d, int E, bool inv, int k, int router, bool capacity);
hipError_t launch_router(int act, const void *x, const float *Wr, const float *bias, int T, int d, int E, int k,
                         float lambda, int32_t *idx, float *w, double *gap, void *ws, bool inv, int router, int C,
                         hipStream_t stream);

// permute.hip
size_t permute_lds_bytes(int E);
size_t permute_workspace_bytes(int A, int E);  // the multi-block path's histograms (0 below its threshold)
hipError_t launch_permute(const int32_t *idx, int A, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                          int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, hipStream_t stream);

// ffn_decode.hip: decode path, int8 MFMA with exact integer accumulation (h kept in fp32 in the workspace)
const char *decode_unsupported(const FfnParams &P);  // nullptr when the decode kernels take the shape
size_t decode_workspace_bytes(const FfnParams &P);
hipError_t launch_ffn_decode(const FfnParams &P, void *ws, hipStream_t stream);

// ffn_gemm.hip: MFMA grouped-GEMM path (bf16 activations, d and I multiples of 64)
bool gemm_supported(const FfnParams &P);
size_t gemm_workspace_bytes(const FfnParams &P);
hipError_t launch_ffn_gemm(const FfnParams &P, void *ws, hipStream_t stream);

// dsa_index.hip: sparse-attention indexer scores and top-K causal keys
size_t index_workspace_bytes(int T, int S);
const char *index_unsupported(int T, int S, int H, int D);
hipError_t launch_index_topk(const int8_t *q, const float *w, const int8_t *k, const float *kscale, int T, int S,
                             int H, int D, int K, int pos0, int32_t *top, double *gap, void *ws, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const float *y_perm, const float *y_shared, const int32_t *inv, const float *w, int T,
                          int d, int k, float *y, hipStream_t stream);

}  // namespace moe
