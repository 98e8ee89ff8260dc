// Weighted combine: y[t] = y_shared[t] + sum_j w[t][j] * y_perm[inv[t*k + j]], fp32, fixed order.
//
// HBM-bound gather: each workgroup handles one token and 1024 consecutive
// hidden columns (float4 per thread), reading the k routed rows of that token
// from wherever the permutation put them.
#include "common.h"
#include "kernels.h"

namespace moe {

// grid: (T, ceil(d/1024)); block 256.  The k routed rows are taken in batches of CB: the batch's row
// numbers and weights are read together (one round trip), then its row loads are issued together (a
// second), then added in order j = 0, 1, ...; with k <= CB the whole gather is two round trips deep.
// Every y_perm and y_shared element is read once and every y element written once, so they move with
// non-temporal loads and stores (T = 8192: 478 -> 415 us for the 2.35 GB).
constexpr int CB = 8;

typedef float nt4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float *p) {
    const nt4_t v = __builtin_nontemporal_load((const nt4_t *)p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(float *p, float4 a) {
    const nt4_t v = {a.x, a.y, a.z, a.w};
    __builtin_nontemporal_store(v, (nt4_t *)p);
}

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_perm,
                                                      const float *__restrict__ y_shared,
                                                      const int32_t *__restrict__ inv, const float *__restrict__ w,
                                                      int d, int k, float *__restrict__ y) {
    const int t = blockIdx.x;
    const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    // the shared row is requested unconditionally (from y itself when there is none, then discarded), so
    // that it travels with the first batch instead of ahead of it
    const float4 s4 = load_nt((y_shared ? y_shared : y) + (long)t * d + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += CB) {
        int p[CB];
        float wj[CB];
#pragma unroll
        for (int u = 0; u < CB; u++) {
            const int j = j0 + u;
            p[u] = j < k ? inv[(long)t * k + j] : -1;
            wj[u] = j < k ? w[(long)t * k + j] : 0.f;
        }
        float4 v[CB];
#pragma unroll
        for (int u = 0; u < CB; u++)  // p < 0: assignment dropped by moe_permute (invalid expert id), or past k
            v[u] = p[u] >= 0 ? load_nt(y_perm + (long)p[u] * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 == 0 && y_shared) acc = s4;
#pragma unroll
        for (int u = 0; u < CB; u++) {
            if (p[u] < 0) continue;
            acc.x = fmaf(wj[u], v[u].x, acc.x);
            acc.y = fmaf(wj[u], v[u].y, acc.y);
            acc.z = fmaf(wj[u], v[u].z, acc.z);
            acc.w = fmaf(wj[u], v[u].w, acc.w);
        }
    }
    if (k <= 0 && y_shared) acc = s4;
    store_nt(y + (long)t * d + c, acc);
}

hipError_t launch_combine(const float *y_perm, const float *y_shared, const int32_t *inv, const float *w, int T,
                          int d, int k, float *y, hipStream_t stream) {
    dim3 grid(T, (d + 1023) / 1024);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, y_perm, y_shared, inv, w, d, k, y);
    return hipGetLastError();
}

}  // namespace moe
