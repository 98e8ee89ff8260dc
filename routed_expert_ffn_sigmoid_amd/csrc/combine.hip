// Weighted combine: y[t] = y_shared[t] + sum_j w[t][j] * y_perm[inv[t*k + j]], fp32, fixed order.
//
// HBM-bound gather: each workgroup handles one token and 1024 consecutive
// hidden columns (float4 per thread), reading the k routed rows of that token
// from wherever the permutation put them.
#include "common.h"
#include "kernels.h"

namespace moe {

// grid: (T, ceil(d/1024)); block 256
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_perm,
                                                      const float *__restrict__ y_shared,
                                                      const int32_t *__restrict__ inv, const float *__restrict__ w,
                                                      int d, int k, float *__restrict__ y) {
    const int t = blockIdx.x;
    const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    float4 acc = y_shared ? *(const float4 *)(y_shared + (long)t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
        const float wj = w[(long)t * k + j];
        const int p = inv[(long)t * k + j];
        if (p < 0) continue;  // assignment dropped by moe_permute (invalid expert id)
        const float4 v = *(const float4 *)(y_perm + (long)p * d + c);
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    *(float4 *)(y + (long)t * d + c) = acc;
}

hipError_t launch_combine(const float *y_perm, const float *y_shared, const int32_t *inv, const float *w, int T,
                          int d, int k, float *y, hipStream_t stream) {
    dim3 grid(T, (d + 1023) / 1024);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, y_perm, y_shared, inv, w, d, k, y);
    return hipGetLastError();
}

}  // namespace moe
