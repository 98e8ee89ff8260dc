// Sigmoid + bias top-k router ("25GB 内存跑 744B GLM-5.2 模型" page, sections 三.1 and 四.3).
//
// Two kernels:
//   router_logits  z = x . W_r in fp64, tiled 64 tokens x 64 experts per
//                  workgroup with a K split so small T still spreads the
//                  W_r read over the whole chip; partial sums per split go to
//                  the workspace (no atomics: the reduction order is fixed).
//   router_select  one wavefront per token: sums the splits in order, takes
//                  the sigmoid, adds the bias, and picks the top k+1 by
//                  repeated wave-wide argmax with ties to the lower id.
// Products of an fp32/bf16 activation and an fp32 weight are exact in fp64,
// so the logit differs from any other fp64 summation order only by fp64
// rounding; the choice of experts therefore matches a plain fp64 evaluation
// unless two selection scores agree to ~1e-16.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RL_TT = 64;  // tokens per tile
constexpr int RL_TE = 64;  // experts per tile
constexpr int RL_KS = 32;  // d rows per LDS stage

template <int ACT>
__device__ __forceinline__ double load_act(const void *x, long i) {
    if (ACT == 0) return (double)((const float *)x)[i];
    return (double)bf16_to_f32(((const uint16_t *)x)[i]);
}

// grid: (ceil(E/64), ceil(T/64), nsplit); block 256.
// part[s][t][e] = sum over d rows [s*chunk, min(d,(s+1)*chunk)) of x[t][i]*W_r[i][e]
template <int ACT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ x,
                                                            const float *__restrict__ Wr, int T, int d, int E,
                                                            int chunk, double *__restrict__ part) {
    __shared__ double xs[RL_KS][RL_TT + 2];
    __shared__ double wsm[RL_KS][RL_TE + 2];
    const int tid = threadIdx.x;
    const int e0 = blockIdx.x * RL_TE, t0 = blockIdx.y * RL_TT;
    const int i_begin = blockIdx.z * chunk;
    const int i_end = min(d, i_begin + chunk);
    const int tx = tid & 15, ty = tid >> 4;  // 16 x 16 threads, 4 x 4 outputs each
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = 0.0;

    for (int i0 = i_begin; i0 < i_end; i0 += RL_KS) {
        // x tile: RL_TT tokens x RL_KS rows (stored transposed: [k][token])
        for (int q = tid; q < RL_TT * RL_KS; q += 256) {
            int tt = q / RL_KS, kk = q % RL_KS;
            int t = t0 + tt, i = i0 + kk;
            xs[kk][tt] = (t < T && i < i_end) ? load_act<ACT>(x, (long)t * d + i) : 0.0;
        }
        // W tile: RL_KS rows x RL_TE experts
        for (int q = tid; q < RL_TE * RL_KS; q += 256) {
            int kk = q / RL_TE, ee = q % RL_TE;
            int i = i0 + kk, e = e0 + ee;
            wsm[kk][ee] = (i < i_end && e < E) ? (double)Wr[(long)i * E + e] : 0.0;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < RL_KS; kk++) {
            double a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; u++) a[u] = xs[kk][ty * 4 + u];
#pragma unroll
            for (int u = 0; u < 4; u++) b[u] = wsm[kk][tx * 4 + u];
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int v = 0; v < 4; v++) acc[u][v] = fma(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
    double *out = part + (long)blockIdx.z * T * E;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        int t = t0 + ty * 4 + u;
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            int e = e0 + tx * 4 + v;
            if (e < E) out[(long)t * E + e] = acc[u][v];
        }
    }
}

constexpr int RS_MAXJ = 16;  // experts per lane: E <= 1024

// (v, id) is better than (v2, id2): larger score, then lower id
__device__ __forceinline__ bool better(double v, int id, double v2, int id2) {
    return v > v2 || (v == v2 && id < id2);
}

// grid: ceil(T/4); block 256 (one wavefront per token)
__global__ __launch_bounds__(256) void router_select_kernel(const double *__restrict__ part, int nsplit, int T,
                                                            int E, int k, const float *__restrict__ bias,
                                                            float lambda, int32_t *__restrict__ idx,
                                                            float *__restrict__ w, double *__restrict__ gap) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int nj = (E + 63) >> 6;
    double sel[RS_MAXJ], s[RS_MAXJ];
#pragma unroll
    for (int j = 0; j < RS_MAXJ; j++) {
        int e = lane + 64 * j;
        sel[j] = -INFINITY;
        s[j] = 0.0;
        if (j < nj && e < E) {
            double z = 0.0;
            for (int sp = 0; sp < nsplit; sp++) z += part[((long)sp * T + t) * E + e];
            s[j] = 1.0 / (1.0 + exp(-z));
            sel[j] = s[j] + (double)bias[e];
        }
    }
    uint32_t taken = 0;  // bit j: slot j of this lane already chosen
    double sum_s = 0.0, prev_v = 0.0;
    double my_s = 0.0;  // lane j' < k keeps the score of choice j'
    int my_id = 0;
    const int rounds = (k < E) ? k + 1 : k;
    for (int r = 0; r < rounds; r++) {
        double bv = -INFINITY, bs = 0.0;
        int bid = 0x7fffffff, bj = -1;
#pragma unroll
        for (int j = 0; j < RS_MAXJ; j++) {
            int e = lane + 64 * j;
            if (j < nj && e < E && !((taken >> j) & 1u) && better(sel[j], e, bv, bid)) {
                bv = sel[j];
                bid = e;
                bs = s[j];
                bj = j;
            }
        }
        // wave-wide argmax of (bv, bid)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            double ov = __shfl_xor(bv, o, 64);
            int oid = __shfl_xor(bid, o, 64);
            double os = __shfl_xor(bs, o, 64);
            if (better(ov, oid, bv, bid)) {
                bv = ov;
                bid = oid;
                bs = os;
            }
        }
        if (r < k) {
            if ((bid & 63) == lane && bj >= 0 && lane + 64 * bj == bid) taken |= 1u << bj;
            sum_s += bs;
            if (lane == r) {
                my_s = bs;
                my_id = bid;
            }
            prev_v = bv;
        } else if (lane == 0 && gap) {
            gap[t] = prev_v - bv;
        }
    }
    if (lane == 0 && gap && k >= E) gap[t] = INFINITY;
    if (lane < k) {
        idx[(long)t * k + lane] = my_id;
        w[(long)t * k + lane] = (float)((double)lambda * my_s / sum_s);
    }
}

int router_nsplit(int T, int d, int E) {
    int gx = (E + RL_TE - 1) / RL_TE, gy = (T + RL_TT - 1) / RL_TT;
    int ksteps = (d + RL_KS - 1) / RL_KS;
    int want = 512 / (gx * gy);
    if (want < 1) want = 1;
    if (want > ksteps) want = ksteps;
    return want;
}

size_t router_workspace_bytes(int T, int d, int E) {
    return (size_t)router_nsplit(T, d, E) * (size_t)T * (size_t)E * sizeof(double);
}

hipError_t launch_router(int act, const void *x, const float *Wr, const float *bias, int T, int d, int E, int k,
                         float lambda, int32_t *idx, float *w, double *gap, void *ws, hipStream_t stream) {
    int nsplit = router_nsplit(T, d, E);
    int ksteps = (d + RL_KS - 1) / RL_KS;
    int chunk = ((ksteps + nsplit - 1) / nsplit) * RL_KS;
    nsplit = (d + chunk - 1) / chunk;
    double *part = (double *)ws;
    dim3 grid((E + RL_TE - 1) / RL_TE, (T + RL_TT - 1) / RL_TT, nsplit);
    if (act == 0)
        hipLaunchKernelGGL(router_logits_kernel<0>, grid, dim3(256), 0, stream, x, Wr, T, d, E, chunk, part);
    else
        hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, stream, x, Wr, T, d, E, chunk, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(router_select_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, part, nsplit, T, E, k, bias,
                       lambda, idx, w, gap);
    return hipGetLastError();
}

}  // namespace moe
