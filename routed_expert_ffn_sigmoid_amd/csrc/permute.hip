// Batch union as a stable counting sort ("25GB 内存跑 744B GLM-5.2 模型" page, section 三.4).
//
// One workgroup of 16 wavefronts.  The A assignments are split into 16
// contiguous ranges, one per wavefront, so "earlier range" means "smaller
// assignment id" and stability needs no ordering between waves:
//   1. per-wave histograms in LDS (integer atomics: order-free);
//   2. per expert, an exclusive scan over the 16 waves gives each wave's base
//      inside the expert's bucket; a scan over experts gives the offsets;
//   3. each wave walks its range 64 assignments at a time; lanes with the
//      same expert find each other with one ballot per key bit, take their
//      rank among lower lanes, and the highest lane of each group advances
//      the wave's running count.
// Every output is a function of topk_idx alone, independent of scheduling.  An id of -1 is an empty slot
// (a capacity drop, or no expert in expert choice): skipped like an invalid id, without the error flag.
//
// Above PMB_MIN_A assignments one workgroup would take the whole sort in series (84 us at A = 65536), so
// the work is cut into nb contiguous blocks of about PMB_PER_BLOCK assignments, in three launches:
//   1. per-block histograms (and invalid-key flags) into the workspace;
//   2. one workgroup: per expert the exclusive prefix over blocks, the totals and their scan (offsets),
//      counts and the unique list; the histogram entries become each block's first position per expert;
//   3. per block, the single-workgroup scatter above, its waves' bases starting from those positions.
// Blocks, like waves, own contiguous ranges, so the result is the same stable order.
#include "common.h"
#include "kernels.h"
#include "permute_dev.h"

namespace moe {

__global__ __launch_bounds__(PM_THREADS) void permute_kernel(const int32_t *__restrict__ keys, int A, int E,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                             int32_t *__restrict__ uniq,
                                                             int32_t *__restrict__ n_uniq) {
    extern __shared__ int32_t sm[];
    permute_block(keys, A, E, counts, offsets, perm, inv, uniq, n_uniq, sm);
}

size_t permute_lds_bytes(int E) { return sizeof(int32_t) * ((size_t)PM_WAVES * E + 2 * (size_t)E + 1); }

// ---- multi-block path
constexpr int PMB_MIN_A = 8192;       // assignments above which the sort is split into blocks
constexpr int PMB_PER_BLOCK = 512;    // assignments per block, about
constexpr int PMB_MAXB = 256;         // blocks at most
constexpr int PMB_WAVES = 4;          // wavefronts per block in passes 1 and 3

static int pmb_blocks(int A) {
    const int nb = (A + PMB_PER_BLOCK - 1) / PMB_PER_BLOCK;
    return nb < PMB_MAXB ? nb : PMB_MAXB;
}

size_t permute_workspace_bytes(int A, int E) {
    if (A <= PMB_MIN_A) return 0;
    return sizeof(int32_t) * ((size_t)pmb_blocks(A) * E + PMB_MAXB);
}

__global__ __launch_bounds__(PMB_WAVES * 64) void permute_hist_kernel(const int32_t *__restrict__ keys, int A, int E,
                                                                    int nb, int32_t *__restrict__ hist,
                                                                    int32_t *__restrict__ badb) {
    extern __shared__ int32_t h[];  // [E]
    __shared__ int32_t bad;
    const int b = blockIdx.x, tid = threadIdx.x;
    const long a0 = (long)A * b / nb, a1 = (long)A * (b + 1) / nb;
    for (int e = tid; e < E; e += PMB_WAVES * 64) h[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (long a = a0 + tid; a < a1; a += PMB_WAVES * 64) {
        const int key = keys[a];
        if (key >= 0 && key < E)
            atomicAdd(&h[key], 1);
        else if (key != -1)  // -1: an empty slot, skipped; any other id out of range is an error
            atomicOr(&bad, 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += PMB_WAVES * 64) hist[(long)b * E + e] = h[e];
    if (tid == 0) badb[b] = bad;
}

__global__ __launch_bounds__(PM_THREADS) void permute_scan_kernel(int E, int nb, int32_t *__restrict__ hist,
                                                                const int32_t *__restrict__ badb,
                                                                int32_t *__restrict__ counts,
                                                                int32_t *__restrict__ offsets,
                                                                int32_t *__restrict__ uniq,
                                                                int32_t *__restrict__ n_uniq) {
    extern __shared__ int32_t sm[];
    int32_t *off = sm;           // [E+1]
    int32_t *flag = off + E + 1;  // [E]: unique-expert positions
    __shared__ int32_t bad, nu;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int b = tid; b < nb; b += PM_THREADS)
        if (badb[b]) atomicOr(&bad, 1);
    // per expert: each block's exclusive prefix (in block order) and the total.  The counts are read 16
    // blocks at a time, all loads before any store, so a column of nb blocks costs nb / 16 memory round
    // trips instead of nb (T = 8192, 128 blocks: this kernel took 42 us with one load per trip).
    constexpr int SB = 16;
    for (int e = tid; e < E; e += PM_THREADS) {
        int run = 0;
        for (int b0 = 0; b0 < nb; b0 += SB) {
            int c[SB];
#pragma unroll
            for (int u = 0; u < SB; u++) c[u] = b0 + u < nb ? hist[(long)(b0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < SB; u++) {
                if (b0 + u < nb) hist[(long)(b0 + u) * E + e] = run;
                run += c[u];
            }
        }
        off[e + 1] = run;
        flag[e] = run > 0 ? 1 : 0;
    }
    if (tid == 0) off[0] = 0;
    __syncthreads();
    if (wv == 0) {
        int carry = 0, carry_u = 0;
        for (int base = 0; base < E; base += 64) {
            int e = base + lane;
            int v = (e < E) ? off[e + 1] : 0;
            int f = (e < E) ? flag[e] : 0;
            int sv = v, sf = f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                int tv = __shfl_up(sv, o, 64);
                int tf = __shfl_up(sf, o, 64);
                if (lane >= o) {
                    sv += tv;
                    sf += tf;
                }
            }
            if (e < E) {
                counts[e] = v;
                off[e + 1] = carry + sv;
                flag[e] = f ? (carry_u + sf - 1) : -1;
            }
            carry += __shfl(sv, 63, 64);
            carry_u += __shfl(sf, 63, 64);
        }
        if (lane == 0) {
            *n_uniq = bad ? -1 : carry_u;
            nu = carry_u;
        }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += PM_THREADS) offsets[e] = off[e];
    for (int e = tid; e < E; e += PM_THREADS) {
        if (flag[e] >= 0) uniq[flag[e]] = e;
        if (e >= nu) uniq[e] = -1;
    }
    // each block's first position per expert, again SB blocks per round trip
    for (int e = tid; e < E; e += PM_THREADS) {
        const int o = off[e];
        for (int b0 = 0; b0 < nb; b0 += SB) {
            int c[SB];
#pragma unroll
            for (int u = 0; u < SB; u++) c[u] = b0 + u < nb ? hist[(long)(b0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < SB; u++)
                if (b0 + u < nb) hist[(long)(b0 + u) * E + e] = c[u] + o;
        }
    }
}

__global__ __launch_bounds__(PMB_WAVES * 64) void permute_scatter_kernel(const int32_t *__restrict__ keys, int A,
                                                                       int E, int nb,
                                                                       const int32_t *__restrict__ hist,
                                                                       int32_t *__restrict__ perm,
                                                                       int32_t *__restrict__ inv) {
    extern __shared__ int32_t cnt[];  // [PMB_WAVES][E]: per-wave counts, then running positions
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const long a0 = (long)A * b / nb, a1 = (long)A * (b + 1) / nb;
    const long wa0 = a0 + (a1 - a0) * wv / PMB_WAVES, wa1 = a0 + (a1 - a0) * (wv + 1) / PMB_WAVES;
    for (int i = tid; i < PMB_WAVES * E; i += PMB_WAVES * 64) cnt[i] = 0;
    __syncthreads();
    for (long a = wa0 + lane; a < wa1; a += 64) {
        const int key = keys[a];
        if (key >= 0 && key < E) atomicAdd(&cnt[wv * E + key], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += PMB_WAVES * 64) {
        int run = hist[(long)b * E + e];
        for (int w2 = 0; w2 < PMB_WAVES; w2++) {
            const int c = cnt[w2 * E + e];
            cnt[w2 * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) nbits++;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (long base = wa0; base < wa1; base += 64) {
        const long a = base + lane;
        const int key = (a < wa1) ? keys[a] : -1;
        const bool valid = key >= 0 && key < E;
        uint64_t m = __ballot(valid);
#pragma unroll 1
        for (int bit = 0; bit < nbits; bit++) {
            const uint64_t B = __ballot(valid && ((key >> bit) & 1));
            m &= ((key >> bit) & 1) ? B : ~B;
        }
        if (valid) {
            const int pos = cnt[wv * E + key];
            const int dest = pos + __popcll(m & below);
            perm[dest] = (int32_t)a;
            inv[a] = dest;
            if ((m >> lane) == 1ull) cnt[wv * E + key] = pos + __popcll(m);
        } else if (a < wa1) {
            inv[a] = -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

hipError_t launch_permute(const int32_t *idx, int A, int E, int32_t *counts, int32_t *offsets, int32_t *perm,
                          int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, hipStream_t stream) {
    if (A > PMB_MIN_A) {
        const int nb = pmb_blocks(A);
        int32_t *hist = (int32_t *)ws, *badb = hist + (size_t)nb * E;
        hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(PMB_WAVES * 64), sizeof(int32_t) * E, stream, idx, A,
                           E, nb, hist, badb);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PM_THREADS), sizeof(int32_t) * (2 * E + 1), stream, E,
                           nb, hist, badb, counts, offsets, uniq, n_uniq);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(PMB_WAVES * 64), sizeof(int32_t) * PMB_WAVES * E,
                           stream, idx, A, E, nb, hist, perm, inv);
        return hipGetLastError();
    }
    size_t lds = permute_lds_bytes(E);
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute((const void *)permute_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PM_THREADS), lds, stream, idx, A, E, counts,
                       offsets, perm, inv, uniq, n_uniq);
    return hipGetLastError();
}

}  // namespace moe
