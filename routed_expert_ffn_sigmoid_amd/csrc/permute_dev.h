// Single-workgroup stable counting sort of expert assignments (device code shared by the permutation kernel and
// the router's fused selection and permutation).  See permute.hip for the method.
#pragma once

#include "common.h"

namespace moe {

constexpr int PM_WAVES = 16;
constexpr int PM_THREADS = PM_WAVES * 64;

// The single-workgroup sort, as a device function of a PM_THREADS-thread workgroup (the permutation kernel, and
// the router's fused path); sm: LDS of permute_lds_bytes(E) bytes.  keys may be in global memory or LDS.
__device__ inline void permute_block(const int32_t *keys, int A, int E, int32_t *__restrict__ counts,
                                     int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                     int32_t *__restrict__ inv, int32_t *__restrict__ uniq,
                                     int32_t *__restrict__ n_uniq, int32_t *sm) {
    int32_t *cnt = sm;                       // [PM_WAVES][E]: per-wave counts, then running bases
    int32_t *off = cnt + PM_WAVES * E;       // [E+1]
    int32_t *flag = off + E + 1;             // [E]: unique-expert positions
    __shared__ int32_t bad, nu;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const long a_begin = (long)A * wv / PM_WAVES, a_end = (long)A * (wv + 1) / PM_WAVES;

    for (int i = tid; i < PM_WAVES * E; i += PM_THREADS) cnt[i] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (long a = a_begin + lane; a < a_end; a += 64) {
        int key = keys[a];
        if (key >= 0 && key < E)
            atomicAdd(&cnt[wv * E + key], 1);
        else if (key != -1)  // -1: an empty slot, skipped; any other id out of range is an error
            atomicOr(&bad, 1);
    }
    __syncthreads();
    // per-expert totals and per-wave bases
    for (int e = tid; e < E; e += PM_THREADS) {
        int run = 0;
        for (int w2 = 0; w2 < PM_WAVES; w2++) {
            int c = cnt[w2 * E + e];
            cnt[w2 * E + e] = run;
            run += c;
        }
        off[e + 1] = run;  // total for e, scanned below
        flag[e] = run > 0 ? 1 : 0;
    }
    if (tid == 0) off[0] = 0;
    __syncthreads();
    // inclusive scans of totals (off[1..E]) and of unique flags, by the first wave
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
                flag[e] = f ? (carry_u + sf - 1) : -1;  // position in uniq, or -1
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

    // stable scatter
    int nbits = 0;
    while ((1 << nbits) < E) nbits++;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (long base = a_begin; base < a_end; base += 64) {
        long a = base + lane;
        int key = (a < a_end) ? keys[a] : -1;
        bool valid = key >= 0 && key < E;
        uint64_t m = __ballot(valid);
#pragma unroll 1
        for (int b = 0; b < nbits; b++) {
            uint64_t B = __ballot(valid && ((key >> b) & 1));
            m &= ((key >> b) & 1) ? B : ~B;
        }
        if (valid) {
            int rank = __popcll(m & below);
            int basepos = cnt[wv * E + key];
            int dest = off[key] + basepos + rank;
            perm[dest] = (int32_t)a;
            inv[a] = dest;
            // highest lane of the group advances the running count
            if ((m >> lane) == 1ull) cnt[wv * E + key] = basepos + __popcll(m);
        } else if (a < a_end) {
            inv[a] = -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace moe
