// Exact block-wide top-K by radix selection (device code shared by the expert-choice router and the sparse
// attention indexer).
//
// One workgroup of NT threads selects, among n keys, the K largest in the order "larger key first, equal keys by
// lower index".  Keys are unsigned integers whose order is the order of the scores (fp64 values >= 0 as their bit
// patterns; signed scores through an order-preserving map).  The K-th largest key v is found digit by digit from the
// top, 8 bits per pass, each pass histogramming the keys that share the digits found so far; once those keys fit in
// LDS they are copied there and the remaining passes read only them.  Then every key above v is chosen, and of the
// keys equal to v the `need` of lowest index.  Integer work: the chosen set is exact and unique, whatever the
// order in which threads run.
#pragma once

#include "common.h"

namespace moe {

constexpr int TOPK_UNROLL = 16;    // keys loaded together per thread in the histogram and copy passes
constexpr int TOPK_VISIT = 8;      // consecutive keys per thread per step of the ordered visit
constexpr int TOPK_CAND = 4096;    // keys sharing the digits found so far that LDS holds (32 KB)

struct TopkState {
    uint64_t v;  // the K-th largest key
    int need;    // keys equal to v to take (the lowest indices first)
    int eq;      // keys equal to v in all
    int ncand;   // keys copied to the candidate buffer (-1: not copied)
};

// hist[b] += 1 for every lane of the wavefront with b >= 0.  The leading digits of scores of one magnitude are
// mostly equal: when every active lane has the same bucket one lane adds their count (64 lanes adding to one
// address would serialise); otherwise each lane adds its own.
__device__ __forceinline__ void wave_hist_add(int *hist, int b) {
    const uint64_t act = __ballot(b >= 0);
    if (!act) return;
    const int first = __builtin_ctzll(act);
    const int b0 = __shfl(b, first, 64);
    if (__ballot(b >= 0 && b != b0) == 0) {
        if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], __popcll(act));
    } else if (b >= 0) {
        atomicAdd(&hist[b], 1);
    }
}

// The K-th largest of n keys (1 <= K <= n).  key(i) returns key i.  LDS: hist (256 ints), s (a TopkState), cand
// (TOPK_CAND keys) and *cnt (one int).  All NT threads of the workgroup call it.
template <int NT, int BITS, typename KeyFn>
__device__ TopkState radix_kth_largest(KeyFn key, int n, int K, int *hist, TopkState *s, uint64_t *cand, int *cnt) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint64_t prefix = 0, mask = 0;
    if (tid == 0) {
        s->need = K;
        s->ncand = -1;
        s->eq = n;
    }
    __syncthreads();
    for (int shift = BITS - 8; shift >= 0; shift -= 8) {
        const int nc = s->ncand;  // uniform
        for (int b = tid; b < 256; b += NT) hist[b] = 0;
        __syncthreads();
        if (nc >= 0) {
            for (int i = tid; i < nc; i += NT) {
                const uint64_t k = cand[i];
                wave_hist_add(hist, (k & mask) == prefix ? (int)((k >> shift) & 255u) : -1);
            }
        } else {
            // TOPK_UNROLL independent loads per thread before their histogram updates
            for (int i0 = tid; i0 < n; i0 += NT * TOPK_UNROLL) {
                uint64_t kk[TOPK_UNROLL];
#pragma unroll
                for (int u = 0; u < TOPK_UNROLL; u++) {
                    const int i = i0 + u * NT;
                    kk[u] = i < n ? (uint64_t)key(i) : 0;
                }
#pragma unroll
                for (int u = 0; u < TOPK_UNROLL; u++) {
                    const bool in = i0 + u * NT < n && (kk[u] & mask) == prefix;
                    wave_hist_add(hist, in ? (int)((kk[u] >> shift) & 255u) : -1);
                }
            }
        }
        __syncthreads();
        if (tid < 64) {
            // buckets from the top: lane l holds the counts of buckets 255 - 4l .. 252 - 4l
            int c[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                c[q] = hist[255 - 4 * lane - q];
                sum += c[q];
            }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            const int need = s->need;
            const int before = incl - sum;  // keys in buckets above this lane's
            // the lane whose buckets hold the need-th key from the top
            if (before < need && incl >= need) {
                int acc = before, q = 0;
                while (acc + c[q] < need) acc += c[q++];
                const int bucket = 255 - 4 * lane - q;
                s->v = prefix | ((uint64_t)bucket << shift);
                s->need = need - acc;
                s->eq = c[q];
            }
        }
        if (tid == 0) *cnt = 0;
        __syncthreads();
        prefix = s->v;
        mask |= (uint64_t)255u << shift;
        // the keys that share the digits found so far, copied to LDS once they fit (order does not matter here)
        if (shift > 0 && nc < 0 && s->eq <= TOPK_CAND) {
            for (int i0 = tid; i0 < n; i0 += NT * TOPK_UNROLL) {
                uint64_t kk[TOPK_UNROLL];
#pragma unroll
                for (int u = 0; u < TOPK_UNROLL; u++) {
                    const int i = i0 + u * NT;
                    kk[u] = i < n ? (uint64_t)key(i) : 0;
                }
#pragma unroll
                for (int u = 0; u < TOPK_UNROLL; u++) {
                    const bool in = i0 + u * NT < n && (kk[u] & mask) == prefix;
                    const uint64_t bal = __ballot(in);
                    int base = 0;
                    if (bal) {
                        const int leader = __builtin_ctzll(bal);
                        if (lane == leader) base = atomicAdd(cnt, __popcll(bal));
                        base = __shfl(base, leader, 64);
                    }
                    const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
                    if (in) cand[base + __popcll(bal & lower)] = kk[u];
                }
            }
            __syncthreads();
            if (tid == 0) s->ncand = *cnt;
        }
        __syncthreads();
    }
    return *s;
}

// Visits the keys in index order: f(i, rank) for every chosen i, rank = its place among the chosen (0 .. K-1,
// increasing with i); g(i, k) for every key i not chosen, k its key.  Thread tid takes TOPK_VISIT consecutive keys
// of each step of NT * TOPK_VISIT; one workgroup-wide scan per step gives each thread the counts before its own.
// scan is LDS of NT / 64 + 1 ints.
template <int NT, typename KeyFn, typename F, typename G>
__device__ void visit_topk(KeyFn key, int n, const TopkState &st, int *scan, F f, G g) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NW = NT / 64, U = TOPK_VISIT;
    static_assert(NT * U < (1 << 15), "per-step counts are packed in 16 bits");
    int taken_eq = 0, taken = 0;  // over the steps done so far (uniform)
    uint64_t nxt[U];  // the next step's keys, requested while this step is processed
#pragma unroll
    for (int u = 0; u < U; u++) nxt[u] = tid * U + u < n ? (uint64_t)key(tid * U + u) : 0;
    for (int base = 0; base < n; base += NT * U) {
        const int i0 = base + tid * U;
        uint64_t kk[U];
#pragma unroll
        for (int u = 0; u < U; u++) kk[u] = nxt[u];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int in = i0 + NT * U + u;
            nxt[u] = in < n ? (uint64_t)key(in) : 0;
        }
        int neq = 0, ngt = 0;
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (i0 + u < n) {
                neq += kk[u] == st.v;
                ngt += kk[u] > st.v;
            }
        }
        // exclusive scans over the threads, in index order, of the equal counts and of the greater counts (packed
        // in one int): the equal keys before a thread decide which of its equal keys are taken, and the taken keys
        // before it give its ranks
        const int v = (neq << 16) | ngt;
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        __syncthreads();  // scan is reused
        if (lane == 63) scan[wv] = incl;
        __syncthreads();
        int before = incl - v, step = 0;
        for (int w2 = 0; w2 < NW; w2++) {
            const int sw = scan[w2];
            if (w2 < wv) before += sw;
            step += sw;
        }
        int eq_before = taken_eq + (before >> 16);
        // taken before this thread: every greater key, and the equal keys while they are still needed
        int rank = taken + (before & 0xFFFF) + min(max(st.need - taken_eq, 0), before >> 16);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + u;
            if (i < n) {
                const bool gt = kk[u] > st.v, eq = kk[u] == st.v;
                const bool chosen = gt || (eq && eq_before < st.need);
                if (eq) eq_before++;
                if (chosen)
                    f(i, rank++);
                else
                    g(i, kk[u]);
            }
        }
        const int step_eq = step >> 16, step_gt = step & 0xFFFF;
        taken += step_gt + min(max(st.need - taken_eq, 0), step_eq);
        taken_eq += step_eq;
    }
}

// Largest of one 64-bit value per thread, over the workgroup: a wavefront maximum in lane shuffles, then one LDS
// atomic per wavefront into *out (which the caller has set to 0 and synchronised).
__device__ __forceinline__ void block_max_u64(uint64_t v, unsigned long long *out) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t w = ((uint64_t)(uint32_t)__shfl_xor((int)(v >> 32), o, 64) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
        v = w > v ? w : v;
    }
    if ((threadIdx.x & 63) == 0) atomicMax(out, (unsigned long long)v);
}

}  // namespace moe
