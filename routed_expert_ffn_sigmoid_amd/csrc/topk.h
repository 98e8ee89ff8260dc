// Exact block-wide top-K by radix selection (device code shared by the expert-choice router and the sparse
// attention indexer).
//
// One workgroup of NT threads selects, among n keys, the K largest in the order "larger key first, equal keys by
// lower index".  Keys are unsigned integers whose order is the order of the scores (fp64 values >= 0 as their bit
// patterns; fp32 scores through ordered_f32).  The K-th largest key v is found digit by digit from the top, 8 bits
// per pass, each pass histogramming the keys that share the digits found so far; then every key above v is
// chosen, and of the keys equal to v the `need` of lowest index.  Integer work: the chosen set is exact and
// unique, whatever the order in which threads run.
#pragma once

#include "common.h"

namespace moe {

// fp32 -> uint32 whose unsigned order is the order of the values (-0 below +0; NaN above +inf)
__device__ __forceinline__ uint32_t ordered_f32(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkState {
    uint64_t v;  // the K-th largest key
    int need;    // keys equal to v to take (the lowest indices first)
    int eq;      // keys equal to v in all
};

// The K-th largest of n keys (1 <= K <= n).  key(i) returns key i; hist is LDS of 256 ints; s an LDS TopkState.
// All NT threads of the workgroup call it.
template <int NT, int BITS, typename KeyFn>
__device__ TopkState radix_kth_largest(KeyFn key, int n, int K, int *hist, TopkState *s) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint64_t prefix = 0, mask = 0;
    if (tid == 0) s->need = K;
    for (int shift = BITS - 8; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += NT) hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint64_t k = (uint64_t)key(i);
            if ((k & mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 255u)], 1);
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
            const bool here = before < need && incl >= need;
            if (here) {
                int acc = before, q = 0;
                while (acc + c[q] < need) acc += c[q++];
                const int bucket = 255 - 4 * lane - q;
                s->v = prefix | ((uint64_t)bucket << shift);
                s->need = need - acc;
                s->eq = c[q];
            }
        }
        __syncthreads();
        prefix = s->v;
        mask |= (uint64_t)255u << shift;
        __syncthreads();
    }
    return *s;
}

// Visits the chosen keys in index order: f(i, rank) for every chosen i, rank = its place among the chosen (0 ..
// K-1, increasing with i); g(i) for every key not chosen.  scan is LDS of NT / 64 + 1 ints.
template <int NT, typename KeyFn, typename F, typename G>
__device__ void visit_topk(KeyFn key, int n, const TopkState &st, int *scan, F f, G g) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NW = NT / 64;
    int taken_eq = 0, taken = 0;  // over the chunks done so far (uniform)
    for (int base = 0; base < n; base += NT) {
        const int i = base + tid;
        const uint64_t k = i < n ? (uint64_t)key(i) : 0;
        const bool gt = i < n && k > st.v, eq = i < n && k == st.v;
        // rank of this key among the chunk's equal keys and among its chosen keys, in index order
        const uint64_t beq = __ballot(eq);
        __syncthreads();  // scan is reused
        if (lane == 0) scan[wv] = __popcll(beq);
        __syncthreads();
        int eq_before = taken_eq;
        for (int w2 = 0; w2 < wv; w2++) eq_before += scan[w2];
        const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        eq_before += __popcll(beq & lower);
        const bool chosen = gt || (eq && eq_before < st.need);
        int chunk_eq = 0;
        for (int w2 = 0; w2 < NW; w2++) chunk_eq += scan[w2];
        const uint64_t bch = __ballot(chosen);
        __syncthreads();
        if (lane == 0) scan[wv] = __popcll(bch);
        __syncthreads();
        int rank = taken;
        for (int w2 = 0; w2 < wv; w2++) rank += scan[w2];
        rank += __popcll(bch & lower);
        int chunk_taken = 0;
        for (int w2 = 0; w2 < NW; w2++) chunk_taken += scan[w2];
        if (i < n) {
            if (chosen)
                f(i, rank);
            else
                g(i);
        }
        taken_eq += chunk_eq;
        taken += chunk_taken;
    }
}

}  // namespace moe
