// Sparse-attention indexer: scores of the cached keys for each query and the top K causal keys.
//
// The GLM-5.2 page ("github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！") has the engine run the model's
// lightning indexer and keep the top 2048 causal keys per layer for attention (section 三.3); a light indexer
// scores the history's keys and the top-k entries go to the real attention (section 四.4).  Read here with the
// DSA indexer's published form and integer operands:
//     I[t][s] = kscale[s] * sum_h w[t][h] * max(0, q[t][h] . k[s])
// q and k int8, the dot products exact in int32 on the matrix cores (v_mfma_i32_16x16x64_i8), the head sum an
// fp64 fused multiply-add chain in head order, then one fp64 product by kscale[s]: the same bits as a plain
// evaluation in that order, so the selection matches it exactly.  Query t (position pos0 + t) sees keys s <=
// pos0 + t.  The top K visible keys (larger score first, equal scores by lower position) are found by the exact
// radix selection of topk.h and listed by ascending position.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int IX_WAVES = 4;            // wavefronts per scoring workgroup: 64 keys
constexpr int IX_KEYS = 16 * IX_WAVES;
constexpr int IX_QB = 4;               // queries per scoring workgroup (one per lane group of 16)
constexpr int IX_SEL_THREADS = 1024;

// Scores for the queries [IX_QB y, IX_QB y + IX_QB) and the keys of nkb blocks of 64 from block nkb x.  The
// queries' rows go to LDS once (padded rows: the 16 rows one fragment read touches sit in different banks).  In the
// matrix product of a wavefront the rows (A operand) are (query, head) pairs: row i is query i / 4 of the group and
// head 4 m + i % 4 of head tile m; the columns (B operand) are 16 keys; lane l supplies bytes 16 (l / 16) .. + 15 of
// each 64-byte segment of row or column l % 16.  C[row i][key j] sits in lane 16 (i / 4) + j, register i % 4, so
// lane (g, j) = (l / 16, l % 16) receives the dot products of query g with key j for heads 4 m .. 4 m + 3 in its
// four registers and runs the head chain of that pair tile after tile, in head order, from registers.
constexpr int IX_QPAD = 16;  // bytes of padding per LDS row of q

__global__ __launch_bounds__(IX_WAVES * 64) void index_score_kernel(const int8_t *__restrict__ q,
                                                                    const float *__restrict__ w,
                                                                    const int8_t *__restrict__ k,
                                                                    const float *__restrict__ kscale, int T, int S,
                                                                    int H, int D, int pos0, int nkb,
                                                                    double *__restrict__ scores,
                                                                    double *__restrict__ range) {
    extern __shared__ __align__(16) uint8_t qs[];  // [IX_QB][H][D + IX_QPAD]
    __shared__ double s_rng[IX_WAVES][IX_QB][2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int nseg = D / 64, ntile = H / 4, pitch = D + IX_QPAD;
    const int t0 = blockIdx.y * IX_QB;
    const int tlast = min(T - 1, t0 + IX_QB - 1);
    const int kb0 = blockIdx.x * nkb * IX_KEYS;  // first key of this workgroup
    // range[t][x] = {smallest, largest} score of query t among workgroup x's keys (+inf, -inf: none)
    double *rng = range + ((long)t0 * gridDim.x + blockIdx.x) * 2;
    if (kb0 > pos0 + tlast) {  // no query of the group sees these keys (uniform)
        if (tid < 2 * IX_QB && t0 + tid / 2 < T) rng[(long)(tid / 2) * gridDim.x * 2 + (tid & 1)] = tid & 1 ? -INFINITY : INFINITY;
        return;
    }
    // the group's query rows into LDS (rows of queries past T are zeros)
    const int nq16 = IX_QB * H * D / 16;
    for (int c = tid; c < nq16; c += IX_WAVES * 64) {
        const int row = c / (D / 16), col = c % (D / 16);  // row = query * H + head
        const int tq = t0 + row / H;
        const uint4 v = tq < T ? *(const uint4 *)(q + ((long)t0 * H + row) * D + 16 * col) : make_uint4(0, 0, 0, 0);
        *(uint4 *)(qs + (long)row * pitch + 16 * col) = v;
    }
    __syncthreads();
    const rsrc_t kr = make_rsrc(k, (uint32_t)((long)S * D));
    // this lane's A rows: query j / 4, head 4 m + j % 4 (row j / 4 * H + 4 m + j % 4)
    const uint8_t *arow = qs + (long)((j >> 2) * H + (j & 3)) * pitch + 16 * g;
    const int t = t0 + g;  // this lane's chain: query t, key s0 + j
    const float *wt = w + (long)(t < T ? t : 0) * H;
    double lmn = INFINITY, lmx = -INFINITY;  // this lane's scores' range
    for (int kb = 0; kb < nkb; kb++) {
        const int s0 = kb0 + kb * IX_KEYS + 16 * wv;
        if (s0 > pos0 + tlast || s0 >= S) break;  // uniform over the wavefront
        uint4 b[4];
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
            const int key = s0 + j;
            b[sg] = buf_load16(kr, (sg < nseg && key < S) ? (uint32_t)((long)key * D + 64 * sg + 16 * g) : kOOB);
        }
        double acc = 0.0;
        for (int m = 0; m < ntile; m++) {
            const uint8_t *am = arow + (long)4 * m * pitch;
            const float4 w4 = *(const float4 *)(wt + 4 * m);
            i32x4_t c = {0, 0, 0, 0};
#pragma unroll
            for (int sg = 0; sg < 4; sg++) {
                if (sg >= nseg) break;
                const uint4 a = *(const uint4 *)(am + 64 * sg);
                const i32x4_t A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                const i32x4_t Bv = {(int)b[sg].x, (int)b[sg].y, (int)b[sg].z, (int)b[sg].w};
                c = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bv, c, 0, 0, 0);
            }
            acc = __builtin_fma((double)w4.x, (double)(c[0] > 0 ? c[0] : 0), acc);
            acc = __builtin_fma((double)w4.y, (double)(c[1] > 0 ? c[1] : 0), acc);
            acc = __builtin_fma((double)w4.z, (double)(c[2] > 0 ? c[2] : 0), acc);
            acc = __builtin_fma((double)w4.w, (double)(c[3] > 0 ? c[3] : 0), acc);
        }
        const int key = s0 + j;
        if (t < T && key < S && key <= pos0 + t) {
            const double sc = (double)kscale[key] * acc;
            scores[(long)t * S + key] = sc;
            lmn = fmin(lmn, sc);
            lmx = fmax(lmx, sc);
        }
    }
    // the range of each query over the workgroup's keys: the 16 lanes of its lane group, then the wavefronts
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
        lmn = fmin(lmn, __shfl_xor(lmn, o, 64));
        lmx = fmax(lmx, __shfl_xor(lmx, o, 64));
    }
    if (j == 0) {
        s_rng[wv][g][0] = lmn;
        s_rng[wv][g][1] = lmx;
    }
    __syncthreads();
    if (tid < 2 * IX_QB && t0 + tid / 2 < T) {
        const int gq = tid / 2, hi = tid & 1;
        double v = s_rng[0][gq][hi];
        for (int w2 = 1; w2 < IX_WAVES; w2++) v = hi ? fmax(v, s_rng[w2][gq][hi]) : fmin(v, s_rng[w2][gq][hi]);
        rng[(long)gq * gridDim.x * 2 + hi] = v;
    }
}

// fp64 -> uint64 whose unsigned order is the order of the values
__device__ __forceinline__ uint64_t ordered_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double from_ordered_f64(uint64_t o) {
    const uint64_t u = (o >> 63) ? (o & 0x7FFFFFFFFFFFFFFFull) : ~o;
    return __longlong_as_double((long long)u);
}

// One workgroup per query: the top K of its n = min(S, pos0 + t + 1) visible keys, by ascending position.
//
// The K-th largest score is found in two rounds.  First a histogram of IX_NB buckets spaced evenly between the
// query's smallest and largest score, bucket(s) = floor((s - min) * IX_NB / (max - min)): the map is monotonic in
// s (a subtraction and a product by a positive constant, each rounded), so every key of a higher bucket has a
// larger or equal score, and equal scores share a bucket.  A scan from the top finds the bucket b* holding the
// K-th largest and the count above it; the keys of b* (a few dozen for scores spread like these) are copied to
// LDS and the exact radix selection of topk.h finds, among them, the K-th largest key and how many of its equals
// are taken.  Queries whose b* holds more than TOPK_CAND keys (many equal scores, or a range that does not
// spread) take the radix selection over all keys instead.  Either way the ordered visit writes the positions.
constexpr int IX_NB = 4096;
constexpr int IX_UN = 16;  // scores loaded together per thread in the streaming passes

__device__ __forceinline__ int ix_bucket(double s, double mn, double scale) {
    const double f = (s - mn) * scale;
    return f >= 0.0 ? (f < (double)(IX_NB - 1) ? (int)f : IX_NB - 1) : 0;
}

// The bucket holding the K-th largest key (K <= the keys counted): thread tid sums buckets IX_NB - BPT tid - 1 ..
// IX_NB - BPT tid - BPT (from the top); an inclusive scan over the threads gives the keys above each thread's
// buckets.  Writes the bucket, the keys in buckets above it and its own count.  scan: LDS of the wavefront totals.
__device__ void ix_find_bucket(const int *bhist, int K, int *scan, int *bstar, int *above, int *nb) {
    constexpr int BPT = IX_NB / IX_SEL_THREADS;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int c[BPT], sum = 0;
#pragma unroll
    for (int q = 0; q < BPT; q++) {
        c[q] = bhist[IX_NB - 1 - BPT * tid - q];
        sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t2 = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t2;
    }
    if (lane == 63) scan[wv] = incl;
    __syncthreads();
    int before = incl - sum;
    for (int w2 = 0; w2 < wv; w2++) before += scan[w2];
    if (before < K && before + sum >= K) {
        int acc = before, q = 0;
        while (acc + c[q] < K) acc += c[q++];
        *bstar = IX_NB - 1 - BPT * tid - q;
        *above = acc;
        *nb = c[q];
    }
}

__global__ __launch_bounds__(IX_SEL_THREADS) void index_select_kernel(const double *__restrict__ scores, int S,
                                                                      int K, int pos0, int32_t *__restrict__ top,
                                                                      double *__restrict__ gap,
                                                                      const double *__restrict__ range, int nbx) {
    __shared__ int bhist[IX_NB];
    __shared__ uint64_t bkeys[TOPK_CAND];
    __shared__ int hist[256];
    __shared__ int scan[IX_SEL_THREADS / 64 + 1];
    __shared__ TopkState st;
    __shared__ uint64_t cand[TOPK_CAND];
    __shared__ int ncand, s_nb, s_bstar, s_above;
    __shared__ double s_mn[IX_SEL_THREADS / 64], s_mx[IX_SEL_THREADS / 64];
    __shared__ unsigned long long below;  // ordered key of the largest score not taken
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    long nl = (long)pos0 + t + 1;
    const int n = (int)(nl < 0 ? 0 : (nl > S ? S : nl));
    int32_t *out = top + (long)t * K;
    const double *sc = scores + (long)t * S;
    if (n <= K) {  // every visible key
        for (int i = tid; i < K; i += IX_SEL_THREADS) out[i] = i < n ? i : -1;
        if (tid == 0 && gap) gap[t] = INFINITY;
        return;
    }
    auto key = [&](int i) { return ordered_f64(sc[i]); };
    if (tid == 0) below = 0ull;
    // ---- the query's range of scores, from the scoring workgroups' ranges
    double mn = INFINITY, mx = -INFINITY;
    for (int i = tid; i < nbx; i += IX_SEL_THREADS) {
        mn = fmin(mn, range[((long)t * nbx + i) * 2]);
        mx = fmax(mx, range[((long)t * nbx + i) * 2 + 1]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o, 64));
        mx = fmax(mx, __shfl_xor(mx, o, 64));
    }
    if (lane == 0) {
        s_mn[wv] = mn;
        s_mx[wv] = mx;
    }
    for (int b = tid; b < IX_NB; b += IX_SEL_THREADS) bhist[b] = 0;
    __syncthreads();
    mn = s_mn[0];
    mx = s_mx[0];
    for (int w2 = 1; w2 < IX_SEL_THREADS / 64; w2++) {
        mn = fmin(mn, s_mn[w2]);
        mx = fmax(mx, s_mx[w2]);
    }
    const double scale = (double)IX_NB / (mx - mn);
    bool spread = mx > mn && scale > 0.0 && scale < INFINITY;  // uniform over the workgroup
    TopkState s;
    if (spread) {
        // ---- histogram of the buckets
        for (int i0 = tid; i0 < n; i0 += IX_SEL_THREADS * IX_UN) {
            double v[IX_UN];
#pragma unroll
            for (int u = 0; u < IX_UN; u++) v[u] = i0 + u * IX_SEL_THREADS < n ? sc[i0 + u * IX_SEL_THREADS] : 0.0;
#pragma unroll
            for (int u = 0; u < IX_UN; u++)
                if (i0 + u * IX_SEL_THREADS < n) atomicAdd(&bhist[ix_bucket(v[u], mn, scale)], 1);
        }
        __syncthreads();
        ix_find_bucket(bhist, K, scan, &s_bstar, &s_above, &s_nb);
        if (tid == 0) ncand = 0;
        __syncthreads();
        spread = s_nb <= TOPK_CAND;
    }
    if (spread) {
        // ---- the keys of bucket b* into LDS (any order), then the exact selection among them
        const int bstar = s_bstar;
        for (int i0 = tid; i0 < n; i0 += IX_SEL_THREADS * IX_UN) {
            double v[IX_UN];
#pragma unroll
            for (int u = 0; u < IX_UN; u++) v[u] = i0 + u * IX_SEL_THREADS < n ? sc[i0 + u * IX_SEL_THREADS] : 0.0;
#pragma unroll
            for (int u = 0; u < IX_UN; u++) {
                const bool in = i0 + u * IX_SEL_THREADS < n && ix_bucket(v[u], mn, scale) == bstar;
                const uint64_t bal = __ballot(in);
                int base = 0;
                if (bal) {
                    const int leader = __builtin_ctzll(bal);
                    if (lane == leader) base = atomicAdd(&ncand, __popcll(bal));
                    base = __shfl(base, leader, 64);
                }
                const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
                if (in) bkeys[base + __popcll(bal & lower)] = ordered_f64(v[u]);
            }
        }
        __syncthreads();
        const int nb = s_nb, kb = K - s_above;  // the kb-th largest of the bucket's nb keys
        if (nb <= IX_SEL_THREADS) {
            // few candidates: each thread counts the candidates above and equal to its own; the one with
            // (above < kb <= above + equal) is the K-th largest key
            if (tid < nb) {
                const uint64_t mk = bkeys[tid];
                int gt = 0, eq = 0;
                for (int j = 0; j < nb; j++) {
                    const uint64_t o = bkeys[j];
                    gt += o > mk;
                    eq += o == mk;
                }
                if (gt < kb && kb <= gt + eq) {  // every thread holding this key writes the same values
                    st.v = mk;
                    st.need = kb - gt;
                    st.eq = eq;
                }
            }
            __syncthreads();
            s = st;
        } else {
            s = radix_kth_largest<IX_SEL_THREADS, 64>([&](int i) { return bkeys[i]; }, nb, kb, hist, &st, cand,
                                                      &ncand);
        }
    } else {
        s = radix_kth_largest<IX_SEL_THREADS, 64>(key, n, K, hist, &st, cand, &ncand);
    }
    uint64_t mine = 0;  // this thread's largest key not taken
    visit_topk<IX_SEL_THREADS>(key, n, s, scan, [&](int i, int rank) { out[rank] = i; },
                               [&](int, uint64_t ki) { mine = ki > mine ? ki : mine; });
    block_max_u64(mine, &below);
    __syncthreads();
    if (tid == 0 && gap)
        gap[t] = s.eq > s.need ? 0.0 : from_ordered_f64(s.v) - from_ordered_f64(below);
}

// scores [T][S], then the scoring workgroups' ranges [T][at most ceil(S / IX_KEYS)][2]
size_t index_workspace_bytes(int T, int S) {
    return (size_t)T * (size_t)S * sizeof(double) + (size_t)T * (size_t)((S + IX_KEYS - 1) / IX_KEYS) * 16;
}

const char *index_unsupported(int T, int S, int H, int D) {
    if ((long)S * D >= kMaxDescBytes) return "the keys (S*D bytes) exceed 2^31 bytes";
    if ((long)T * H * D >= kMaxDescBytes) return "the queries (T*H*D bytes) exceed 2^31 bytes";
    return nullptr;
}

hipError_t launch_index_topk(const int8_t *q, const float *w, const int8_t *k, const float *kscale, int T, int S,
                             int H, int D, int K, int pos0, int32_t *top, double *gap, void *ws,
                             hipStream_t stream) {
    double *scores = (double *)ws;
    double *range = scores + (long)T * S;
    int nbx = 0;  // scoring workgroups along the keys
    // key blocks up to the last query's position
    long vis = (long)pos0 + T;
    if (vis > S) vis = S;
    if (vis > 0) {
        // key blocks per workgroup: one for a few queries (every CU streams a share of the keys), more when many
        // query groups each read the keys (the group's query rows then serve more keys)
        const int groups = (T + IX_QB - 1) / IX_QB;
        const int nkb = groups >= 16 ? 8 : 1;
        const long blocks = (vis + IX_KEYS - 1) / IX_KEYS;
        nbx = (int)((blocks + nkb - 1) / nkb);
        const dim3 grid((unsigned)nbx, (unsigned)groups);
        const size_t lds = (size_t)IX_QB * H * (D + IX_QPAD);
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute((const void *)index_score_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(index_score_kernel, grid, dim3(IX_WAVES * 64), lds, stream, q, w, k, kscale, T, S, H, D,
                           pos0, nkb, scores, range);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(index_select_kernel, dim3(T), dim3(IX_SEL_THREADS), 0, stream, scores, S, K, pos0, top, gap,
                       range, nbx);
    return hipGetLastError();
}

}  // namespace moe
