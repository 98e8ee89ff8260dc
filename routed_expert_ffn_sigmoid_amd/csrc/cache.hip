// Expert residency: a per-layer cache of HBM slots over a host tier that holds every expert.
//
// The pwwt.cn Colibri write-up keeps an expert cache of slots, each holding one expert's complete weights, and
// evicts by a weighted LRU: every slot keeps a last-use time and a hit count, and slots with few hits and an old
// last use go first (its section 3.1).  The GLM-5.2 page ("github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！")
// keeps one such cache per layer and reads the next experts while the current ones compute (section 三.5),
// reads each distinct expert of a batch once (三.4) and pins hot experts in the faster tier (五).
//
// Here one step is one layer call.  Its requests are the batch union U (the permutation's list of used experts).
// Resident experts of U are hits (hit count + 1, last use = the step).  The missing ones, in ascending id, take
// the evictable slots in the order: empty (lower slot first), fewest hits, oldest last use, lower expert id (pure
// LRU: the same without the hits); slots of U and pinned slots (0 .. P-1) are not evictable.  A loaded slot
// starts at hit count 1.  All of it runs on the device, in one workgroup, from the device-resident list of used
// experts: no count goes to the host, and the copies that follow read the plan from device memory too.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int CP_THREADS = 1024;  // the planning workgroup: one thread per expert and per slot (E, S <= 1024)

// State layout (device bytes): int64 head[8] = {steps, hits, misses, evictions, unplaced, 0, 0, 0}, then int32
// slot_expert[S] (-1 empty), expert_slot[E] (-1 not resident), uint32 last_used[S], uint32 hits[S].
struct CacheView {
    long long *head;
    int *slot_expert, *expert_slot;
    unsigned *last_used, *hits;
};

__host__ __device__ inline CacheView cache_view(void *state, int E, int S) {
    CacheView v;
    uint8_t *p = (uint8_t *)state;
    v.head = (long long *)p;
    v.slot_expert = (int *)(p + 64);
    v.expert_slot = v.slot_expert + S;
    v.last_used = (unsigned *)(v.expert_slot + E);
    v.hits = v.last_used + S;
    return v;
}

size_t cache_state_bytes(int E, int S) { return 64 + 4 * ((size_t)3 * S + E); }

const int32_t *cache_slot_map(const void *state, int E, int S) {
    return cache_view(const_cast<void *>(state), E, S).expert_slot;
}

// Initial state: slot i < P holds pinned[i]; the pinned experts become the miss list (to be copied once).
__global__ __launch_bounds__(CP_THREADS) void cache_init_kernel(void *state, int E, int S, int P,
                                                               int32_t *__restrict__ miss, int32_t *__restrict__ n_miss) {
    const CacheView v = cache_view(state, E, S);
    const int tid = threadIdx.x;
    if (tid < 8) v.head[tid] = 0;
    for (int e = tid; e < E; e += CP_THREADS) v.expert_slot[e] = -1;
    __syncthreads();
    for (int s = tid; s < S; s += CP_THREADS) {
        const int e = s < P ? miss[s] : -1;  // the pinned ids, copied into the miss list by the host
        v.slot_expert[s] = e;
        v.last_used[s] = 0;
        v.hits[s] = 0;
        if (e >= 0) v.expert_slot[e] = s;
    }
    __syncthreads();
    for (int i = P + tid; i < E; i += CP_THREADS) miss[i] = -1;
    if (tid == 0) *n_miss = P;
}

// Exclusive scan of one flag per thread over the workgroup, in thread order; *total = the number of flags.
__device__ int block_scan_flag(bool f, int *wsum, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint64_t b = __ballot(f);
    const int before_in_wave = __popcll(b & (lane == 0 ? 0ull : (~0ull >> (64 - lane))));
    __syncthreads();  // wsum is reused
    if (lane == 0) wsum[wv] = __popcll(b);
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < CP_THREADS / 64; w++) {
        const int c = wsum[w];
        if (w < wv) before += c;
        all += c;
    }
    *total = all;
    return before + before_in_wave;
}

// One step: hit and miss lists (ascending expert id, -1 past their counts, E entries each), state updated.  The
// slots' state is worked on in LDS and written back at the end.
__global__ __launch_bounds__(CP_THREADS) void cache_plan_kernel(void *state, int E, int S, int P, int policy,
                                                               const int32_t *__restrict__ uniq,
                                                               const int32_t *__restrict__ n_uniq,
                                                               int32_t *__restrict__ hit, int32_t *__restrict__ n_hit,
                                                               int32_t *__restrict__ miss,
                                                               int32_t *__restrict__ n_miss) {
    __shared__ unsigned char req[1024];          // expert requested in this step
    __shared__ int l_expert[1024];               // slot -> expert
    __shared__ unsigned l_last[1024], l_hits[1024];
    __shared__ unsigned long long key_hi[1024];  // per slot: (hits, last use) of an occupied slot
    __shared__ int key_lo[1024];                 // per slot: expert id, or the slot for an empty one
    __shared__ unsigned char key_cls[1024];      // 0 empty, 1 occupied, 2 not evictable
    __shared__ int l_miss[1024];
    __shared__ int wsum[CP_THREADS / 64];
    __shared__ int s_nu;
    const CacheView v = cache_view(state, E, S);
    const int tid = threadIdx.x;
    const long long now = v.head[0] + 1;
    if (tid == 0) {
        int nu = n_uniq[0];
        if (nu < 0) {  // invalid ids in the routing: the valid experts are the non-negative prefix of uniq
            nu = 0;
            while (nu < E && uniq[nu] >= 0) nu++;
        }
        s_nu = nu < E ? nu : E;
    }
    for (int e = tid; e < E; e += CP_THREADS) req[e] = 0;
    const int s = tid;  // slot of this thread (S <= CP_THREADS)
    if (s < S) {
        const int se = v.slot_expert[s];
        l_expert[s] = se >= 0 && se < E ? se : -1;
        l_last[s] = v.last_used[s];
        l_hits[s] = v.hits[s];
    }
    __syncthreads();
    const int nu = s_nu;
    for (int i = tid; i < nu; i += CP_THREADS) {
        const int e = uniq[i];
        if (e >= 0 && e < E) req[e] = 1;
    }
    __syncthreads();
    // ---- hits and misses, thread e = expert e (E <= CP_THREADS)
    const int e = tid;
    int es = -1;
    bool is_hit = false, is_miss = false;
    if (e < E && req[e]) {
        es = v.expert_slot[e];
        is_hit = es >= 0 && es < S && l_expert[es] == e;
        is_miss = !is_hit;
    }
    int nh, nm;
    const int ph = block_scan_flag(is_hit, wsum, &nh);
    const int pm = block_scan_flag(is_miss, wsum, &nm);
    if (is_hit) {
        hit[ph] = e;
        l_hits[es] += 1u;
        l_last[es] = (unsigned)now;
    }
    if (is_miss) l_miss[pm] = e;
    __syncthreads();
    // ---- victim order of the slots, thread s = slot s
    if (s < S) {
        const int se = l_expert[s];
        if (s < P || (se >= 0 && req[se])) {
            key_cls[s] = 2;
        } else if (se < 0) {
            key_cls[s] = 0;
            key_hi[s] = 0;
            key_lo[s] = s;
        } else {
            key_cls[s] = 1;
            key_hi[s] = ((unsigned long long)(policy == 0 ? l_hits[s] : 0u) << 32) | l_last[s];
            key_lo[s] = se;
        }
    }
    __syncthreads();
    // rank of slot s among the evictable slots (keys are distinct: (0, slot) or (1, ..., expert))
    int rank = -1;
    if (s < S && key_cls[s] < 2) {
        const int c = key_cls[s];
        const unsigned long long kh = key_hi[s];
        const int kl = key_lo[s];
        rank = 0;
        for (int t = 0; t < S; t++) {
            const int ct = key_cls[t];
            if (ct == 2 || t == s) continue;
            rank += ct != c ? ct < c : (key_hi[t] != kh ? key_hi[t] < kh : key_lo[t] < kl);
        }
    }
    int nev;  // evictable slots
    block_scan_flag(rank >= 0, wsum, &nev);
    const int placed = nm < nev ? nm : nev;
    bool evicted = false;
    if (rank >= 0 && rank < placed) {
        const int ne = l_miss[rank];  // the rank-th miss in ascending id
        const int old = l_expert[s];
        if (old >= 0) {
            v.expert_slot[old] = -1;  // not requested in this step, so no miss writes this entry
            evicted = true;
        }
        l_expert[s] = ne;
        v.expert_slot[ne] = s;
        l_hits[s] = 1u;
        l_last[s] = (unsigned)now;
    }
    int nevict;
    block_scan_flag(evicted, wsum, &nevict);  // (its barriers also order the LDS updates above)
    if (s < S) {
        v.slot_expert[s] = l_expert[s];
        v.last_used[s] = l_last[s];
        v.hits[s] = l_hits[s];
    }
    // lists past their counts hold -1 (the misses that found no slot, beyond `placed`, too)
    for (int i = tid; i < E; i += CP_THREADS) {
        if (i >= nh) hit[i] = -1;
        miss[i] = i < placed ? l_miss[i] : -1;
    }
    if (tid == 0) {
        *n_hit = nh;
        *n_miss = placed;
        v.head[0] = now;
        v.head[1] += nh;
        v.head[2] += placed;
        v.head[3] += nevict;
        v.head[4] += nm - placed;
    }
}

// Copies the missed experts' weights (nine tensors each) from the host tier to their slots.  Work unit: 16 KB of
// one tensor of one expert (256 threads x 4 x 16 bytes, four loads in flight per thread), dealt round-robin to
// the workgroups so that neighbouring workgroups stream neighbouring bytes.
constexpr int CF_THREADS = 256;
constexpr int CF_UNROLL = 4;
constexpr int CF_CHUNK = CF_THREADS * CF_UNROLL * 16;

struct FetchArgs {
    const uint8_t *src[9];  // device view of the host tier, tensor j of expert e at src[j] + e * bytes[j]
    uint8_t *dst[9];        // the slots, tensor j of slot s at dst[j] + s * bytes[j]
    long bytes[9];          // per expert
    int cfirst[10];         // first unit of tensor j within an expert; cfirst[9] = units per expert
};

__global__ __launch_bounds__(CF_THREADS) void cache_fetch_kernel(FetchArgs a, const int32_t *__restrict__ miss,
                                                                const int32_t *__restrict__ n_miss,
                                                                const int32_t *__restrict__ slot_of, int E, int S) {
    int nm = n_miss[0];
    nm = nm < 0 ? 0 : (nm > E ? E : nm);
    const int per = a.cfirst[9];
    const long units = (long)nm * per;
    for (long u = blockIdx.x; u < units; u += gridDim.x) {
        const int i = (int)(u / per), c = (int)(u % per);
        const int e = miss[i];
        if (e < 0 || e >= E) continue;
        const int s = slot_of[e];
        if (s < 0 || s >= S) continue;
        // tensor of unit c (unrolled selects: constant offsets into the argument block)
        const uint8_t *sb = a.src[0];
        uint8_t *db = a.dst[0];
        long nb = a.bytes[0];
        int c0 = 0;
#pragma unroll
        for (int q = 1; q < 9; q++)
            if (c >= a.cfirst[q]) {
                sb = a.src[q];
                db = a.dst[q];
                nb = a.bytes[q];
                c0 = a.cfirst[q];
            }
        const long off = (long)(c - c0) * CF_CHUNK;
        const uint4 *src = (const uint4 *)(sb + (long)e * nb + off);
        uint4 *dst = (uint4 *)(db + (long)s * nb + off);
        const long n16 = (nb - off) / 16;  // 16-byte words left in the tensor from this unit
        uint4 r[CF_UNROLL];
#pragma unroll
        for (int q = 0; q < CF_UNROLL; q++) {
            const long w = threadIdx.x + (long)q * CF_THREADS;
            if (w < n16) r[q] = src[w];
        }
#pragma unroll
        for (int q = 0; q < CF_UNROLL; q++) {
            const long w = threadIdx.x + (long)q * CF_THREADS;
            if (w < n16) dst[w] = r[q];
        }
    }
}

hipError_t launch_cache_init(void *state, int E, int S, int P, int32_t *miss, int32_t *n_miss, hipStream_t stream) {
    hipLaunchKernelGGL(cache_init_kernel, dim3(1), dim3(CP_THREADS), 0, stream, state, E, S, P, miss, n_miss);
    return hipGetLastError();
}

hipError_t launch_cache_plan(void *state, int E, int S, int P, int policy, const int32_t *uniq,
                             const int32_t *n_uniq, int32_t *hit, int32_t *n_hit, int32_t *miss, int32_t *n_miss,
                             hipStream_t stream) {
    hipLaunchKernelGGL(cache_plan_kernel, dim3(1), dim3(CP_THREADS), 0, stream, state, E, S, P, policy, uniq, n_uniq,
                       hit, n_hit, miss, n_miss);
    return hipGetLastError();
}

hipError_t launch_cache_fetch(const QW &src, const QW &dst, const long bytes[9], const int32_t *miss,
                              const int32_t *n_miss, const void *state, int E, int S, int workgroups,
                              hipStream_t stream) {
    FetchArgs a;
    const void *sp[9] = {src.qg, src.qu, src.qd, src.sg, src.su, src.sd, src.zg, src.zu, src.zd};
    const void *dp[9] = {dst.qg, dst.qu, dst.qd, dst.sg, dst.su, dst.sd, dst.zg, dst.zu, dst.zd};
    int c = 0;
    for (int j = 0; j < 9; j++) {
        a.src[j] = (const uint8_t *)sp[j];
        a.dst[j] = (uint8_t *)const_cast<void *>(dp[j]);
        a.bytes[j] = bytes[j];
        a.cfirst[j] = c;
        c += (int)((bytes[j] + CF_CHUNK - 1) / CF_CHUNK);
    }
    a.cfirst[9] = c;
    hipLaunchKernelGGL(cache_fetch_kernel, dim3(workgroups), dim3(CF_THREADS), 0, stream, a, miss, n_miss,
                       cache_slot_map(state, E, S), E, S);
    return hipGetLastError();
}

}  // namespace moe
