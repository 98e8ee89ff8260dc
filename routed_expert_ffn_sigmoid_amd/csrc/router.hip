// Sigmoid + bias top-k router ("25GB 内存跑 744B GLM-5.2 模型" page, sections 三.1 and 四.3).
//
// Two kernels:
//   logits  z = x . W_r in fp64, split over blocks of d rows (and, for few
//           tokens, of 32 experts) so that even one token spreads the W_r read
//           over the whole chip.  T <= 4: 1024-thread workgroups each stream a
//           block of at least 8 KB of W_r once for all tokens, at most 32 row
//           blocks so the partials are few; larger T: fp64 matrix cores on tiles
//           of 64 tokens x 256 experts.  Partial sums per block go to the
//           workspace (no atomics: the reduction order is fixed).
//   select  one workgroup per token (for one token whose permutation is asked
//           for, that workgroup also sorts): adds the partials in a fixed order,
//           takes the sigmoid, adds the bias, and picks the top k+1 by repeated
//           wave-wide argmax with ties to the lower id.  The selection's device
//           code (select_dev.h) also serves the decode gate/up launch that
//           routes one token itself.
// Products of an fp32/bf16 activation and an fp32 weight are exact in fp64,
// so the logit differs from any other fp64 summation order only by fp64
// rounding; the choice of experts therefore matches a plain fp64 evaluation
// unless two selection scores agree to ~1e-16.
#include "common.h"
#include "kernels.h"
#include "permute_dev.h"
#include "select_dev.h"
#include "topk.h"

#include <type_traits>

namespace moe {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int RM_TT = 64;           // tokens per workgroup tile
constexpr int RM_TE = 256;          // experts per workgroup tile (4 wavefronts x 64)
constexpr int RM_KS = 16;           // d rows per LDS stage
constexpr int RM_XP = RM_TT + 16;   // LDS row pitch of the activation tile, floats
constexpr int RM_WP = RM_TE + 16;   // LDS row pitch of the W_r tile, floats
constexpr int RM_MAXSPLIT = 64;

template <int ACT>
__device__ __forceinline__ float load_act(const void *x, long i) {
    if (ACT == 0) return ((const float *)x)[i];
    return bf16_to_f32(((const uint16_t *)x)[i]);
}

// Logits on the fp64 matrix cores (v_mfma_f64_16x16x4f64; lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16], and D[4 i + l / 16][l % 16] in register i).  grid: (ceil(E/256), ceil(T/64), nsplit),
// block 256: wavefront w owns experts 64 w .. 64 w + 63 of the tile for all 64 tokens, as 4 x 4 blocks of
// 16 x 16.  The d rows [s*chunk, min(d,(s+1)*chunk)) go through a double-buffered LDS stage of 16 rows
// (fp32: both operands convert to fp64 exactly).  part[s][t][e] = the partial dot product.
template <int ACT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ x,
                                                            const float *__restrict__ Wr, int T, int d, int E,
                                                            int chunk, double *__restrict__ part) {
    __shared__ float xs[2][RM_KS][RM_XP];  // [stage][row][token]
    __shared__ float wsm[2][RM_KS][RM_WP]; // [stage][row][expert]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e0 = blockIdx.x * RM_TE, t0 = blockIdx.y * RM_TT;
    const int i_begin = blockIdx.z * chunk;
    const int i_end = min(d, i_begin + chunk);
    const int nsteps = (i_end - i_begin + RM_KS - 1) / RM_KS;
    // staging map: activations of token tid / 4, rows 4 (tid % 4) .. + 3; W_r row tid / 16, experts
    // 16 (tid % 16) .. + 15
    const int xt = tid >> 2, xk = 4 * (tid & 3);
    const int wk = tid >> 4, we = 16 * (tid & 15);
    const bool vec4 = (E & 3) == 0;
    float xr[4], wr[16];
    auto load = [&](int step) {
        const int i = i_begin + step * RM_KS;
        const int t = t0 + xt;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int k = i + xk + u;
            xr[u] = (t < T && k < i_end) ? load_act<ACT>(x, (long)t * d + k) : 0.f;
        }
        const int k = i + wk;
        const float *row = Wr + (long)k * E + e0 + we;
        if (vec4 && k < i_end && e0 + we + 16 <= E) {
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float4 q = ((const float4 *)row)[v];
                wr[4 * v] = q.x;
                wr[4 * v + 1] = q.y;
                wr[4 * v + 2] = q.z;
                wr[4 * v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; v++) wr[v] = (k < i_end && e0 + we + v < E) ? row[v] : 0.f;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 4; u++) xs[buf][xk + u][xt] = xr[u];
#pragma unroll
        for (int v = 0; v < 4; v++)
            *(float4 *)&wsm[buf][wk][we + 4 * v] = make_float4(wr[4 * v], wr[4 * v + 1], wr[4 * v + 2], wr[4 * v + 3]);
    };

    f64x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = (f64x4_t){0.0, 0.0, 0.0, 0.0};

    const int kr = lane >> 4, cl = lane & 15;
    load(0);
    store(0);
    __syncthreads();
    for (int step = 0; step < nsteps; step++) {
        const int buf = step & 1;
        if (step + 1 < nsteps) load(step + 1);
#pragma unroll
        for (int q = 0; q < RM_KS / 4; q++) {
            double a[4], b[4];
#pragma unroll
            for (int tb = 0; tb < 4; tb++) a[tb] = (double)xs[buf][4 * q + kr][16 * tb + cl];
#pragma unroll
            for (int eb = 0; eb < 4; eb++) b[eb] = (double)wsm[buf][4 * q + kr][64 * wv + 16 * eb + cl];
#pragma unroll
            for (int tb = 0; tb < 4; tb++)
#pragma unroll
                for (int eb = 0; eb < 4; eb++)
                    acc[tb][eb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[tb], b[eb], acc[tb][eb], 0, 0, 0);
        }
        if (step + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }
    double *out = part + (long)blockIdx.z * T * E;
#pragma unroll
    for (int tb = 0; tb < 4; tb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + 16 * tb + 4 * i + kr;
            if (t >= T) continue;
#pragma unroll
            for (int eb = 0; eb < 4; eb++) {
                const int e = e0 + 64 * wv + 16 * eb + cl;
                if (e < E) out[(long)t * E + e] = acc[tb][eb][i];
            }
        }
}

// Small-T logits: 1024-thread workgroups each stream a block of W_r (a range of rows, and of the experts a
// block of at most RSK_EB columns) once for all T <= RS_TMAX tokens.  Thread (row group rg, expert quad q)
// handles rows rg, rg+R, ... (at most RSK_MAXR) of the block for the block's experts 4q..4q+3; all of its
// W_r loads are issued before the block's activations are staged in LDS.  Splitting the experts as well as
// the rows spreads the read over about RSK_WGS workgroups of at least RSK_MIN_BYTES each (one CU streams
// only about 20 GB/s), while the row splits stay at most RSK_SPLITS, so the select kernel reads few
// partials.
constexpr int RS_TMAX = 4;
constexpr int RSK_THREADS = 1024;
constexpr int RSK_SPLITS = 32;
constexpr int RSK_MIN_BYTES = 8 * 1024;   // W_r bytes per workgroup at least
constexpr int RSK_EB = 32;                // experts per workgroup column block
constexpr int RSK_WGS = 256;              // workgroups aimed at
constexpr int RSK_MAXR = 12;              // W_r rows per thread (1024 threads: 128 VGPRs each)
constexpr int RSK_MAX_ROWS = 2048;        // rows per block (LDS holds RS_TMAX x rows activations)
// The selection kernel's permutation (moe_route_permute at T <= RS_FUSE_TMAX): with perm set, one workgroup selects
// every token and sorts the assignments.  The tokens' selections then run one after another, each adding about the
// cost of a separate sort launch, so only the single-token call is fused.
constexpr int RS_FUSE_TMAX = 1;
struct FusedPerm {
    int32_t *counts, *offsets, *perm, *inv, *uniq, *n_uniq;  // perm = nullptr: no permutation
};

// One workgroup (1024 threads) per token.  Thread (e, g) sums the splits s = g, g+4, ... of expert e
// (fixed order); thread (e, 0) adds the four groups in order and takes sigmoid and bias (one expert per
// thread, so the code holds one copy of exp and the sigmoids run in parallel); then the first wavefront
// picks the top k+1.  Each lane holds EJ experts (e = lane + 64 j), sorts them once, and exposes its
// best unchosen one; each round is one wave-wide argmax and the winning lane moves to its next.
constexpr int RSEL_THREADS = 1024;

// mode 0: sigmoid scores, selection by s + bias.  mode 1: softmax gate, selection by the logits and weights
// lambda * exp(z_j - z_max) / sum over the selected (the max-subtracted softmax renormalised over them).
// Token t's selection by a workgroup of RSEL_THREADS threads (all of them call it); zs: LDS of 4 E doubles.
// keys (optional, LDS or global): receives idx[t][0 .. k).
template <int EJ>
__device__ inline void select_token(const double *__restrict__ part, int nsplit, int T, int E, int k,
                                    const float *__restrict__ bias, float lambda, int mode, int t,
                                    int32_t *__restrict__ idx, float *__restrict__ w, double *__restrict__ gap,
                                    double *zs, int32_t *keys) {
    token_scores<RSEL_THREADS>(part, nsplit, T, E, bias, mode, t, zs);
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    int my_id;
    float my_w;
    double g;
    topk_pick<EJ>(zs, E, k, lambda, mode, my_id, my_w, g);
    if (lane == 0 && gap) gap[t] = g;
    if (lane < k) {
        idx[(long)t * k + lane] = my_id;
        w[(long)t * k + lane] = my_w;
        if (keys) keys[t * k + lane] = my_id;
    }
}

// One workgroup per token; with F.perm set (T <= RS_FUSE_TMAX) one workgroup selects the T tokens one after the other
// and then sorts the assignments from LDS, so the permutation needs no launch of its own and no workgroup waits
// for another.
template <int EJ, int MODE>
__global__ __launch_bounds__(RSEL_THREADS) void router_select_kernel(const double *__restrict__ part, int nsplit,
                                                                     int T, int E, int k,
                                                                     const float *__restrict__ bias, float lambda,
                                                                     int32_t *__restrict__ idx,
                                                                     float *__restrict__ w,
                                                                     double *__restrict__ gap, FusedPerm F) {
    extern __shared__ double zs[];  // [4][E], then (with F.perm) the sort's LDS and the T k chosen ids
    if (!F.perm) {
        select_token<EJ>(part, nsplit, T, E, k, bias, lambda, MODE, blockIdx.x, idx, w, gap, zs, nullptr);
        return;
    }
    int32_t *psm = (int32_t *)(zs + 4 * E);
    int32_t *keys = psm + 18 * E + 1;
    for (int t = 0; t < T; t++) {
        select_token<EJ>(part, nsplit, T, E, k, bias, lambda, MODE, t, idx, w, gap, zs, keys);
        __syncthreads();  // zs is reused; the ids are complete
    }
    permute_block(keys, T * k, E, F.counts, F.offsets, F.perm, F.inv, F.uniq, F.n_uniq, psm);
}

template <int ACT>
__global__ __launch_bounds__(RSK_THREADS) void router_logits_skinny_kernel(const void *__restrict__ x,
                                                                           const float *__restrict__ Wr, int T,
                                                                           int d, int E, int rows,
                                                                           double *__restrict__ part) {
    __shared__ double red[RSK_THREADS / 64][256];
    __shared__ float xs[RS_TMAX * RSK_MAX_ROWS];  // [t][row in block], row pitch = rows
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tg = blockIdx.z * RS_TMAX, ng = min(RS_TMAX, T - tg);  // this workgroup's tokens tg .. tg + ng
    const int EB = E < RSK_EB ? E : RSK_EB, e0 = blockIdx.y * EB;  // this workgroup's experts
    const int nq = EB >> 2;            // expert quads: a power of two <= 8
    const int R = RSK_THREADS / nq;    // row groups (>= 16: every wave holds at least one)
    const int q = tid % nq, rg = tid / nq;
    const int i0 = blockIdx.x * rows, i1 = min(d, i0 + rows);
    const rsrc_t wsrc = make_rsrc(Wr, (uint32_t)((long)d * E * 4));
    const rsrc_t xsrc = make_rsrc(x, (uint32_t)((long)T * d * (ACT == 0 ? 4 : 2)));
    // activations first (few, branch-free), then every W_r row of this thread: waiting for the
    // activations does not wait for the weights
    constexpr int XPT = RS_TMAX * RSK_MAX_ROWS / RSK_THREADS;
    uint32_t xr[XPT];
#pragma unroll
    for (int c = 0; c < XPT; c++) {
        const int o = tid + c * RSK_THREADS;
        const int t = o / rows, i = i0 + o % rows;
        const uint32_t xo = (t < ng && i < i1) ? (uint32_t)(((long)(tg + t) * d + i) * (ACT == 0 ? 4 : 2)) : kOOB;
        xr[c] = ACT == 0 ? buf_load4(xsrc, xo) : (uint32_t)buf_load2(xsrc, xo);
    }
    uint4 w[RSK_MAXR];
#pragma unroll
    for (int u = 0; u < RSK_MAXR; u++) {
        const int i = i0 + rg + u * R;
        w[u] = buf_load16(wsrc, i < i1 ? (uint32_t)(((long)i * E + e0 + 4 * q) * 4) : kOOB);
    }
#pragma unroll
    for (int c = 0; c < XPT; c++)  // unconditional: entries past T*rows are zeros nobody reads
        xs[tid + c * RSK_THREADS] = ACT == 0 ? __uint_as_float(xr[c]) : bf16_to_f32((uint16_t)xr[c]);
    __syncthreads();
    double acc[RS_TMAX][4];
#pragma unroll
    for (int t = 0; t < RS_TMAX; t++)
#pragma unroll
        for (int v = 0; v < 4; v++) acc[t][v] = 0.0;
#pragma unroll
    for (int u = 0; u < RSK_MAXR; u++) {
        const int li = rg + u * R;  // row inside the block (the weights are zero past its end)
        if (li < rows) {
            const double w4[4] = {(double)__uint_as_float(w[u].x), (double)__uint_as_float(w[u].y),
                                  (double)__uint_as_float(w[u].z), (double)__uint_as_float(w[u].w)};
#pragma unroll
            for (int t = 0; t < RS_TMAX; t++) {
                const double xd = (double)xs[t * rows + li];
#pragma unroll
                for (int v = 0; v < 4; v++) acc[t][v] = fma(xd, w4[v], acc[t][v]);
            }
        }
    }
    // fixed-order reduction over row groups: the lanes holding the same quad inside a wave, then the 16
    // waves in order, one token at a time
    for (int t = 0; t < ng; t++) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const double a = sum_congruent(acc[t][v], nq);
            if (lane < nq) red[wv][lane * 4 + v] = a;
        }
        __syncthreads();
        if (tid < EB) {
            double z = 0.0;
            for (int w2 = 0; w2 < RSK_THREADS / 64; w2++) z += red[w2][tid];
            part[((long)blockIdx.x * T + tg + t) * E + e0 + tid] = z;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------- router variants

// Logit of (t, e) from the split partials, in the order the select kernel adds them: splits g, g + 4, g + 8, ...
// summed for each g in 0..3, then the four sums left to right.
__device__ __forceinline__ double logit_of(const double *part, int nsplit, int T, int E, int t, int e) {
    double zg[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int g = 0; g < 4; g++)
        for (int sp = g; sp < nsplit; sp += 4) zg[g] += part[((long)sp * T + t) * E + e];
    return ((zg[0] + zg[1]) + zg[2]) + zg[3];
}

// Expert choice, step 1: pT[e][t] = softmax over the experts of token t (E <= 32), the maximum subtracted and the
// sum taken over e ascending.  One thread per token.
__global__ __launch_bounds__(256) void ec_softmax_kernel(const double *__restrict__ part, int nsplit, int T, int E,
                                                         double *__restrict__ pT) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    double z[32];
    double m = -INFINITY;
    for (int e = 0; e < E; e++) {
        z[e] = logit_of(part, nsplit, T, E, t, e);
        m = fmax(m, z[e]);
    }
    double sum = 0.0;
    for (int e = 0; e < E; e++) sum += exp(z[e] - m);
    for (int e = 0; e < E; e++) pT[(long)e * T + t] = exp(z[e] - m) / sum;
}

// Expert choice, step 2: one workgroup per expert takes the C tokens of largest p (equal p by lower token) by an
// exact radix selection over the bit patterns of the fp64 probabilities (non-negative: they order as the values).
// Writes column e of idx [T][E] (e or -1) and w (lambda p or 0), and gap[e] (p of the C-th minus the (C+1)-th).
constexpr int EC_THREADS = 1024;

__global__ __launch_bounds__(EC_THREADS) void ec_select_kernel(const double *__restrict__ pT, int T, int E, int C,
                                                               float lambda, int32_t *__restrict__ idx,
                                                               float *__restrict__ w, double *__restrict__ gap) {
    __shared__ int hist[256];
    __shared__ int scan[EC_THREADS / 64 + 1];
    __shared__ TopkState st;
    __shared__ uint64_t cand[TOPK_CAND];
    __shared__ int ncand;
    __shared__ unsigned long long below;  // largest key not chosen
    const int e = blockIdx.x;
    const double *p = pT + (long)e * T;
    auto key = [&](int i) { return (uint64_t)__double_as_longlong(p[i]); };
    if (threadIdx.x == 0) below = 0ull;
    const TopkState s = radix_kth_largest<EC_THREADS, 64>(key, T, C, hist, &st, cand, &ncand);
    uint64_t mine = 0;  // this thread's largest key not taken
    visit_topk<EC_THREADS>(
        key, T, s, scan,
        [&](int i, int) {
            idx[(long)i * E + e] = e;
            w[(long)i * E + e] = (float)((double)lambda * p[i]);
        },
        [&](int i, uint64_t ki) {
            idx[(long)i * E + e] = -1;
            w[(long)i * E + e] = 0.f;
            mine = ki > mine ? ki : mine;
        });
    block_max_u64(mine, &below);
    __syncthreads();
    if (threadIdx.x == 0 && gap)
        gap[e] = C >= T ? INFINITY : (s.eq > s.need ? 0.0 : __longlong_as_double((long long)s.v) -
                                                              __longlong_as_double((long long)below));
}

// Capacity, step 1: the assignments in (choice, token) order, idxT[j * T + t] = idx[t * k + j].
__global__ __launch_bounds__(256) void cap_transpose_kernel(const int32_t *__restrict__ idx, int T, int k,
                                                            int32_t *__restrict__ idxT) {
    const long a = (long)blockIdx.x * 256 + threadIdx.x;
    if (a >= (long)T * k) return;
    const int t = (int)(a / k), j = (int)(a % k);
    idxT[(long)j * T + t] = idx[a];
}

// Capacity, step 3: after the stable counting sort of idxT, an assignment's place within its expert is its rank in
// (choice, token) order; places C and beyond become empty slots.
__global__ __launch_bounds__(256) void cap_drop_kernel(int32_t *__restrict__ idx, int T, int k, int C,
                                                       const int32_t *__restrict__ invT,
                                                       const int32_t *__restrict__ offT) {
    const long a = (long)blockIdx.x * 256 + threadIdx.x;
    if (a >= (long)T * k) return;
    const int e = idx[a];
    if (e < 0) return;
    const int t = (int)(a / k), j = (int)(a % k);
    if (invT[(long)j * T + t] - offT[e] >= C) idx[a] = -1;
}

static bool skinny_fits(int E) { return E >= 4 && E <= 256 && (E & (E - 1)) == 0; }

// The skinny kernel takes T <= RS_TMAX; in the batch-invariant mode it takes every T (in groups of RS_TMAX tokens,
// each group reading W_r again, mostly from the caches), so that a token's sums never depend on T.
static bool use_skinny(int T, int E, bool inv) { return (inv || T <= RS_TMAX) && skinny_fits(E); }

static int skinny_eb(int E) { return E < RSK_EB ? E : RSK_EB; }

static int skinny_rows(int d, int E) {
    const int eb = skinny_eb(E), neb = E / eb;
    long nsplit = (RSK_WGS + neb - 1) / neb;                // about RSK_WGS workgroups in all
    const long by_bytes = (long)d * eb * 4 / RSK_MIN_BYTES;  // each with at least RSK_MIN_BYTES
    if (nsplit > by_bytes) nsplit = by_bytes;
    if (nsplit > RSK_SPLITS) nsplit = RSK_SPLITS;
    if (nsplit < 1) nsplit = 1;
    long rows = (d + nsplit - 1) / nsplit;
    const long cap = (long)RSK_MAXR * (RSK_THREADS / (eb / 4));  // rows the threads of a block can hold
    if (rows > cap) rows = cap;
    if (rows > RSK_MAX_ROWS) rows = RSK_MAX_ROWS;
    return (int)rows;
}

int router_nsplit(int T, int d, int E, bool inv) {
    if (use_skinny(T, E, inv)) {
        const int rows = skinny_rows(d, E);
        return (d + rows - 1) / rows;
    }
    // about two workgroups per CU, at least 4 stages of rows per split; the batch-invariant mode counts one
    // token tile whatever T is, so the split (and each token's order of sums) depends on (d, E) alone
    const int gx = (E + RM_TE - 1) / RM_TE, gy = inv ? 1 : (T + RM_TT - 1) / RM_TT;
    const int ksteps = (d + RM_KS - 1) / RM_KS;
    int want = (512 + gx * gy - 1) / (gx * gy);
    if (want > ksteps / 4) want = ksteps / 4;
    if (want > RM_MAXSPLIT) want = RM_MAXSPLIT;
    if (want < 1) want = 1;
    const int chunk = ((ksteps + want - 1) / want) * RM_KS;
    return (d + chunk - 1) / chunk;
}

const char *router_unsupported(int T, int d, int E, int act, bool inv) {
    if ((long)T * d * (act == 0 ? 4 : 2) >= kMaxDescBytes) return "x exceeds 2^31 bytes";
    if ((long)d * E * 4 >= kMaxDescBytes) return "W_r exceeds 2^31 bytes";
    if (T > 0 && (long)router_nsplit(T, d, E, inv) * T * E * 8 >= kMaxDescBytes)
        return "the router's fp64 partial sums (splits x T x E) exceed 2^31 bytes";
    return nullptr;
}

static size_t r_al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace after the partials: the capacity step's transposed assignments, its counting sort (counts, offsets,
// perm, inv, uniq, n_uniq) and that sort's own workspace; or expert choice's probabilities pT [E][T].
static size_t variant_bytes(int T, int E, int k, int router, bool capacity) {
    const size_t A = (size_t)T * k;
    if (router == 2) return r_al256((size_t)E * T * sizeof(double));
    if (!capacity) return 0;
    return r_al256(A * 4) * 3 + r_al256((size_t)E * 4) * 2 + r_al256((size_t)(E + 1) * 4) + r_al256(4) +
           r_al256(permute_workspace_bytes((int)A, E));
}

size_t router_workspace_bytes(int T, int d, int E, bool inv, int k, int router, bool capacity) {
    if (T <= 0) return 0;
    return r_al256((size_t)router_nsplit(T, d, E, inv) * (size_t)T * (size_t)E * sizeof(double)) +
           variant_bytes(T, E, k, router, capacity);
}

bool router_fused(int T, int E, bool inv, int router, int C) {
    (void)E;
    (void)inv;
    return T >= 1 && T <= RS_FUSE_TMAX && router != 2 && C <= 0;
}

size_t router_partials_bytes(int T, int d, int E, bool inv) {
    return r_al256((size_t)router_nsplit(T, d, E, inv) * (size_t)T * (size_t)E * sizeof(double));
}

hipError_t launch_router_logits(int act, const void *x, const float *Wr, int T, int d, int E, bool inv, double *part,
                                int *nsplit_out, hipStream_t stream) {
    int nsplit;
    if (use_skinny(T, E, inv)) {
        const int rows = skinny_rows(d, E);
        nsplit = (d + rows - 1) / rows;
        const dim3 grid(nsplit, E / skinny_eb(E), (T + RS_TMAX - 1) / RS_TMAX);
        if (act == 0)
            hipLaunchKernelGGL(router_logits_skinny_kernel<0>, grid, dim3(RSK_THREADS), 0, stream, x, Wr, T, d, E,
                               rows, part);
        else
            hipLaunchKernelGGL(router_logits_skinny_kernel<1>, grid, dim3(RSK_THREADS), 0, stream, x, Wr, T, d, E,
                               rows, part);
    } else {
        nsplit = router_nsplit(T, d, E, inv);
        const int chunk = (((d + RM_KS - 1) / RM_KS + nsplit - 1) / nsplit) * RM_KS;
        dim3 grid((E + RM_TE - 1) / RM_TE, (T + RM_TT - 1) / RM_TT, nsplit);
        if (act == 0)
            hipLaunchKernelGGL(router_logits_kernel<0>, grid, dim3(256), 0, stream, x, Wr, T, d, E, chunk, part);
        else
            hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, stream, x, Wr, T, d, E, chunk, part);
    }
    *nsplit_out = nsplit;
    return hipGetLastError();
}

hipError_t launch_router(int act, const void *x, const float *Wr, const float *bias, int T, int d, int E, int k,
                         float lambda, int32_t *idx, float *w, double *gap, void *ws, bool inv, int router, int C,
                         hipStream_t stream, const PermOut *po) {
    double *part = (double *)ws;
    char *vws = (char *)ws + router_partials_bytes(T, d, E, inv);
    int nsplit = 0;
    hipError_t err = launch_router_logits(act, x, Wr, T, d, E, inv, part, &nsplit, stream);
    if (err != hipSuccess) return err;
    if (router == 2) {
        // expert choice: per-token softmax, then per expert the C tokens of largest probability
        double *pT = (double *)vws;
        hipLaunchKernelGGL(ec_softmax_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, part, nsplit, T, E, pT);
        hipLaunchKernelGGL(ec_select_kernel, dim3(E), dim3(EC_THREADS), 0, stream, pT, T, E, C, lambda, idx, w, gap);
        return hipGetLastError();
    }
    const bool fuse = po && router_fused(T, E, inv, router, C);
    FusedPerm F{};
    size_t lds = 4 * E * sizeof(double);
    if (fuse) {
        F = FusedPerm{po->counts, po->offsets, po->perm, po->inv, po->uniq, po->n_uniq};
        lds += sizeof(int32_t) * ((size_t)18 * E + 1 + (size_t)T * k);
    }
    const dim3 sgrid(fuse ? 1 : T);
    auto select = [&](auto mode) {
        constexpr int M = decltype(mode)::value;
        if (E <= 64)
            hipLaunchKernelGGL((router_select_kernel<1, M>), sgrid, dim3(RSEL_THREADS), lds, stream, part, nsplit, T,
                               E, k, bias, lambda, idx, w, gap, F);
        else if (E <= 256)
            hipLaunchKernelGGL((router_select_kernel<4, M>), sgrid, dim3(RSEL_THREADS), lds, stream, part, nsplit, T,
                               E, k, bias, lambda, idx, w, gap, F);
        else
            hipLaunchKernelGGL((router_select_kernel<16, M>), sgrid, dim3(RSEL_THREADS), lds, stream, part, nsplit,
                               T, E, k, bias, lambda, idx, w, gap, F);
    };
    if (router == 1)
        select(std::integral_constant<int, 1>{});
    else
        select(std::integral_constant<int, 0>{});
    err = hipGetLastError();
    if (err != hipSuccess || C <= 0) return err;
    // capacity: rank every assignment within its expert in (choice, token) order by the stable counting sort of
    // the transposed assignments, then empty the slots ranked C and beyond
    const long A = (long)T * k;
    char *p = vws;
    auto take = [&](size_t b) {
        char *q = p;
        p += r_al256(b);
        return q;
    };
    int32_t *idxT = (int32_t *)take(A * 4), *permT = (int32_t *)take(A * 4), *invT = (int32_t *)take(A * 4);
    int32_t *cntT = (int32_t *)take((size_t)E * 4), *uniqT = (int32_t *)take((size_t)E * 4);
    int32_t *offT = (int32_t *)take((size_t)(E + 1) * 4), *nuT = (int32_t *)take(4);
    void *pws = take(permute_workspace_bytes((int)A, E));
    const unsigned g = (unsigned)((A + 255) / 256);
    hipLaunchKernelGGL(cap_transpose_kernel, dim3(g), dim3(256), 0, stream, idx, T, k, idxT);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = launch_permute(idxT, (int)A, E, cntT, offT, permT, invT, uniqT, nuT, pws, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(cap_drop_kernel, dim3(g), dim3(256), 0, stream, idx, T, k, C, invT, offT);
    return hipGetLastError();
}

}  // namespace moe
