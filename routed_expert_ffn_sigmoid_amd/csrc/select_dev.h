// Device code of the router's selection, shared by the router's kernels and the decode gate/up kernel that
// routes a single token for itself: fixed-order wave reductions, the wave-wide argmax with ties to the lower
// id, a token's scores from the split partial sums of its logits, and the top-k pick ("25GB 内存跑 744B
// GLM-5.2 模型" page, sections 三.1 and 四.3: sigmoid scores, selection by score plus bias, weights normalised
// over the chosen and scaled).
#pragma once

#include <math.h>

#include "common.h"

namespace moe {

// Sum of a over the lanes whose index is congruent to this lane's modulo nq (a power of two <= 64), every
// lane getting the result, in a fixed order: neighbours and pairs inside quads (DPP quad permutes), lanes 4
// and 8 apart inside rows of 16 (DPP row rotations), then the other row of each 32 and the other half of the
// wavefront (16- and 32-lane swaps).  All steps are register moves; the steps below nq are skipped.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double a) {
    const int2 b = __builtin_bit_cast(int2, a);
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_update_dpp(0, b.x, CTRL, 0xF, 0xF, false),
                                                __builtin_amdgcn_update_dpp(0, b.y, CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ double swap_add_f64(double a, bool sixteen) {
    const int2 b = __builtin_bit_cast(int2, a);
    int2 p, q;
    if (sixteen) {
        const auto x = __builtin_amdgcn_permlane16_swap((uint32_t)b.x, (uint32_t)b.x, false, false);
        const auto y = __builtin_amdgcn_permlane16_swap((uint32_t)b.y, (uint32_t)b.y, false, false);
        p = make_int2((int)x[0], (int)y[0]);
        q = make_int2((int)x[1], (int)y[1]);
    } else {
        const auto x = __builtin_amdgcn_permlane32_swap((uint32_t)b.x, (uint32_t)b.x, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap((uint32_t)b.y, (uint32_t)b.y, false, false);
        p = make_int2((int)x[0], (int)y[0]);
        q = make_int2((int)x[1], (int)y[1]);
    }
    // the two results hold this lane's value and its partner's, the lower row or half first
    return __builtin_bit_cast(double, p) + __builtin_bit_cast(double, q);
}
__device__ __forceinline__ double sum_congruent(double a, int nq) {
    if (nq <= 1) a += dpp_f64<0xB1>(a);   // quad_perm 1,0,3,2
    if (nq <= 2) a += dpp_f64<0x4E>(a);   // quad_perm 2,3,0,1
    if (nq <= 4) a += dpp_f64<0x124>(a);  // row_ror:4
    if (nq <= 8) a += dpp_f64<0x128>(a);  // row_ror:8
    if (nq <= 16) a = swap_add_f64(a, true);
    if (nq <= 32) a = swap_add_f64(a, false);
    return a;
}

// (v, id) is better than (v2, id2): larger score, then lower id
__device__ __forceinline__ bool better(double v, int id, double v2, int id2) {
    return v > v2 || (v == v2 && id < id2);
}

// One DPP step of a wave-wide argmax of (v, id): take the partner's pair when it is better.
// bound_ctrl off and old = own value: lanes without a partner keep what they have.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(double &v, int &id) {
    const int2 b = __builtin_bit_cast(int2, v);
    const int lo = __builtin_amdgcn_update_dpp(b.x, b.x, CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(b.y, b.y, CTRL, ROW_MASK, 0xF, false);
    const int oid = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
    const double ov = __builtin_bit_cast(double, make_int2(lo, hi));
    if (better(ov, oid, v, id)) {
        v = ov;
        id = oid;
    }
}

// Wave-wide argmax (larger v, then lower id); the result is returned to every lane.
__device__ __forceinline__ void wave_argmax(double &v, int &id) {
    argmax_step<0xB1, 0xF>(v, id);   // quad_perm [1,0,3,2]
    argmax_step<0x4E, 0xF>(v, id);   // quad_perm [2,3,0,1]
    argmax_step<0x141, 0xF>(v, id);  // row_half_mirror
    argmax_step<0x140, 0xF>(v, id);  // row_mirror: lane 15 of each row holds the row's best
    argmax_step<0x142, 0xA>(v, id);  // row_bcast15: rows 1 and 3 take the last lane of rows 0 and 2
    argmax_step<0x143, 0xC>(v, id);  // row_bcast31: rows 2 and 3 take lane 31
    const int2 b = __builtin_bit_cast(int2, v);
    v = __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(b.x, 63), __builtin_amdgcn_readlane(b.y, 63)));
    id = __builtin_amdgcn_readlane(id, 63);
}

constexpr int RSEL_LOADS = 8;

// Scores of token t from the router's split partial sums part[nsplit][T][E], by a workgroup of NT threads (all
// of them call it; E <= NT).  Thread (e, g) sums the splits g, g+4, ... of expert e in split order, in batches
// of RSEL_LOADS loads; thread e then adds the four group sums left to right and writes zs[e] = the weight's
// score and zs[E + e] = the selection value: for mode 0 the sigmoid and sigmoid + bias, for mode 1 (softmax
// gate) the logit twice.  One expert per thread, so the code holds one copy of exp.  zs: LDS of 4 E doubles;
// ends with a barrier.
template <int NT>
__device__ inline void token_scores(const double *__restrict__ part, int nsplit, int T, int E,
                                    const float *__restrict__ bias, int mode, int t, double *zs) {
    constexpr int NG = NT / 4;  // threads per split group
    const int tid = threadIdx.x;
    const int ept = (E + NG - 1) / NG;  // experts per thread column
    const rsrc_t psrc = make_rsrc(part, (uint32_t)((long)nsplit * T * E * 8));
    const float bz = (mode == 0 && tid < E) ? bias[tid] : 0.f;  // requested now, used after the sums
    for (int j = 0; j < ept; j++) {
        const int e = tid % NG + NG * j;
        const int g = tid / NG;
        if (e >= E) continue;
        double z = 0.0;
        int sp = g;
        for (; sp < nsplit; sp += 4 * RSEL_LOADS) {
            double a[RSEL_LOADS];
#pragma unroll
            for (int m = 0; m < RSEL_LOADS; m++) {
                const int s2 = sp + 4 * m;
                a[m] = buf_load_f64(psrc, s2 < nsplit ? (uint32_t)((((long)s2 * T + t) * E + e) * 8) : kOOB);
            }
#pragma unroll
            for (int m = 0; m < RSEL_LOADS; m++) z += a[m];
        }
        zs[g * E + e] = z;
    }
    __syncthreads();
    // s and sel of expert e replace its first two partial sums (each thread touches only its own entries)
    if (tid < E) {
        const int e = tid;
        const double z = ((zs[e] + zs[E + e]) + zs[2 * E + e]) + zs[3 * E + e];
        if (mode == 0) {
            const double sv = 1.0 / (1.0 + exp(-z));
            zs[e] = sv;
            zs[E + e] = sv + (double)bz;
        } else {
            zs[e] = z;
            zs[E + e] = z;
        }
    }
    __syncthreads();
}

// The top k by selection value of the scores token_scores left in zs, by one wavefront (call from lanes 0..63
// of one wavefront only).  Each lane holds EJ experts (e = lane + 64 j, E <= 64 EJ), sorts them once and
// exposes its best unchosen one; each of the k + 1 rounds is one wave-wide argmax, the winning lane moving to
// its next.  Lane r < k receives choice r: its id and its weight lambda u_r / (u_0 + ... + u_{k-1}), with u
// the sigmoid score (mode 0) or exp(z - z_max) (mode 1), summed in choice order and divided in fp64, rounded
// once to fp32.  gap (every lane): the k-th selection value less the (k+1)-th, infinity when k >= E.
template <int EJ>
__device__ inline void topk_pick(const double *zs, int E, int k, float lambda, int mode, int &id_out, float &w_out,
                                 double &gap) {
    const int lane = threadIdx.x & 63;
    double cv[EJ], cs[EJ];
    int ci[EJ];
#pragma unroll
    for (int j = 0; j < EJ; j++) {
        const int e = lane + 64 * j;
        cv[j] = -INFINITY;
        cs[j] = 0.0;
        ci[j] = 0x7fffffff;
        if (e < E) {
            cs[j] = zs[e];
            cv[j] = zs[E + e];
            ci[j] = e;
        }
    }
#pragma unroll
    for (int a2 = 0; a2 < EJ; a2++)  // insertion sort, fully unrolled (EJ <= 16)
#pragma unroll
        for (int b2 = EJ - 1; b2 > a2; b2--)
            if (better(cv[b2], ci[b2], cv[b2 - 1], ci[b2 - 1])) {
                const double tv = cv[b2], ts = cs[b2];
                const int ti = ci[b2];
                cv[b2] = cv[b2 - 1];
                cs[b2] = cs[b2 - 1];
                ci[b2] = ci[b2 - 1];
                cv[b2 - 1] = tv;
                cs[b2 - 1] = ts;
                ci[b2 - 1] = ti;
            }
    int head = 0;  // next unchosen candidate of this lane
    double sum_s = 0.0, prev_v = 0.0, top_z = 0.0;
    double my_s = 0.0;  // lane r < k keeps the score of choice r
    int my_id = 0;
    gap = INFINITY;
    const int rounds = (k < E) ? k + 1 : k;
    for (int r = 0; r < rounds; r++) {
        double hv = -INFINITY, hs = 0.0;
        int hid = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EJ; j++)
            if (head == j) {
                hv = cv[j];
                hs = cs[j];
                hid = ci[j];
            }
        double bv = hv;
        int bid = hid;
        wave_argmax(bv, bid);
        const int wl = bid & 63;  // lane that owns the winner
        const int2 sb = __builtin_bit_cast(int2, hs);
        const double bs = __builtin_bit_cast(
            double, make_int2(__builtin_amdgcn_readlane(sb.x, wl), __builtin_amdgcn_readlane(sb.y, wl)));
        if (r < k) {
            if (lane == wl) head++;
            // the weight's numerator: the sigmoid score, or exp(z - z_max) of the softmax gate
            if (mode == 1 && r == 0) top_z = bs;
            const double u = mode == 0 ? bs : exp(bs - top_z);
            sum_s += u;
            if (lane == r) {
                my_s = u;
                my_id = bid;
            }
            prev_v = bv;
        } else {
            gap = prev_v - bv;
        }
    }
    id_out = my_id;
    w_out = (float)((double)lambda * my_s / sum_s);
}

}  // namespace moe
