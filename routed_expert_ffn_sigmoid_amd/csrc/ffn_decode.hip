// Decode path of the expert FFNs: a bandwidth-bound dequant-GEMV run on the
// matrix cores with exact integer accumulation.
//
// Experts are SwiGLU FFNs quantised per output channel with a scale and a
// zero point ("企业官网建设流程全解析" page, Colibri walk-through, section 3.4);
// each unique expert runs once for all tokens routed to it (batch union,
// "25GB 内存跑 744B GLM-5.2 模型" page, section 三.4).
//
// Arithmetic.  For an output row with quantised weights q, zero point z and
// scale s, and an input row x:
//     out = s * (sum_k q_k x_k  -  z * sum_k x_k).
// The input row is put into 24-bit fixed point with a power-of-two scale per
// token and K part (the inputs one wavefront covers), x_k ~= X_k * 2^-e
// (|X_k| < 2^22), and X_k is written as three signed
// 8-bit digits, X = 65536 D2 + 256 D1 + D0.  sum_k q_k X_k is then three
// v_mfma_i32_16x16x64_i8 products with exact int32 accumulation: int8 weights
// feed the MFMA as loaded, int4 weights need two bit operations per 8
// weights (low and high nibbles as bytes 0..15).  The only rounding in the
// dot product is the 24-bit fixed point of the input (relative 2^-23 of the
// row's largest element); everything after it is done in fp64 and rounded
// once to fp32.
//
// Mapping (16x16x64 MFMA: M = 16 tokens, N = 16 weight rows, K = 64 inputs):
//   lane l holds weight row l%16; lane group g = l/16 loads bytes
//   [16g, 16g+16) of each 64-byte segment of the row (one dwordx4 per
//   segment, 16 rows x 64 contiguous bytes per instruction);
//   the activation digits for token l%16 come from LDS at the same inputs;
//   C[token i][row j] lands in lane 16*(i/4) + j, register i%4.
// Two kernels use this arithmetic.  decode_persistent_kernel (the default)
// runs one workgroup of 8 wavefronts per CU over a range of (slot, tile) items
// with the weight stream running across items; a slot with more tokens than
// its digit planes hold (at most 16) is taken in token passes.  With the
// routing of one token given to it, its gate/up launch also selects and sorts,
// and its down launch may also combine.  decode_kernel (routing tables beyond
// the persistent kernel's LDS) runs a grid of (row block, slot) workgroups of
// 4 wavefronts covering TPW = 4/S tiles of 16 rows, tokens in passes.  In both, the S wavefronts of a tile
// split K and add their fp64 partials in a fixed order, and the segment loop
// is padded to a multiple of PF with out-of-range (zero) loads, so it is
// straight-line code with PF segments in flight per row.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "select_dev.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int DK_THREADS = 256;
constexpr int DK_GMAX = 16;               // tokens per pass: the MFMA M dimension
constexpr int DK_LDS_BUDGET = 150 * 1024; // digit planes + reduction buffer

struct DSlot {
    int e, w, I;  // expert, its weight row, intermediate size
    bool shared;
};

// Expert of a grid slot; routed slots past the unique list hold -1 and exit.
__device__ __forceinline__ bool dk_slot(const FfnParams &P, int slot, DSlot &s) {
    if (slot < P.n_routed_slots) {
        const int e = P.uniq[slot];
        if (e < 0) return false;
        s.e = e;
        s.w = weight_row(P, e);
        if (s.w < 0) return false;  // weights not resident: rows left unwritten
        s.I = P.I;
        s.shared = false;
    } else {
        s.e = 0;
        s.w = 0;
        s.I = P.Is;
        s.shared = true;
        if (!P.y_sh) return false;  // the shared expert left out (y_sh = nullptr)
    }
    return s.I > 0;
}

// Plane byte position of input k: natural for int8 weights; for int4 weights the 32 inputs of each
// 16-byte weight chunk are stored as their 16 even inputs followed by their 16 odd inputs.
template <int WBITS>
__device__ __forceinline__ int plane_pos(int k) {
    if (WBITS == 8) return k;
    return (k & ~31) + ((k & 1) << 4) + ((k & 31) >> 1);
}

// Eight consecutive source values (fp32, or bf16 bit patterns) as fp32 from byte offset off of the
// source descriptor; an out-of-range offset gives zeros.
template <int SRC>
__device__ __forceinline__ void load8(rsrc_t src, uint32_t off, float (&v)[8]) {
    if (SRC == 0) {
        const uint4 a = buf_load16(src, off);
        const uint4 b = buf_load16(src, off == kOOB ? kOOB : off + 16);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
        v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    } else {
        const uint4 q = buf_load16(src, off);
        const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[2 * j] = __uint_as_float(qq[j] << 16);
            v[2 * j + 1] = __uint_as_float(qq[j] & 0xFFFF0000u);
        }
    }
}

// Wave-private staging: the inputs [k0, k0 + kpart) of ng source rows (fp32 or bf16) become three
// signed 8-bit digit planes of their 24-bit fixed-point values, with one power-of-two scale per
// (row, wavefront): x ~= X * 2^-expo[i], |X| < 2^22.  xsum[i] = sum of X (exact).  Positions past
// kpart up to the padded length are zero.  Only this wavefront reads what it writes, so the only
// synchronisation is the wavefront's own LDS ordering.
//
// A row is staged in two steps so that its loads can be issued ahead of other memory traffic:
// stage_issue requests the row's first 4 x 64 groups of 8 inputs (all in flight at once) and
// stage_finish turns them into digits; longer K parts are loaded there in further rounds of 4 groups
// per lane (read twice: once for the maximum, once for the digits).
template <int SRC>
struct StageRaw {
    static constexpr int G = 4;  // groups of 8 inputs per lane
    static constexpr int W = SRC == 0 ? 2 : 1;  // 16-byte loads per group
    uint4 q[G][W];
};

template <int SRC>
__device__ __forceinline__ void stage_issue(rsrc_t src, long ro, int m0, int ngr, int kpart, StageRaw<SRC> &r) {
    const int lane = threadIdx.x & 63;
    const int esz = SRC == 0 ? 4 : 2;
#pragma unroll
    for (int c = 0; c < StageRaw<SRC>::G; c++) {
        const int m = m0 + lane + 64 * c;
        const uint32_t off = (m < ngr && m * 8 < kpart) ? (uint32_t)((ro + (long)m * 8) * esz) : kOOB;
#pragma unroll
        for (int w = 0; w < StageRaw<SRC>::W; w++) r.q[c][w] = buf_load16(src, off == kOOB ? kOOB : off + 16 * w);
    }
}

template <int SRC>
__device__ __forceinline__ void raw_to_f32(const uint4 (&q)[StageRaw<SRC>::W], float (&v)[8]) {
    if (SRC == 0) {
        const uint4 a = q[0], b = q[StageRaw<SRC>::W - 1];
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
        v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    } else {
        const uint32_t qq[4] = {q[0].x, q[0].y, q[0].z, q[0].w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[2 * j] = __uint_as_float(qq[j] << 16);
            v[2 * j + 1] = __uint_as_float(qq[j] & 0xFFFF0000u);
        }
    }
}

template <int SRC>
__device__ __forceinline__ float raw_absmax(const StageRaw<SRC> &r, float mx) {
#pragma unroll
    for (int c = 0; c < StageRaw<SRC>::G; c++) {
        float v[8];
        raw_to_f32<SRC>(r.q[c], v);
#pragma unroll
        for (int t = 0; t < 8; t++) mx = fmaxf(mx, fabsf(v[t]));
    }
    return mx;
}

// Wave-wide reductions in DPP steps (neighbours, pairs, mirrored halves of 8 and 16 lanes, then rows 0-1
// into 1 and 2-3 into 3, then row 1 into rows 2-3): lane 63 ends with the result.  Low latency next to
// shuffles through LDS, which matters on the start-up path.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float wave_max_nonneg(float x) {  // x >= 0: the bit patterns order as the values
    uint32_t v = __float_as_uint(x);
    v = max(v, dpp_u32<0xB1, 0xF>(v, v));
    v = max(v, dpp_u32<0x4E, 0xF>(v, v));
    v = max(v, dpp_u32<0x141, 0xF>(v, v));
    v = max(v, dpp_u32<0x140, 0xF>(v, v));
    v = max(v, dpp_u32<0x142, 0xA>(v, v));
    v = max(v, dpp_u32<0x143, 0xC>(v, v));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 63));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_add_f64(double v) {
    const int2 b = __builtin_bit_cast(int2, v);
    const int2 o = make_int2((int)dpp_u32<CTRL, ROWS>((uint32_t)b.x, 0u), (int)dpp_u32<CTRL, ROWS>((uint32_t)b.y, 0u));
    return v + __builtin_bit_cast(double, o);  // lanes of rows outside ROWS add +0
}
__device__ __forceinline__ double wave_sum_f64(double v) {  // exact when every partial sum is (integers below 2^53)
    v = dpp_add_f64<0xB1, 0xF>(v);
    v = dpp_add_f64<0x4E, 0xF>(v);
    v = dpp_add_f64<0x141, 0xF>(v);
    v = dpp_add_f64<0x140, 0xF>(v);
    v = dpp_add_f64<0x142, 0xA>(v);
    v = dpp_add_f64<0x143, 0xC>(v);
    const int2 b = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(b.x, 63), __builtin_amdgcn_readlane(b.y, 63)));
}

template <int WBITS, int SRC>
__device__ void stage_finish(const StageRaw<SRC> &r, rsrc_t src, long ro, int i, int ngr, int kpart, int stride,
                             long plane_bytes, int8_t *planes, int *expo, double *xsum) {
    constexpr int RG = 64 * StageRaw<SRC>::G;  // groups per round
    const int lane = threadIdx.x & 63;
    float mx = raw_absmax<SRC>(r, 0.f);
    for (int m0 = RG; m0 < ngr; m0 += RG) {
        StageRaw<SRC> r2;
        stage_issue<SRC>(src, ro, m0, ngr, kpart, r2);
        mx = raw_absmax<SRC>(r2, mx);
    }
    mx = wave_max_nonneg(mx);
    int e = 0;
    if (mx > 0.f) {
        int ex;
        frexpf(mx, &ex);  // mx < 2^ex
        e = 22 - ex;
    }
    const float sc = ldexpf(1.f, e);
    long ssum = 0;
    int8_t *p0 = planes + (long)i * stride, *p1 = p0 + plane_bytes, *p2 = p1 + plane_bytes;
    auto put = [&](int m, const float (&xv)[8]) {
        // Digits: for |X| < 2^22 the bytes of (X + 0x808080) ^ 0x808080 are the signed base-256 digits
        // d0, d1, d2 of X (each in [-128, 127], the representation being unique).  Planes are packed with
        // byte permutes: for int8 weights two words per plane in input order, for int4 weights one word
        // of even inputs and one of odd inputs.
        uint32_t V[8];
        int gs = 0;  // |sum| < 2^25
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int X = (int)rintf(xv[t] * sc);
            gs += X;
            V[t] = ((uint32_t)X + 0x808080u) ^ 0x808080u;
        }
        ssum += gs;
        uint32_t w[3][2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            // the four inputs of word q: q*4 + 0..3 (int8) or q, q + 2, q + 4, q + 6 (int4)
            const uint32_t a0 = WBITS == 8 ? V[4 * q] : V[q], a1 = WBITS == 8 ? V[4 * q + 1] : V[q + 2];
            const uint32_t a2 = WBITS == 8 ? V[4 * q + 2] : V[q + 4], a3 = WBITS == 8 ? V[4 * q + 3] : V[q + 6];
            const uint32_t A = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.b0 a1.b0 a0.b1 a1.b1
            const uint32_t B = __builtin_amdgcn_perm(a3, a2, 0x05010400u);  // a2.b0 a3.b0 a2.b1 a3.b1
            const uint32_t C = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.b2 a1.b2 ...
            const uint32_t D = __builtin_amdgcn_perm(a3, a2, 0x07030602u);  // a2.b2 a3.b2 ...
            w[0][q] = __builtin_amdgcn_perm(B, A, 0x05040100u);             // byte 0 of a0..a3
            w[1][q] = __builtin_amdgcn_perm(B, A, 0x07060302u);             // byte 1
            w[2][q] = __builtin_amdgcn_perm(D, C, 0x05040100u);             // byte 2
        }
        if (WBITS == 8) {
            const int pos = m * 8;
            *(uint2 *)(p0 + pos) = make_uint2(w[0][0], w[0][1]);
            *(uint2 *)(p1 + pos) = make_uint2(w[1][0], w[1][1]);
            *(uint2 *)(p2 + pos) = make_uint2(w[2][0], w[2][1]);
        } else {
            // inputs 8m..8m+7: evens go to plane_pos(8m), odds to plane_pos(8m+1)
            const int pe = plane_pos<4>(m * 8), po = plane_pos<4>(m * 8 + 1);
            *(uint32_t *)(p0 + pe) = w[0][0];
            *(uint32_t *)(p0 + po) = w[0][1];
            *(uint32_t *)(p1 + pe) = w[1][0];
            *(uint32_t *)(p1 + po) = w[1][1];
            *(uint32_t *)(p2 + pe) = w[2][0];
            *(uint32_t *)(p2 + po) = w[2][1];
        }
    };
    auto put_round = [&](const StageRaw<SRC> &rr, int m0) {
#pragma unroll
        for (int c = 0; c < StageRaw<SRC>::G; c++) {
            const int m = m0 + lane + 64 * c;
            float v[8];
            raw_to_f32<SRC>(rr.q[c], v);
            if (m < ngr) put(m, v);
        }
    };
    put_round(r, 0);
    for (int m0 = RG; m0 < ngr; m0 += RG) {
        StageRaw<SRC> r2;
        stage_issue<SRC>(src, ro, m0, ngr, kpart, r2);
        put_round(r2, m0);
    }
    const double ds = wave_sum_f64((double)ssum);  // exact: integers below 2^53
    if (lane == 0) {
        xsum[i] = ds;
        expo[i] = e;
    }
}

// make this wavefront's LDS writes visible to its own later reads
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Source row of staged token i: through the permutation (gate/up of a routed expert reads row
// perm[base + i] / k of x), or directly (row base + i of h, or of x for the shared expert).  The index
// is wave-uniform, so the permutation is read with scalar loads.
struct RowMap {
    const int32_t *perm;  // nullptr: direct
    int base, k;
    long len;  // elements per source row
    __device__ __forceinline__ long row_off(int i) const {
        return perm ? (long)(ld_const(perm, base + i) / k) * len : (long)(base + i) * len;
    }
};

// All ng rows, one after the other (each row's loads in flight together).
template <int WBITS, int SRC>
__device__ void wave_stage(rsrc_t src, const RowMap &rm, int ng, int k0, int kpart, int kpad, int stride,
                           long plane_bytes, int8_t *planes, int *expo, double *xsum) {
    const int ngr = kpad / 8;  // groups of 8 inputs, zero past kpart
    for (int i = 0; i < ng; i++) {
        const long ro = rm.row_off(i) + k0;  // element offset of this row's first input
        StageRaw<SRC> r;
        stage_issue<SRC>(src, ro, 0, ngr, kpart, r);
        stage_finish<WBITS, SRC>(r, src, ro, i, ngr, kpart, stride, plane_bytes, planes, expo, xsum);
    }
    wave_lds_sync();
}

__device__ __forceinline__ float zp_val(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
}

// One 64-byte segment of a wavefront's 16 rows (NM matrices) through the matrix cores:
// C[m][p] += digits of plane p (A, 16 tokens x 64 inputs) . weights of matrix m (B, 64 inputs x 16 rows).
template <int WBITS, int NM>
__device__ __forceinline__ void consume_segment(const uint4 (&wq)[NM], const int8_t *xrow, long pstep, int gstep,
                                                int seg, int g, i32x4_t (&C)[NM][3]) {
    if (WBITS == 8) {
        i32x4_t A[3];
        const int8_t *xa = xrow + gstep * (64 * seg + 16 * g);
#pragma unroll
        for (int p = 0; p < 3; p++) {
            const uint4 v = *(const uint4 *)(xa + p * pstep);
            A[p] = (i32x4_t){(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int m = 0; m < NM; m++) {
            const uint4 q = wq[m];
            const i32x4_t Bq = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
#pragma unroll
            for (int p = 0; p < 3; p++) C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[p], Bq, C[m][p], 0, 0, 0);
        }
    } else {
        i32x4_t Ae[3], Ao[3];
        const int8_t *xa = xrow + gstep * (128 * seg + 32 * g);
#pragma unroll
        for (int p = 0; p < 3; p++) {
            const uint4 ve = *(const uint4 *)(xa + p * pstep);
            const uint4 vo = *(const uint4 *)(xa + p * pstep + 16);
            Ae[p] = (i32x4_t){(int)ve.x, (int)ve.y, (int)ve.z, (int)ve.w};
            Ao[p] = (i32x4_t){(int)vo.x, (int)vo.y, (int)vo.z, (int)vo.w};
        }
#pragma unroll
        for (int m = 0; m < NM; m++) {
            const uint4 q = wq[m];
            const i32x4_t Be = {(int)(q.x & 0x0F0F0F0Fu), (int)(q.y & 0x0F0F0F0Fu), (int)(q.z & 0x0F0F0F0Fu),
                                (int)(q.w & 0x0F0F0F0Fu)};
            const i32x4_t Bo = {(int)((q.x >> 4) & 0x0F0F0F0Fu), (int)((q.y >> 4) & 0x0F0F0F0Fu),
                                (int)((q.z >> 4) & 0x0F0F0F0Fu), (int)((q.w >> 4) & 0x0F0F0F0Fu)};
#pragma unroll
            for (int p = 0; p < 3; p++) {
                C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ae[p], Be, C[m][p], 0, 0, 0);
                C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ao[p], Bo, C[m][p], 0, 0, 0);
            }
        }
    }
}

// MODE 0: gate/up -> h (fp32); MODE 1: down -> y_perm / y_shared.
// grid: (ceil(rows / (16 * 4/S)), slots); block 256; dynamic LDS from dk_lds_bytes.
template <int MODE, int WBITS, int SRC, int S>
__global__ __launch_bounds__(DK_THREADS, 3) void decode_kernel(FfnParams P, float *__restrict__ h,
                                                            float *__restrict__ h_sh, int gmax, int kpad) {
    constexpr int TPW = 4 / S;
    constexpr int NM = MODE == 0 ? 2 : 1;  // matrices per wave: gate and up, or down
    constexpr int PF = MODE == 0 ? 4 : 8;  // 64-byte segments in flight per row
    extern __shared__ __align__(16) uint8_t dk_lds[];
    __shared__ int wexpo[4][DK_GMAX];
    __shared__ double wxsum[4][DK_GMAX];
    __shared__ uint32_t zero_area[8];

    DSlot s;
    if (!dk_slot(P, blockIdx.y, s)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tile = wv / S, kp = wv % S;
    const int nout = MODE == 0 ? s.I : P.d;
    const int row_base = (blockIdx.x * TPW) * 16;
    if (row_base >= nout) return;
    const int K = MODE == 0 ? P.d : s.I;
    const long rb = (long)K * WBITS / 8;
    const int kpart = K / S;                          // inputs per wavefront
    const int kpart_bytes = kpart * WBITS / 8;
    const int nseg = (kpart_bytes + 63) / 64;
    const int g = lane >> 4, j = lane & 15;
    const int row = min(row_base + tile * 16 + j, nout - 1);
    const QW &W = s.shared ? P.shared : P.routed;
    // one descriptor per weight matrix of this expert; lane offsets inside it
    rsrc_t wr[NM];
    const int mrows = MODE == 0 ? s.I : P.d;
    const uint32_t mbytes = (uint32_t)((long)mrows * rb);
    if (MODE == 0) {
        wr[0] = make_rsrc(W.qg + (long)s.w * s.I * rb, mbytes);
        wr[NM - 1] = make_rsrc(W.qu + (long)s.w * s.I * rb, mbytes);
    } else {
        wr[0] = make_rsrc(W.qd + (long)s.w * P.d * rb, mbytes);
    }
    const uint32_t lane_off = (uint32_t)((long)row * rb) + (uint32_t)(kp * kpart_bytes + 16 * g);
    const int nseg_pad = (nseg + PF - 1) / PF * PF;

    uint4 wbuf[PF][NM];
    auto ldw = [&](int b, int seg) {
        const uint32_t off = (64 * seg + 16 * g < kpart_bytes) ? lane_off + 64 * seg : kOOB;
#pragma unroll
        for (int m = 0; m < NM; m++) wbuf[b][m] = buf_load16(wr[m], off);
    };
#pragma unroll
    for (int b = 0; b < PF; b++) ldw(b, b);  // the weight stream starts here

    const int p0 = s.shared ? 0 : P.offsets[s.e];
    const int n = s.shared ? P.T : P.offsets[s.e + 1] - p0;
    const int stride = kpad + 16;
    const long pb = (long)gmax * stride;             // bytes per digit plane of one wavefront
    int8_t *planes = (int8_t *)dk_lds + (long)wv * 3 * pb;
    double *red = (double *)dk_lds;                  // cross-wave partials, after the planes are done
    if (tid < 8) zero_area[tid] = 0u;
    const rsrc_t src = MODE == 0 ? make_rsrc(P.x, (uint32_t)((long)P.T * P.d * (SRC == 0 ? 4 : 2)))
                                 : make_rsrc(s.shared ? h_sh : h,
                                             (uint32_t)((long)(s.shared ? P.T : P.A) * K * 4));
    // z of this lane's output row (the same row for every token)
    float zrow[NM];
    if (MODE == 0) {
        zrow[0] = zp_val(W.zg, WBITS, (long)s.w * s.I + row);
        zrow[NM - 1] = zp_val(W.zu, WBITS, (long)s.w * s.I + row);
    } else {
        zrow[0] = zp_val(W.zd, WBITS, (long)s.w * P.d + row);
    }
    __syncthreads();  // zero_area

    for (int g0 = 0; g0 < n; g0 += gmax) {
        const int ng = min(gmax, n - g0);
        if (g0 != 0) {
#pragma unroll
            for (int b = 0; b < PF; b++) ldw(b, b);
        }
        RowMap rm;
        rm.perm = (MODE == 0 && !s.shared) ? P.perm : nullptr;
        rm.base = (s.shared ? 0 : p0) + g0;
        rm.k = P.k;
        rm.len = MODE == 0 ? P.d : K;
        if (MODE == 0)
            wave_stage<WBITS, SRC>(src, rm, ng, kp * kpart, kpart, kpad, stride, pb, planes, wexpo[wv], wxsum[wv]);
        else
            wave_stage<WBITS, 0>(src, rm, ng, kp * kpart, kpart, kpad, stride, pb, planes, wexpo[wv], wxsum[wv]);

        // ---- stream the wavefront's K part through the matrix cores
        i32x4_t C[NM][3];
#pragma unroll
        for (int m = 0; m < NM; m++)
#pragma unroll
            for (int p = 0; p < 3; p++) C[m][p] = (i32x4_t){0, 0, 0, 0};
        // A-operand rows: token j of this lane; lanes without a token read a zeroed LDS area
        const bool tok_ok = j < ng;
        const int8_t *xrow = tok_ok ? planes + (long)j * stride : (const int8_t *)zero_area;
        const long pstep = tok_ok ? pb : 0;
        const int gstep = tok_ok ? 1 : 0;
        for (int seg0 = 0; seg0 < nseg_pad; seg0 += PF) {
#pragma unroll
            for (int b = 0; b < PF; b++) {
                const int seg = seg0 + b;
                consume_segment<WBITS, NM>(wbuf[b], xrow, pstep, gstep, seg, g, C);
                // refill this slot right away (past the end: out of range, zeros, no memory traffic);
                // the scheduling barrier keeps the compiler from sinking the refill to the end of the
                // unrolled block, which would let the in-flight queue drain every PF segments
                __builtin_amdgcn_sched_barrier(0);
                ldw(b, seg + PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- this wavefront's exact partial, zero point applied and scale undone, in fp64
        double v[NM][4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int i = 4 * g + r;  // token of this register
            const bool ok = i < ng;
            const double unit = ok ? ldexp(1.0, -wexpo[wv][i]) : 0.0;
            const double xs = ok ? wxsum[wv][i] : 0.0;
#pragma unroll
            for (int m = 0; m < NM; m++) {
                const double dot = (double)C[m][2][r] * 65536.0 + (double)C[m][1][r] * 256.0 + (double)C[m][0][r];
                v[m][r] = (dot - (double)zrow[m] * xs) * unit;
            }
        }
        // the S wavefronts of a tile add their partials in a fixed order
        if (S > 1) {
            __syncthreads();  // every wavefront is done with its planes: red may overwrite them
#pragma unroll
            for (int m = 0; m < NM; m++)
#pragma unroll
                for (int r = 0; r < 4; r++) red[((wv * NM + m) * 4 + r) * 64 + lane] = v[m][r];
            __syncthreads();
            if (kp == 0) {
#pragma unroll
                for (int m = 0; m < NM; m++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        double a = v[m][r];
                        for (int q = 1; q < S; q++) a += red[(((wv + q) * NM + m) * 4 + r) * 64 + lane];
                        v[m][r] = a;
                    }
            }
        }
        if (kp == 0) {
            const int o = row_base + tile * 16 + j;
            if (o < nout) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int i = 4 * g + r;  // token of this register
                    if (i < ng) {
                        if (MODE == 0) {
                            const long ch = (long)s.w * s.I + o;
                            const float gf = (float)((double)W.sg[ch] * v[0][r]);
                            const float uf = (float)((double)W.su[ch] * v[NM - 1][r]);
                            const float hv = gf / (1.f + expf(-gf)) * uf;
                            if (s.shared)
                                h_sh[(long)(g0 + i) * s.I + o] = hv;
                            else
                                h[(long)(p0 + g0 + i) * s.I + o] = hv;
                        } else {
                            const long ch = (long)s.w * P.d + o;
                            const float y = (float)((double)W.sd[ch] * v[0][r]);
                            if (s.shared)
                                P.y_sh[(long)(g0 + i) * P.d + o] = y;
                            else
                                P.y_perm[(long)(p0 + g0 + i) * P.d + o] = y;
                        }
                    }
                }
            }
        }
        if (S > 1 || g0 + gmax < n) __syncthreads();  // red / planes are reused by the next token group
    }
}

// ---------------------------------------------------------------------------- persistent variant
// Decode with one workgroup of DKP_WAVES wavefronts per CU.  Work items are (slot, row tile) pairs,
// slot-major over the unique experts and then the shared expert; CU c takes the contiguous items
// [c*N/ncu, (c+1)*N/ncu).  The S wavefronts of a tile split its K range and TPW = DKP_WAVES / S
// tiles share an item, so every wavefront of a CU works on the same item and the CU's items end
// together.  Each wavefront's weight stream runs across items: while it consumes the last batch of
// an item, the refills already fetch the first segments of the next item.  PF loads per matrix are in
// flight (16 KB per wavefront); the host picks PF among two depths so that the item's segments fill
// whole batches where they can.
//
// Start-up takes two memory round trips: the routing tables (unique list, offsets, permutation) go to
// LDS in one round together with the first activation rows; the weight stream starts right after.
// Gate/up stages the digit planes of all T tokens once where they fit (slots only remap lanes to tokens); down,
// and gate/up in token passes, stage the rows of each (virtual) slot when it changes.
struct DItem {
    int slot, e, w, tile, I, kpart_bytes, nseg_pad, row, p0, ng;  // w: weight row (-1: not resident)
    bool shared, row_ok;
};

constexpr int DKP_WAVES = 8;
constexpr int DKP_TAB_PER_THREAD = 6;  // routing-table words loaded per thread (>= 1 + 1024 + 1025 + 512)

// Words of the routing table kept in LDS: n_uniq, uniq[n_routed_slots], offsets[E + 1], perm[A] (gate/up).
__host__ __device__ inline int dkp_tab_words(int mode, int n_routed_slots, int E, int A) {
    return 1 + n_routed_slots + E + 1 + (mode == 0 ? A : 0);
}

// One token's routing inside the gate/up launch (FfnParams::route): its scores from the router's split partial
// sums, the top k by wavefront 0 (the selection kernel's order of sums and picks, so the same bits), and the
// permutation of those k distinct experts straight into the LDS routing table.  For one token the stable
// counting sort reduces to ranks: choice j goes to place r_j = the number of chosen ids below its own, uniq
// lists the chosen ids in increasing order, and offsets[e] counts the chosen ids below e.  Workgroup 0 also
// writes the routing outputs.  zs: LDS of 4 E doubles and k ints, free until the table barrier.  Every thread
// calls it; E <= 256, k <= 64.
__device__ void route_one_token(const FfnParams &P, int *tab, double *zs) {
    const FfnParams::Route &R = P.route;
    const int E = P.E, k = P.k;
    const int tid = threadIdx.x, lane = tid & 63;
    const bool out = blockIdx.x == 0;
    token_scores<DKP_WAVES * 64>(R.part, R.nsplit, 1, E, R.bias, R.mode, 0, zs);  // ends with a barrier
    int *ids = (int *)(zs + 4 * E);
    if (tid < 64) {
        int id;
        float wt;
        double gp;
        topk_pick<4>(zs, E, k, R.lambda, R.mode, id, wt, gp);
        if (lane < k) ids[lane] = id;
        if (out) {
            if (lane < k) {
                R.idx[lane] = id;
                R.w[lane] = wt;
            }
            if (lane == 0 && R.gap) R.gap[0] = gp;
        }
    }
    __syncthreads();
    int *t_uniq = tab + 1, *t_off = tab + 1 + k, *t_perm = tab + 2 + k + E;  // n_routed_slots = k for one token
    if (tid < k) {
        const int id = ids[tid];
        int r = 0;
        for (int i = 0; i < k; i++) r += ids[i] < id;
        t_uniq[r] = id;
        t_perm[r] = tid;
        if (out) {
            R.uniq[r] = id;
            R.perm[r] = tid;
            R.inv[tid] = r;
        }
    }
    for (int e = tid; e <= E; e += DKP_WAVES * 64) {
        int c = 0, chosen = 0;
        for (int i = 0; i < k; i++) {
            const int v = ids[i];
            c += v < e;
            chosen |= v == e;
        }
        t_off[e] = c;
        if (out) {
            R.offsets[e] = c;
            if (e < E) R.counts[e] = chosen;
            if (e >= k && e < E) R.uniq[e] = -1;
        }
    }
    if (tid == 0) {
        tab[0] = k;
        if (out) *R.n_uniq = k;
    }
}

// PASSES: the digit planes hold gcap < T token rows, so a slot with more rows is taken as several virtual slots
// of at most gcap rows each, in row order, each streaming the expert's rows again (the mid workload's down pass at
// T = 4: 3 x 14336 inputs of planes fit the LDS, 4 do not; gate/up of the 256-expert layer at T = 8: 5 x 7168).
// Down stages the virtual slot's rows of h, gate/up its tokens' activation rows (planes row r = its r-th row).
// COMB (down only, one token, FfnParams::comb_y set): the combine runs in this launch.  The h rows of all
// nsl = n_uniq + shared slots are staged at once (planes row s = slot s, gcap = nsl), items are numbered
// tile-major (item i = tile i / nsl of slot i % nsl) and ranges are cut at tiles, so a workgroup takes every
// slot of its rows in turn.  The wavefront that finishes a row of a slot keeps its output in LDS; after the
// tile's last slot it adds, as the combine kernel does, y = y_shared + w_0 Y_0 + w_1 Y_1 + ... in fp32 fmaf
// (choice j's output is slot inv[j]'s: one row per slot at T = 1).
template <int MODE, int WBITS, int SRC, int S, int PF, bool PASSES, bool COMB>
__global__ __launch_bounds__(DKP_WAVES * 64, 1) void decode_persistent_kernel(FfnParams P, float *__restrict__ h,
                                                                           float *__restrict__ h_sh, int kpad,
                                                                           int tiles_r, int tiles_s, int ncu,
                                                                           int gcap) {
    constexpr int NW = DKP_WAVES;
    constexpr int TPW = NW / S;
    constexpr int NM = MODE == 0 ? 2 : 1;
    constexpr int SRCX = MODE == 0 ? SRC : 0;
    extern __shared__ __align__(16) uint8_t dk_lds[];
    __shared__ int wexpo[NW][DK_GMAX];
    __shared__ double wxsum[NW][DK_GMAX];
    __shared__ uint32_t zero_area[8];
    // COMB: each wavefront's outputs of its 16 rows per slot, and the token's choices (inv, w)
    __shared__ float ycomb[COMB ? NW : 1][COMB ? DK_GMAX : 1][16];
    __shared__ int c_inv[COMB ? DK_GMAX : 1];
    __shared__ float c_w[COMB ? DK_GMAX : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave indices stay scalar
    const int tile_w = wv / S, kp = wv % S;
    const int g = lane >> 4, j = lane & 15;
    const int T = P.T;

    // ---- LDS layout: routing table, digit planes (one copy per K part), cross-wave partials
    const int nrs = P.n_routed_slots;
    const int tab_words = dkp_tab_words(MODE, nrs, P.E, P.A);
    int *tab = (int *)dk_lds;
    const int *t_uniq = tab + 1, *t_off = tab + 1 + nrs, *t_perm = tab + 2 + nrs + P.E;
    const int stride = kpad + 16;
    const long pb = (long)(PASSES || COMB ? gcap : T) * stride;  // bytes per digit plane of one K part
    const int vwords = PASSES ? nrs + 2 : 0;               // first virtual slot of each slot (PASSES)
    int *vpre = tab + tab_words;
    const long pl0 = ((long)(tab_words + vwords) * 4 + 15) & ~15L;
    int8_t *planes = (int8_t *)dk_lds + pl0 + (long)kp * 3 * pb;
    double *red = (double *)(dk_lds + pl0 + (long)S * 3 * pb);

    // ---- this workgroup's range of units [ra, rb) for nu_ routed slots (nvr_ and nvs_ routed and shared virtual
    // slots).  With one tile per item (S = NW) the ranges are cut in half tiles (8 rows): every CU gets the same
    // number of rows to within 8, and a range may begin or end in the middle of a tile, whose rows outside it
    // read and store nothing.  Otherwise the ranges are cut in items.
    constexpr bool HALVES = TPW == 1;
    auto urange = [&](int nu_, int nvr_, int nvs_, int &ra, int &rb) {
        const int N = COMB ? tiles_r : nvr_ * tiles_r + nvs_ * tiles_s;  // COMB: ranges count tiles
        const int NU = HALVES ? 2 * N : N;
        if (MODE == 0 || HALVES || COMB) {
            const int G = gridDim.x, b = blockIdx.x;
            if (G % ncu == 0 && NU >= G) {
                const int m = G / ncu, c = b % ncu, r = b / ncu;
                const int c0 = c * NU / ncu, c1 = (c + 1) * NU / ncu;
                ra = c0 + r * (c1 - c0) / m;
                rb = c0 + (r + 1) * (c1 - c0) / m;
            } else {
                ra = b * NU / G;
                rb = (b + 1) * NU / G;
            }
        } else {
            // Down with items of several tiles: it restages the rows of h whenever a range moves to another
            // slot, and that request would queue behind the weights already in flight, a long delay next to
            // coarse items.  So the range boundaries are moved to slot starts: each slot is shared by the
            // workgroups whose plain boundary c * NU / G falls inside it, in equal parts; a slot that no
            // boundary falls into goes to the workgroup before it.  (With half-tile units the plain split is
            // kept: it balances to 8 rows, and one restage per crossing range costs less than the rounding
            // of slot-aligned shares.)
            const int G = gridDim.x;
            const int ur = HALVES ? 2 * tiles_r : tiles_r;
            const int us = P.Is > 0 ? (HALVES ? 2 * tiles_s : tiles_s) : 0;
            auto bound = [&](int c) -> int {
                if (c <= 0 || NU == 0) return 0;
                if (c >= G) return NU;
                const int p = (int)((long)c * NU / G);
                int st, len;
                if (PASSES || p < nu_ * ur) {
                    st = p / ur * ur;
                    len = ur;
                } else {
                    st = nu_ * ur;
                    len = us;
                }
                const int first = (int)(((long)st * G + NU - 1) / NU);
                const int n = (int)(((long)(st + len) * G + NU - 1) / NU) - first;  // >= 1: c is one of them
                return st + (int)((long)(c - first) * len / n);
            };
            ra = bound(blockIdx.x);
            rb = bound(blockIdx.x + 1);
        }
    };

    // ---- first memory round trip: routing table and (gate/up) this wavefront's first activation row, all
    // requested before any of them is waited for
    const int kd = MODE == 0 ? P.d : 0;
    const rsrc_t xsrc0 = make_rsrc(P.x, (uint32_t)((long)T * P.d * (SRC == 0 ? 4 : 2)));
    StageRaw<SRCX> raw0;
    // Down at one token: slot s's row of h is row s (each chosen expert has the one assignment, so offsets of the
    // slot's expert is s), and the shared expert's is row 0 of its own.  So the rows of h this wavefront stages
    // first are requested with the routing table, for the range it would have with every routed slot used; they
    // are checked against the real ones once the table is in.  raw1 / raw2: the rows' data; e_ro1 / e_ro2: their
    // element offsets (-1: none requested) and e_sh1 / e_sh2 whether they are the shared expert's.
    const bool early = MODE == 1 && !PASSES && T == 1;
    StageRaw<SRCX> raw1, raw2;
    long e_ro1 = -1, e_ro2 = -1;
    bool e_sh1 = false, e_sh2 = false;
    int eu0 = 0, eu1 = 0;
    auto h_row_src = [&](bool sh) {
        return make_rsrc(sh ? h_sh : h, (uint32_t)((long)(sh ? T : P.A) * (sh ? P.Is : P.I) * 4));
    };
    if (MODE == 0 && P.route.part) {
        // one token routed here: its activation row is requested first, then the partial sums
        const int kpart = kd / S;
        stage_issue<SRCX>(xsrc0, (long)tile_w * kd + kp * kpart, tile_w < T ? 0 : kpad, kpad / 8, kpart, raw0);
        route_one_token(P, tab, (double *)(dk_lds + pl0));
    } else {
        const rsrc_t r_nu = make_rsrc(P.n_uniq, 4), r_uq = make_rsrc(P.uniq, (uint32_t)nrs * 4);
        const rsrc_t r_of = make_rsrc(P.offsets, (uint32_t)(P.E + 1) * 4);
        const rsrc_t r_pm = make_rsrc(P.perm, (uint32_t)P.A * 4);
        uint32_t v[DKP_TAB_PER_THREAD];
#pragma unroll
        for (int q = 0; q < DKP_TAB_PER_THREAD; q++) {
            const int w = tid + q * NW * 64;
            // one source per word; words past the table read nothing
            const int b1 = 1, b2 = 1 + nrs, b3 = 2 + nrs + P.E;
            rsrc_t r = r_nu;
            uint32_t off = kOOB;
            if (w < b1) { r = r_nu; off = 0; }
            else if (w < b2) { r = r_uq; off = (uint32_t)(w - b1) * 4; }
            else if (w < b3) { r = r_of; off = (uint32_t)(w - b2) * 4; }
            else if (w < tab_words) { r = r_pm; off = (uint32_t)(w - b3) * 4; }
            v[q] = buf_load4(r, off);
        }
        if (MODE == 0) {
            // token row tile_w (if any), this wavefront's K part
            const int kpart = kd / S;
            const long ro = (long)tile_w * kd + kp * kpart;
            stage_issue<SRCX>(xsrc0, ro, tile_w < T && !PASSES ? 0 : kpad, kpad / 8, kpart, raw0);
        }
        if (early) {
            auto issue = [&](int slot, StageRaw<SRCX> &raw, bool &sh, long &ro) {
                sh = slot >= nrs;
                const int I = sh ? P.Is : P.I;
                ro = (sh ? 0 : (long)slot * I) + kp * (I / S);
                stage_issue<SRCX>(h_row_src(sh), ro, 0, kpad / 8, I / S, raw);
            };
            const int nsl_all = nrs + (P.Is > 0 ? 1 : 0);
            if (COMB) {  // planes row r = slot r: rows tile_w and tile_w + TPW
                if (tile_w < nsl_all) issue(tile_w, raw1, e_sh1, e_ro1);
                if (tile_w + TPW < nsl_all) issue(tile_w + TPW, raw2, e_sh2, e_ro2);
            } else {  // the first item's slot, staged by the wavefronts of token row 0
                urange(nrs, nrs, P.Is > 0 ? 1 : 0, eu0, eu1);
                const int i0p = HALVES ? eu0 >> 1 : eu0;
                if (eu0 < eu1 && tile_w == 0) issue(i0p < nrs * tiles_r ? i0p / tiles_r : nrs, raw1, e_sh1, e_ro1);
            }
        }
        if (COMB && tid < P.k) {
            c_inv[tid] = P.comb_inv[tid];
            c_w[tid] = P.comb_w[tid];
        }
#pragma unroll
        for (int q = 0; q < DKP_TAB_PER_THREAD; q++) {
            const int w = tid + q * NW * 64;
            if (w < tab_words) tab[w] = (int)v[q];
        }
    }
    if (tid < 8) zero_area[tid] = 0u;
    __syncthreads();  // table in LDS (the compiler waits for the table loads before the stores)

    int nu = __builtin_amdgcn_readfirstlane(tab[0]);
    if (nu < 0) {
        // invalid expert ids in the routing (n_uniq = -1): the valid experts are the non-negative prefix of uniq
        nu = 0;
        while (nu < nrs && t_uniq[nu] >= 0) nu++;
        nu = __builtin_amdgcn_readfirstlane(nu);
    }
    nu = nu > nrs ? nrs : nu;
    int nvr = nu, nvs = P.Is > 0 ? 1 : 0;  // routed and shared (virtual) slots
    if constexpr (PASSES) {
        // vpre[s] = first virtual slot of routed slot s (exclusive prefix of its passes), vpre[nu] = their total
        if (tid < 64) {
            int carry = 0;
            for (int b = 0; b < nu; b += 64) {
                const int sl = b + lane;
                int np = 0;
                if (sl < nu) {
                    const int e = t_uniq[sl];
                    np = (t_off[e + 1] - t_off[e] + gcap - 1) / gcap;
                }
                int incl = np;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int t2 = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += t2;
                }
                if (sl < nu) vpre[sl] = carry + incl - np;
                carry += __shfl(incl, 63, 64);
            }
            if (lane == 0) vpre[nu] = carry;
        }
        __syncthreads();
        nvr = __builtin_amdgcn_readfirstlane(vpre[nu]);
        nvs = P.Is > 0 ? (T + gcap - 1) / gcap : 0;
    }
    // item counts stay far below 2^31 / ncu (at most 1025 slots x 2^16 tiles), so 32-bit index math
    const int nsl = nu + (P.Is > 0 ? 1 : 0);  // COMB: slots per tile
    int u0, u1;
    if (early && nu == nrs && !COMB) {
        u0 = eu0;  // the range the early rows were requested for
        u1 = eu1;
    } else {
        urange(nu, nvr, nvs, u0, u1);
    }
    const int i0 = (HALVES ? u0 >> 1 : u0) * (COMB ? nsl : 1), i1 = (HALVES ? (u1 + 1) >> 1 : u1) * (COMB ? nsl : 1);
    if (i0 >= i1) return;  // uniform over the workgroup

    auto decode = [&](int i) {
        DItem it;
        const int tile = COMB ? i / nsl : 0;
        if (COMB) {
            const int sl = i - tile * nsl;
            it.slot = sl;
            it.tile = tile;
            it.ng = 1;
            if (sl < nu) {
                it.e = __builtin_amdgcn_readfirstlane(t_uniq[sl]);
                it.w = weight_row(P, it.e);
                it.shared = false;
                it.I = P.I;
                it.p0 = __builtin_amdgcn_readfirstlane(t_off[it.e]);
            } else {
                it.e = 0;
                it.w = 0;
                it.shared = true;
                it.I = P.Is;
                it.p0 = 0;
            }
        } else if (PASSES) {
            const int vs = i / tiles_r;
            it.slot = vs;
            it.tile = i % tiles_r;
            if (vs < nvr) {
                // routed slot of virtual slot vs: the last s with vpre[s] <= vs
                int lo = 0, hi = nu - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (vpre[mid] <= vs) lo = mid; else hi = mid - 1;
                }
                const int sl = __builtin_amdgcn_readfirstlane(lo);
                const int q = vs - __builtin_amdgcn_readfirstlane(vpre[sl]);
                it.e = __builtin_amdgcn_readfirstlane(t_uniq[sl]);
                it.w = weight_row(P, it.e);
                it.shared = false;
                it.I = P.I;
                const int o0 = __builtin_amdgcn_readfirstlane(t_off[it.e]);
                const int c = __builtin_amdgcn_readfirstlane(t_off[it.e + 1]) - o0;
                it.p0 = o0 + q * gcap;
                it.ng = min(gcap, c - q * gcap);
            } else {
                const int q = vs - nvr;
                it.e = 0;
                it.w = P.y_sh ? 0 : -1;  // y_sh = nullptr: the shared expert left out
                it.shared = true;
                it.I = P.Is;
                it.p0 = q * gcap;
                it.ng = min(gcap, T - q * gcap);
            }
        } else if (i < nu * tiles_r) {
            it.slot = i / tiles_r;
            it.tile = i % tiles_r;
            it.e = __builtin_amdgcn_readfirstlane(t_uniq[it.slot]);
            it.w = weight_row(P, it.e);
            it.shared = false;
            it.I = P.I;
            it.p0 = __builtin_amdgcn_readfirstlane(t_off[it.e]);
            it.ng = __builtin_amdgcn_readfirstlane(t_off[it.e + 1]) - it.p0;
        } else {
            it.slot = nrs;
            it.tile = i - nu * tiles_r;
            it.e = 0;
            it.w = P.y_sh ? 0 : -1;
            it.shared = true;
            it.I = P.Is;
            it.p0 = 0;
            it.ng = T;
        }
        const int K = MODE == 0 ? P.d : it.I;
        const int nout = MODE == 0 ? it.I : P.d;
        it.kpart_bytes = K / S * WBITS / 8;
        it.nseg_pad = ((it.kpart_bytes + 63) / 64 + PF - 1) / PF * PF;
        it.row = (it.tile * TPW + tile_w) * 16 + j;
        const int u = 2 * (COMB ? tile : i) + (j >> 3);  // half tile of this lane's row
        it.row_ok = it.row < nout && (!HALVES || (u >= u0 && u < u1)) && it.w >= 0;
        if (it.w < 0) it.w = 0;  // not resident: reads nothing (row_ok false), writes nothing
        return it;
    };
    auto weights = [&](const DItem &it, rsrc_t (&wr)[NM], uint32_t &lane_off) {
        const QW &W = it.shared ? P.shared : P.routed;
        const int K = MODE == 0 ? P.d : it.I;
        const int nout = MODE == 0 ? it.I : P.d;
        const long rb = (long)K * WBITS / 8;
        const uint32_t mbytes = (uint32_t)((long)nout * rb);
        if (MODE == 0) {
            wr[0] = make_rsrc(W.qg + (long)it.w * it.I * rb, mbytes);
            wr[NM - 1] = make_rsrc(W.qu + (long)it.w * it.I * rb, mbytes);
        } else {
            wr[0] = make_rsrc(W.qd + (long)it.w * P.d * rb, mbytes);
        }
        // rows past the output or outside this CU's half tiles read nothing
        lane_off = it.row_ok ? (uint32_t)((long)it.row * rb) + (uint32_t)(kp * it.kpart_bytes + 16 * g) : kOOB;
    };
    // down: rows of h of a slot (row r of the slot is h row p0 + r, or h_sh row r)
    auto h_src = [&](const DItem &it) {
        return make_rsrc(it.shared ? h_sh : h, (uint32_t)((long)(it.shared ? T : P.A) * it.I * 4));
    };

    // gate/up with token passes: the token of row r of an item's virtual slot (the shared expert's rows are the
    // tokens in order; a routed slot's are its assignments' tokens)
    auto gu_token = [&](const DItem &it, int r) -> int {
        return it.shared ? it.p0 + r : __builtin_amdgcn_readfirstlane(t_perm[it.p0 + r]) / P.k;
    };

    DItem cur = decode(i0);
    rsrc_t wr_cur[NM], wr_nxt[NM];
    uint32_t off_cur, off_nxt;
    weights(cur, wr_cur, off_cur);
    uint4 wbuf[PF][NM];
    auto ld = [&](int b, const rsrc_t (&wr)[NM], uint32_t lane_off, int kpart_bytes, int seg) {
        const uint32_t off = (64 * seg + 16 * g < kpart_bytes) ? lane_off + 64 * seg : kOOB;
#pragma unroll
        for (int m = 0; m < NM; m++) wbuf[b][m] = buf_load16(wr[m], off);
    };

    // ---- activations of the first item and the weight stream.  Gate/up stages first (its rows were
    // requested with the table): the staging code is cold at launch, and fetching it behind the whole
    // chip's first burst of weight requests costs more than the short gap before the stream starts.
    if (MODE == 0 && PASSES) {
        // token passes: the planes hold the rows of the first item's virtual slot (row r = its r-th token)
        const int kpart = kd / S;
        for (int r = tile_w; r < cur.ng; r += TPW) {
            const long ro = (long)gu_token(cur, r) * kd + kp * kpart;
            StageRaw<SRCX> raw;
            stage_issue<SRCX>(xsrc0, ro, 0, kpad / 8, kpart, raw);
            stage_finish<WBITS, SRCX>(raw, xsrc0, ro, r, kpad / 8, kpart, stride, pb, planes, wexpo[kp], wxsum[kp]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < PF; b++) ld(b, wr_cur, off_cur, cur.kpart_bytes, b);
    } else if (MODE == 0) {
        // rows tile_w, tile_w + TPW, ...: the next row is requested before this one is turned into digits
        const int kpart = kd / S;
        StageRaw<SRCX> rb;
        for (int r = tile_w; r < T; r += 2 * TPW) {
            const int r1 = r + TPW, r2 = r + 2 * TPW;
            if (r1 < T) stage_issue<SRCX>(xsrc0, (long)r1 * kd + kp * kpart, 0, kpad / 8, kpart, rb);
            stage_finish<WBITS, SRCX>(raw0, xsrc0, (long)r * kd + kp * kpart, r, kpad / 8, kpart, stride, pb, planes,
                                      wexpo[kp], wxsum[kp]);
            if (r1 < T) {
                if (r2 < T) stage_issue<SRCX>(xsrc0, (long)r2 * kd + kp * kpart, 0, kpad / 8, kpart, raw0);
                stage_finish<WBITS, SRCX>(rb, xsrc0, (long)r1 * kd + kp * kpart, r1, kpad / 8, kpart, stride, pb,
                                          planes, wexpo[kp], wxsum[kp]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < PF; b++) ld(b, wr_cur, off_cur, cur.kpart_bytes, b);
    } else if (COMB) {
        // the h rows of every slot, planes row r = slot r: each wavefront stages rows tile_w and
        // tile_w + TPW (the host keeps nsl <= 2 TPW), both requested before the weights
        auto row_src = [&](int r, rsrc_t &src, long &ro, int &kpart) {
            const bool sh = r >= nu;
            const int I = sh ? P.Is : P.I;
            kpart = I / S;
            const long p0 = sh ? 0 : __builtin_amdgcn_readfirstlane(t_off[__builtin_amdgcn_readfirstlane(t_uniq[r])]);
            src = make_rsrc(sh ? h_sh : h, (uint32_t)((long)(sh ? T : P.A) * I * 4));
            ro = p0 * I + kp * kpart;
        };
        const int r1 = tile_w, r2 = tile_w + TPW;
        const bool st1 = r1 < nsl, st2 = r2 < nsl;
        rsrc_t src1, src2;
        long ro1, ro2;
        int kpart1, kpart2;
        row_src(st1 ? r1 : 0, src1, ro1, kpart1);
        row_src(st2 ? r2 : 0, src2, ro2, kpart2);
        // rows requested with the table (one token) are used when they are the ones needed
        if (!(st1 && e_ro1 == ro1 && e_sh1 == (r1 >= nu)))
            stage_issue<SRCX>(src1, ro1, st1 ? 0 : kpad, kpad / 8, kpart1, raw1);
        if (!(st2 && e_ro2 == ro2 && e_sh2 == (r2 >= nu)))
            stage_issue<SRCX>(src2, ro2, st2 ? 0 : kpad, kpad / 8, kpart2, raw2);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < PF; b++) ld(b, wr_cur, off_cur, cur.kpart_bytes, b);
        __builtin_amdgcn_sched_barrier(0);
        if (st1)
            stage_finish<WBITS, SRCX>(raw1, src1, ro1, r1, kpad / 8, kpart1, stride, pb, planes, wexpo[kp],
                                      wxsum[kp]);
        if (st2)
            stage_finish<WBITS, SRCX>(raw2, src2, ro2, r2, kpad / 8, kpart2, stride, pb, planes, wexpo[kp],
                                      wxsum[kp]);
    } else {
        // Rows of h: those of the slot are known only after the table round.  Each staging wavefront's
        // first row is requested before any wavefront starts its weights (when fewer rows than tiles
        // per item leave wavefronts without staging work, their weight requests would otherwise
        // queue ahead of the rows in the CU's memory pipeline); the digits are made while the weight
        // stream starts.
        const rsrc_t src = h_src(cur);
        const int kpart = cur.I / S;
        const long base = cur.p0;
        const bool st1 = tile_w < cur.ng;
        const long ro1 = (base + tile_w) * cur.I + kp * kpart;
        // the row requested with the table (one token) is used when it is the one needed
        if (!(st1 && e_ro1 == ro1 && e_sh1 == cur.shared))
            stage_issue<SRCX>(src, ro1, st1 ? 0 : kpad, kpad / 8, kpart, raw1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < PF; b++) ld(b, wr_cur, off_cur, cur.kpart_bytes, b);
        __builtin_amdgcn_sched_barrier(0);
        if (st1) stage_finish<WBITS, SRCX>(raw1, src, ro1, tile_w, kpad / 8, kpart, stride, pb, planes, wexpo[kp], wxsum[kp]);
        for (int r = tile_w + TPW; r < cur.ng; r += TPW) {
            const long ro = (base + r) * cur.I + kp * kpart;
            StageRaw<SRCX> raw;
            stage_issue<SRCX>(src, ro, 0, kpad / 8, kpart, raw);
            stage_finish<WBITS, SRCX>(raw, src, ro, r, kpad / 8, kpart, stride, pb, planes, wexpo[kp], wxsum[kp]);
        }
    }
    __syncthreads();  // planes and exponents

    int staged_slot = cur.slot;
    for (int i = i0; i < i1; i++) {
        const bool has_next = i + 1 < i1;
        DItem nxt = cur;
        if (has_next) {
            nxt = decode(i + 1);
            weights(nxt, wr_nxt, off_nxt);
        } else {
            // no next item: keep a valid descriptor; its refills use an out-of-range offset
#pragma unroll
            for (int m = 0; m < NM; m++) wr_nxt[m] = wr_cur[m];
            off_nxt = off_cur;
        }
        // ---- gate/up with token passes: the activation rows of a new virtual slot
        if (MODE == 0 && PASSES && cur.slot != staged_slot) {
            const int kpart = kd / S;
            __syncthreads();  // every wavefront is done reading the previous planes
            for (int r = tile_w; r < cur.ng; r += TPW) {
                const long ro = (long)gu_token(cur, r) * kd + kp * kpart;
                StageRaw<SRCX> raw;
                stage_issue<SRCX>(xsrc0, ro, 0, kpad / 8, kpart, raw);
                stage_finish<WBITS, SRCX>(raw, xsrc0, ro, r, kpad / 8, kpart, stride, pb, planes, wexpo[kp],
                                          wxsum[kp]);
            }
            __syncthreads();
        }
        // ---- down: the rows of h of a new slot
        if (MODE == 1 && !COMB && cur.slot != staged_slot) {
            const rsrc_t src = h_src(cur);
            const int kpart = cur.I / S;
            const long base = cur.p0;
            __syncthreads();  // every wavefront is done reading the previous planes
            for (int r = tile_w; r < cur.ng; r += TPW) {
                const long ro = (base + r) * cur.I + kp * kpart;
                StageRaw<SRCX> raw;
                stage_issue<SRCX>(src, ro, 0, kpad / 8, kpart, raw);
                stage_finish<WBITS, SRCX>(raw, src, ro, r, kpad / 8, kpart, stride, pb, planes, wexpo[kp],
                                          wxsum[kp]);
            }
            __syncthreads();
        }
        staged_slot = cur.slot;

        // ---- A-operand row of this lane: the token (gate/up) or slot row (down) at position j
        int trow = -1;
        if (j < cur.ng) trow = MODE == 0 && !PASSES ? (cur.shared ? j : t_perm[cur.p0 + j] / P.k) : (COMB ? cur.slot : j);
        const bool tok_ok = trow >= 0;
        const int8_t *xrow = tok_ok ? planes + (long)trow * stride : (const int8_t *)zero_area;
        const long pstep = tok_ok ? pb : 0;
        const int gstep = tok_ok ? 1 : 0;

        // ---- the item's segments
        i32x4_t C[NM][3];
#pragma unroll
        for (int m = 0; m < NM; m++)
#pragma unroll
            for (int p = 0; p < 3; p++) C[m][p] = (i32x4_t){0, 0, 0, 0};
        int seg0 = 0;
        for (; seg0 + PF < cur.nseg_pad; seg0 += PF) {
#pragma unroll
            for (int b = 0; b < PF; b++) {
                consume_segment<WBITS, NM>(wbuf[b], xrow, pstep, gstep, seg0 + b, g, C);
                __builtin_amdgcn_sched_barrier(0);
                ld(b, wr_cur, off_cur, cur.kpart_bytes, seg0 + PF + b);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // last batch, peeled: the per-row zero points and scales are requested first, then the refills
        // start the next item (or read nothing), so the epilogue waits only for what it uses
        const QW &W = cur.shared ? P.shared : P.routed;
        const int nout = MODE == 0 ? cur.I : P.d;
        const int rowc = cur.row_ok ? min(cur.row, nout - 1) : 0;
        float zrow[NM], srow[NM];
        if (MODE == 0) {
            const long ch = (long)cur.w * cur.I + rowc;
            zrow[0] = zp_val(W.zg, WBITS, ch);
            zrow[NM - 1] = zp_val(W.zu, WBITS, ch);
            srow[0] = W.sg[ch];
            srow[NM - 1] = W.su[ch];
        } else {
            const long ch = (long)cur.w * P.d + rowc;
            zrow[0] = zp_val(W.zd, WBITS, ch);
            srow[0] = W.sd[ch];
        }
        __builtin_amdgcn_sched_barrier(0);
        const int kpb_nxt = has_next ? nxt.kpart_bytes : 0;
#pragma unroll
        for (int b = 0; b < PF; b++) {
            consume_segment<WBITS, NM>(wbuf[b], xrow, pstep, gstep, seg0 + b, g, C);
            __builtin_amdgcn_sched_barrier(0);
            ld(b, wr_nxt, off_nxt, kpb_nxt, b);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- exact partial of this wavefront, zero point applied and scale undone, in fp64; register r
        // of lane group g holds position 4g + r of the slot
        double v[NM][4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int i2 = 4 * g + r;
            const bool ok = i2 < cur.ng;
            const int pr = ok ? (MODE == 0 && !PASSES ? (cur.shared ? i2 : t_perm[cur.p0 + i2] / P.k) : (COMB ? cur.slot : i2))
                              : 0;
            const double unit = ok ? ldexp(1.0, -wexpo[kp][pr]) : 0.0;
            const double xs = ok ? wxsum[kp][pr] : 0.0;
#pragma unroll
            for (int m = 0; m < NM; m++) {
                const double dot = (double)C[m][2][r] * 65536.0 + (double)C[m][1][r] * 256.0 + (double)C[m][0][r];
                v[m][r] = (dot - (double)zrow[m] * xs) * unit;
            }
        }
        if (S > 1) {
            __syncthreads();  // the previous item's partials have been read
#pragma unroll
            for (int m = 0; m < NM; m++)
#pragma unroll
                for (int r = 0; r < 4; r++) red[((wv * NM + m) * 4 + r) * 64 + lane] = v[m][r];
            __syncthreads();
            if (kp == 0) {
#pragma unroll
                for (int m = 0; m < NM; m++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        double a = v[m][r];
                        for (int q = 1; q < S; q++) a += red[(((wv + q) * NM + m) * 4 + r) * 64 + lane];
                        v[m][r] = a;
                    }
            }
        }
        if (kp == 0 && cur.row_ok) {
            const int o = cur.row;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int i2 = 4 * g + r;
                if (i2 < cur.ng) {
                    if (MODE == 0) {
                        const float gf = (float)((double)srow[0] * v[0][r]);
                        const float uf = (float)((double)srow[NM - 1] * v[NM - 1][r]);
                        const float hv = gf / (1.f + expf(-gf)) * uf;
                        if (cur.shared)
                            h_sh[(long)(cur.p0 + i2) * cur.I + o] = hv;
                        else
                            h[(long)(cur.p0 + i2) * cur.I + o] = hv;
                    } else {
                        const float y = (float)((double)srow[0] * v[0][r]);
                        if (cur.shared)
                            P.y_sh[(long)(cur.p0 + i2) * P.d + o] = y;
                        else
                            P.y_perm[(long)(cur.p0 + i2) * P.d + o] = y;
                        if (COMB) {
                            // the same lane holds row o for every slot of the tile: the last slot combines
                            ycomb[wv][cur.slot][j] = y;
                            if (cur.slot == nsl - 1) {
                                float acc = P.Is > 0 ? ycomb[wv][nu][j] : 0.f;
                                for (int c = 0; c < P.k; c++) {
                                    const int p = c_inv[c];
                                    if (p >= 0 && p < nu) acc = fmaf(c_w[c], ycomb[wv][p][j], acc);
                                }
                                P.comb_y[o] = acc;
                            }
                        }
                    }
                }
            }
        }
        cur = nxt;
#pragma unroll
        for (int m = 0; m < NM; m++) wr_cur[m] = wr_nxt[m];
        off_cur = off_nxt;
    }
}

// ---------------------------------------------------------------------------- host side

static int pad_k(int K, int wbits) {
    const int seg_inputs = wbits == 8 ? 64 : 128;
    return (K + seg_inputs - 1) / seg_inputs * seg_inputs;
}

// K split: the largest S in {4, 2, 1} that keeps whole 16-byte chunks per wavefront and leaves each
// wavefront at least 16 segments of 64 bytes per row (short rows: one wavefront per tile over the
// whole row, no cross-wave reduction).
static int pick_s(int mode, int K, int wbits) {
    (void)mode;
    const int chunk_inputs = wbits == 8 ? 16 : 32;
    const int nseg_full = (K * wbits / 8 + 63) / 64;
    for (int S = 4; S >= 2; S >>= 1) {
        if (K % (S * chunk_inputs)) continue;
        if (nseg_full / S < 16) continue;
        return S;
    }
    return 1;
}

// bytes of cross-wave partials (fp64): 4 wavefronts x NM matrices x 4 registers x 64 lanes
static size_t dk_red_bytes(int mode) { return (size_t)4 * (mode == 0 ? 2 : 1) * 4 * 64 * 8; }

// Tokens per pass: as many as the digit planes of the four wavefronts can hold, at most DK_GMAX.
static int dk_gmax(int T, int kpad) {
    int fit = DK_LDS_BUDGET / (4 * 3 * (kpad + 16));
    if (fit > DK_GMAX) fit = DK_GMAX;
    if (fit < 1) fit = 1;
    return T < fit ? T : fit;
}

static size_t dk_lds_bytes(int mode, int kpad, int gmax) {
    const size_t planes = (size_t)4 * 3 * gmax * (kpad + 16);
    const size_t red = dk_red_bytes(mode);
    return planes > red ? planes : red;
}

const char *decode_unsupported(const FfnParams &P) {
    const long Imax = P.I > P.Is ? P.I : P.Is;
    if ((long)P.T * P.d * (P.act == 0 ? 4 : 2) >= kMaxDescBytes) return "x exceeds 2^31 bytes";
    if (Imax * ((long)P.d * P.wbits / 8) >= kMaxDescBytes) return "one expert weight matrix exceeds 2^31 bytes";
    if ((long)P.A * P.I * 4 >= kMaxDescBytes) return "h of the routed rows (T*k*I fp32) exceeds 2^31 bytes";
    if ((long)P.T * P.Is * 4 >= kMaxDescBytes) return "h of the shared expert (T*I_shared fp32) exceeds 2^31 bytes";
    return nullptr;
}

size_t decode_workspace_bytes(const FfnParams &P) {
    const size_t hb = ((size_t)P.A * P.I * sizeof(float) + 255) & ~(size_t)255;
    const size_t hs = ((size_t)P.T * P.Is * sizeof(float) + 255) & ~(size_t)255;
    return hb + hs;
}

static int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    return n;
}

template <typename F>
static hipError_t allow_lds(F fn, size_t lds) {
    if (lds <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// ---- persistent path (every slot's tokens fit one pass of the digit-plane LDS)

constexpr size_t DKP_LDS_BUDGET = 150 * 1024;  // routing table + digit planes (one copy per K part) + partials

static size_t dkp_red_bytes(int mode) { return (size_t)DKP_WAVES * (mode == 0 ? 2 : 1) * 4 * 64 * 8; }

// Weight loads in flight per wavefront and matrix: 8 or 7 for gate/up (two matrices), 16 or 14 for down, 16
// loads of 1 KB either way.  An item's segments are consumed in batches of PF, the last one padded with
// loads that read nothing; a padded place carries no data, so fewer bytes are in flight while it waits.
// The depth that pads least is taken (7 for the 7 segments of the large workload's gate/up wavefronts, 14
// for the 28 of the mid workload's down wavefronts); ties go to the deeper one.
static int dkp_pf(int mode, int nseg) {
    const int a = mode == 0 ? 8 : 16, b = mode == 0 ? 7 : 14;
    const int pad_a = (nseg + a - 1) / a * a - nseg, pad_b = (nseg + b - 1) / b * b - nseg;
    return pad_b < pad_a ? b : a;
}

// K split of the persistent kernel: the S in {8, 4, 2, 1} (whole 16-byte chunks per wavefront).
// Gate/up: the least work on the busiest CU at the largest possible slot count, counted as items x tiles
// per item x segments padded to the prefetch depth; ties go to the smaller S.  Down: a wavefront streams
// items x segments padded to the prefetch depth (a padded segment costs its place in the stream though it
// reads nothing), at the expected number of slots -- uniform routing hits E (1 - (1 - k/E)^T) experts, and
// skewed routing fewer -- with items counted in half tiles when a tile is an item (its ranges are cut in
// half tiles); ties go to the larger S.
static int dkp_pick_s(int mode, int K, int nout, int slots, double slots_exp, int wbits, int ncu, int smax = DKP_WAVES) {
    const int chunk_inputs = wbits == 8 ? 16 : 32;
    const int nseg_full = (K * wbits / 8 + 63) / 64;
    int best = 1;
    double best_cost = -1;
    for (int i = 0; i < 4; i++) {
        const int S = mode == 0 ? 1 << i : DKP_WAVES >> i;
        if (S > smax || K % (S * chunk_inputs)) continue;
        const int tpw = DKP_WAVES / S;
        const int nseg = (nseg_full + S - 1) / S;
        const int pf = dkp_pf(mode, nseg);
        const int nseg_pad = (nseg + pf - 1) / pf * pf;
        const long tiles = (nout + 16 * tpw - 1) / (16 * tpw);
        double cost;
        if (mode == 0) {
            const long items = (long)slots * tiles;
            cost = (double)((items + ncu - 1) / ncu) * tpw * nseg_pad;
        } else {
            const double items = slots_exp * (double)tiles;
            const double per_cu = tpw == 1 ? std::ceil(2.0 * items / ncu) / 2.0 : std::ceil(items / ncu);
            cost = per_cu * nseg_pad;
        }
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = S;
        }
    }
    return best;
}

// K split of pass `mode` in the batch-invariant mode: the split dkp_pick_s's cost rule gives for one token, capped
// at 4 (the token-group kernel's largest), and dividing both the routed and the shared K range.  It depends on the
// layer's shape alone, so a token's staged fixed point and its order of sums are the same at every T.
static int decode_pinned_s(int mode, const FfnParams &P) {
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int K = mode == 0 ? P.d : Imax;
    const int Kmin = mode == 0 ? P.d : (P.Is > 0 && P.Is < P.I ? P.Is : P.I);
    const int nout = mode == 0 ? Imax : P.d;
    const int shared = P.Is > 0 ? 1 : 0;
    const int rslots = P.E < P.k ? P.E : P.k;  // routed slots of one token
    int S = dkp_pick_s(mode, K, nout, rslots + shared, (double)rslots + shared, P.wbits, device_cus(), 4);
    while (S > 1 && (Kmin % (S * (P.wbits == 8 ? 16 : 32)) || K % (S * (P.wbits == 8 ? 16 : 32)))) S >>= 1;
    return S;
}

// LDS of the persistent kernel with digit planes for g token rows (g < T: token passes, which add the
// virtual-slot prefix after the routing table)
static size_t dkp_lds_bytes(int mode, int S, const FfnParams &P, int kpad, int g) {
    const int words = dkp_tab_words(mode, P.n_routed_slots, P.E, P.A) + (g < P.T ? P.n_routed_slots + 2 : 0);
    const size_t tab = ((size_t)words * 4 + 15) & ~(size_t)15;
    return tab + (size_t)S * 3 * g * (kpad + 16) + dkp_red_bytes(mode);
}

// Gate/up split outside the batch-invariant mode.  The weight stream is the bound, and it runs at full rate
// while most CUs stream, so fewer and longer items win (less per-item work: the cross-wavefront sum of the K
// parts, the epilogue, the refill across items) as long as the last round of items keeps most CUs busy.
// One token (the slot count is exact): the smallest S in {1, 2, 4} whose items per CU, R = items / CUs, are at
// least 1.5 with the last round at least 3/4 full.  The mid workload's token (2 slots of 14336 rows) takes
// S = 2, R = 1.75; the 256-expert layer's (9 slots of 2048 rows) keeps S = 8, whose half-tile ranges balance to
// 8 rows where S = 4 would leave a last round a quarter full.  Several tokens (the slot count is an estimate,
// which skewed routing lowers): S = 4 while R >= 3 at the expected slot count.  Measured at 2 to 16 tokens on
// both layers, S = 4 beat S = 8 by 1.6-4 % at 2 and 4 tokens and on the mid layer at 8, and tied elsewhere;
// S = 2 also beat S = 8, by less than S = 4 on the mid layer; S = 1 lost up to 7 % to S = 8 on the mid layer
// (it won on the 256-expert layer at 4 tokens).  0: none qualifies (dkp_pick_s decides).  The planes must hold
// one token row; tokens beyond what they hold are taken in passes.
static int dkp_pick_s0(const FfnParams &P, double slots) {
    const int chunk = P.wbits == 8 ? 16 : 32, ncu = device_cus();
    const double shared = P.Is > 0 ? 1.0 : 0.0;
    for (int S = P.T == 1 ? 1 : 4; S <= 4; S <<= 1) {
        if (P.d % (S * chunk)) continue;
        const int rows = 16 * (DKP_WAVES / S);
        const double items = (slots - shared) * ((P.I + rows - 1) / rows) + shared * ((P.Is + rows - 1) / rows);
        const double R = items / ncu, fill = R - std::floor(R);
        const bool ok = P.T == 1 ? R >= 1.5 && (fill == 0.0 || fill >= 0.75) : R >= 3.0;
        // the planes must hold one token row at least (more tokens than fit are taken in passes)
        if (ok && dkp_lds_bytes(0, S, P, pad_k(P.d / S, P.wbits), 1) <= DKP_LDS_BUDGET) return S;
    }
    return 0;
}

template <int MODE, int WBITS, int SRC, int S, int PF, bool PASSES, bool COMB = false>
static hipError_t dkp_launch_s(const FfnParams &P, float *h, float *h_sh, int kpad, int gcap, hipStream_t stream) {
    const int rows_per_item = 16 * (DKP_WAVES / S);
    int tiles_r = ((MODE == 0 ? P.I : P.d) + rows_per_item - 1) / rows_per_item;
    int tiles_s = P.Is > 0 ? ((MODE == 0 ? P.Is : P.d) + rows_per_item - 1) / rows_per_item : 0;
    // token passes number every virtual slot's items alike: gate/up counts the larger of the two expert widths
    if (MODE == 0 && PASSES && tiles_s > tiles_r) tiles_r = tiles_s;
    if (MODE == 0 && PASSES && tiles_s > 0) tiles_s = tiles_r;
    const size_t lds = dkp_lds_bytes(MODE, S, P, kpad, gcap);
    auto fn = decode_persistent_kernel<MODE, WBITS, SRC, S, PF, PASSES, COMB>;
    hipError_t err = allow_lds(fn, lds);
    if (err != hipSuccess) return err;
    const int ncu = device_cus();
    // at most: every routed assignment its own virtual slot when passes split the slots
    const long vslots = PASSES ? (long)P.A + (P.Is > 0 ? (P.T + gcap - 1) / gcap : 0) : 0;
    const long items = PASSES ? vslots * tiles_r : (long)P.n_routed_slots * tiles_r + tiles_s;
    long grid = ncu;
    if (grid > items) grid = items;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(DKP_WAVES * 64), lds, stream, P, h, h_sh, kpad, tiles_r,
                       tiles_s, ncu, gcap);
    return hipGetLastError();
}

// The down pass with token passes (instantiated for the down kernel only).
template <int MODE, int WBITS, int SRC>
static hipError_t dkp_launch_pass(const FfnParams &P, float *h, float *h_sh, int kpad, int gcap, int S, bool deep,
                                  hipStream_t stream) {
    constexpr int PFA = MODE == 0 ? 8 : 16, PFB = MODE == 0 ? 7 : 14;
    switch (S) {
        case 8: return deep ? dkp_launch_s<MODE, WBITS, SRC, 8, PFA, true>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 8, PFB, true>(P, h, h_sh, kpad, gcap, stream);
        case 4: return deep ? dkp_launch_s<MODE, WBITS, SRC, 4, PFA, true>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 4, PFB, true>(P, h, h_sh, kpad, gcap, stream);
        case 2: return deep ? dkp_launch_s<MODE, WBITS, SRC, 2, PFA, true>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 2, PFB, true>(P, h, h_sh, kpad, gcap, stream);
        default: return deep ? dkp_launch_s<MODE, WBITS, SRC, 1, PFA, true>(P, h, h_sh, kpad, gcap, stream)
                             : dkp_launch_s<MODE, WBITS, SRC, 1, PFB, true>(P, h, h_sh, kpad, gcap, stream);
    }
}

// The persistent kernel's K split, padded K part and token rows per pass for pass `mode`; false when the
// token-group kernel takes the pass instead.  With the combine in the down launch (P.comb_y), the planes hold
// the rows of every slot of the token, and false means that form does not fit.
struct DkpPlan {
    int S, kpad, gcap;
};
static bool dkp_plan(int mode, const FfnParams &P, DkpPlan *pl) {
    const int wbits = P.wbits;
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int K = mode == 0 ? P.d : Imax;
    const int Kmin = mode == 0 ? P.d : (P.Is > 0 && P.Is < P.I ? P.Is : P.I);
    const int nout = mode == 0 ? Imax : P.d;
    const int slots = P.n_routed_slots + (P.Is > 0 ? 1 : 0);
    const double uniq_exp = (double)P.E * (1.0 - std::pow(1.0 - (double)P.k / P.E, (double)P.T));
    const double slots_exp = std::min((double)P.n_routed_slots, uniq_exp) + (P.Is > 0 ? 1 : 0);
    // routed and shared expert split alike: the split must divide both K ranges
    int S = P.invariant || mode == 1 ? 0 : dkp_pick_s0(P, P.T == 1 ? slots : slots_exp);
    if (S == 0)
        S = P.invariant ? decode_pinned_s(mode, P) : dkp_pick_s(mode, K, nout, slots, slots_exp, wbits, device_cus());
    while (S > 1 && (Kmin % (S * (wbits == 8 ? 16 : 32)))) S >>= 1;
    const int kpad = pad_k(K / S, wbits);
    if (dkp_tab_words(mode, P.n_routed_slots, P.E, P.A) > DKP_TAB_PER_THREAD * DKP_WAVES * 64) return false;
    if (mode == 1 && P.comb_y) {
        // each wavefront stages at most two rows (nsl <= 2 TPW), and the ranges, cut at tiles so that a
        // workgroup holds every slot of its rows, give the busiest CU no more items than the plain split
        const int nsl = P.n_routed_slots + (P.Is > 0 ? 1 : 0);
        const int tpw = DKP_WAVES / S, ncu = device_cus();
        const long tiles = (P.d + 16 * tpw - 1) / (16 * tpw), units = tpw == 1 ? 2 * tiles : tiles;
        if (P.T != 1 || nsl > DK_GMAX || nsl > 2 * tpw || dkp_lds_bytes(1, S, P, kpad, nsl) > DKP_LDS_BUDGET)
            return false;
        if ((units + ncu - 1) / ncu * nsl > (units * nsl + ncu - 1) / ncu) return false;
        *pl = DkpPlan{S, kpad, nsl};
        return true;
    }
    // token rows the planes hold: all T, or fewer (at most DK_GMAX, the MFMA rows), with the slots taken in passes
    int gcap = P.T < DK_GMAX ? P.T : DK_GMAX;
    while (gcap > 0 && dkp_lds_bytes(mode, S, P, kpad, gcap) > DKP_LDS_BUDGET) gcap--;
    if (gcap < 1) return false;
    *pl = DkpPlan{S, kpad, gcap};
    return true;
}

bool decode_combines(const FfnParams &P) {
    DkpPlan pl;
    return P.T == 1 && P.comb_y && P.k <= DK_GMAX && dkp_plan(1, P, &pl);
}

bool decode_routes(const FfnParams &P) {
    DkpPlan pl;
    if (P.T != 1 || P.E > 256 || P.k > 64 || !dkp_plan(0, P, &pl)) return false;
    // the selection's scores and ids borrow the digit planes' LDS before the activations are staged
    return (size_t)pl.S * 3 * pl.gcap * (pl.kpad + 16) >= (size_t)32 * P.E + (size_t)4 * P.k;
}

// Launches the persistent kernel if the digit planes of all T tokens fit (for the down pass: of at least one
// token, the slots then taken in passes); *done tells whether it did.
template <int MODE, int WBITS, int SRC>
static hipError_t dkp_try(const FfnParams &P, float *h, float *h_sh, hipStream_t stream, bool *done) {
    *done = false;
    DkpPlan pl;
    if (!dkp_plan(MODE, P, &pl)) return hipSuccess;
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int K = MODE == 0 ? P.d : Imax;
    const int S = pl.S, kpad = pl.kpad, gcap = pl.gcap;
    *done = true;
    constexpr int PFA = MODE == 0 ? 8 : 16, PFB = MODE == 0 ? 7 : 14;
    const bool deep = dkp_pf(MODE, (K / S * WBITS / 8 + 63) / 64) == PFA;
    if (gcap < P.T) return dkp_launch_pass<MODE, WBITS, SRC>(P, h, h_sh, kpad, gcap, S, deep, stream);
    if constexpr (MODE == 1) {
        if (P.comb_y) {
            switch (S) {
                case 8: return deep ? dkp_launch_s<1, WBITS, SRC, 8, PFA, false, true>(P, h, h_sh, kpad, gcap, stream)
                                    : dkp_launch_s<1, WBITS, SRC, 8, PFB, false, true>(P, h, h_sh, kpad, gcap, stream);
                case 4: return deep ? dkp_launch_s<1, WBITS, SRC, 4, PFA, false, true>(P, h, h_sh, kpad, gcap, stream)
                                    : dkp_launch_s<1, WBITS, SRC, 4, PFB, false, true>(P, h, h_sh, kpad, gcap, stream);
                case 2: return deep ? dkp_launch_s<1, WBITS, SRC, 2, PFA, false, true>(P, h, h_sh, kpad, gcap, stream)
                                    : dkp_launch_s<1, WBITS, SRC, 2, PFB, false, true>(P, h, h_sh, kpad, gcap, stream);
                default: return deep ? dkp_launch_s<1, WBITS, SRC, 1, PFA, false, true>(P, h, h_sh, kpad, gcap, stream)
                                     : dkp_launch_s<1, WBITS, SRC, 1, PFB, false, true>(P, h, h_sh, kpad, gcap, stream);
            }
        }
    }
    switch (S) {
        case 8: return deep ? dkp_launch_s<MODE, WBITS, SRC, 8, PFA, false>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 8, PFB, false>(P, h, h_sh, kpad, gcap, stream);
        case 4: return deep ? dkp_launch_s<MODE, WBITS, SRC, 4, PFA, false>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 4, PFB, false>(P, h, h_sh, kpad, gcap, stream);
        case 2: return deep ? dkp_launch_s<MODE, WBITS, SRC, 2, PFA, false>(P, h, h_sh, kpad, gcap, stream)
                            : dkp_launch_s<MODE, WBITS, SRC, 2, PFB, false>(P, h, h_sh, kpad, gcap, stream);
        default: return deep ? dkp_launch_s<MODE, WBITS, SRC, 1, PFA, false>(P, h, h_sh, kpad, gcap, stream)
                             : dkp_launch_s<MODE, WBITS, SRC, 1, PFB, false>(P, h, h_sh, kpad, gcap, stream);
    }
}

// ---- token-group path (large T): one workgroup per (row block, slot), tokens in passes of gmax

template <int MODE, int WBITS, int SRC, int S>
static hipError_t dk_launch_s(const FfnParams &P, float *h, float *h_sh, int kpad, int gmax, hipStream_t stream) {
    const int slots = P.n_routed_slots + (P.Is > 0 ? 1 : 0);
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int rows_per_item = 16 * (4 / S);
    const size_t lds = dk_lds_bytes(MODE, kpad, gmax);
    auto fn = decode_kernel<MODE, WBITS, SRC, S>;
    hipError_t err = allow_lds(fn, lds);
    if (err != hipSuccess) return err;
    const int nout = MODE == 0 ? Imax : P.d;
    dim3 grid((nout + rows_per_item - 1) / rows_per_item, slots);
    hipLaunchKernelGGL(fn, grid, dim3(DK_THREADS), lds, stream, P, h, h_sh, gmax, kpad);
    return hipGetLastError();
}

template <int MODE, int WBITS, int SRC>
static hipError_t dk_launch_mode(const FfnParams &P, float *h, float *h_sh, hipStream_t stream) {
    // only the persistent kernel routes, and combines
    if (MODE == 0 && P.route.part && !decode_routes(P)) return hipErrorInvalidValue;
    if (MODE == 1 && P.comb_y && !decode_combines(P)) return hipErrorInvalidValue;
    bool done = false;
    hipError_t err = dkp_try<MODE, WBITS, SRC>(P, h, h_sh, stream, &done);
    if (done || err != hipSuccess) return err;
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int K = MODE == 0 ? P.d : Imax;
    // both the routed and the shared expert must split the same way: use the smaller intermediate size
    const int Kmin = MODE == 0 ? P.d : (P.Is > 0 && P.Is < P.I ? P.Is : P.I);
    const int S = P.invariant ? decode_pinned_s(MODE, P)
                  : pick_s(MODE, Kmin, WBITS) < pick_s(MODE, K, WBITS) ? pick_s(MODE, Kmin, WBITS)
                                                                      : pick_s(MODE, K, WBITS);
    const int kpad = pad_k(K / S, WBITS);  // the largest wavefront K part, padded to whole segments
    const int gmax = dk_gmax(P.T, kpad);
    if (S == 4) return dk_launch_s<MODE, WBITS, SRC, 4>(P, h, h_sh, kpad, gmax, stream);
    if (S == 2) return dk_launch_s<MODE, WBITS, SRC, 2>(P, h, h_sh, kpad, gmax, stream);
    return dk_launch_s<MODE, WBITS, SRC, 1>(P, h, h_sh, kpad, gmax, stream);
}

template <int WBITS, int SRC>
static hipError_t dk_launch(const FfnParams &P, float *h, float *h_sh, hipStream_t stream) {
    hipError_t err = dk_launch_mode<0, WBITS, SRC>(P, h, h_sh, stream);
    if (err != hipSuccess) return err;
    return dk_launch_mode<1, WBITS, 0>(P, h, h_sh, stream);
}

hipError_t launch_ffn_decode(const FfnParams &P, void *ws, hipStream_t stream) {
    float *h = (float *)ws;
    float *h_sh = (float *)((char *)ws + (((size_t)P.A * P.I * sizeof(float) + 255) & ~(size_t)255));
    if (P.wbits == 4)
        return P.act == 0 ? dk_launch<4, 0>(P, h, h_sh, stream) : dk_launch<4, 1>(P, h, h_sh, stream);
    return P.act == 0 ? dk_launch<8, 0>(P, h, h_sh, stream) : dk_launch<8, 1>(P, h, h_sh, stream);
}

}  // namespace moe
