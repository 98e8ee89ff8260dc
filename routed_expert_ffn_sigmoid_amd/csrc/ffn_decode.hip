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
// The input row is put into 24-bit fixed point with a per-token power-of-two
// scale, x_k ~= X_k * 2^-e (|X_k| < 2^22), and X_k is written as three signed
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
// A workgroup is 4 wavefronts covering TPW = 4/S tiles of 16 rows; the S
// wavefronts of a tile split K and add their fp64 partials in a fixed order.
// The first PF segments of every row are requested before the slot's token
// list is read and before the activations are staged; the segment loop is
// padded to a multiple of PF with out-of-range (zero) loads, so it is
// straight-line code with PF segments in flight per row.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int DK_THREADS = 256;
constexpr int DK_GMAX = 16;               // tokens per pass: the MFMA M dimension
constexpr int DK_LDS_BUDGET = 150 * 1024; // digit planes + reduction buffer

struct DSlot {
    int e, I;
    bool shared;
};

// Expert of a grid slot; routed slots past the unique list hold -1 and exit.
__device__ __forceinline__ bool dk_slot(const FfnParams &P, int slot, DSlot &s) {
    if (slot < P.n_routed_slots) {
        const int e = P.uniq[slot];
        if (e < 0) return false;
        s.e = e;
        s.I = P.I;
        s.shared = false;
    } else {
        s.e = 0;
        s.I = P.Is;
        s.shared = true;
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
template <int WBITS, int SRC>
__device__ void wave_stage(rsrc_t src, long rowoff_lane, int ng, int k0, int kpart, int kpad, int stride,
                           long plane_bytes, int8_t *planes, int *expo, double *xsum) {
    const int lane = threadIdx.x & 63;
    const int ngr = kpad / 8;  // groups of 8 inputs, zero past kpart
    constexpr int MAXG = 2;    // groups per lane held in registers (kpart <= 1024)
    const int esz = SRC == 0 ? 4 : 2;
    for (int i = 0; i < ng; i++) {
        const long ro = __shfl(rowoff_lane, i, 64) + k0;  // element offset of this row's first input
        float v[MAXG][8];
        float mx = 0.f;
#pragma unroll
        for (int c = 0; c < MAXG; c++) {
            const int m = lane + 64 * c;
            load8<SRC>(src, (m < ngr && m * 8 < kpart) ? (uint32_t)((ro + (long)m * 8) * esz) : kOOB, v[c]);
#pragma unroll
            for (int t = 0; t < 8; t++) mx = fmaxf(mx, fabsf(v[c][t]));
        }
        for (int m = lane + 64 * MAXG; m < ngr; m += 64) {  // K parts longer than 1024 inputs
            float xv[8];
            load8<SRC>(src, m * 8 < kpart ? (uint32_t)((ro + (long)m * 8) * esz) : kOOB, xv);
#pragma unroll
            for (int t = 0; t < 8; t++) mx = fmaxf(mx, fabsf(xv[t]));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
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
            int d0[8], d1[8], d2[8];
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int X = (int)rintf(xv[t] * sc);
                ssum += X;
                d0[t] = (X << 24) >> 24;
                const int r = (X - d0[t]) >> 8;
                d1[t] = (r << 24) >> 24;
                d2[t] = (r - d1[t]) >> 8;
            }
            auto pack4 = [](const int *d) {
                return (uint32_t)(d[0] & 255) | ((uint32_t)(d[1] & 255) << 8) | ((uint32_t)(d[2] & 255) << 16) |
                       ((uint32_t)(d[3] & 255) << 24);
            };
            if (WBITS == 8) {
                const int pos = m * 8;
                *(uint2 *)(p0 + pos) = make_uint2(pack4(d0), pack4(d0 + 4));
                *(uint2 *)(p1 + pos) = make_uint2(pack4(d1), pack4(d1 + 4));
                *(uint2 *)(p2 + pos) = make_uint2(pack4(d2), pack4(d2 + 4));
            } else {
                // inputs 8m..8m+7: evens go to plane_pos(8m), odds to plane_pos(8m+1)
                const int pe = plane_pos<4>(m * 8), po = plane_pos<4>(m * 8 + 1);
                int ev[4], od[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    ev[t] = d0[2 * t];
                    od[t] = d0[2 * t + 1];
                }
                *(uint32_t *)(p0 + pe) = pack4(ev);
                *(uint32_t *)(p0 + po) = pack4(od);
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    ev[t] = d1[2 * t];
                    od[t] = d1[2 * t + 1];
                }
                *(uint32_t *)(p1 + pe) = pack4(ev);
                *(uint32_t *)(p1 + po) = pack4(od);
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    ev[t] = d2[2 * t];
                    od[t] = d2[2 * t + 1];
                }
                *(uint32_t *)(p2 + pe) = pack4(ev);
                *(uint32_t *)(p2 + po) = pack4(od);
            }
        };
#pragma unroll
        for (int c = 0; c < MAXG; c++) {
            const int m = lane + 64 * c;
            if (m < ngr) put(m, v[c]);
        }
        for (int m = lane + 64 * MAXG; m < ngr; m += 64) {
            float xv[8];
            load8<SRC>(src, m * 8 < kpart ? (uint32_t)((ro + (long)m * 8) * esz) : kOOB, xv);
            put(m, xv);
        }
        double ds = (double)ssum;  // exact: integers below 2^53
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ds += __shfl_xor(ds, o, 64);
        if (lane == 0) {
            xsum[i] = ds;
            expo[i] = e;
        }
    }
    // make this wavefront's LDS writes visible to its own later reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float zp_val(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
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
        wr[0] = make_rsrc(W.qg + (long)s.e * s.I * rb, mbytes);
        wr[NM - 1] = make_rsrc(W.qu + (long)s.e * s.I * rb, mbytes);
    } else {
        wr[0] = make_rsrc(W.qd + (long)s.e * P.d * rb, mbytes);
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
        zrow[0] = zp_val(W.zg, WBITS, (long)s.e * s.I + row);
        zrow[NM - 1] = zp_val(W.zu, WBITS, (long)s.e * s.I + row);
    } else {
        zrow[0] = zp_val(W.zd, WBITS, (long)s.e * P.d + row);
    }
    __syncthreads();  // zero_area

    for (int g0 = 0; g0 < n; g0 += gmax) {
        const int ng = min(gmax, n - g0);
        if (g0 != 0) {
#pragma unroll
            for (int b = 0; b < PF; b++) ldw(b, b);
        }
        long rowoff_lane = 0;  // lane i < ng: element offset of token i's source row
        if (lane < ng) {
            if (MODE == 0) {
                const int t = s.shared ? (g0 + lane) : (P.perm[p0 + g0 + lane] / P.k);
                rowoff_lane = (long)t * P.d;
            } else {
                rowoff_lane = (long)((s.shared ? 0 : p0) + g0 + lane) * K;
            }
        }
        if (MODE == 0)
            wave_stage<WBITS, SRC>(src, rowoff_lane, ng, kp * kpart, kpart, kpad, stride, pb, planes,
                                   wexpo[wv], wxsum[wv]);
        else
            wave_stage<WBITS, 0>(src, rowoff_lane, ng, kp * kpart, kpart, kpad, stride, pb, planes, wexpo[wv],
                                 wxsum[wv]);

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
                        const uint4 q = wbuf[b][m];
                        const i32x4_t Bq = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
#pragma unroll
                        for (int p = 0; p < 3; p++)
                            C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[p], Bq, C[m][p], 0, 0, 0);
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
                        const uint4 q = wbuf[b][m];
                        const i32x4_t Be = {(int)(q.x & 0x0F0F0F0Fu), (int)(q.y & 0x0F0F0F0Fu),
                                            (int)(q.z & 0x0F0F0F0Fu), (int)(q.w & 0x0F0F0F0Fu)};
                        const i32x4_t Bo = {(int)((q.x >> 4) & 0x0F0F0F0Fu), (int)((q.y >> 4) & 0x0F0F0F0Fu),
                                            (int)((q.z >> 4) & 0x0F0F0F0Fu), (int)((q.w >> 4) & 0x0F0F0F0Fu)};
#pragma unroll
                        for (int p = 0; p < 3; p++) {
                            C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ae[p], Be, C[m][p], 0, 0, 0);
                            C[m][p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ao[p], Bo, C[m][p], 0, 0, 0);
                        }
                    }
                }
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
                            const long ch = (long)s.e * s.I + o;
                            const float gf = (float)((double)W.sg[ch] * v[0][r]);
                            const float uf = (float)((double)W.su[ch] * v[NM - 1][r]);
                            const float hv = gf / (1.f + expf(-gf)) * uf;
                            if (s.shared)
                                h_sh[(long)(g0 + i) * s.I + o] = hv;
                            else
                                h[(long)(p0 + g0 + i) * s.I + o] = hv;
                        } else {
                            const long ch = (long)s.e * P.d + o;
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

// ---------------------------------------------------------------------------- host side

static int pad_k(int K, int wbits) {
    const int seg_inputs = wbits == 8 ? 64 : 128;
    return (K + seg_inputs - 1) / seg_inputs * seg_inputs;
}

// K split: the largest S in {4, 2, 1} that keeps whole 16-byte chunks per wavefront and, for the
// down projection, at least 8 segments per wavefront.
static int pick_s(int mode, int K, int wbits) {
    const int chunk_inputs = wbits == 8 ? 16 : 32;
    const int nseg_full = (K * wbits / 8 + 63) / 64;
    for (int S = 4; S >= 2; S >>= 1) {
        if (K % (S * chunk_inputs)) continue;
        if (mode == 1 && nseg_full / S < 8) continue;
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

size_t decode_workspace_bytes(const FfnParams &P) {
    const size_t hb = ((size_t)P.A * P.I * sizeof(float) + 255) & ~(size_t)255;
    const size_t hs = ((size_t)P.T * P.Is * sizeof(float) + 255) & ~(size_t)255;
    return hb + hs;
}

template <int MODE, int WBITS, int SRC>
static hipError_t dk_launch_mode(const FfnParams &P, float *h, float *h_sh, hipStream_t stream) {
    const int slots = P.n_routed_slots + (P.Is > 0 ? 1 : 0);
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int K = MODE == 0 ? P.d : Imax;
    // both the routed and the shared expert must split the same way: use the smaller intermediate size
    const int Kmin = MODE == 0 ? P.d : (P.Is > 0 && P.Is < P.I ? P.Is : P.I);
    const int S = pick_s(MODE, Kmin, WBITS) < pick_s(MODE, K, WBITS) ? pick_s(MODE, Kmin, WBITS)
                                                                        : pick_s(MODE, K, WBITS);
    const int kpad = pad_k(K / S, WBITS);  // the largest wavefront K part, padded to whole segments
    const int gmax = dk_gmax(P.T, kpad);
    const size_t lds = dk_lds_bytes(MODE, kpad, gmax);
    const int nout = MODE == 0 ? Imax : P.d;
    const int rows_per_wg = 16 * (4 / S);
    dim3 grid((nout + rows_per_wg - 1) / rows_per_wg, slots);
    const void *fn;
    if (S == 4)
        fn = (const void *)decode_kernel<MODE, WBITS, SRC, 4>;
    else if (S == 2)
        fn = (const void *)decode_kernel<MODE, WBITS, SRC, 2>;
    else
        fn = (const void *)decode_kernel<MODE, WBITS, SRC, 1>;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    if (S == 4)
        hipLaunchKernelGGL((decode_kernel<MODE, WBITS, SRC, 4>), grid, dim3(DK_THREADS), lds, stream, P, h, h_sh,
                           gmax, kpad);
    else if (S == 2)
        hipLaunchKernelGGL((decode_kernel<MODE, WBITS, SRC, 2>), grid, dim3(DK_THREADS), lds, stream, P, h, h_sh,
                           gmax, kpad);
    else
        hipLaunchKernelGGL((decode_kernel<MODE, WBITS, SRC, 1>), grid, dim3(DK_THREADS), lds, stream, P, h, h_sh,
                           gmax, kpad);
    return hipGetLastError();
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
