// MFMA grouped-GEMM path of the expert FFNs (large token counts).
//
// Batch union (page "github一周涨11k⭐️！25GB 内存跑 744B GLM-5.2 模型！", section 三.4) leaves each used
// expert with a dense block of rows: its c_e assignments (rows of x gathered through the permutation)
// times its weight matrices.  That block is a plain GEMM, run here on the fp16 matrix cores:
//
//   gate/up:  G = X_e (Qg_e)^T,  U = X_e (Qu_e)^T,   h = silu(s_g (G - z_g sum x)) * (s_u (U - z_u sum x))
//   down:     Y = H_e (Qd_e)^T,  y = s_d (Y - z_d sum h)
//
// Weights are the integers q of the per-channel quantisation (page "企业官网建设流程全解析", section
// 3.4): w = s (q - z).  They enter the MFMA as fp16 values of q, exact for int8 and int4, dequantised in
// registers from the packed bytes; the zero point is applied once per output through the row sum of the
// activations, and the scale in the epilogue.  Activations: x is bf16 (exact in fp16 save for values
// below 2^-14 in magnitude); h is kept in fp32 and enters the down GEMM as fp16 hi + lo (two MFMAs into
// one accumulator, about 22 significant bits: a single fp16 rounding of h moves the largest down
// outputs by up to 3e-3 of their RMS).  Accumulation is fp32.
//
// Tiles: 128 rows x (4 wavefronts x 2 subtiles x 32 outputs); gate/up pairs the gate and up rows of
// the same channels in one wavefront.  A persistent grid walks the tiles (slot-major, then output
// tile, then row tile) from a table built on the device from n_uniq / uniq / offsets, so one launch
// shape serves every routing.  Row tiles with fewer than 128 rows skip the empty 32-row MFMA blocks.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t_ __attribute__((ext_vector_type(16)));

constexpr int GG_M = 128;       // rows per tile
constexpr int GG_WAVES = 4;
constexpr int GG_K = 64;        // K per pipeline step
constexpr int GG_LDA = 72;      // LDS row stride of the activation tile, in halfs (64 + 8 of padding)
constexpr int GG_MAXSLOTS = 1025;

// fp16 values of eight int4 weights from one word of packed nibbles (input k in the low nibble of byte
// k/2), in the order k = 0,4,1,5,2,6,3,7: 0x6400 | n is the fp16 bit pattern of 1024 + n.
__device__ __forceinline__ h8_t deq_int4(uint32_t w) {
    const uint32_t M = 0x000F000Fu, B = 0x64006400u;
    const h2_t off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const h2_t p0 = __builtin_bit_cast(h2_t, (w & M) | B) + off;
    const h2_t p1 = __builtin_bit_cast(h2_t, ((w >> 4) & M) | B) + off;
    const h2_t p2 = __builtin_bit_cast(h2_t, ((w >> 8) & M) | B) + off;
    const h2_t p3 = __builtin_bit_cast(h2_t, ((w >> 12) & M) | B) + off;
    return (h8_t){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// fp16 values of eight int8 weights from two words, in input order: bytes are offset to unsigned
// (q + 128) and placed under the fp16 exponent of 1024 (0x64), then 1152 is subtracted.
__device__ __forceinline__ h8_t deq_int8(uint32_t w0, uint32_t w1) {
    const h2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const h2_t p0 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) + off;
    const h2_t p1 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) + off;
    const h2_t p2 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) + off;
    const h2_t p3 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) + off;
    return (h8_t){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ float gg_zp(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
}

// MODE 0: gate/up (A = x rows through the permutation, B = gate and up rows of 32 channels per
// wavefront, output h in fp16).  MODE 1: down (A = h rows of the slot, B = 64 down rows per wavefront,
// output y_perm / y_shared in fp32).
template <int MODE, int WBITS>
__global__ __launch_bounds__(GG_WAVES * 64, 1) void gemm_kernel(FfnParams P, float *__restrict__ hbuf,
                                                                float *__restrict__ hbuf_sh, int tiles_n) {
    constexpr int NOUT_W = MODE == 0 ? 32 : 64;  // output columns per wavefront
    constexpr int NOUT_G = NOUT_W * GG_WAVES;     // per tile
    constexpr int NA = MODE == 0 ? 1 : 2;         // activation planes: x, or h hi and lo
    constexpr int AW = MODE == 0 ? 4 : 8;         // 16-byte activation loads per thread per step
    // activation tiles in dynamic LDS: [2 buffers][NA planes][GG_M rows][GG_LDA halfs]
    extern __shared__ __align__(16) _Float16 As_dyn[];
    __shared__ float rsum[GG_M];
    __shared__ int s_e[GG_MAXSLOTS], s_p0[GG_MAXSLOTS], s_c[GG_MAXSLOTS], s_t0[GG_MAXSLOTS + 1];
    __shared__ int s_nslot;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, lr = lane & 31;

    // ---- tile table: slot s (used experts in uniq order, then the shared expert) has
    // mt_s = ceil(c_s / 128) row tiles and tiles_n output tiles; s_t0 is the exclusive prefix
    if (wv == 0) {
        int nu = *P.n_uniq;
        nu = nu < 0 ? 0 : (nu > P.n_routed_slots ? P.n_routed_slots : nu);
        const bool has_sh = P.Is > 0;
        const int ns = nu + (has_sh ? 1 : 0);
        int carry = 0;
        for (int b = 0; b < ns; b += 64) {
            const int s = b + lane;
            int mt = 0;
            if (s < ns) {
                int e = 0, p0 = 0, c = P.T;
                if (s < nu) {
                    e = P.uniq[s];
                    p0 = P.offsets[e];
                    c = P.offsets[e + 1] - p0;
                }
                s_e[s] = e;
                s_p0[s] = p0;
                s_c[s] = c;
                mt = (c + GG_M - 1) / GG_M;
            }
            int v = mt * tiles_n, incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (s < ns) s_t0[s] = carry + incl - v;
            carry += __shfl(incl, 63, 64);
        }
        if (lane == 0) {
            s_t0[ns] = carry;
            s_nslot = ns;
        }
    }
    __syncthreads();
    const int nslot = s_nslot;
    const int ntiles = s_t0[nslot];

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        // ---- locate the tile: slot (binary search), output tile, row tile
        int lo = 0, hi = nslot - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_t0[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int slot = lo;
        const bool shared = slot >= nslot - (P.Is > 0 ? 1 : 0) && P.Is > 0;
        const int e = s_e[slot], p0 = s_p0[slot], cnt = s_c[slot];
        const int mt_n = (cnt + GG_M - 1) / GG_M;
        const int local = tile - s_t0[slot];
        const int ntile = local / mt_n, mtile = local % mt_n;
        const int r0 = mtile * GG_M;                     // first row of the tile within the slot
        const int rows = min(GG_M, cnt - r0);
        const int nm32 = (rows + 31) >> 5;               // 32-row MFMA blocks with data
        const int I = shared ? P.Is : P.I;
        const int KK = MODE == 0 ? P.d : I;              // contraction length
        const int nout = MODE == 0 ? I : P.d;
        const int nsteps = KK / GG_K;
        const QW &W = shared ? P.shared : P.routed;

        // ---- activation rows staged by this thread: row am = tid / 2, inputs [32*ah, 32*ah + 32) of each step
        const int am = tid >> 1, ah = tid & 1;
        long arow = -1;  // element offset of the source row, -1: padding row
        if (am < rows) {
            if (MODE == 0) {
                const int t = shared ? (r0 + am) : (P.perm[p0 + r0 + am] / P.k);
                arow = (long)t * P.d;
            } else {
                arow = (long)((shared ? 0 : p0) + r0 + am) * I;
            }
        }
        rsrc_t asrc;
        constexpr int AES = MODE == 0 ? 2 : 4;  // bytes per activation element (bf16 x, fp32 h)
        if (MODE == 0)
            asrc = make_rsrc(P.x, (uint32_t)((long)P.T * P.d * 2));
        else
            asrc = make_rsrc(shared ? (const void *)hbuf_sh : (const void *)hbuf,
                             (uint32_t)((long)(shared ? P.T : P.A) * I * 4));
        auto a_off = [&](int step) -> uint32_t {
            return arow < 0 ? kOOB : (uint32_t)((arow + (long)step * GG_K + 32 * ah) * AES);
        };

        // ---- weight rows of this lane: subtile j (gate/up: j = 0 gate, 1 up of channel c; down: outputs
        // o and o + 32)
        const long rb = (long)KK * WBITS / 8;  // bytes per weight row
        rsrc_t wsrc[2];
        uint32_t wrow[2];
        int ocol[2];
        {
            const int nbase = ntile * NOUT_G + wv * NOUT_W;
            if (MODE == 0) {
                const int c = nbase + lr;
                ocol[0] = ocol[1] = c;
                const uint32_t mb = (uint32_t)((long)I * rb);
                wsrc[0] = make_rsrc(W.qg + (long)e * I * rb, mb);
                wsrc[1] = make_rsrc(W.qu + (long)e * I * rb, mb);
                wrow[0] = wrow[1] = c < I ? (uint32_t)(c * rb) : kOOB;
            } else {
                const uint32_t mb = (uint32_t)((long)P.d * rb);
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int o = nbase + 32 * j + lr;
                    ocol[j] = o;
                    wsrc[j] = make_rsrc(W.qd + (long)e * P.d * rb, mb);
                    wrow[j] = o < P.d ? (uint32_t)(o * rb) : kOOB;
                }
            }
        }
        constexpr int WL = WBITS == 8 ? 2 : 1;  // 16-byte weight loads per subtile per step
        auto w_off = [&](int j, int step, int q) -> uint32_t {
            return wrow[j] == kOOB ? kOOB : wrow[j] + (uint32_t)(step * (GG_K * WBITS / 8) + kg * (16 * WL) + 16 * q);
        };

        // ---- pipeline: loads for step s+1 are in flight while step s computes
        uint4 araw[AW];
        uint4 wraw[2][WL];
        auto issue = [&](int step) {
            const uint32_t ao = a_off(step);
#pragma unroll
            for (int q = 0; q < AW; q++) araw[q] = buf_load16(asrc, ao == kOOB ? kOOB : ao + 16 * q);
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < WL; q++) wraw[j][q] = buf_load16(wsrc[j], w_off(j, step, q));
        };
        float rs = 0.f;
        f32x16_t_ acc[4][2];
#pragma unroll
        for (int mm = 0; mm < 4; mm++)
#pragma unroll
            for (int j = 0; j < 2; j++) acc[mm][j] = (f32x16_t_){};

        issue(0);
        for (int step = 0; step < nsteps; step++) {
            _Float16 *Ab = As_dyn + (step & 1) * NA * GG_M * GG_LDA;
            // activations of this step -> fp16 planes in LDS (int4 weights: each group of 8 inputs stored
            // in the order 0,4,1,5,2,6,3,7 to match the weight registers)
            {
                _Float16 v[NA][32];
                if (MODE == 0) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const uint32_t ww[4] = {araw[q].x, araw[q].y, araw[q].z, araw[q].w};
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float lo = __uint_as_float(ww[i] << 16), hi = __uint_as_float(ww[i] & 0xFFFF0000u);
                            v[0][8 * q + 2 * i] = (_Float16)lo;
                            v[0][8 * q + 2 * i + 1] = (_Float16)hi;
                            rs += lo + hi;
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < AW; q++) {
                        const float f[4] = {__uint_as_float(araw[q].x), __uint_as_float(araw[q].y),
                                            __uint_as_float(araw[q].z), __uint_as_float(araw[q].w)};
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const _Float16 hi = (_Float16)f[i];
                            v[0][4 * q + i] = hi;
                            v[NA - 1][4 * q + i] = (_Float16)(f[i] - (float)hi);
                            rs += f[i];
                        }
                    }
                }
#pragma unroll
                for (int pl = 0; pl < NA; pl++) {
                    h8_t o[4];
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) {
                        const _Float16 *vv = v[pl] + 8 * gq;
                        if (WBITS == 4)
                            o[gq] = (h8_t){vv[0], vv[4], vv[1], vv[5], vv[2], vv[6], vv[3], vv[7]};
                        else
                            o[gq] = (h8_t){vv[0], vv[1], vv[2], vv[3], vv[4], vv[5], vv[6], vv[7]};
                    }
                    h8_t *dst = (h8_t *)(Ab + pl * GG_M * GG_LDA + am * GG_LDA + 32 * ah);
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) dst[gq] = o[gq];
                }
            }
            uint4 wcur[2][WL];
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < WL; q++) wcur[j][q] = wraw[j][q];
            __syncthreads();  // the step's activations are in LDS; the other buffer is free
            if (step + 1 < nsteps) issue(step + 1);

#pragma unroll
            for (int s = 0; s < 4; s++) {
                h8_t bq[2];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    if (WBITS == 4) {
                        const uint32_t ww[4] = {wcur[j][0].x, wcur[j][0].y, wcur[j][0].z, wcur[j][0].w};
                        bq[j] = deq_int4(ww[s]);
                    } else {
                        const uint4 q = wcur[j][s >> 1];
                        bq[j] = (s & 1) ? deq_int8(q.z, q.w) : deq_int8(q.x, q.y);
                    }
                }
#pragma unroll
                for (int mm = 0; mm < 4; mm++) {
                    if (mm < nm32) {
#pragma unroll
                        for (int pl = 0; pl < NA; pl++) {
                            const h8_t a =
                                *(const h8_t *)(Ab + pl * GG_M * GG_LDA + (mm * 32 + lr) * GG_LDA + 32 * kg + 8 * s);
#pragma unroll
                            for (int j = 0; j < 2; j++)
                                acc[mm][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq[j], acc[mm][j], 0, 0, 0);
                        }
                    }
                }
            }
        }

        // ---- row sums of the staged activations (fixed order: the two halves of a row)
        __syncthreads();
        {
            const float other = __shfl_xor(rs, 1, 64);
            if (ah == 0) rsum[am] = rs + other;
        }
        __syncthreads();

        // ---- epilogue: lane column ocol[j], register r holds row 8*(r/4) + 4*kg + (r%4) of block mm
        float sc[2], zp[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int cc = min(ocol[j], nout - 1);
            if (MODE == 0) {
                const long ch = (long)e * I + cc;
                sc[j] = j == 0 ? W.sg[ch] : W.su[ch];
                zp[j] = gg_zp(j == 0 ? W.zg : W.zu, WBITS, ch);
            } else {
                const long ch = (long)e * P.d + cc;
                sc[j] = W.sd[ch];
                zp[j] = gg_zp(W.zd, WBITS, ch);
            }
        }
#pragma unroll
        for (int mm = 0; mm < 4; mm++) {
            if (mm >= nm32) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = mm * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (m >= rows) continue;
                const float xs = rsum[m];
                const long prow = (long)(shared ? 0 : p0) + r0 + m;  // output row
                if (MODE == 0) {
                    if (ocol[0] < nout) {
                        const float gv = sc[0] * (acc[mm][0][r] - zp[0] * xs);
                        const float uv = sc[1] * (acc[mm][1][r] - zp[1] * xs);
                        const float hv = gv / (1.f + expf(-gv)) * uv;
                        (shared ? hbuf_sh : hbuf)[prow * I + ocol[0]] = hv;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        if (ocol[j] < nout) {
                            const float y = sc[j] * (acc[mm][j][r] - zp[j] * xs);
                            (shared ? P.y_sh : P.y_perm)[prow * P.d + ocol[j]] = y;
                        }
                    }
                }
            }
        }
        __syncthreads();  // rsum and the activation buffers are reused by the next tile
    }
}

// ---------------------------------------------------------------------------- host side

size_t gemm_workspace_bytes(const FfnParams &P) {
    const size_t hb = ((size_t)P.A * P.I * 4 + 255) & ~(size_t)255;
    const size_t hs = ((size_t)P.T * P.Is * 4 + 255) & ~(size_t)255;
    return hb + hs;
}

bool gemm_supported(const FfnParams &P) {
    if (P.act != 1) return false;  // bf16 activations
    if (P.d % GG_K || P.I % GG_K || (P.Is > 0 && P.Is % GG_K)) return false;
    if (P.n_routed_slots + 1 > GG_MAXSLOTS) return false;
    // 32-bit buffer offsets
    const long wb = (long)(P.wbits == 8 ? 1 : 2);
    if ((long)P.I * P.d / (P.wbits == 8 ? 1 : 2) * wb > 0x7FFFFFFFL) return false;
    if ((long)P.A * P.I * 4 > 0x7FFFFFFFL || (long)P.T * P.d * 2 > 0x7FFFFFFFL) return false;
    return true;
}

static int gg_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    return n;
}

template <int MODE, int WBITS>
static hipError_t gg_launch_mode(const FfnParams &P, float *h, float *h_sh, int tiles_n, hipStream_t stream) {
    const size_t lds = (size_t)2 * (MODE == 0 ? 1 : 2) * GG_M * GG_LDA * sizeof(_Float16);
    auto fn = gemm_kernel<MODE, WBITS>;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(fn, dim3(gg_cus()), dim3(GG_WAVES * 64), lds, stream, P, h, h_sh, tiles_n);
    return hipGetLastError();
}

template <int WBITS>
static hipError_t gg_launch(const FfnParams &P, float *h, float *h_sh, hipStream_t stream) {
    const int Imax = P.I > P.Is ? P.I : P.Is;
    hipError_t err = gg_launch_mode<0, WBITS>(P, h, h_sh, (Imax + 32 * GG_WAVES - 1) / (32 * GG_WAVES), stream);
    if (err != hipSuccess) return err;
    return gg_launch_mode<1, WBITS>(P, h, h_sh, (P.d + 64 * GG_WAVES - 1) / (64 * GG_WAVES), stream);
}

hipError_t launch_ffn_gemm(const FfnParams &P, void *ws, hipStream_t stream) {
    if (!gemm_supported(P)) return hipErrorNotSupported;
    float *h = (float *)ws;
    float *h_sh = (float *)((char *)ws + (((size_t)P.A * P.I * 4 + 255) & ~(size_t)255));
    return P.wbits == 4 ? gg_launch<4>(P, h, h_sh, stream) : gg_launch<8>(P, h, h_sh, stream);
}

}  // namespace moe
