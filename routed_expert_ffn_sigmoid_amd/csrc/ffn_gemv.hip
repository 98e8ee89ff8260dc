// Decode path of the expert FFNs: dequant-GEMV, bound by HBM bandwidth.
//
// Experts are SwiGLU FFNs quantised per output channel with a scale and a
// zero point ("企业官网建设流程全解析" page, Colibri walk-through, section 3.4),
// run once per unique expert for every token routed to it (batch union,
// "25GB 内存跑 744B GLM-5.2 模型" page, section 三.4).
//
// Grid: (row blocks, slots).  Slots 0..min(E,A)-1 read the device-side unique
// expert list (slots past n_uniq exit at once); one more slot is the shared
// expert.  Each wavefront streams a few weight rows with 16-byte loads (lane l
// takes chunks l, l+64, ...), the activations of up to 4 tokens sit in LDS,
// and the zero point is folded out of the inner loop:
//     sum_i (q_i - z) x_i = sum_i (q_i + M) x_i - (M + z) sum_i x_i
// with M chosen so that q + M is a cheap non-negative number:
//   int4: each nibble pair becomes a packed bf16 pair 128+q by OR-ing the
//         exponent bits 0x43 in (exact), and v_dot2c_f32_bf16 multiplies it
//         with a packed pair of activations -- 7 bit-ops + 4 dot2 per 8
//         weights.  Activations are bf16 (exact for bf16 input; fp32 input
//         and the fp32 h are split as hi + lo bf16, two dot2 per pair).
//   int8: q ^ 0x80 = q + 128 as an unsigned byte, v_cvt_f32_ubyteN, fp32 FMA
//         against fp32 activations.
// Pair order inside each group of 8 inputs: the packed weight dword holds
// nibbles n0..n7; (w >> 4p) & 0x000F000F gives (n_p, n_{p+4}), so the
// activation pairs are staged as (x_p, x_{p+4}) for p = 0..3.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GV_WAVES = 4;
constexpr int GV_THREADS = GV_WAVES * 64;
constexpr int GV_G = 4;                       // tokens per pass over the weights
constexpr int GV_LDS_BUDGET = 32 * 1024;      // activation staging per workgroup
constexpr int GV_RPW_GATEUP = 2;              // channels per wave (gate + up rows each)
constexpr int GV_RPW_DOWN = 4;                // output rows per wave

struct Slot {
    int e, p0, n, I;
    bool shared;
};

__device__ __forceinline__ bool decode_slot(const FfnParams &P, int slot, Slot &s) {
    if (slot < P.n_routed_slots) {
        const int nu = *P.n_uniq;
        if (slot >= nu) return false;
        const int e = P.uniq[slot];
        s.e = e;
        s.p0 = P.offsets[e];
        s.n = P.offsets[e + 1] - s.p0;
        s.I = P.I;
        s.shared = false;
    } else {
        s.e = 0;
        s.p0 = 0;
        s.n = P.T;
        s.I = P.Is;
        s.shared = true;
    }
    return s.n > 0 && s.I > 0;
}

__device__ __forceinline__ float zp_value(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
}

// LDS words per token for kc inputs
template <int WBITS, bool SPLIT>
__host__ __device__ constexpr int stage_words(int kc) {
    return WBITS == 4 ? (SPLIT ? kc : kc / 2) : kc;
}

// Stage inputs [k0, k0+kcur) of ng source rows into LDS in the format the dot loop reads and add
// each row's sum of the staged values to sums[i] (sums[i] is reset when k0 == 0).
// SRC: 0 = fp32 source, 1 = bf16 source.  Deterministic: fixed per-thread order, fixed reduction tree.
template <int WBITS, int SRC, bool SPLIT>
__device__ __forceinline__ void stage_rows(const void *__restrict__ base, const long *rowoff, int ng, int gmax, int k0,
                                           int kcur, int kc, uint32_t *lds, float *sums, float (*red)[GV_G]) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ngroups = kcur / 8;
    float part[GV_G];
#pragma unroll
    for (int i = 0; i < GV_G; i++) part[i] = 0.f;
#pragma unroll
    for (int i = 0; i < GV_G; i++) {
        if (i >= ng) break;
        for (int m = tid; m < ngroups; m += GV_THREADS) {
            float v[8];
            const long off = rowoff[i] + k0 + (long)m * 8;
            if (SRC == 0) {
                const float4 a = *(const float4 *)((const float *)base + off);
                const float4 b = *(const float4 *)((const float *)base + off + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            } else {
                const uint4 q = *(const uint4 *)((const uint16_t *)base + off);
                const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[2 * j] = __uint_as_float(qq[j] << 16);
                    v[2 * j + 1] = __uint_as_float(qq[j] & 0xFFFF0000u);
                }
            }
            if (WBITS == 4) {
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    if (SPLIT) {
                        split_bf16(v[j], hi[j], lo[j]);
                        part[i] += __uint_as_float(hi[j] << 16) + __uint_as_float(lo[j] << 16);
                    } else {
                        hi[j] = __float_as_uint(v[j]) >> 16;  // bf16 source: exact
                        part[i] += v[j];
                    }
                }
                uint32_t *dst = lds + (long)i * stage_words<WBITS, SPLIT>(kc) + (long)m * (SPLIT ? 8 : 4);
                uint4 ph = make_uint4(hi[0] | (hi[4] << 16), hi[1] | (hi[5] << 16), hi[2] | (hi[6] << 16),
                                      hi[3] | (hi[7] << 16));
                *(uint4 *)dst = ph;
                if (SPLIT) {
                    uint4 pl = make_uint4(lo[0] | (lo[4] << 16), lo[1] | (lo[5] << 16), lo[2] | (lo[6] << 16),
                                          lo[3] | (lo[7] << 16));
                    *(uint4 *)(dst + 4) = pl;
                }
            } else {
                float *dst = (float *)lds + (long)i * kc + (long)m * 8;
                *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
                *(float4 *)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
                for (int j = 0; j < 8; j++) part[i] += v[j];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < GV_G; i++) {
        float sv = wave_sum(part[i]);
        if (lane == 0) red[wv][i] = sv;
    }
    __syncthreads();
    if (tid < ng) {
        float s = red[0][tid];
#pragma unroll
        for (int w = 1; w < GV_WAVES; w++) s += red[w][tid];
        sums[tid] = (k0 == 0 ? 0.f : sums[tid]) + s;
    }
    (void)gmax;
}

// acc[r][i] += sum over the chunks of this lane of (q + M) * staged activation, NR rows, up to GV_G tokens.
template <int WBITS, bool SPLIT, int NR>
__device__ __forceinline__ void dot_chunks(const uint8_t *const (&rowp)[NR], int nch, const uint32_t *lds, int kc,
                                           int ng, float (&acc)[NR][GV_G]) {
    const int lane = threadIdx.x & 63;
    const int words = stage_words<WBITS, SPLIT>(kc);
    for (int ci = lane; ci < nch; ci += 64) {
        uint4 wq[NR];
#pragma unroll
        for (int r = 0; r < NR; r++) wq[r] = *(const uint4 *)(rowp[r] + (long)ci * 16);
        if (WBITS == 4) {
            // 16 packed bf16 weight pairs per row
            uint32_t pw[NR][16];
#pragma unroll
            for (int r = 0; r < NR; r++) {
                const uint32_t w4[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int p = 0; p < 4; p++) pw[r][m * 4 + p] = ((w4[m] >> (4 * p)) & 0x000F000Fu) | 0x43004300u;
            }
#pragma unroll
            for (int i = 0; i < GV_G; i++) {
                if (i >= ng) break;
                const uint32_t *xp = lds + (long)i * words + (long)ci * (SPLIT ? 32 : 16);
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const uint4 xh = *(const uint4 *)(xp + m * (SPLIT ? 8 : 4));
                    const uint32_t xa[4] = {xh.x, xh.y, xh.z, xh.w};
#pragma unroll
                    for (int r = 0; r < NR; r++)
#pragma unroll
                        for (int p = 0; p < 4; p++) acc[r][i] = dot2_bf16(pw[r][m * 4 + p], xa[p], acc[r][i]);
                    if (SPLIT) {
                        const uint4 xl = *(const uint4 *)(xp + m * 8 + 4);
                        const uint32_t xb[4] = {xl.x, xl.y, xl.z, xl.w};
#pragma unroll
                        for (int r = 0; r < NR; r++)
#pragma unroll
                            for (int p = 0; p < 4; p++) acc[r][i] = dot2_bf16(pw[r][m * 4 + p], xb[p], acc[r][i]);
                    }
                }
            }
        } else {
            float fw[NR][16];
#pragma unroll
            for (int r = 0; r < NR; r++) {
                const uint32_t w4[4] = {wq[r].x ^ 0x80808080u, wq[r].y ^ 0x80808080u, wq[r].z ^ 0x80808080u,
                                        wq[r].w ^ 0x80808080u};
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int b = 0; b < 4; b++) fw[r][m * 4 + b] = (float)((w4[m] >> (8 * b)) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < GV_G; i++) {
                if (i >= ng) break;
                const float *xp = (const float *)lds + (long)i * kc + (long)ci * 16;
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const float4 xv = *(const float4 *)(xp + m * 4);
                    const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int r = 0; r < NR; r++)
#pragma unroll
                        for (int b = 0; b < 4; b++) acc[r][i] = fmaf(fw[r][m * 4 + b], xa[b], acc[r][i]);
                }
            }
        }
    }
}

template <int WBITS>
__device__ __forceinline__ constexpr float offset_M() {
    return 128.f;  // int4: bf16 0x43.. pattern = 128 + q;  int8: (q ^ 0x80) = q + 128
}

// gate/up: h[row][c] = silu(g_c) * u_c for the slot's tokens.
// grid: (ceil(max(I, Is) / (4*RPW)), slots); block 256; dynamic LDS = gmax * stage_words(kc) * 4
template <int WBITS, int SRC>
__global__ __launch_bounds__(GV_THREADS) void gateup_gemv_kernel(FfnParams P, float *__restrict__ h,
                                                                 float *__restrict__ h_sh, int kc, int gmax) {
    constexpr int RPW = GV_RPW_GATEUP;
    constexpr bool SPLIT = (WBITS == 4 && SRC == 0);
    extern __shared__ uint32_t lds[];
    __shared__ float sums[GV_G];
    __shared__ float red[GV_WAVES][GV_G];
    __shared__ long rowoff[GV_G];
    Slot s;
    if (!decode_slot(P, blockIdx.y, s)) return;
    const int c0 = blockIdx.x * (GV_WAVES * RPW);
    if (c0 >= s.I) return;
    const QW &W = s.shared ? P.shared : P.routed;
    const long rb = (long)P.d * WBITS / 8;
    const uint8_t *qg = W.qg + (long)s.e * s.I * rb;
    const uint8_t *qu = W.qu + (long)s.e * s.I * rb;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;

    for (int g0 = 0; g0 < s.n; g0 += gmax) {
        const int ng = min(gmax, s.n - g0);
        float acc[2 * RPW][GV_G];
#pragma unroll
        for (int r = 0; r < 2 * RPW; r++)
#pragma unroll
            for (int i = 0; i < GV_G; i++) acc[r][i] = 0.f;
        __syncthreads();  // previous pass is done with rowoff / sums
        if (tid < ng) {
            const int t = s.shared ? (g0 + tid) : (P.perm[s.p0 + g0 + tid] / P.k);
            rowoff[tid] = (long)t * P.d;
        }
        for (int k0 = 0; k0 < P.d; k0 += kc) {
            const int kcur = min(kc, P.d - k0);
            __syncthreads();
            stage_rows<WBITS, SRC, SPLIT>(P.x, rowoff, ng, gmax, k0, kcur, kc, lds, sums, red);
            __syncthreads();
            const uint8_t *rowp[2 * RPW];
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const int c = min(c0 + wv * RPW + r, s.I - 1);
                rowp[2 * r] = qg + (long)c * rb + (long)k0 * WBITS / 8;
                rowp[2 * r + 1] = qu + (long)c * rb + (long)k0 * WBITS / 8;
            }
            dot_chunks<WBITS, SPLIT, 2 * RPW>(rowp, kcur * WBITS / 8 / 16, lds, kc, ng, acc);
        }
#pragma unroll
        for (int r = 0; r < 2 * RPW; r++)
#pragma unroll
            for (int i = 0; i < GV_G; i++) acc[r][i] = wave_sum(acc[r][i]);
        const float M = offset_M<WBITS>();
#pragma unroll
        for (int r = 0; r < RPW; r++) {
#pragma unroll
            for (int i = 0; i < GV_G; i++) {
                const int c = c0 + wv * RPW + r;
                if (lane == r * GV_G + i && i < ng && c < s.I) {
                    const long ch = (long)s.e * s.I + c;
                    const float g = W.sg[ch] * (acc[2 * r][i] - (M + zp_value(W.zg, WBITS, ch)) * sums[i]);
                    const float u = W.su[ch] * (acc[2 * r + 1][i] - (M + zp_value(W.zu, WBITS, ch)) * sums[i]);
                    const float hv = g / (1.f + expf(-g)) * u;
                    if (s.shared)
                        h_sh[(long)(g0 + i) * s.I + c] = hv;
                    else
                        h[(long)(s.p0 + g0 + i) * s.I + c] = hv;
                }
            }
        }
    }
}

// down: y[row][r] = s_r * ((q_r - z_r) . h[row]).
// grid: (ceil(d / (4*RPW)), slots); block 256; dynamic LDS = gmax * stage_words(kc) * 4
template <int WBITS>
__global__ __launch_bounds__(GV_THREADS) void down_gemv_kernel(FfnParams P, const float *__restrict__ h,
                                                               const float *__restrict__ h_sh, int kc, int gmax) {
    constexpr int RPW = GV_RPW_DOWN;
    constexpr bool SPLIT = (WBITS == 4);
    extern __shared__ uint32_t lds[];
    __shared__ float sums[GV_G];
    __shared__ float red[GV_WAVES][GV_G];
    __shared__ long rowoff[GV_G];
    Slot s;
    if (!decode_slot(P, blockIdx.y, s)) return;
    const int r0 = blockIdx.x * (GV_WAVES * RPW);
    if (r0 >= P.d) return;
    const QW &W = s.shared ? P.shared : P.routed;
    const int K = s.I;
    const long rb = (long)K * WBITS / 8;
    const uint8_t *qd = W.qd + (long)s.e * P.d * rb;
    const float *hsrc = s.shared ? h_sh : h;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;

    for (int g0 = 0; g0 < s.n; g0 += gmax) {
        const int ng = min(gmax, s.n - g0);
        float acc[RPW][GV_G];
#pragma unroll
        for (int r = 0; r < RPW; r++)
#pragma unroll
            for (int i = 0; i < GV_G; i++) acc[r][i] = 0.f;
        __syncthreads();
        if (tid < ng) rowoff[tid] = (long)((s.shared ? 0 : s.p0) + g0 + tid) * K;
        for (int k0 = 0; k0 < K; k0 += kc) {
            const int kcur = min(kc, K - k0);
            __syncthreads();
            stage_rows<WBITS, 0, SPLIT>(hsrc, rowoff, ng, gmax, k0, kcur, kc, lds, sums, red);
            __syncthreads();
            const uint8_t *rowp[RPW];
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const int o = min(r0 + wv * RPW + r, P.d - 1);
                rowp[r] = qd + (long)o * rb + (long)k0 * WBITS / 8;
            }
            dot_chunks<WBITS, SPLIT, RPW>(rowp, kcur * WBITS / 8 / 16, lds, kc, ng, acc);
        }
#pragma unroll
        for (int r = 0; r < RPW; r++)
#pragma unroll
            for (int i = 0; i < GV_G; i++) acc[r][i] = wave_sum(acc[r][i]);
        const float M = offset_M<WBITS>();
#pragma unroll
        for (int r = 0; r < RPW; r++) {
#pragma unroll
            for (int i = 0; i < GV_G; i++) {
                const int o = r0 + wv * RPW + r;
                if (lane == r * GV_G + i && i < ng && o < P.d) {
                    const long ch = (long)s.e * P.d + o;
                    const float y = W.sd[ch] * (acc[r][i] - (M + zp_value(W.zd, WBITS, ch)) * sums[i]);
                    if (s.shared)
                        P.y_sh[(long)(g0 + i) * P.d + o] = y;
                    else
                        P.y_perm[(long)(s.p0 + g0 + i) * P.d + o] = y;
                }
            }
        }
    }
}

// Largest staged k-range (multiple of the 16-byte chunk's element count) that fits the LDS budget.
static int pick_kc(int K, int wbits, bool split, int gmax) {
    const int per_elem_words_x2 = wbits == 4 ? (split ? 2 : 1) : 2;  // LDS words per 2 elements
    const int chunk = wbits == 4 ? 32 : 16;
    long max_elems = (long)GV_LDS_BUDGET / 4 * 2 / per_elem_words_x2 / gmax;
    long kc = (max_elems / chunk) * chunk;
    if (kc >= K) return K;
    if (kc < chunk) kc = chunk;
    return (int)kc;
}

static size_t h_bytes(const FfnParams &P) { return (size_t)P.A * P.I * sizeof(float); }
static size_t hsh_bytes(const FfnParams &P) { return (size_t)P.T * (size_t)P.Is * sizeof(float); }

size_t gemv_workspace_bytes(const FfnParams &P) {
    return ((h_bytes(P) + 255) & ~(size_t)255) + ((hsh_bytes(P) + 255) & ~(size_t)255);
}

template <int WBITS, int SRC>
static hipError_t launch_t(const FfnParams &P, float *h, float *h_sh, hipStream_t stream) {
    const int gmax = P.T < GV_G ? P.T : GV_G;
    const int slots = P.n_routed_slots + (P.Is > 0 ? 1 : 0);
    const int Imax = P.I > P.Is ? P.I : P.Is;
    {
        constexpr bool split = (WBITS == 4 && SRC == 0);
        const int kc = pick_kc(P.d, WBITS, split, gmax);
        const size_t lds = (size_t)gmax * stage_words<WBITS, split>(kc) * 4;
        dim3 grid((Imax + GV_WAVES * GV_RPW_GATEUP - 1) / (GV_WAVES * GV_RPW_GATEUP), slots);
        hipLaunchKernelGGL((gateup_gemv_kernel<WBITS, SRC>), grid, dim3(GV_THREADS), lds, stream, P, h, h_sh, kc, gmax);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        constexpr bool split = (WBITS == 4);
        const int kc = pick_kc(Imax, WBITS, split, gmax);
        const size_t lds = (size_t)gmax * stage_words<WBITS, split>(kc) * 4;
        dim3 grid((P.d + GV_WAVES * GV_RPW_DOWN - 1) / (GV_WAVES * GV_RPW_DOWN), slots);
        hipLaunchKernelGGL((down_gemv_kernel<WBITS>), grid, dim3(GV_THREADS), lds, stream, P, h, h_sh, kc, gmax);
        return hipGetLastError();
    }
}

hipError_t launch_ffn_gemv(const FfnParams &P, void *ws, hipStream_t stream) {
    float *h = (float *)ws;
    float *h_sh = (float *)((char *)ws + ((h_bytes(P) + 255) & ~(size_t)255));
    if (P.wbits == 4)
        return P.act == 0 ? launch_t<4, 0>(P, h, h_sh, stream) : launch_t<4, 1>(P, h, h_sh, stream);
    return P.act == 0 ? launch_t<8, 0>(P, h, h_sh, stream) : launch_t<8, 1>(P, h, h_sh, stream);
}

}  // namespace moe
