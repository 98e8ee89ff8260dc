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
// activations, and the scale in the epilogue.  Activations: bf16 x is converted once to fp16 under a
// power-of-two scale per token (exact for every value above 2^-29 of the row's largest; any range fits),
// undone in the gate/up epilogue; fp32 x becomes two fp16 values hi + lo under that scale (about 22
// significant bits), and gate/up runs every weight step against both.  h is stored under a power-of-two scale per row, 2^-r, chosen from a bound
// on |h| that x's L1 norm and the expert's scales give (see x16_kernel), so it never overflows fp16 either;
// the down epilogue multiplies by 2^r.  h enters the down GEMM as an fp16 plane plus the residual
// h - fp16(h) in fp6 e2m3 under one E8M0 exponent per row and 32 channels (the block form of the scaled
// matrix-core product), about 15-16 significant bits for the larger values of a block: a single fp16
// rounding of h would move the largest down outputs by up to 3e-3 of their RMS.  The residual product
// is one scaled e2m3 MFMA per K step and 32x32 block, a quarter of the matrix-core time of the fp16
// plane's four; its weights are the same dequantised values in e2m3 under a per-column power of two
// (exact for int4 with zero points in 0..15, 4 significant bits for larger values, which the residual's
// own 4 bits already bound).  Accumulation is fp32.
//
// Layout of the activation planes (x16, h and its residual): row-major, and for int4 weights the 8
// inputs of each group are stored in the order 0,4,1,5,2,6,3,7, the order in which the nibble
// dequantisation below produces the weights.  The residual plane keeps one byte per channel: each block
// of 32 channels holds their 24 bytes of e2m3 codes, then the fp32 sum of the rounded residuals, then 4
// unused bytes.  Residual exponents: per row tile (over all slots) and K step, 256 bytes
// [block][row % 32][row / 32], the order in which one 32-bit LDS read gives a lane the exponents of its
// four row blocks.
//
// Tiles: 128 rows x 512 weight rows; each of the 8 wavefronts covers all 128 rows (as up to 4 blocks of
// 32) and 64 weight rows as 2 subtiles of 32 columns.  Gate/up pairs the gate and up rows of the same 32
// channels in one wavefront (256 channels per tile), down takes 64 outputs per wavefront (512 per tile).
// A persistent grid (one workgroup per CU) walks the tiles (slot-major, then output tile, then row tile)
// from a table built on the device from n_uniq / uniq / offsets, so one launch shape serves every
// routing.  Activations and weights are copied from memory straight into an LDS ring of 2-8 K steps
// (more for tiles with fewer rows).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16v_t __attribute__((ext_vector_type(16)));

constexpr int GG_M = 128;          // rows per tile
constexpr int GG_WAVES = 8;        // wavefronts per workgroup, one workgroup per CU
constexpr int GG_K = 64;           // K per pipeline step
constexpr int GG_NW = 64;          // weight rows per wavefront and tile (two 32-column subtiles)
constexpr int GG_MAXSLOTS = 1025;
constexpr int GG_XCDS = 8;         // XCDs of the chip; workgroups are dealt to them round-robin
constexpr int GG_GROUP = 16;       // consecutive tiles handed to one XCD at a time
constexpr int GG_RING = 152 * 1024;  // LDS for the staging ring (the rest of the 160 KB holds the tables)
constexpr int GG_JUNK = 1024;        // end of the ring: sink of the copies a tile does not need (they read nothing)

// storage position, within its group of 8, of input i of the group (int4 weights)
__device__ __forceinline__ int pos8(int i) { return ((i & 3) << 1) | (i >> 2); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "s"(o));
    return r;
}

// fp16 values of eight int4 weights from one word (input k in the low nibble of byte k/2 for even k, the
// high nibble for odd k), in the order k = 0,4,1,5,2,6,3,7.  A nibble under the exponent of 1024
// (0x6400) is the fp16 value 1024 + n; a high nibble is left in place, giving 1024 + 16 n, and scaled
// by 1/16 in a fused multiply-add.  off = -(1024 + z), off16 = -(64 + z), z the folded integral zero
// point (or 0).  Exact: every intermediate is an integer or a multiple of 1/16 below 2048.
__device__ __forceinline__ h8_t deq_int4(uint32_t w, uint32_t mlo, uint32_t mhi, h2_t off, h2_t off16) {
    const uint32_t B = 0x64006400u;
    const h2_t sixteenth = (h2_t){(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    const h2_t p0 = __builtin_bit_cast(h2_t, and_or(w, mlo, B)) + off;
    const h2_t p1 = __builtin_bit_cast(h2_t, and_or(w, mhi, B)) * sixteenth + off16;
    const h2_t p2 = __builtin_bit_cast(h2_t, and_or(w8, mlo, B)) + off;
    const h2_t p3 = __builtin_bit_cast(h2_t, and_or(w8, mhi, B)) * sixteenth + off16;
    return (h8_t){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// fp16 values of eight int8 weights from two words, in input order: bytes are offset to unsigned
// (q + 128) and placed under the fp16 exponent of 1024 (0x64), then off = -(1152 + z) is added (z the
// folded zero point, or 0).  Exact: integers below 2048 in magnitude.
__device__ __forceinline__ h8_t deq_int8(uint32_t w0, uint32_t w1, h2_t off) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const h2_t p0 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) + off;
    const h2_t p1 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) + off;
    const h2_t p2 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) + off;
    const h2_t p3 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) + off;
    return (h8_t){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

typedef int i2v_t __attribute__((ext_vector_type(2)));
typedef int i4v_t __attribute__((ext_vector_type(4)));
typedef int i8v_t __attribute__((ext_vector_type(8)));
typedef _Float16 h32_t __attribute__((ext_vector_type(32)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef unsigned int u6v_t __attribute__((ext_vector_type(6)));
typedef float f32x32v_t __attribute__((ext_vector_type(32)));

// fp6 e2m3 (1 sign, 2 exponent bits of bias 1, 3 mantissa bits): magnitudes 0.125 m below 1 and
// (1 + m/8) 2^(e-1) up to 7.5, i.e. 4 significant bits over three binades.  32 values of one lane
// take six words, value i at bits 6i..6i+5 of their little-endian concatenation; the conversions
// divide by their scale, round to nearest even and saturate at 7.5.

// One scaled e2m3 x e2m3 product of a 32x32x64 block (format code 2 for both operands).  Lane half h
// holds the 32 inputs 32h..32h+31 of its row (A) or column (B) in order, and scales them by an E8M0
// exponent: byte OPS of sa for A, byte OPB of sb for B.
template <int OPS, int OPB>
__device__ __forceinline__ f32x16v_t mfma_lo(i8v_t a, i8v_t b, f32x16v_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, OPS, sa, OPB, sb);
}

__device__ __forceinline__ float gg_zp(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
}

// Buffer -> LDS copy of one wavefront: lane L's 16 bytes at voff land at LDS address lds + 16 L.  Written
// as inline assembly so that the compiler's wait-count pass, which cannot tell the stages of the ring
// apart, does not make every LDS read wait for every copy in flight; the pipeline below waits for the
// exact count itself.  M0 (the LDS base of the copy) is saved and restored, with a wait state after
// each write of it.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds), "s"(r)
        : "memory");
}

// s_waitcnt with only the vector-memory count (gfx9 encoding; expcnt and lgkmcnt left at their maxima)
#define GG_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// x (bf16 [T][d]) -> x16 (fp16 [T][d], int4 order within groups of 8), one workgroup per row at a time.  Each
// row is multiplied by the power of two 2^e that puts its largest magnitude into [2^14, 2^15), and xinv[t] =
// 2^-e, which the gate/up epilogue applies (exactly).  bf16 carries 8 significant bits and fp16 11, so every
// value of the row down to 2^-29 of its largest converts exactly, and no row overflows fp16 whatever its range.
//
// The same launch bounds h, so that it too is stored in fp16 without overflow whatever the range of x or of
// the weights.  For channel c of an expert, |g_c| = |s_c sum_i (q_ci - z_c) x_i| <= |s_c| M_c ||x||_1 with
// M_c = max |q - z| over the weight range, likewise |u_c|, and |silu(g)| <= |g|, so
//     |h_c| = |silu(g_c) u_c| <= 2^(G_e + U_e + 2 L_t),
// with 2^G_e >= max_c |s^g_c| M^g_c, 2^U_e likewise (hexp[e] = G_e + U_e; e = E for the shared expert) and
// 2^L_t >= ||x_t||_1 (xl[t] = L_t).  The gate/up pass stores h of row t, expert e times 2^-r with
// r = G_e + U_e + 2 L_t - 15 (below 2^15 in magnitude) and the down epilogue multiplies by 2^r.  The bound is
// loose by about sqrt(d) max|q - z| / std(q) per factor (2^16 to 2^20 for h), which leaves typical values of h
// far above fp16's subnormal range.  Workgroups [0, nrb) take rows, the next E (+1) experts.
constexpr int XK_KEEP = 4;  // 16-byte chunks per thread held in registers between the two passes

__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t w, uint32_t m) {
    // magnitude bit patterns of the two bf16 halves (they order as the magnitudes)
    return max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
}

// exponent ex + 1 with v < 2^ex (v >= 0): a power of two at least twice v, so fp32 rounding of v cannot reach it
__device__ __forceinline__ int exp_bound(float v) {
    int ex = 0;
    if (v > 0.f && v <= 3.0e38f) frexpf(v, &ex);
    else if (v > 3.0e38f) ex = 128;
    return ex + 1;
}

// ACT 1: x bf16 -> x16 [T][d].  ACT 0: x fp32 -> x16 [T][2 d], per K step of 64 inputs the 64 values of
// hi = fp16(x 2^e) and then the 64 of lo = fp16(x 2^e - hi) (x 2^e - hi is exact in fp32), about 22 significant
// bits in all; the gate/up pass runs every weight step against both.
template <int WBITS, int ACT>
__global__ __launch_bounds__(256) void x16_kernel(FfnParams P, _Float16 *__restrict__ x16, float *__restrict__ xinv,
                                                  int *__restrict__ xl, int *__restrict__ hexp, int nrb,
                                                  int *__restrict__ tile_ctr) {
    __shared__ float wred[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    auto block_max2 = [&](float &a, float &b) {  // workgroup-wide maxima of two non-negative values
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            a = fmaxf(a, __shfl_xor(a, o, 64));
            b = fmaxf(b, __shfl_xor(b, o, 64));
        }
        if (lane == 0) {
            wred[0][wv] = a;
            wred[1][wv] = b;
        }
        __syncthreads();
        a = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
        b = fmaxf(fmaxf(wred[1][0], wred[1][1]), fmaxf(wred[1][2], wred[1][3]));
        __syncthreads();  // wred is rewritten next
    };
    if (blockIdx.x >= nrb) {
        // ---- expert exponents: e < E routed, e == E the shared expert
        const int e = blockIdx.x - nrb;  // the weight row (routed) or E (shared)
        const bool sh = e == P.E;
        if (!sh && e >= P.n_wrows) return;  // fewer weight rows than experts (an expert cache's slots)
        const int I = sh ? P.Is : P.I;
        const long base = sh ? 0 : (long)e * I;
        const QW &W = sh ? P.shared : P.routed;
        float mg = 0.f, mu = 0.f;
        for (int c = tid; c < I; c += 256) {
            float zg, zu;
            if (WBITS == 8) {
                zg = (float)((const int8_t *)W.zg)[base + c];
                zu = (float)((const int8_t *)W.zu)[base + c];
            } else {
                zg = ((const float *)W.zg)[base + c];
                zu = ((const float *)W.zu)[base + c];
            }
            const float Mg = WBITS == 4 ? fmaxf(fabsf(zg), fabsf(15.f - zg)) : 128.f + fabsf(zg);
            const float Mu = WBITS == 4 ? fmaxf(fabsf(zu), fabsf(15.f - zu)) : 128.f + fabsf(zu);
            mg = fmaxf(mg, fabsf(W.sg[base + c]) * Mg);
            mu = fmaxf(mu, fabsf(W.su[base + c]) * Mu);
        }
        block_max2(mg, mu);
        if (tid == 0) hexp[e] = exp_bound(mg) + exp_bound(mu);
        return;
    }
    // the tile queues of the two GEMM launches that follow start empty
    if (blockIdx.x == 0 && tid < 2 * GG_XCDS) tile_ctr[tid] = 0;
    const int d = P.d, nch = d / 8;
    auto order8 = [](const _Float16 (&v)[8]) -> h8_t {
        if (WBITS == 4) return (h8_t){v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};
        return (h8_t){v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    };
    auto row_exp = [](float m) {  // 2^e puts the row maximum m into [2^14, 2^15); see below
        int e = 0;
        if (m > 0.f && m <= 3.4e38f) {
            int ex;
            frexpf(m, &ex);
            e = min(max(15 - ex, -120), 120);
        }
        return e;
    };
    if constexpr (ACT == 0) {
        const float *xf = (const float *)P.x;
        for (int t = blockIdx.x; t < P.T; t += nrb) {
            const float4 *row = (const float4 *)(xf + (long)t * d);
            float m = 0.f, unused = 0.f;
            for (int c = tid; c < 2 * nch; c += 256) {
                const float4 v = row[c];
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            block_max2(m, unused);
            const int e = row_exp(m);
            const float sc = __builtin_ldexpf(1.f, e);
            float l1 = 0.f;
            h8_t *out = (h8_t *)(x16 + (long)t * 2 * d);
            for (int c = tid; c < nch; c += 256) {
                const float4 a = row[2 * c], b = row[2 * c + 1];
                const float v[8] = {a.x * sc, a.y * sc, a.z * sc, a.w * sc, b.x * sc, b.y * sc, b.z * sc, b.w * sc};
                _Float16 hi[8], lo[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    hi[i] = (_Float16)v[i];
                    lo[i] = (_Float16)(v[i] - (float)hi[i]);
                    l1 += fabsf(v[i]);
                }
                // K step c / 8 holds 8 chunks of hi, then 8 of lo
                out[16 * (c >> 3) + (c & 7)] = order8(hi);
                out[16 * (c >> 3) + 8 + (c & 7)] = order8(lo);
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) l1 += __shfl_xor(l1, o, 64);
            if (lane == 0) wred[0][wv] = l1;
            __syncthreads();
            if (tid == 0) {
                xinv[t] = __builtin_ldexpf(1.f, -e);
                xl[t] = exp_bound((wred[0][0] + wred[0][1]) + (wred[0][2] + wred[0][3])) - e;
            }
            __syncthreads();  // wred is rewritten by the next row
        }
        return;
    }
    const uint16_t *x = (const uint16_t *)P.x;
    for (int t = blockIdx.x; t < P.T; t += nrb) {
        const uint4 *row = (const uint4 *)(x + (long)t * d);
        uint4 keep[XK_KEEP];
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < XK_KEEP; i++) {
            const int c = tid + 256 * i;
            keep[i] = c < nch ? row[c] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < XK_KEEP; i++)
            mx = bf16x2_absmax(keep[i].w, bf16x2_absmax(keep[i].z, bf16x2_absmax(keep[i].y, bf16x2_absmax(keep[i].x, mx))));
        for (int c = tid + 256 * XK_KEEP; c < nch; c += 256) {
            const uint4 q = row[c];
            mx = bf16x2_absmax(q.w, bf16x2_absmax(q.z, bf16x2_absmax(q.y, bf16x2_absmax(q.x, mx))));
        }
        float m = __uint_as_float(mx << 16), unused = 0.f;
        block_max2(m, unused);
        // 2^e with the row maximum m in [2^(ex-1), 2^ex): e = 15 - ex; rows of zeros (and non-finite rows,
        // whose outputs are not finite anyway) keep e = 0; e stays where 2^e and 2^-e are normal fp32
        int e = 0;
        if (m > 0.f && m <= 3.4e38f) {
            int ex;
            frexpf(m, &ex);
            e = min(max(15 - ex, -120), 120);
        }
        const float sc = __builtin_ldexpf(1.f, e);
        float l1 = 0.f;  // sum of the scaled magnitudes (each below 2^15: no overflow)
        auto put = [&](int c, uint4 q) {
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
            _Float16 v[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float a = __uint_as_float(w[i] << 16) * sc, b = __uint_as_float(w[i] & 0xFFFF0000u) * sc;
                l1 += fabsf(a) + fabsf(b);
                v[2 * i] = (_Float16)a;
                v[2 * i + 1] = (_Float16)b;
            }
            h8_t o;
            if (WBITS == 4)
                o = (h8_t){v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};
            else
                o = (h8_t){v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
            ((h8_t *)(x16 + (long)t * d))[c] = o;
        };
#pragma unroll
        for (int i = 0; i < XK_KEEP; i++) {
            const int c = tid + 256 * i;
            if (c < nch) put(c, keep[i]);
        }
        for (int c = tid + 256 * XK_KEEP; c < nch; c += 256) put(c, row[c]);
        // the row's L1 norm only enters through its exponent (the sum's rounding is covered by exp_bound's
        // factor 2), so a maximum-style reduction of partial sums would not do: sum them
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l1 += __shfl_xor(l1, o, 64);
        if (lane == 0) wred[0][wv] = l1;
        __syncthreads();
        if (tid == 0) {
            xinv[t] = __builtin_ldexpf(1.f, -e);
            xl[t] = exp_bound((wred[0][0] + wred[0][1]) + (wred[0][2] + wred[0][3])) - e;
        }
        __syncthreads();  // wred is rewritten by the next row
    }
}

// r for the h of a row: G_e + U_e + 2 L_t - 15, kept in [-126, 126] where 2^r and 2^-r are normal fp32.  At the
// upper clamp any finite fp32 h times 2^-126 is below 4, so a finite h never overflows fp16; at the lower clamp
// the bound is below 2^-111 and h times 2^126 stays below 2^15.
__device__ __forceinline__ int h_row_exp(int he, int lt) { return min(max(he + 2 * lt - 15, -126), 126); }

template <int V>
struct GgInt {
    static constexpr int value = V;
};

struct GemmBufs {
    const _Float16 *x16;       // [T][d], row t scaled by 1 / xinv[t]
    float *xinv;               // [T] the power of two that undoes the scale of row t of x16
    int *xl;                   // [T] L_t: 2^L_t >= ||x_t||_1
    int *hexp;                 // [E + 1] G_e + U_e (e = E: the shared expert); see x16_kernel
    _Float16 *hhi;             // [A][I] h rounded to fp16
    uint8_t *hlo;              // [A][I] its residual h - hi: per 32 channels, 24 bytes of e2m3, their sum (fp32), 4 unused
    _Float16 *hshi;            // [T][I_shared], the same for the shared expert
    uint8_t *hslo;
    uint8_t *hsc;              // residual exponents (E8M0): [row tile][K step][block 2][row 32][row block 4]
    uint32_t hsc_bytes;
    int ksmax;                 // K steps per row tile in hsc
    int *tile_ctr;             // [2][GG_XCDS] tile queue counters (zeroed by the x16 pass)
};

// Stage layout of the LDS ring.  Activation planes: 128 rows x 128 bytes (64 fp16); weights: each
// wavefront's 64 rows x RB bytes.  The 16-byte chunks of a row are permuted (XOR with a function of the
// row) so that the 16 lanes that a 128-bit LDS read serves together (16 consecutive rows, one chunk
// column) hit 16 different 16-byte slots of the 64 banks.  XOR is its own inverse: the same map takes a
// logical chunk to its slot and a slot back to the chunk.
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ ((r >> 1) & 7); }   // 128-byte rows
__device__ __forceinline__ int swz_b4(int r, int c) { return c ^ ((r >> 3) & 1); }  // 32-byte rows
__device__ __forceinline__ int swz_b8(int r, int c) { return c ^ ((r >> 2) & 3); }  // 64-byte rows

template <int MODE, int WBITS>
struct GgCfg {
    static constexpr bool RES = MODE == 1;                  // h residual plane (e2m3 + block exponents)
    static constexpr int RB = GG_K * WBITS / 8;             // weight bytes per row and step
    static constexpr int B_BYTES = GG_WAVES * GG_NW * RB;
    static constexpr int NLA = 2;                           // 1 KB copies per wavefront and step, fp16 plane
    static constexpr int NLB = GG_NW * RB / 1024;           // 1 KB weight copies per wavefront and step
    static constexpr int NL = NLA + (RES ? 2 : 0) + NLB;    // + one residual and one exponent copy
    static constexpr int NOUT_W = MODE == 0 ? 32 : 64;      // distinct output columns per wavefront
    static constexpr int NOUT_G = NOUT_W * GG_WAVES;        // per tile
    static_assert(GG_M * 128 / 1024 == NLA * GG_WAVES, "activation copies");
    // Stage layout of a tile with MU blocks of 32 rows: the fp16 plane (x or h hi; MU x 32 rows x 128 bytes),
    // the residual plane (MU x 32 rows x 64 bytes) and the 1 KB exponent copy, then the weights (each
    // wavefront's 64 rows x RB bytes); as many stages as the ring holds, at most 8.  Short tiles thus keep
    // more steps of weights in flight, which is what bounds them.
    template <int MU>
    struct Lay {
        static constexpr int PLANE = MU * 32 * GG_K * 2;
        static constexpr int LO_BYTES = RES ? MU * 32 * GG_K : 0;
        static constexpr int SC_BYTES = RES ? 1024 : 0;
        static constexpr int A_BYTES = PLANE + LO_BYTES + SC_BYTES;
        static constexpr int STAGE = A_BYTES + B_BYTES;
        static constexpr int STAGES = (GG_RING - GG_JUNK) / STAGE > 8 ? 8 : (GG_RING - GG_JUNK) / STAGE;
        static constexpr int NAC = 4 * MU;           // 1 KB copies of the fp16 plane per step
        static constexpr int NLC = RES ? 2 * MU : 0;  // of the residual plane
        static_assert(STAGES >= 2, "LDS ring");
    };
};

// MODE 0: gate/up (A = x16 rows through the permutation; each wavefront owns 32 channels, subtile 0 their
// gate rows and subtile 1 their up rows; output h as an fp16 plane plus the e2m3 residual plane and its
// exponents).  MODE 1: down (A = the h planes of the slot's rows; 64 down rows per wavefront; output
// y_perm / y_shared in fp32).  Its K step is four fp16 MFMAs on h hi and one scaled e2m3 MFMA on the
// residual, whose weights are the same dequantised values converted to e2m3.
//
// Zero points: when every zero point of the tile's weight rows is an integer (int8 always; int4 when
// its fp32 zero points are integral), it is folded into the dequantisation (B = q - z, exact in fp16);
// otherwise B = q and the epilogue subtracts z times the row sum of the activations, summed from the
// staged tiles.
// XLO (gate/up with fp32 activations): x16 holds each row as 2d fp16 values, K step by K step the step's 64
// values of hi = fp16(x) and then of lo = fp16(x - hi) (about 22 significant bits together); the K loop runs
// twice the steps and virtual step v multiplies weight step v / 2, so every weight fragment meets hi and lo.
template <int MODE, int WBITS, bool XLO>
__global__ __launch_bounds__(GG_WAVES * 64, 1) void gemm_kernel(FfnParams P, GemmBufs G, int tiles_n) {
    using C = GgCfg<MODE, WBITS>;
    constexpr bool RES = C::RES;
    constexpr int RB = C::RB;
    constexpr int NLB = C::NLB, NL = C::NL;
    constexpr int WL = WBITS == 8 ? 2 : 1;   // 16-byte weight fragments per subtile and step
    constexpr float QBIAS = WBITS == 8 ? 1152.f : 1024.f;
    extern __shared__ __align__(16) unsigned char gg_ring[];
    __shared__ int s_t0[GG_MAXSLOTS + 1];
    __shared__ float rsum[GG_M];
    // per tile row: gate/up, the power of two that undoes the scale of x, and 2^-r that scales h; down, 2^r
    __shared__ float rscale[GG_M];
    __shared__ float hscale[GG_M];
    __shared__ int s_nslot;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, lr = lane & 31;
    const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)gg_ring;

    // ---- tile table: slot s (used experts in uniq order, then the shared expert) has
    // ceil(c_s / 128) row tiles times tiles_n output tiles; s_t0 is the exclusive prefix
    if (wv == 0) {
        int nu = *P.n_uniq;
        if (nu < 0) {
            // invalid expert ids in the routing (n_uniq = -1): the valid experts are the non-negative prefix of uniq
            nu = 0;
            for (int b = 0; b < P.n_routed_slots; b += 64) {
                const int s = b + lane;
                nu += __popcll(__ballot(s < P.n_routed_slots && P.uniq[s] >= 0));
            }
        }
        nu = nu > P.n_routed_slots ? P.n_routed_slots : nu;
        const int ns = nu + (P.Is > 0 ? 1 : 0);
        int carry = 0;
        for (int b = 0; b < ns; b += 64) {
            const int s = b + lane;
            int mt = 0;
            if (s < ns) {
                int c = P.T;
                if (s < nu) {
                    const int e = P.uniq[s];
                    c = P.offsets[e + 1] - P.offsets[e];
                }
                mt = (c + GG_M - 1) / GG_M;
            }
            const int v = mt * tiles_n;
            int incl = v;
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
    const int nslot = __builtin_amdgcn_readfirstlane(s_nslot);
    const int ntiles = __builtin_amdgcn_readfirstlane(s_t0[nslot]);

    // Tile queue.  The tile list (slot-major, then output tile, then row tile: consecutive tiles share
    // weights or activations) is cut into groups of GG_GROUP tiles, dealt round-robin to the XCDs; each
    // XCD's workgroups take the tiles of its groups in order from its own counter, so the data that
    // neighbouring tiles share is read through one L2.  A workgroup whose XCD has run out takes tiles
    // from the other XCDs' queues.  The next tile is claimed while the current one runs.
    __shared__ int s_tile[2];
    int *ctr = G.tile_ctr + MODE * GG_XCDS;
    const int xcd = (int)(blockIdx.x % GG_XCDS);
    auto claim = [&]() -> int {
        for (int k = 0; k < GG_XCDS; k++) {
            const int xx = (xcd + k) % GG_XCDS;
            const int c = atomicAdd(ctr + xx, 1);
            const long t = ((long)(c / GG_GROUP) * GG_XCDS + xx) * GG_GROUP + c % GG_GROUP;
            if (t < ntiles) return (int)t;
        }
        return -1;
    };
    if (tid == 0) s_tile[0] = claim();
    __syncthreads();
    int tsel = 0;
    for (int tile = __builtin_amdgcn_readfirstlane(s_tile[0]); tile >= 0;
         tile = __builtin_amdgcn_readfirstlane(s_tile[tsel])) {
        if (tid == 0) s_tile[tsel ^ 1] = claim();  // read after the barriers of this tile
        tsel ^= 1;
        // ---- locate the tile: slot (binary search), output tile, row tile
        int lo = 0, hi = nslot - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_t0[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int slot = __builtin_amdgcn_readfirstlane(lo);
        const bool shared = P.Is > 0 && slot == nslot - 1;
        int e = 0, wr = 0, p0 = 0, cnt = P.T;
        bool resident = P.y_sh != nullptr;  // (shared) y_sh = nullptr: the shared expert left out
        if (!shared) {
            e = ld_const(P.uniq, slot);
            p0 = ld_const(P.offsets, e);
            cnt = ld_const(P.offsets, e + 1) - p0;
            wr = weight_row(P, e);
            resident = wr >= 0;
            if (!resident) wr = 0;
        }
        const int mt_n = (cnt + GG_M - 1) / GG_M;
        const int local = tile - __builtin_amdgcn_readfirstlane(s_t0[slot]);
        const int ntile = local / mt_n, mtile = local % mt_n;
        const int r0 = mtile * GG_M;                     // first row of the tile within the slot
        // an expert whose weights are not resident: a tile of no rows (reads and writes nothing)
        const int rows = resident ? min(GG_M, cnt - r0) : 0;
        // row tile number over all slots (the same in both passes: the prefix counts row tiles times
        // tiles_n); it indexes the residual exponents
        const int rt = __builtin_amdgcn_readfirstlane(s_t0[slot]) / tiles_n + mtile;
        const int I = shared ? P.Is : P.I;
        const int KK = MODE == 0 ? P.d : I;              // contraction length
        const int KX = MODE == 0 && XLO ? 2 * KK : KK;   // activation values per row (hi and lo with XLO)
        const int nout = MODE == 0 ? I : P.d;
        const int nsteps = KX / GG_K;
        // field by field: a reference into the by-value parameter block would make the compiler copy it
        // to private memory and read these pointers back into vector registers
        QW W;
        W.qg = shared ? P.shared.qg : P.routed.qg;
        W.qu = shared ? P.shared.qu : P.routed.qu;
        W.qd = shared ? P.shared.qd : P.routed.qd;
        W.sg = shared ? P.shared.sg : P.routed.sg;
        W.su = shared ? P.shared.su : P.routed.su;
        W.sd = shared ? P.shared.sd : P.routed.sd;
        W.zg = shared ? P.shared.zg : P.routed.zg;
        W.zu = shared ? P.shared.zu : P.routed.zu;
        W.zd = shared ? P.shared.zd : P.routed.zd;
        const long rbf = (long)KK * WBITS / 8;           // bytes per weight row

        // ---- copy sources.  fp16 activations: this lane fills slot lane & 7 of row 8 (2 wv + i) + lane / 8
        // (i = 0, 1), i.e. it moves the logical chunk that the swizzle puts there.  Residual plane: slot
        // lane & 3 of row 16 wv + lane / 4.  Exponents (wavefront 0): lanes 0..15 copy the 256 bytes of the
        // step, the other lanes' out-of-range copies fill the rest of the 1 KB with zeros.
        rsrc_t ars, alrs, scrs;
        uint32_t asrc[2], alsrc = kOOB, scsrc = kOOB;
        {
            if (MODE == 0) {
                ars = make_rsrc(G.x16, (uint32_t)((long)P.T * KX * 2));
                alrs = scrs = ars;  // unused
            } else {
                const long nr = shared ? P.T : P.A;
                ars = make_rsrc(shared ? G.hshi : G.hhi, (uint32_t)(nr * I * 2));
                alrs = make_rsrc(shared ? G.hslo : G.hlo, (uint32_t)(nr * I));
                scrs = make_rsrc(G.hsc, G.hsc_bytes);
                const int m = 16 * wv + (lane >> 2);
                if (m < rows) alsrc = (uint32_t)(((long)(shared ? 0 : p0) + r0 + m) * I) + 16 * swz_b8(m, lane & 3);
                if (wv == 0 && lane < 16) scsrc = (uint32_t)rt * (uint32_t)G.ksmax * 256u + 16 * lane;
            }
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = 8 * (2 * wv + i) + (lane >> 3);
                const uint32_t alc = (uint32_t)swz_a(m, lane & 7);
                uint32_t off = kOOB;
                if (m < rows) {
                    long row;
                    if (MODE == 0) row = shared ? (r0 + m) : (P.perm[p0 + r0 + m] / P.k);
                    else row = (long)(shared ? 0 : p0) + r0 + m;
                    off = (uint32_t)(row * KX * 2) + 16 * alc;
                    // one lane per row brings the row's scales (read in the epilogue, after the K loop's barriers;
                    // the previous tile's epilogue is done with them since the barrier that ends it)
                    if ((lane & 7) == 0) {
                        const int he = G.hexp[shared ? P.E : wr];
                        if (MODE == 0) {
                            rscale[m] = G.xinv[row];
                            hscale[m] = __builtin_ldexpf(1.f, -h_row_exp(he, G.xl[row]));
                        } else {
                            const int tok = shared ? r0 + m : P.perm[p0 + r0 + m] / P.k;
                            rscale[m] = __builtin_ldexpf(1.f, h_row_exp(he, G.xl[tok]));
                        }
                    }
                }
                asrc[i] = off;
            }
        }
        // Weights: 1 KB copy i of this wavefront holds rows 32 i + lane / 2 (int4) or 16 i + lane / 4
        // (int8) of its 64; row r of subtile j = r / 32 is column 32 j + r % 32 of the wavefront.
        rsrc_t brs[2];
        uint32_t bsrc[NLB];
        const int nbase = ntile * C::NOUT_G + wv * C::NOUT_W;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const uint8_t *base = MODE == 0 ? (j == 0 ? W.qg : W.qu) + (long)wr * I * rbf : W.qd + (long)wr * P.d * rbf;
            brs[j] = make_rsrc(base, (uint32_t)(nout * rbf));
        }
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            int rl, lc;
            if (WBITS == 4) {
                rl = 32 * i + (lane >> 1);
                lc = swz_b4(rl, lane & 1);
            } else {
                rl = 16 * i + (lane >> 2);
                lc = swz_b8(rl, lane & 3);
            }
            const int j = rl >> 5, col = rl & 31;
            const int o = MODE == 0 ? nbase + col : nbase + 32 * j + col;
            bsrc[i] = o < nout ? (uint32_t)(o * rbf) + 16 * lc : kOOB;
        }

        // ---- epilogue columns, scales and zero points of this lane (column lr of subtile j)
        int ocol[2];
        float sc[2], zp[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int o = MODE == 0 ? nbase + lr : nbase + 32 * j + lr;
            ocol[j] = o;
            const long ncol = MODE == 0 ? I : P.d;
            const long ch = (long)wr * ncol + min(o, nout - 1);
            if (MODE == 0) {
                sc[j] = j == 0 ? W.sg[ch] : W.su[ch];
                zp[j] = gg_zp(j == 0 ? W.zg : W.zu, WBITS, ch);
            } else {
                sc[j] = W.sd[ch];
                zp[j] = gg_zp(W.zd, WBITS, ch);
            }
        }
        // (|z| <= 256 keeps the folded weights q - z and the offsets below exact in fp16)
        bool my_int = true;
#pragma unroll
        for (int j = 0; j < 2; j++) my_int = my_int && zp[j] == rintf(zp[j]) && fabsf(zp[j]) <= 256.f;
        const bool fold = __syncthreads_and(my_int);  // uniform over the workgroup
        h2_t boff[2], boff16[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const float z = fold ? zp[j] : 0.f;
            const _Float16 o = (_Float16)(-(QBIAS + z)), o16 = (_Float16)(-(64.f + z));
            boff[j] = (h2_t){o, o};
            boff16[j] = (h2_t){o16, o16};
        }
        // Weights of the residual product: the dequantised values divided by 2^be, the smallest power of two
        // that brings the column's largest possible |B| to 7.5 or less (e2m3 keeps no more); exact for int4
        // with an integral z in 0..15 (be = 1), 4 significant bits above 2^be otherwise.
        // Its E8M0 exponent 127 + be of subtile j sits in byte j of sbp.
        int sbp = 0;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const float z = fold ? zp[j] : 0.f;
            const float mx = WBITS == 4 ? fmaxf(fabsf(z), fabsf(15.f - z)) : 128.f + fabsf(z);
            int be = -1;
            while (7.5f * __builtin_ldexpf(1.f, be) < mx) be++;
            sbp |= (127 + be) << (8 * j);
        }
        // nibble masks kept in registers (the three-operand and-or cannot take two literals)
        const uint32_t mlo = __builtin_amdgcn_readfirstlane(0x000F000Fu), mhi = __builtin_amdgcn_readfirstlane(0x00F000F0u);

        // ---- LDS read offsets within a stage
        uint32_t ard[4];  // activation fragment of substep s: row lr (+ 32 mm), chunk 4 kg + s
#pragma unroll
        for (int s = 0; s < 4; s++) ard[s] = (uint32_t)(lr * 128 + swz_a(lr, 4 * kg + s) * 16);
        // ---- the tile, with the number of 32-row blocks that hold data as a compile-time constant
        auto run = [&](auto muc) {
            constexpr int MU = decltype(muc)::value;
            using Y = typename C::template Lay<MU>;
            constexpr int PLANE = Y::PLANE, STAGE = Y::STAGE, STAGES = Y::STAGES;
            uint32_t brd[2][WL];  // weight fragment of subtile j: row 32 j + lr of the wavefront, bytes 32 kg ...
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int h = 0; h < WL; h++) {
                    const int rl = 32 * j + lr;
                    const int pc = WBITS == 4 ? swz_b4(rl, kg) : swz_b8(rl, 2 * kg + h);
                    brd[j][h] = (uint32_t)(Y::A_BYTES + wv * GG_NW * RB + rl * RB + pc * 16);
                }
            // Copies of step `step` into stage `stg`.  Every wavefront issues the same number per step (so one
            // wait count serves all): the activation rows past MU x 32 and the exponents of wavefronts other
            // than 0 go to the junk area and read nothing, and so does every copy of a step past the end of K.
            const uint32_t junk = ring0 + (uint32_t)(GG_RING - GG_JUNK);
            auto issue = [&](int step, int stg) {
                const uint32_t sb = ring0 + (uint32_t)(stg * STAGE);
                const bool live = step < nsteps;
                auto src = [&](uint32_t base, uint32_t adv) { return live ? base + adv : kOOB; };
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const int c = 2 * wv + i;
                    dma16(ars, c < Y::NAC ? sb + c * 1024 : junk, src(asrc[i], (uint32_t)(step * 128)));
                }
                if constexpr (RES) {
                    dma16(alrs, wv < Y::NLC ? sb + PLANE + wv * 1024 : junk, src(alsrc, (uint32_t)(step * 64)));
                    dma16(scrs, wv == 0 ? sb + PLANE + Y::LO_BYTES : junk, src(scsrc, (uint32_t)(step * 256)));
                }
#pragma unroll
                for (int i = 0; i < NLB; i++)
                    dma16(brs[WBITS == 4 ? i : i >> 1], sb + Y::A_BYTES + wv * GG_NW * RB + i * 1024,
                          src(bsrc[i], (uint32_t)((XLO ? step >> 1 : step) * RB)));
            };
            f32x16v_t acc[MU][2];
#pragma unroll
            for (int mm = 0; mm < MU; mm++)
#pragma unroll
                for (int j = 0; j < 2; j++) acc[mm][j] = (f32x16v_t){};
            float rs = 0.f;

            // Operand registers: activation fragments of two substeps, the raw weights of a step and their
            // dequantised values (two substeps; with the residual plane all four, which its e2m3 weights are
            // converted from at once); with the residual plane, its fragments and its exponent word.
            constexpr int NBR = 2 * WL;  // raw weight reads per step
            constexpr int NBQ = RES ? 4 : 2;
            uint4 braw[2][WL];
            h8_t af[2][MU];
            h8_t bq[NBQ][2];
            i8v_t al[MU], bl[2];
            int scw = 0;
            auto bqi = [](int sub) { return RES ? sub : (sub & 1); };
            auto rd_b = [&](const unsigned char *p) {
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int h = 0; h < WL; h++) braw[j][h] = *(const uint4 *)(p + brd[j][h]);
            };
            auto rd_a = [&](const unsigned char *p, int sub, int buf) {
#pragma unroll
                for (int mm = 0; mm < MU; mm++) af[buf][mm] = *(const h8_t *)(p + mm * 4096 + ard[sub]);
            };
            auto deq = [&](int sub, int buf) {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    if (WBITS == 4) {
                        const uint32_t ww[4] = {braw[j][0].x, braw[j][0].y, braw[j][0].z, braw[j][0].w};
                        bq[buf][j] = deq_int4(ww[sub], mlo, mhi, boff[j], boff16[j]);
                    } else {
                        const uint4 q = braw[j][sub >> 1];
                        bq[buf][j] = (sub & 1) ? deq_int8(q.z, q.w, boff[j]) : deq_int8(q.x, q.y, boff[j]);
                    }
                }
            };
            auto mfmas = [&](int sub) {
#pragma unroll
                for (int mm = 0; mm < MU; mm++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[mm][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[sub & 1][mm], bq[bqi(sub)][j],
                                                                            acc[mm][j], 0, 0, 0);
            };
            // Residual product.  Lane half kg dequantises inputs 32 kg + 8 s .. + 7 in substep s, so after four
            // substeps it holds inputs 32 kg .. 32 kg + 31 in order: the operand layout of the e2m3 product.
            auto pk6 = [&]() {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    h32_t v;
#pragma unroll
                    for (int q = 0; q < 4; q++)
#pragma unroll
                        for (int i = 0; i < 8; i++) v[8 * q + i] = bq[q][j][i];
                    const float bx = __builtin_bit_cast(float, (((uint32_t)sbp >> (8 * j)) & 0xFFu) << 23);  // 2^be
                    const u6v_t r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(v, bx);
                    bl[j] = (i8v_t){(int)r[0], (int)r[1], (int)r[2], (int)r[3], (int)r[4], (int)r[5], 0, 0};
                }
            };
            // residual fragment: row lr (+ 32 mm), the 24 bytes of inputs 32 kg .. 32 kg + 31 (chunk 2 kg and the
            // first 8 bytes of chunk 2 kg + 1); the exponent word of row block kg, rows lr + 32 mm in byte mm.
            // The offsets are recomputed at each use (from an opaque copy of the lane index), which costs a few
            // instructions per step instead of registers held across the loop.
            auto rd_lo = [&](const unsigned char *p) {
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int r = ln & 31, h = ln >> 5;
                uint32_t ald[2];
#pragma unroll
                for (int i = 0; i < 2; i++) ald[i] = (uint32_t)(PLANE + r * 64 + swz_b8(r, 2 * h + i) * 16);
                const uint32_t scd = (uint32_t)(PLANE + Y::LO_BYTES + h * 128 + r * 4);
#pragma unroll
                for (int mm = 0; mm < MU; mm++) {
                    const i4v_t u0 = *(const i4v_t *)(p + mm * 2048 + ald[0]);
                    const i2v_t u1 = *(const i2v_t *)(p + mm * 2048 + ald[1]);
                    al[mm] = (i8v_t){u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], 0, 0};
                }
                scw = *(const int *)(p + scd);
            };
            auto mfmas_lo = [&]() {
#pragma unroll
                for (int mm = 0; mm < MU; mm++)
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        if (mm == 0) acc[mm][j] = j == 0 ? mfma_lo<0, 0>(al[mm], bl[j], acc[mm][j], scw, sbp) : mfma_lo<0, 1>(al[mm], bl[j], acc[mm][j], scw, sbp);
                        else if (mm == 1) acc[mm][j] = j == 0 ? mfma_lo<1, 0>(al[mm], bl[j], acc[mm][j], scw, sbp) : mfma_lo<1, 1>(al[mm], bl[j], acc[mm][j], scw, sbp);
                        else if (mm == 2) acc[mm][j] = j == 0 ? mfma_lo<2, 0>(al[mm], bl[j], acc[mm][j], scw, sbp) : mfma_lo<2, 1>(al[mm], bl[j], acc[mm][j], scw, sbp);
                        else acc[mm][j] = j == 0 ? mfma_lo<3, 0>(al[mm], bl[j], acc[mm][j], scw, sbp) : mfma_lo<3, 1>(al[mm], bl[j], acc[mm][j], scw, sbp);
                    }
            };
            auto wait_steps = [&](auto nc) {  // all but the copies of the last n steps issued have landed
                constexpr int n = decltype(nc)::value;
                GG_WAIT_VM(n * NL);
            };

            // ---- prologue: STAGES steps in flight, the operands of step 0 in registers
#pragma unroll
            for (int i = 0; i < STAGES; i++) issue(i, i);
            wait_steps(GgInt<STAGES - 1>{});
            __syncthreads();
            rd_b(gg_ring);
            rd_a(gg_ring, 0, 0);
            deq(0, 0);

            // ---- K loop.  Step t's data sit in stage t % STAGES.  The copies of step t + STAGES are issued
            // into the stage of step t once every wavefront has passed the barrier of step t, which comes
            // after the last read of that stage (the fragments of the last phase are read one phase ahead).
            int stg = 0;
            for (int step = 0; step < nsteps; step++) {
                const unsigned char *sp = gg_ring + stg * STAGE;
                const int nstg = stg + 1 == STAGES ? 0 : stg + 1;
                if (!fold) {
                    // row sums of the staged activations: row tid / 4, fp16 chunks 2 (tid % 4) and
                    // 2 (tid % 4) + 1, residual chunk tid % 4 (times its block exponent)
                    const int m = tid >> 2;
                    if (m < MU * 32) {
#pragma unroll
                        for (int h = 0; h < 2; h++) {
                            const int pc = swz_a(m, 2 * (tid & 3) + h);
                            const h8_t v = *(const h8_t *)(sp + m * 128 + pc * 16);
#pragma unroll
                            for (int i = 0; i < 8; i++) rs += (float)v[i];
                        }
                        if constexpr (RES) {
                            // the residual block sums of the step (bytes 24..27 of each 32-byte block)
                            const int q = tid & 3;
                            if (q < 2) rs += *(const float *)(sp + PLANE + m * 64 + swz_b8(m, 2 * q + 1) * 16 + 8);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // substeps but the last: the MFMAs of substep s run interleaved with the fragment reads and
                // the dequantisation of substep s + 1
#pragma unroll
                for (int ph = 0; ph < 3; ph++) {
                    rd_a(sp, ph + 1, (ph + 1) & 1);
                    deq(ph + 1, bqi(ph + 1));
                    mfmas(ph);
#pragma unroll
                    for (int i = 0; i < 2 * MU; i++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
                        if (i < MU) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);            // VALU
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (RES) {
                    // substep 3 (with the reads of the residual fragments and the e2m3 conversion of the
                    // step's weights), then the residual product; step + 1 has landed everywhere after the
                    // barrier, and its operands are read while the residual MFMAs run
                    rd_lo(sp);
                    pk6();
                    mfmas(3);
#pragma unroll
                    for (int i = 0; i < 2 * MU; i++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (i < MU) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    wait_steps(GgInt<STAGES - 2>{});
                    __syncthreads();
                    issue(step + STAGES, stg);
                    const unsigned char *np = gg_ring + nstg * STAGE;
                    rd_b(np);
                    rd_a(np, 0, 0);
                    mfmas_lo();
                    deq(0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, NBR + MU, 0);  // the reads first
#pragma unroll
                    for (int i = 0; i < 2 * MU; i++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (i >= MU / 2) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    // last substep: step + 1 has landed everywhere after the barrier; its operands are read
                    // while the MFMAs of this substep run
                    wait_steps(GgInt<STAGES - 2>{});
                    __syncthreads();
                    issue(step + STAGES, stg);
                    const unsigned char *np = gg_ring + nstg * STAGE;
                    rd_b(np);
                    rd_a(np, 0, 0);
                    mfmas(3);
                    deq(0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, NBR + MU, 0);  // the reads first
#pragma unroll
                    for (int i = 0; i < 2 * MU; i++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (i >= MU / 2) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                stg = nstg;
            }
            GG_WAIT_VM(0);  // the copies issued past the end land before the ring is reused
            {
                // row sums (zeros when the zero points are folded: the epilogue reads them either way)
                float t = rs;
                t += __shfl_xor(t, 1, 64);
                t += __shfl_xor(t, 2, 64);
                if ((tid & 3) == 0) rsum[tid >> 2] = t;
            }
            __syncthreads();

            // ---- epilogue: lane column ocol[j]; register r holds row 8 (r / 4) + 4 kg + r % 4 of block mm.
            // The lane's row offset is made opaque here so that the compiler does not hoist the 64 row
            // indices that derive from it out of the tile loop (they would occupy registers throughout).
            // Stores go through buffer descriptors based at the tile's first row and ending after its last,
            // so rows past the tile fall out of range, as do columns past the output (their offsets are
            // made out of range): the bounds check drops them, with no branch around the stores.
            int mk = 4 * kg;
            asm volatile("" : "+v"(mk));
            const long prow0 = (long)(shared ? 0 : p0) + r0;  // output row of tile row 0
            float zpe[2];  // zero point still to apply (0 when folded)
#pragma unroll
            for (int j = 0; j < 2; j++) zpe[j] = fold ? 0.f : zp[j];
            // tile row of register r of block mm: the lane part mk plus a uniform part
            auto mrow = [](int mm, int r) { return mm * 32 + 8 * (r >> 2) + (r & 3); };
            if constexpr (MODE == 0) {
                const int c = ocol[0];
                // stored at the planes' position of channel c (int4 order within groups of 8)
                const uint32_t hp = (uint32_t)(WBITS == 4 ? ((c & ~7) | pos8(c & 7)) : c);
                const uint32_t o2 = c < nout ? 2 * hp : kOOB;
                const rsrc_t hhr = make_rsrc((shared ? G.hshi : G.hhi) + prow0 * I, (uint32_t)(rows * I * 2));
                const rsrc_t hlr = make_rsrc((shared ? G.hslo : G.hlo) + prow0 * I, (uint32_t)(rows * I));
                // The 32 channels of this wavefront (positions nbase .. nbase + 31) form one residual block of K
                // step nbase / 64 of the down pass (block (nbase / 32) % 2).  The residuals go through LDS, this
                // wavefront's 128 rows x 32 fp32, so that one lane holds a row's block: position p sits in
                // column 16 (p % 2) + p / 2 (the operand order of the paired conversion below), and the 16-byte
                // chunks of a row are XOR-swizzled by the row so that the row reads spread over the banks.
                const long scbase = ((long)rt * G.ksmax + (nbase >> 6)) * 256 + ((nbase >> 5) & 1) * 128;
                const rsrc_t hsr = make_rsrc(G.hsc + scbase, 128);
                const bool blk_ok = nbase < nout;
                const uint32_t mkI = (uint32_t)mk * (uint32_t)I;
                float *tr = (float *)(gg_ring + wv * (GG_M * 128));
                const int pc = (int)(hp & 31);
                const int tcol = ((pc & 1) << 4) | (pc >> 1);
                auto tix = [](int m, int col) { return m * 32 + ((((col >> 2) ^ m) & 7) << 2) + (col & 3); };
                uint32_t nonfinite = 0;  // h values of this lane that fp16 cannot hold
#pragma unroll
                for (int mm = 0; mm < MU; mm++) {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int m = mrow(mm, r) + mk;
                        const float xs = rsum[m], xr = rscale[m];
                        // (x was scaled by 1 / xr, a power of two: these products are exact)
                        const float gv = sc[0] * ((acc[mm][0][r] - zpe[0] * xs) * xr);
                        const float uv = sc[1] * ((acc[mm][1][r] - zpe[1] * xs) * xr);
                        // silu through the hardware exp2 and reciprocal (relative error ~1e-6, below the
                        // precision that h keeps); h is stored times 2^-r (exact: a power of two)
                        const float hv = gv * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504f * gv)) * uv *
                                         hscale[m];
                        const _Float16 hh = (_Float16)hv;
                        const uint32_t mo = mkI + (uint32_t)mrow(mm, r) * (uint32_t)I;
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hh), hhr, (int)(2 * mo + o2), 0, 0);
                        // rows past the tile and columns past the output give zeros (the block maximum ignores them)
                        const bool valid = c < nout && m < rows;
                        tr[tix(m, tcol)] = valid ? hv - (float)hh : 0.f;
                        nonfinite += (valid && (__builtin_bit_cast(uint16_t, hh) & 0x7C00u) == 0x7C00u) ? 1u : 0u;
                    }
                }
                if (P.diag && nonfinite) atomicAdd(P.diag, nonfinite);
                __syncthreads();
                // Lane L takes rows L and L + 64 (those of the MU blocks): the block exponent S puts the largest
                // residual magnitude into [4, 7.75), the top binade of e2m3 (into [2, 4) where it would round
                // past 7.5); the values, divided by 2^(S - 127), become e2m3 codes (nearest even).  32 bytes
                // per row and block: the 24 of the codes, their sum in fp32, 4 unused.
#pragma unroll
                for (int rr = 0; rr < 2; rr++) {
                    const int m = lane + 64 * rr;
                    if (64 * rr < MU * 32 && m < MU * 32) {
                        // (the maximum is taken from the loaded scalars: a bit cast of a vector element
                        // compiles to a read of element 0 with this compiler)
                        f16v_t b0, b1;
                        uint32_t mx = 0;
                        auto amax = [&](float f) { mx = max(mx, __builtin_bit_cast(uint32_t, f) & 0x7FFFFFFFu); };
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float4 u = *(const float4 *)(tr + tix(m, 4 * i));
                            const float4 v = *(const float4 *)(tr + tix(m, 16 + 4 * i));
                            b0[4 * i] = u.x; b0[4 * i + 1] = u.y; b0[4 * i + 2] = u.z; b0[4 * i + 3] = u.w;
                            b1[4 * i] = v.x; b1[4 * i + 1] = v.y; b1[4 * i + 2] = v.z; b1[4 * i + 3] = v.w;
                            amax(u.x); amax(u.y); amax(u.z); amax(u.w);
                            amax(v.x); amax(v.y); amax(v.z); amax(v.w);
                        }
                        int S = (int)(mx >> 23) - 2 + ((mx & 0x7FFFFFu) >= 0x780000u ? 1 : 0);
                        S = min(max(S, 1), 254);
                        const float X = __builtin_bit_cast(float, (uint32_t)S << 23);
                        const u6v_t q = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(b0, b1, X);
                        // the sum of the stored (rounded) residuals, for the zero-point term of the down pass:
                        // exact, as every value is a multiple of X / 8 below 7.5 X
                        const f32x32v_t dq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(q, X);
                        float bs = 0.f;
#pragma unroll
                        for (int i = 0; i < 32; i++) bs += dq[i];
                        const uint32_t ro = blk_ok ? (uint32_t)m * (uint32_t)I + (uint32_t)nbase : kOOB;
                        typedef int i32x4 __attribute__((ext_vector_type(4)));
                        __builtin_amdgcn_raw_buffer_store_b128((i32x4){(int)q[0], (int)q[1], (int)q[2], (int)q[3]}, hlr, (int)ro, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b128((i32x4){(int)q[4], (int)q[5], __builtin_bit_cast(int, bs), 0}, hlr, (int)(ro + 16), 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)S, hsr, (int)((m & 31) * 4 + (m >> 5) + (blk_ok ? 0u : kOOB)), 0, 0);
                    }
                }
            } else {
                const rsrc_t yr = make_rsrc((shared ? P.y_sh : P.y_perm) + prow0 * P.d, (uint32_t)(rows * P.d * 4));
                uint32_t yo[2];
#pragma unroll
                for (int j = 0; j < 2; j++) yo[j] = ocol[j] < nout ? 4 * (uint32_t)ocol[j] : kOOB;
                const uint32_t rowb = 4 * (uint32_t)P.d, mkd = (uint32_t)mk * rowb;
#pragma unroll
                for (int mm = 0; mm < MU; mm++) {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float xs = rsum[mrow(mm, r) + mk], hr = rscale[mrow(mm, r) + mk];
                        const uint32_t mo = mkd + (uint32_t)mrow(mm, r) * rowb;
#pragma unroll
                        for (int j = 0; j < 2; j++) {
                            // (h was stored times 2^-r: the product by 2^r is exact, and comes last so that
                            // a large 2^r cannot overflow ahead of the scale)
                            const float y = (sc[j] * (acc[mm][j][r] - zpe[j] * xs)) * hr;
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, y), yr, (int)(mo + yo[j]), 0, 0);
                        }
                    }
                }
            }
        };
        const int nm32 = (rows + 31) >> 5;  // 32-row MFMA blocks with data
        if (nm32 >= 4) run(GgInt<4>{});
        else if (nm32 == 3) run(GgInt<3>{});
        else if (nm32 == 2) run(GgInt<2>{});
        else run(GgInt<1>{});
        __syncthreads();  // rsum and the ring are reused by the next tile
    }
}

// ---------------------------------------------------------------------------- host side

static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Row tiles over all slots: at most A / 128 + (used experts) routed ones, plus T / 128 shared ones.
static long gg_row_tiles(const FfnParams &P) {
    return ((long)P.A + GG_M - 1) / GG_M + P.n_routed_slots + (P.Is > 0 ? ((long)P.T + GG_M - 1) / GG_M : 0);
}
static long gg_ksmax(const FfnParams &P) { return (P.I > P.Is ? P.I : P.Is) / GG_K; }
static size_t gg_hsc_bytes(const FfnParams &P) { return (size_t)gg_row_tiles(P) * gg_ksmax(P) * 256; }

// fp16 activation values per row: d, or 2 d (hi and lo) for fp32 activations
static long gg_xrow(const FfnParams &P) { return P.act == 1 ? P.d : 2L * P.d; }

size_t gemm_workspace_bytes(const FfnParams &P) {
    return al256((size_t)P.T * gg_xrow(P) * 2) + 2 * al256((size_t)P.T * 4) + al256((size_t)(P.E + 1) * 4) +
           al256((size_t)P.A * P.I * 2) + al256((size_t)P.A * P.I) +
           al256((size_t)P.T * P.Is * 2) + al256((size_t)P.T * P.Is) + al256(gg_hsc_bytes(P)) +
           al256(2 * GG_XCDS * sizeof(int));
}

bool gemm_supported(const FfnParams &P) {
    if (P.act != 0 && P.act != 1) return false;  // fp32 or bf16 activations
    if (P.d % GG_K || P.I % GG_K || (P.Is > 0 && P.Is % GG_K)) return false;
    if (P.n_routed_slots + 1 > GG_MAXSLOTS) return false;
    // 32-bit buffer offsets
    const long Imax = P.I > P.Is ? P.I : P.Is;
    if (Imax * ((long)P.d * P.wbits / 8) > 0x7FFFFFFFL) return false;
    if ((long)P.A * Imax * 2 > 0x7FFFFFFFL || (long)P.T * gg_xrow(P) * 2 > 0x7FFFFFFFL) return false;
    if ((long)gg_hsc_bytes(P) > 0x7FFFFFFFL) return false;
    // epilogue stores: 32-bit offsets within one 128-row tile (out-of-range marker added on top)
    if ((long)GG_M * Imax * 2 > 0x7FFFFFFFL || (long)GG_M * P.d * 4 > 0x7FFFFFFFL) return false;
    return true;
}

static int gg_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    return n;
}

template <int MODE, int WBITS, bool XLO>
static hipError_t gg_launch_mode(const FfnParams &P, const GemmBufs &G, hipStream_t stream) {
    using C = GgCfg<MODE, WBITS>;
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int tiles_n = ((MODE == 0 ? Imax : P.d) + C::NOUT_G - 1) / C::NOUT_G;
    const size_t lds = GG_RING;  // every tile shape lays its stages (and the junk area) out in the ring
    auto fn = gemm_kernel<MODE, WBITS, XLO>;
    hipError_t err = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(fn, dim3(gg_cus()), dim3(GG_WAVES * 64), lds, stream, P, G, tiles_n);
    return hipGetLastError();
}

template <int WBITS>
static hipError_t gg_launch(const FfnParams &P, const GemmBufs &G, hipStream_t stream) {
    long nrb = P.T;  // row workgroups, a row per workgroup at a time; then one per expert
    if (nrb > (long)gg_cus() * 8) nrb = (long)gg_cus() * 8;
    const long grid = nrb + P.E + (P.Is > 0 ? 1 : 0);
    if (P.act == 1)
        hipLaunchKernelGGL((x16_kernel<WBITS, 1>), dim3((unsigned)grid), dim3(256), 0, stream, P, (_Float16 *)G.x16,
                           G.xinv, G.xl, G.hexp, (int)nrb, G.tile_ctr);
    else
        hipLaunchKernelGGL((x16_kernel<WBITS, 0>), dim3((unsigned)grid), dim3(256), 0, stream, P, (_Float16 *)G.x16,
                           G.xinv, G.xl, G.hexp, (int)nrb, G.tile_ctr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = P.act == 1 ? gg_launch_mode<0, WBITS, false>(P, G, stream) : gg_launch_mode<0, WBITS, true>(P, G, stream);
    if (err != hipSuccess) return err;
    return gg_launch_mode<1, WBITS, false>(P, G, stream);
}

hipError_t launch_ffn_gemm(const FfnParams &P, void *ws, hipStream_t stream) {
    if (!gemm_supported(P)) return hipErrorNotSupported;
    char *p = (char *)ws;
    GemmBufs G;
    G.x16 = (const _Float16 *)p;
    p += al256((size_t)P.T * gg_xrow(P) * 2);
    G.xinv = (float *)p;
    p += al256((size_t)P.T * 4);
    G.xl = (int *)p;
    p += al256((size_t)P.T * 4);
    G.hexp = (int *)p;
    p += al256((size_t)(P.E + 1) * 4);
    G.hhi = (_Float16 *)p;
    p += al256((size_t)P.A * P.I * 2);
    G.hlo = (uint8_t *)p;
    p += al256((size_t)P.A * P.I);
    G.hshi = (_Float16 *)p;
    p += al256((size_t)P.T * P.Is * 2);
    G.hslo = (uint8_t *)p;
    p += al256((size_t)P.T * P.Is);
    G.hsc = (uint8_t *)p;
    G.hsc_bytes = (uint32_t)gg_hsc_bytes(P);
    G.ksmax = (int)gg_ksmax(P);
    p += al256(gg_hsc_bytes(P));
    G.tile_ctr = (int *)p;
    return P.wbits == 4 ? gg_launch<4>(P, G, stream) : gg_launch<8>(P, G, stream);
}

}  // namespace moe
