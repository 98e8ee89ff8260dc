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
// activations, and the scale in the epilogue.  Activations: x is bf16 and is converted once to fp16
// (exact save for magnitudes below 2^-14); h enters the down GEMM as fp16 hi + lo planes (two MFMAs into
// one accumulator, about 22 significant bits: a single fp16 rounding of h moves the largest down outputs
// by up to 3e-3 of their RMS).  Accumulation is fp32.
//
// Layout of the activation planes (x16, h hi/lo): row-major, and for int4 weights the 8 inputs of each
// group are stored in the order 0,4,1,5,2,6,3,7, the order in which the nibble dequantisation below
// produces the weights.
//
// Tiles: 128 rows; 8 wavefronts as 2 (rows) x 4 (columns), each 64 rows x 2 subtiles of 32 columns.
// Gate/up pairs the gate and up rows of the same 32 channels in one wavefront (128 channels per tile),
// down takes 64 outputs per wavefront (256 per tile).  A persistent grid (one workgroup per CU) walks
// the tiles (slot-major, then output tile, then row tile) from a table built on the device from
// n_uniq / uniq / offsets, so one launch shape
// serves every routing.  Activations go through registers to LDS and weights to registers, both two
// K steps ahead.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16v_t __attribute__((ext_vector_type(16)));

constexpr int GG_M = 128;       // rows per tile
constexpr int GG_WAVES = 8;
constexpr int GG_K = 64;        // K per pipeline step
constexpr int GG_LDA = 72;      // LDS row stride of an activation plane, in halfs (64 + 8 of padding)
constexpr int GG_MAXSLOTS = 1025;

// storage position, within its group of 8, of input i of the group (int4 weights)
__device__ __forceinline__ int pos8(int i) { return ((i & 3) << 1) | (i >> 2); }

// fp16 values of eight int4 weights from one word of packed nibbles (input k in the low nibble of byte
// k/2), in the order k = 0,4,1,5,2,6,3,7: 0x6400 | n is the fp16 bit pattern of 1024 + n, and off is
// -(1024 + z) with z the integral zero point folded in (or 0).  Exact: |q - z| <= 1024 + 15.
__device__ __forceinline__ h8_t deq_int4(uint32_t w, h2_t off) {
    const uint32_t M = 0x000F000Fu, B = 0x64006400u;
    const h2_t p0 = __builtin_bit_cast(h2_t, (w & M) | B) + off;
    const h2_t p1 = __builtin_bit_cast(h2_t, ((w >> 4) & M) | B) + off;
    const h2_t p2 = __builtin_bit_cast(h2_t, ((w >> 8) & M) | B) + off;
    const h2_t p3 = __builtin_bit_cast(h2_t, ((w >> 12) & M) | B) + off;
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

__device__ __forceinline__ float gg_zp(const void *z, int wbits, long i) {
    return wbits == 8 ? (float)((const int8_t *)z)[i] : ((const float *)z)[i];
}

// x (bf16 [T][d]) -> x16 (fp16 [T][d], int4 order within groups of 8).
template <int WBITS>
__global__ __launch_bounds__(256) void x16_kernel(const uint16_t *__restrict__ x, _Float16 *__restrict__ x16,
                                                  long nchunks) {
    for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (long)gridDim.x * 256) {
        const uint4 q = ((const uint4 *)x)[c];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        _Float16 v[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
            v[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xFFFF0000u);
        }
        h8_t o;
        if (WBITS == 4)
            o = (h8_t){v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};
        else
            o = (h8_t){v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
        ((h8_t *)x16)[c] = o;
    }
}

template <int V>
struct GgSet {
    static constexpr int value = V;
};

struct GemmBufs {
    const _Float16 *x16;       // [T][d]
    _Float16 *hhi, *hlo;       // [A][I]
    _Float16 *hshi, *hslo;     // [T][I_shared]
};

// MODE 0: gate/up (A = x16 rows through the permutation; B = the gate and up rows of 32 channels per
// wavefront; output h as fp16 hi/lo planes).  MODE 1: down (A = h hi/lo rows of the slot; B = 64 down
// rows per wavefront; output y_perm / y_shared in fp32).
//
// Zero points: when every zero point of the tile's weight rows is an integer (int8 always; int4 when
// its fp32 zero points are integral), it is folded into the dequantisation (B = q - z, exact in fp16);
// otherwise B = q and the epilogue subtracts z times the row sum of the activations, which the
// staging threads then accumulate.
template <int MODE, int WBITS, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_kernel(FfnParams P, GemmBufs G, int tiles_n) {
    constexpr int NA = MODE == 0 ? 1 : 2;         // activation planes: x, or h hi and lo
    constexpr int MM = WAVES == 4 ? 4 : 2;        // 32-row blocks per wavefront
    constexpr int NJ = WAVES == 4 ? 4 : 2;        // 32-column subtiles per wavefront
    constexpr int WM = 4 / MM;                    // wavefront rows
    constexpr int WN = WAVES / WM;                // wavefront columns
    constexpr int NOUT_W = MODE == 0 ? 16 * NJ : 32 * NJ;  // distinct output columns per wavefront
    constexpr int NOUT_G = NOUT_W * WN;           // per tile
    constexpr int CPT = 1024 / (WAVES * 64);      // activation chunks per thread per plane and step
    constexpr int TPR = 8 / CPT;                  // staging threads per row
    constexpr int ACH = CPT * NA;                 // 16-byte activation chunks per thread per step
    constexpr int WL = WBITS == 8 ? 2 : 1;        // 16-byte weight loads per subtile per step
    constexpr int PLANE = GG_M * GG_LDA;          // halfs per activation plane
    constexpr float QBIAS = WBITS == 8 ? 1152.f : 1024.f;
    // activation planes in dynamic LDS: [2 stages][NA planes][GG_M rows][GG_LDA halfs]
    extern __shared__ __align__(16) _Float16 As_dyn[];
    __shared__ float rsum[GG_M];
    __shared__ int s_e[GG_MAXSLOTS], s_p0[GG_MAXSLOTS], s_c[GG_MAXSLOTS], s_t0[GG_MAXSLOTS + 1];
    __shared__ int s_nslot;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 5, lr = lane & 31;
    const int wm = wv / WN, wn = wv % WN;

    // ---- tile table: slot s (used experts in uniq order, then the shared expert) has
    // mt_s = ceil(c_s / 128) row tiles and tiles_n output tiles; s_t0 is the exclusive prefix
    if (wv == 0) {
        int nu = *P.n_uniq;
        nu = nu < 0 ? 0 : (nu > P.n_routed_slots ? P.n_routed_slots : nu);
        const int ns = nu + (P.Is > 0 ? 1 : 0);
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
    const int nslot = s_nslot;
    const int ntiles = s_t0[nslot];

    // staging thread map: row srow of the tile, chunks CPT*sq .. CPT*sq + CPT - 1 (of 8 per row and
    // step) of every plane
    const int srow = tid / TPR, sq = tid % TPR;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        // ---- locate the tile: slot (binary search), output tile, row tile
        int lo = 0, hi = nslot - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_t0[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int slot = lo;
        const bool shared = P.Is > 0 && slot == nslot - 1;
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

        // ---- activation source of this thread's staging row
        rsrc_t asrc[NA];
        long arow = -1;  // element offset of the row, -1: padding
        if (MODE == 0) {
            asrc[0] = make_rsrc(G.x16, (uint32_t)((long)P.T * P.d * 2));
            if (srow < rows) {
                const int t = shared ? (r0 + srow) : (P.perm[p0 + r0 + srow] / P.k);
                arow = (long)t * P.d;
            }
        } else {
            const uint32_t nb = (uint32_t)((long)(shared ? P.T : P.A) * I * 2);
            asrc[0] = make_rsrc(shared ? G.hshi : G.hhi, nb);
            asrc[NA - 1] = make_rsrc(shared ? G.hslo : G.hlo, nb);
            if (srow < rows) arow = (long)((shared ? 0 : p0) + r0 + srow) * I;
        }

        // ---- weight rows of this lane: subtile j.  Gate/up: j < NJ/2 the gate rows of channels
        // c0 + 32 j + lr, j >= NJ/2 the up rows of the same channels; down: outputs o0 + 32 j + lr.
        const long rb = (long)KK * WBITS / 8;  // bytes per weight row
        rsrc_t wsrc[NJ];
        uint32_t wrow[NJ];
        int ocol[NJ];
        float sc[NJ], zp[NJ];
        {
            const int nbase = ntile * NOUT_G + wn * NOUT_W;
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                const bool gate = j < NJ / 2;
                const int o = MODE == 0 ? nbase + 32 * (j % (NJ / 2)) + lr : nbase + 32 * j + lr;
                ocol[j] = o;
                const long ncol = MODE == 0 ? I : P.d;
                const uint8_t *base = MODE == 0 ? (gate ? W.qg : W.qu) + (long)e * I * rb : W.qd + (long)e * P.d * rb;
                wsrc[j] = make_rsrc(base, (uint32_t)(ncol * rb));
                wrow[j] = o < nout ? (uint32_t)(o * rb) : kOOB;
                const long ch = (long)e * ncol + min(o, nout - 1);
                if (MODE == 0) {
                    sc[j] = gate ? W.sg[ch] : W.su[ch];
                    zp[j] = gg_zp(gate ? W.zg : W.zu, WBITS, ch);
                } else {
                    sc[j] = W.sd[ch];
                    zp[j] = gg_zp(W.zd, WBITS, ch);
                }
            }
        }
        bool my_int = true;
#pragma unroll
        for (int j = 0; j < NJ; j++) my_int = my_int && zp[j] == rintf(zp[j]) && fabsf(zp[j]) <= 512.f;
        const bool fold = __syncthreads_and(my_int);  // uniform over the workgroup
        h2_t boff[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const _Float16 o = (_Float16)(-(QBIAS + (fold ? zp[j] : 0.f)));
            boff[j] = (h2_t){o, o};
        }

        // ---- two-step register pipeline (set = step parity).  Steps past the end (the prefetch of the
        // last two steps, and the padding step of an odd count) load nothing and read as zeros, so every
        // step issues the same number of loads.
        uint4 araw[2][ACH];
        uint4 wraw[2][NJ][WL];
        auto issue = [&](int step, int set) {
            const bool live = step < nsteps;
            const uint32_t ao =
                (arow < 0 || !live) ? kOOB : (uint32_t)((arow + (long)step * GG_K + 8 * CPT * sq) * 2);
#pragma unroll
            for (int pl = 0; pl < NA; pl++)
#pragma unroll
                for (int c = 0; c < CPT; c++)
                    araw[set][CPT * pl + c] = buf_load16(asrc[pl], ao == kOOB ? kOOB : ao + 16 * c);
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int q = 0; q < WL; q++)
                    wraw[set][j][q] = buf_load16(
                        wsrc[j], (wrow[j] == kOOB || !live)
                                     ? kOOB
                                     : wrow[j] + (uint32_t)(step * (GG_K * WBITS / 8) + kg * (16 * WL) + 16 * q));
        };
        float rs = 0.f;
        f32x16v_t acc[MM][NJ];
#pragma unroll
        for (int mm = 0; mm < MM; mm++)
#pragma unroll
            for (int j = 0; j < NJ; j++) acc[mm][j] = (f32x16v_t){};

        issue(0, 0);
        issue(1, 1);
        // one pipeline step; the register set is a compile-time constant (the loop runs two steps per
        // iteration) so that every wait counts only the loads it needs
        auto one_step = [&](int step, auto setc) {
            constexpr int set = decltype(setc)::value;
            _Float16 *Ab = As_dyn + set * NA * PLANE;
            // activation chunks of this step -> LDS (and, without folded zero points, their row sums)
#pragma unroll
            for (int pl = 0; pl < NA; pl++)
#pragma unroll
                for (int c = 0; c < CPT; c++)
                    *(uint4 *)(Ab + pl * PLANE + srow * GG_LDA + 8 * (CPT * sq + c)) = araw[set][CPT * pl + c];
            if (!fold) {
#pragma unroll
                for (int q = 0; q < ACH; q++) {
                    const uint32_t ww[4] = {araw[set][q].x, araw[set][q].y, araw[set][q].z, araw[set][q].w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const h2_t hh = __builtin_bit_cast(h2_t, ww[i]);
                        rs += (float)hh.x + (float)hh.y;
                    }
                }
            }
            uint4 wcur[NJ][WL];
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int q = 0; q < WL; q++) wcur[j][q] = wraw[set][j][q];
            __syncthreads();  // this step's activations are in LDS; the other stage is free
            issue(step + 2, set);

#pragma unroll
            for (int s = 0; s < 4; s++) {
                h8_t bq[NJ];
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    if (WBITS == 4) {
                        const uint32_t ww[4] = {wcur[j][0].x, wcur[j][0].y, wcur[j][0].z, wcur[j][0].w};
                        bq[j] = deq_int4(ww[s], boff[j]);
                    } else {
                        const uint4 q = wcur[j][s >> 1];
                        bq[j] = (s & 1) ? deq_int8(q.z, q.w, boff[j]) : deq_int8(q.x, q.y, boff[j]);
                    }
                }
                // every block runs, also the all-padding ones of a short row tile (their rows are zero): a
                // branch around an MFMA would make the compiler copy the accumulator to merge the paths
#pragma unroll
                for (int mm = 0; mm < MM; mm++) {
#pragma unroll
                    for (int pl = 0; pl < NA; pl++) {
                        const h8_t a = *(const h8_t *)(Ab + pl * PLANE + ((MM * wm + mm) * 32 + lr) * GG_LDA +
                                                       32 * kg + 8 * s);
#pragma unroll
                        for (int j = 0; j < NJ; j++)
                            acc[mm][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq[j], acc[mm][j], 0, 0, 0);
                    }
                }
                // keep each substep's fragment loads next to its MFMAs (bounded register use)
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int step = 0; step < nsteps; step += 2) {
            one_step(step, GgSet<0>{});
            one_step(step + 1, GgSet<1>{});
        }

        // ---- row sums (the staging threads of a row, fixed order), only without folded zero points
        if (!fold) {
            float t = rs;
#pragma unroll
            for (int o = 1; o < TPR; o <<= 1) t = t + __shfl_xor(t, o, 64);
            if (sq == 0) rsum[srow] = t;
        }
        __syncthreads();

        // ---- epilogue: lane column ocol[j]; register r holds row 8*(r/4) + 4*kg + (r%4) of block mm
#pragma unroll
        for (int mm = 0; mm < MM; mm++) {
            if (MM * wm + mm >= nm32) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = (MM * wm + mm) * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (m >= rows) continue;
                const float xs = fold ? 0.f : rsum[m];
                const long prow = (long)(shared ? 0 : p0) + r0 + m;  // output row
                if (MODE == 0) {
#pragma unroll
                    for (int jj = 0; jj < NJ / 2; jj++) {
                        const int c = ocol[jj];
                        if (c < nout) {
                            const int ju = jj + NJ / 2;
                            const float gv = sc[jj] * (acc[mm][jj][r] - (fold ? 0.f : zp[jj]) * xs);
                            const float uv = sc[ju] * (acc[mm][ju][r] - (fold ? 0.f : zp[ju]) * xs);
                            const float hv = gv / (1.f + expf(-gv)) * uv;
                            const _Float16 h_hi = (_Float16)hv;
                            const _Float16 h_lo = (_Float16)(hv - (float)h_hi);
                            // stored at the planes' position of channel c (int4 order within groups of 8)
                            const int hp = WBITS == 4 ? ((c & ~7) | pos8(c & 7)) : c;
                            (shared ? G.hshi : G.hhi)[prow * I + hp] = h_hi;
                            (shared ? G.hslo : G.hlo)[prow * I + hp] = h_lo;
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < NJ; j++) {
                        if (ocol[j] < nout) {
                            const float y = sc[j] * (acc[mm][j][r] - (fold ? 0.f : zp[j]) * xs);
                            (shared ? P.y_sh : P.y_perm)[prow * P.d + ocol[j]] = y;
                        }
                    }
                }
            }
        }
        __syncthreads();  // rsum and the activation stages are reused by the next tile
    }
}

// ---------------------------------------------------------------------------- host side

static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t gemm_workspace_bytes(const FfnParams &P) {
    return al256((size_t)P.T * P.d * 2) + 2 * al256((size_t)P.A * P.I * 2) + 2 * al256((size_t)P.T * P.Is * 2);
}

bool gemm_supported(const FfnParams &P) {
    if (P.act != 1) return false;  // bf16 activations
    if (P.d % GG_K || P.I % GG_K || (P.Is > 0 && P.Is % GG_K)) return false;
    if (P.n_routed_slots + 1 > GG_MAXSLOTS) return false;
    // 32-bit buffer offsets
    const long Imax = P.I > P.Is ? P.I : P.Is;
    if (Imax * ((long)P.d * P.wbits / 8) > 0x7FFFFFFFL) return false;
    if ((long)P.A * Imax * 2 > 0x7FFFFFFFL || (long)P.T * P.d * 2 > 0x7FFFFFFFL) return false;
    return true;
}

static int gg_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    return n;
}

template <int MODE, int WBITS, int WAVES>
static hipError_t gg_launch_mode(const FfnParams &P, const GemmBufs &G, hipStream_t stream) {
    constexpr int NJ = WAVES == 4 ? 4 : 2, MM = WAVES == 4 ? 4 : 2;
    constexpr int WN = WAVES / (4 / MM);
    constexpr int NOUT_G = (MODE == 0 ? 16 * NJ : 32 * NJ) * WN;
    const int Imax = P.I > P.Is ? P.I : P.Is;
    const int tiles_n = ((MODE == 0 ? Imax : P.d) + NOUT_G - 1) / NOUT_G;
    const size_t lds = (size_t)2 * (MODE == 0 ? 1 : 2) * GG_M * GG_LDA * sizeof(_Float16);
    auto fn = gemm_kernel<MODE, WBITS, WAVES>;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(fn, dim3(gg_cus()), dim3(WAVES * 64), lds, stream, P, G, tiles_n);
    return hipGetLastError();
}

template <int WBITS>
static hipError_t gg_launch(const FfnParams &P, const GemmBufs &G, hipStream_t stream) {
    const long nchunks = (long)P.T * P.d / 8;
    long grid = (nchunks + 255) / 256;
    if (grid > (long)gg_cus() * 8) grid = (long)gg_cus() * 8;
    hipLaunchKernelGGL(x16_kernel<WBITS>, dim3((unsigned)grid), dim3(256), 0, stream, (const uint16_t *)P.x,
                       (_Float16 *)G.x16, nchunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = gg_launch_mode<0, WBITS, GG_WAVES>(P, G, stream);
    if (err != hipSuccess) return err;
    return gg_launch_mode<1, WBITS, GG_WAVES>(P, G, stream);
}

hipError_t launch_ffn_gemm(const FfnParams &P, void *ws, hipStream_t stream) {
    if (!gemm_supported(P)) return hipErrorNotSupported;
    char *p = (char *)ws;
    GemmBufs G;
    G.x16 = (const _Float16 *)p;
    p += al256((size_t)P.T * P.d * 2);
    G.hhi = (_Float16 *)p;
    p += al256((size_t)P.A * P.I * 2);
    G.hlo = (_Float16 *)p;
    p += al256((size_t)P.A * P.I * 2);
    G.hshi = (_Float16 *)p;
    p += al256((size_t)P.T * P.Is * 2);
    G.hslo = (_Float16 *)p;
    return P.wbits == 4 ? gg_launch<4>(P, G, stream) : gg_launch<8>(P, G, stream);
}

}  // namespace moe
