// C ABI of the MoE-layer forward: argument validation, workspace layout and kernel launches.
// Nothing here allocates device memory or waits on the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/dsa_index.h"
#include "../../include/moe.h"
#include "../../include/moe_cache.h"
#include "kernels.h"

// Scratch memory of moe_forward_static: one copy per device, at its own address on each, held until the process
// ends.  Host code never passes this name to a kernel (on the host it is a stand-in, not a device address): it
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE_PTR(p, name)                                                     \
    do {                                                                         \
        if (!(p)) return fail(MOE_EINVAL, "%s: %s is NULL", fn, name);           \
        if (!aligned((p), 16)) return fail(MOE_EALIGN, "%s: %s is not 16-byte aligned", fn, name); \
    } while (0)
// a pointer to T-sized data: may be NULL when T = 0 (nothing is read or written through it then)
#define REQUIRE_PTR_T(p, name)                                                   \
    do {                                                                         \
        if (s->T > 0 || (p)) REQUIRE_PTR(p, name);                               \
    } while (0)

int check_shape(const char *fn, const moe_shape *s) {
    if (!s) return fail(MOE_EINVAL, "%s: shape is NULL", fn);
    if (s->T < 0 || s->d < 1 || s->E < 1 || s->k < 1 || s->I < 1 || s->I_shared < 0)
        return fail(MOE_EINVAL, "%s: d, E, k, I must be >= 1 and T, I_shared >= 0", fn);
    if (s->k > s->E || s->k > 32) return fail(MOE_EINVAL, "%s: k=%d must be <= min(E, 32)", fn, s->k);
    if (s->E > 1024) return fail(MOE_EINVAL, "%s: E=%d exceeds 1024", fn, s->E);
    if ((long)s->T * s->k >= (1L << 31)) return fail(MOE_EINVAL, "%s: T*k overflows int32", fn);
    // the decode path sums a K part of up to a whole row of int8 weight x 8-bit digit products in int32
    if (s->d >= MOE_MAX_DIM || s->I >= MOE_MAX_DIM || s->I_shared >= MOE_MAX_DIM)
        return fail(MOE_EUNSUPPORTED, "%s: d, I and I_shared must be below %d", fn, MOE_MAX_DIM);
    if (s->act_dtype != MOE_ACT_F32 && s->act_dtype != MOE_ACT_BF16)
        return fail(MOE_EUNSUPPORTED, "%s: act_dtype %d not supported", fn, s->act_dtype);
    if (s->wbits != 8 && s->wbits != 4) return fail(MOE_EUNSUPPORTED, "%s: wbits %d not supported", fn, s->wbits);
    const int m = s->wbits == 4 ? 32 : 16;
    if (s->d % m || s->I % m || s->I_shared % m)
        return fail(MOE_EINVAL, "%s: d, I and I_shared must be multiples of %d for %d-bit weights", fn, m, s->wbits);
    if (s->path != MOE_PATH_AUTO && s->path != MOE_PATH_GEMV && s->path != MOE_PATH_GEMM)
        return fail(MOE_EINVAL, "%s: unknown path %d", fn, s->path);
    if (s->flags & ~MOE_FLAG_BATCH_INVARIANT) return fail(MOE_EINVAL, "%s: unknown flags 0x%x", fn, s->flags);
    if (s->router != MOE_ROUTER_SIGMOID_BIAS && s->router != MOE_ROUTER_SOFTMAX && s->router != MOE_ROUTER_EXPERT_CHOICE)
        return fail(MOE_EINVAL, "%s: unknown router %d", fn, s->router);
    if (!(s->capacity_factor >= 0.f && s->capacity_factor <= 1e6f))
        return fail(MOE_EINVAL, "%s: capacity_factor must be in [0, 1e6]", fn);
    if (s->router == MOE_ROUTER_EXPERT_CHOICE && (s->k != s->E || !(s->capacity_factor > 0.f)))
        return fail(MOE_EINVAL, "%s: expert choice needs k = E (one slot per expert) and capacity_factor > 0", fn);
    return MOE_OK;
}

int check_ws(const char *fn, const moe_shape *s, void *ws, size_t ws_bytes) {
    size_t need = moe_workspace_size(s);
    if (need == 0) return MOE_OK;
    if (!ws) return fail(MOE_EWORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned(ws, 256)) return fail(MOE_EALIGN, "%s: workspace is not 256-byte aligned", fn);
    if (ws_bytes < need) return fail(MOE_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    return MOE_OK;
}

int check_qffn(const char *fn, const moe_qffn *q, const char *which) {
    if (!q) return fail(MOE_EINVAL, "%s: %s weights are NULL", fn, which);
    const void *ptrs[9] = {q->q_gate, q->q_up, q->q_down, q->s_gate, q->s_up, q->s_down, q->z_gate, q->z_up, q->z_down};
    static const char *names[9] = {"q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down"};
    for (int i = 0; i < 9; i++) {
        if (!ptrs[i]) return fail(MOE_EINVAL, "%s: %s.%s is NULL", fn, which, names[i]);
        if (!aligned(ptrs[i], 16)) return fail(MOE_EALIGN, "%s: %s.%s is not 16-byte aligned", fn, which, names[i]);
    }
    return MOE_OK;
}

moe::QW to_qw(const moe_qffn *q) {
    moe::QW w{};
    if (!q) return w;
    w.qg = (const uint8_t *)q->q_gate;
    w.qu = (const uint8_t *)q->q_up;
    w.qd = (const uint8_t *)q->q_down;
    w.sg = q->s_gate;
    w.su = q->s_up;
    w.sd = q->s_down;
    w.zg = q->z_gate;
    w.zu = q->z_up;
    w.zd = q->z_down;
    return w;
}

moe::FfnParams ffn_params(const moe_shape *s) {
    moe::FfnParams P{};
    P.T = s->T;
    P.d = s->d;
    P.k = s->k;
    P.E = s->E;
    P.A = s->T * s->k;
    P.I = s->I;
    P.Is = s->I_shared;
    P.wbits = s->wbits;
    P.act = s->act_dtype;
    P.n_routed_slots = s->E < P.A ? s->E : P.A;
    P.wslot = nullptr;
    P.n_wrows = s->E;
    P.invariant = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
    return P;
}

// Path the forward call takes for this shape: the matrix-core grouped GEMM once there are enough rows
// per expert to reuse each weight (more than MOE_AUTO_DECODE_MAX_T tokens), the bandwidth-bound decode kernels
// otherwise; the batch-invariant mode keeps every T on the decode kernels, so a token's bits never depend on the
// batch.
int forward_path(const moe_shape *s) {
    if (s->path != MOE_PATH_AUTO) return s->path;
    if (s->flags & MOE_FLAG_BATCH_INVARIANT) return MOE_PATH_GEMV;
    moe::FfnParams P = ffn_params(s);
    if (s->T > MOE_AUTO_DECODE_MAX_T && moe::gemm_supported(P)) return MOE_PATH_GEMM;
    return MOE_PATH_GEMV;
}

// Capacity the router applies: top-k routers, ceil(cf T k / E) (0 = none); expert choice, the tokens each expert
// takes, min(T, ceil(cf T / E)).
int router_capacity(const moe_shape *s) {
    if (s->capacity_factor <= 0.f || s->T == 0) return 0;
    const double cf = (double)s->capacity_factor;
    if (s->router == MOE_ROUTER_EXPERT_CHOICE) {
        const double c = ceil(cf * s->T / s->E);
        return c >= s->T ? s->T : (int)c;
    }
    const double c = ceil(cf * s->T * s->k / s->E);
    return c >= (double)s->T * s->k ? s->T * s->k : (int)c;
}

// Workspace bytes of moe_forward alone for this shape (the path it takes).
size_t forward_workspace_bytes(const moe_shape *s) {
    const moe::FfnParams P = ffn_params(s);
    return forward_path(s) == MOE_PATH_GEMM ? moe::gemm_workspace_bytes(P) : moe::decode_workspace_bytes(P);
}

// Device address of `scratch` on the current device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

int scratch_address(const char *fn, void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MOE_EDEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EDEVICE, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return fail(MOE_EDEVICE, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(err));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

int launch_status(const char *fn, hipError_t err) {
    if (err != hipSuccess) return fail(MOE_EDEVICE, "%s: launch failed: %s", fn, hipGetErrorString(err));
    g_err[0] = 0;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return 4; }

const char *moe_last_error(void) { return g_err; }

size_t moe_workspace_size(const moe_shape *s) {
    if (check_shape("moe_workspace_size", s) != MOE_OK) return 0;
    moe::FfnParams P = ffn_params(s);
    const bool inv = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
    size_t r = moe::router_workspace_bytes(s->T, s->d, s->E, inv, s->k, s->router, router_capacity(s) > 0);
    size_t g = moe::decode_workspace_bytes(P);
    size_t need = r > g ? r : g;
    size_t m = moe::gemm_workspace_bytes(P);
    if (m > need) need = m;
    const size_t pm = moe::permute_workspace_bytes(s->T * s->k, s->E);
    if (pm > need) need = pm;
    // moe_layer with the routing inside the forward: the router's partial sums after the forward's workspace
    if (s->T == 1) {
        const size_t lr = g + moe::router_partials_bytes(s->T, s->d, s->E, inv);
        if (lr > need) need = lr;
    }
    return (need + 255) & ~(size_t)255;
}

int moe_route(const moe_shape *s, const void *x, const float *W_r, const float *bias, int32_t *topk_idx,
              float *topk_w, double *gap, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_route";
    int rc = check_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(x, "x");
    REQUIRE_PTR(W_r, "W_r");
    if (s->router == MOE_ROUTER_SIGMOID_BIAS || bias) REQUIRE_PTR(bias, "bias");  // the other routers take no bias
    REQUIRE_PTR_T(topk_idx, "topk_idx");
    REQUIRE_PTR_T(topk_w, "topk_w");
    if (gap && !aligned(gap, 16)) return fail(MOE_EALIGN, "%s: gap is not 16-byte aligned", fn);
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    if (s->T == 0) return MOE_OK;  // empty batch: nothing to route
    const bool inv = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
    if (const char *why = moe::router_unsupported(s->T, s->d, s->E, s->act_dtype, inv))
        return fail(MOE_EUNSUPPORTED, "%s: %s", fn, why);
    return launch_status(fn, moe::launch_router(s->act_dtype, x, W_r, bias, s->T, s->d, s->E, s->k, s->routed_scale,
                                                topk_idx, topk_w, gap, ws, inv, s->router, router_capacity(s),
                                                (hipStream_t)stream, nullptr));
}

int moe_permute(const moe_shape *s, const int32_t *topk_idx, int32_t *counts, int32_t *offsets, int32_t *perm,
                int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_permute";
    int rc = check_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(topk_idx, "topk_idx");
    REQUIRE_PTR(counts, "counts");
    REQUIRE_PTR(offsets, "offsets");
    REQUIRE_PTR_T(perm, "perm");
    REQUIRE_PTR_T(inv, "inv");
    REQUIRE_PTR(uniq, "uniq");
    REQUIRE_PTR(n_uniq, "n_uniq");
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    return launch_status(fn, moe::launch_permute(topk_idx, s->T * s->k, s->E, counts, offsets, perm, inv, uniq,
                                                 n_uniq, ws, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// moe_route_permute's argument checks (all but the workspace)
int check_route_permute(const char *fn, const moe_shape *s, const void *x, const float *W_r, const float *bias,
                        int32_t *topk_idx, float *topk_w, double *gap, int32_t *counts, int32_t *offsets,
                        int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq) {
    int rc = check_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(x, "x");
    REQUIRE_PTR(W_r, "W_r");
    if (s->router == MOE_ROUTER_SIGMOID_BIAS || bias) REQUIRE_PTR(bias, "bias");
    REQUIRE_PTR_T(topk_idx, "topk_idx");
    REQUIRE_PTR_T(topk_w, "topk_w");
    if (gap && !aligned(gap, 16)) return fail(MOE_EALIGN, "%s: gap is not 16-byte aligned", fn);
    REQUIRE_PTR(counts, "counts");
    REQUIRE_PTR(offsets, "offsets");
    REQUIRE_PTR_T(perm, "perm");
    REQUIRE_PTR_T(inv, "inv");
    REQUIRE_PTR(uniq, "uniq");
    REQUIRE_PTR(n_uniq, "n_uniq");
    if (s->T > 0) {
        const bool invariant = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
        if (const char *why = moe::router_unsupported(s->T, s->d, s->E, s->act_dtype, invariant))
            return fail(MOE_EUNSUPPORTED, "%s: %s", fn, why);
    }
    return MOE_OK;
}

// moe_route_permute's kernels, after its checks
hipError_t run_route_permute(const moe_shape *s, const void *x, const float *W_r, const float *bias,
                             int32_t *topk_idx, float *topk_w, double *gap, int32_t *counts, int32_t *offsets,
                             int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq, void *ws, void *stream) {
    const bool invariant = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
    const int C = router_capacity(s);
    if (s->T > 0) {
        const moe::PermOut po{counts, offsets, perm, inv, uniq, n_uniq};
        hipError_t err = moe::launch_router(s->act_dtype, x, W_r, bias, s->T, s->d, s->E, s->k, s->routed_scale,
                                            topk_idx, topk_w, gap, ws, invariant, s->router, C,
                                            (hipStream_t)stream, &po);
        if (err != hipSuccess || moe::router_fused(s->T, s->E, invariant, s->router, C)) return err;
    }
    return moe::launch_permute(topk_idx, s->T * s->k, s->E, counts, offsets, perm, inv, uniq, n_uniq, ws,
                               (hipStream_t)stream);
}

}  // namespace

extern "C" {

int moe_route_permute(const moe_shape *s, const void *x, const float *W_r, const float *bias, int32_t *topk_idx,
                      float *topk_w, double *gap, int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                      int32_t *uniq, int32_t *n_uniq, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_route_permute";
    int rc = check_route_permute(fn, s, x, W_r, bias, topk_idx, topk_w, gap, counts, offsets, perm, inv, uniq,
                                 n_uniq);
    if (rc) return rc;
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    return launch_status(fn, run_route_permute(s, x, W_r, bias, topk_idx, topk_w, gap, counts, offsets, perm, inv,
                                               uniq, n_uniq, ws, stream));
}

}  // extern "C"

namespace {

// moe_forward's argument checks (all but the workspace); MOE_OK when the call may go ahead
// (y_shared_optional: y_shared = NULL leaves the shared expert out, as moe_forward_cached allows)
int check_forward(const char *fn, const moe_shape *s, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                  const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                  float *y_perm, float *y_shared, uint32_t *diag, bool y_shared_optional = false) {
    int rc = check_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(x, "x");
    rc = check_qffn(fn, routed, "routed");
    if (rc) return rc;
    if (s->I_shared > 0) {
        rc = check_qffn(fn, shared, "shared");
        if (rc) return rc;
        if (!y_shared_optional) REQUIRE_PTR_T(y_shared, "y_shared");
        else if (y_shared && !aligned(y_shared, 16)) return fail(MOE_EALIGN, "%s: y_shared is not 16-byte aligned", fn);
    }
    REQUIRE_PTR(offsets, "offsets");
    REQUIRE_PTR_T(perm, "perm");
    REQUIRE_PTR(uniq, "uniq");
    REQUIRE_PTR(n_uniq, "n_uniq");
    REQUIRE_PTR_T(y_perm, "y_perm");
    if (diag && !aligned(diag, 4)) return fail(MOE_EALIGN, "%s: diag is not 4-byte aligned", fn);
    if (s->T == 0) return MOE_OK;
    const moe::FfnParams P = ffn_params(s);
    if (forward_path(s) == MOE_PATH_GEMM) {
        if (!moe::gemm_supported(P))
            return fail(MOE_EUNSUPPORTED,
                        "%s: the matrix-core path takes d, I and I_shared multiples of 64 and "
                        "buffers below 2^31 bytes", fn);
    } else if (const char *why = moe::decode_unsupported(P)) {
        return fail(MOE_EUNSUPPORTED, "%s: %s", fn, why);
    }
    return MOE_OK;
}

moe::FfnParams forward_params(const moe_shape *s, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                              const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                              float *y_perm, float *y_shared, uint32_t *diag) {
    moe::FfnParams P = ffn_params(s);
    P.x = x;
    P.routed = to_qw(routed);
    P.shared = to_qw(s->I_shared > 0 ? shared : nullptr);
    P.offsets = offsets;
    P.perm = perm;
    P.uniq = uniq;
    P.n_uniq = n_uniq;
    P.y_perm = y_perm;
    P.y_sh = s->I_shared > 0 ? y_shared : nullptr;
    P.diag = diag;
    return P;
}

// moe_layer routes inside the forward's gate/up launch: one token on the decode path, a top-k router without
// capacity (the selection the router's own fused form takes)
bool layer_routes_in_forward(const moe_shape *s) {
    if (s->T != 1 || forward_path(s) != MOE_PATH_GEMV) return false;
    if (!moe::router_fused(s->T, s->E, (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0, s->router, router_capacity(s)))
        return false;
    return moe::decode_routes(ffn_params(s));
}

// the forward kernels, after check_forward and a workspace check
// (wslot, n_wrows: the routed weights are an expert cache's n_wrows slots, expert e in slot wslot[e])
int run_forward(const char *fn, const moe_shape *s, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                float *y_perm, float *y_shared, uint32_t *diag, void *ws, void *stream,
                const int32_t *wslot = nullptr, int n_wrows = 0) {
    if (s->T == 0) return MOE_OK;  // empty batch: no rows to transform
    moe::FfnParams P = forward_params(s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag);
    if (wslot) {
        P.wslot = wslot;
        P.n_wrows = n_wrows;
    }
    const hipError_t err = forward_path(s) == MOE_PATH_GEMM ? moe::launch_ffn_gemm(P, ws, (hipStream_t)stream)
                                                             : moe::launch_ffn_decode(P, ws, (hipStream_t)stream);
    return launch_status(fn, err);
}

}  // namespace

extern "C" {

int moe_forward(const moe_shape *s, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                float *y_perm, float *y_shared, uint32_t *diag, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_forward";
    int rc = check_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag);
    if (rc) return rc;
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    return run_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag, ws, stream);
}

int moe_forward_static(const moe_shape *s, const void *x, const moe_qffn *routed, const moe_qffn *shared,
                       const int32_t *offsets, const int32_t *perm, const int32_t *uniq, const int32_t *n_uniq,
                       float *y_perm, float *y_shared, uint32_t *diag, void *stream) {
    const char *fn = "moe_forward_static";
    int rc = check_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag);
    if (rc) return rc;
    const size_t need = forward_workspace_bytes(s);
    if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
        return fail(MOE_EWORKSPACE, "%s: this shape needs %zu bytes of scratch, above the static %u", fn, need,
                    (unsigned)MOE_STATIC_SCRATCH_BYTES);
    if (s->T == 0) return MOE_OK;
    void *ws = nullptr;
    rc = scratch_address(fn, &ws);
    if (rc) return rc;
    return run_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag, ws, stream);
}

}  // extern "C"

namespace {

int check_index_shape(const char *fn, const dsa_index_shape *s) {
    if (!s) return fail(MOE_EINVAL, "%s: shape is NULL", fn);
    if (s->T < 0 || s->S < 0 || s->K < 1 || s->pos0 < 0) return fail(MOE_EINVAL, "%s: T, S, pos0 >= 0 and K >= 1", fn);
    if (s->H < 16 || s->H > 64 || s->H % 16) return fail(MOE_EUNSUPPORTED, "%s: H must be 16, 32, 48 or 64", fn);
    if (s->D < 64 || s->D > 256 || s->D % 64) return fail(MOE_EUNSUPPORTED, "%s: D must be 64, 128, 192 or 256", fn);
    if (const char *why = moe::index_unsupported(s->T, s->S, s->H, s->D)) return fail(MOE_EUNSUPPORTED, "%s: %s", fn, why);
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t dsa_index_workspace_size(const dsa_index_shape *s) {
    if (check_index_shape("dsa_index_workspace_size", s) != MOE_OK) return 0;
    return (moe::index_workspace_bytes(s->T, s->S) + 255) & ~(size_t)255;
}

int dsa_index_topk(const dsa_index_shape *s, const int8_t *q, const float *w, const int8_t *k, const float *kscale,
                   int32_t *top, double *gap, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "dsa_index_topk";
    int rc = check_index_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(q, "q");
    REQUIRE_PTR_T(w, "w");
    REQUIRE_PTR_T(top, "top");
    if (s->S > 0 || k) REQUIRE_PTR(k, "k");
    if (s->S > 0 || kscale) REQUIRE_PTR(kscale, "kscale");
    if (gap && !aligned(gap, 16)) return fail(MOE_EALIGN, "%s: gap is not 16-byte aligned", fn);
    const size_t need = dsa_index_workspace_size(s);
    if (need > 0) {
        if (!ws) return fail(MOE_EWORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
        if (!aligned(ws, 256)) return fail(MOE_EALIGN, "%s: workspace is not 256-byte aligned", fn);
        if (ws_bytes < need) return fail(MOE_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    }
    if (s->T == 0) return MOE_OK;
    return launch_status(fn, moe::launch_index_topk(q, w, k, kscale, s->T, s->S, s->H, s->D, s->K, s->pos0, top, gap,
                                                    ws, (hipStream_t)stream));
}

int moe_combine(const moe_shape *s, const float *y_perm, const float *y_shared, const int32_t *inv,
                const float *topk_w, float *y, void *stream) {
    const char *fn = "moe_combine";
    int rc = check_shape(fn, s);
    if (rc) return rc;
    REQUIRE_PTR_T(y_perm, "y_perm");
    REQUIRE_PTR_T(inv, "inv");
    REQUIRE_PTR_T(topk_w, "topk_w");
    REQUIRE_PTR_T(y, "y");
    if (y_shared && !aligned(y_shared, 16)) return fail(MOE_EALIGN, "%s: y_shared is not 16-byte aligned", fn);
    if (s->T == 0) return MOE_OK;  // empty batch
    return launch_status(fn, moe::launch_combine(y_perm, y_shared, inv, topk_w, s->T, s->d, s->k, y,
                                                 (hipStream_t)stream));
}

int moe_layer(const moe_shape *s, const void *x, const float *W_r, const float *bias, const moe_qffn *routed,
              const moe_qffn *shared, int32_t *topk_idx, float *topk_w, double *gap, int32_t *counts,
              int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *uniq, int32_t *n_uniq, float *y_perm,
              float *y_shared, float *y, uint32_t *diag, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_layer";
    int rc = check_route_permute(fn, s, x, W_r, bias, topk_idx, topk_w, gap, counts, offsets, perm, inv, uniq,
                                 n_uniq);
    if (rc) return rc;
    rc = check_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag);
    if (rc) return rc;
    REQUIRE_PTR_T(y, "y");
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    const hipStream_t st = (hipStream_t)stream;
    hipError_t err;
    if (layer_routes_in_forward(s)) {
        // logits, then the gate/up launch selects and sorts for itself (workgroup 0 writes the routing
        // outputs), the down launch, the combine; the partial sums sit past the forward's workspace
        moe::FfnParams P = forward_params(s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag);
        double *part = (double *)((char *)ws + moe::decode_workspace_bytes(P));
        const bool invariant = (s->flags & MOE_FLAG_BATCH_INVARIANT) != 0;
        int nsplit = 0;
        err = moe::launch_router_logits(s->act_dtype, x, W_r, s->T, s->d, s->E, invariant, part, &nsplit, st);
        if (err != hipSuccess) return launch_status(fn, err);
        P.route = moe::FfnParams::Route{part, nsplit, s->router == MOE_ROUTER_SOFTMAX ? 1 : 0, bias,
                                        s->routed_scale, topk_idx, topk_w, gap, counts, offsets, perm, inv, uniq,
                                        n_uniq};
        // the combine in the down launch when the token's slots fit its LDS
        P.comb_inv = inv;
        P.comb_w = topk_w;
        P.comb_y = y;
        if (!moe::decode_combines(P)) P.comb_y = nullptr;
        err = moe::launch_ffn_decode(P, ws, st);
        if (err != hipSuccess || P.comb_y) return launch_status(fn, err);
    } else {
        err = run_route_permute(s, x, W_r, bias, topk_idx, topk_w, gap, counts, offsets, perm, inv, uniq, n_uniq, ws,
                                stream);
        if (err != hipSuccess) return launch_status(fn, err);
        if (s->T == 0) return launch_status(fn, hipSuccess);
        rc = run_forward(fn, s, x, routed, shared, offsets, perm, uniq, n_uniq, y_perm, y_shared, diag, ws, stream);
        if (rc) return rc;
        err = hipSuccess;
    }
    if (err != hipSuccess) return launch_status(fn, err);
    return launch_status(fn, moe::launch_combine(y_perm, s->I_shared > 0 ? y_shared : nullptr, inv, topk_w, s->T,
                                                 s->d, s->k, y, st));
}

}  // extern "C"

namespace {

int check_cache_shape(const char *fn, const moe_cache_shape *c) {
    if (!c) return fail(MOE_EINVAL, "%s: cache shape is NULL", fn);
    if (c->E < 1 || c->E > 1024) return fail(MOE_EINVAL, "%s: cache E=%d must be in [1, 1024]", fn, c->E);
    if (c->slots < 1 || c->slots > c->E) return fail(MOE_EINVAL, "%s: slots=%d must be in [1, E]", fn, c->slots);
    if (c->pinned < 0 || c->pinned >= c->slots)
        return fail(MOE_EINVAL, "%s: pinned=%d must be in [0, slots)", fn, c->pinned);
    if (c->policy != MOE_CACHE_WEIGHTED_LRU && c->policy != MOE_CACHE_LRU)
        return fail(MOE_EINVAL, "%s: unknown policy %d", fn, c->policy);
    return MOE_OK;
}

// Per-expert bytes of the nine tensors, in moe_qffn's order.
void expert_tensor_bytes(const moe_shape *s, long b[9]) {
    const long d = s->d, I = s->I, wb = s->wbits, zb = s->wbits == 8 ? 1 : 4;
    b[0] = b[1] = I * d * wb / 8;
    b[2] = d * I * wb / 8;
    b[3] = b[4] = 4 * I;
    b[5] = 4 * d;
    b[6] = b[7] = zb * I;
    b[8] = zb * d;
}

// Device address of a host-tier pointer: pinned host memory (its device view) or device memory.
int tier_address(const char *fn, const void *p, const char *name, const void **out) {
    hipPointerAttribute_t a;
    const hipError_t err = hipPointerGetAttributes(&a, p);
    if (err != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of the failed lookup
        return fail(MOE_EINVAL, "%s: host_tier.%s is neither pinned host memory nor device memory", fn, name);
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        *out = a.devicePointer;
    } else if (a.type == hipMemoryTypeDevice) {
        *out = p;
    } else {
        return fail(MOE_EINVAL, "%s: host_tier.%s is neither pinned host memory nor device memory", fn, name);
    }
    return MOE_OK;
}

constexpr int kFetchWorkgroups = 128;

}  // namespace

extern "C" {

size_t moe_cache_state_size(const moe_cache_shape *c) {
    if (check_cache_shape("moe_cache_state_size", c) != MOE_OK) return 0;
    return (moe::cache_state_bytes(c->E, c->slots) + 255) & ~(size_t)255;
}

int moe_cache_init(const moe_cache_shape *c, const int32_t *pinned_ids, void *state, int32_t *miss, int32_t *n_miss,
                   void *stream) {
    const char *fn = "moe_cache_init";
    int rc = check_cache_shape(fn, c);
    if (rc) return rc;
    REQUIRE_PTR(state, "state");
    REQUIRE_PTR(miss, "miss");
    REQUIRE_PTR(n_miss, "n_miss");
    if (c->pinned > 0) {
        if (!pinned_ids) return fail(MOE_EINVAL, "%s: pinned_ids is NULL", fn);
        unsigned char seen[1024] = {0};
        for (int i = 0; i < c->pinned; i++) {
            const int e = pinned_ids[i];
            if (e < 0 || e >= c->E) return fail(MOE_EINVAL, "%s: pinned_ids[%d]=%d outside [0, E)", fn, i, e);
            if (seen[e]) return fail(MOE_EINVAL, "%s: expert %d pinned twice", fn, e);
            seen[e] = 1;
        }
        const hipError_t err = hipMemcpyAsync(miss, pinned_ids, sizeof(int32_t) * (size_t)c->pinned,
                                              hipMemcpyHostToDevice, (hipStream_t)stream);
        if (err != hipSuccess) return fail(MOE_EDEVICE, "%s: copy of the pinned ids: %s", fn, hipGetErrorString(err));
    }
    hipError_t err = moe::launch_cache_init(state, c->E, c->slots, c->pinned, miss, n_miss, (hipStream_t)stream);
    if (err == hipSuccess) err = hipStreamSynchronize((hipStream_t)stream);
    return launch_status(fn, err);
}

int moe_cache_plan(const moe_cache_shape *c, int32_t T, int32_t k, const int32_t *uniq, const int32_t *n_uniq,
                   void *state, int32_t *hit, int32_t *n_hit, int32_t *miss, int32_t *n_miss, void *stream) {
    const char *fn = "moe_cache_plan";
    int rc = check_cache_shape(fn, c);
    if (rc) return rc;
    if (T < 0 || k < 1) return fail(MOE_EINVAL, "%s: T >= 0 and k >= 1", fn);
    const long need = (long)T * k < c->E ? (long)T * k : c->E;
    if (c->slots - c->pinned < need)
        return fail(MOE_EINVAL, "%s: %d unpinned slots cannot take a step of up to %ld missing experts", fn,
                    c->slots - c->pinned, need);
    REQUIRE_PTR(uniq, "uniq");
    REQUIRE_PTR(n_uniq, "n_uniq");
    REQUIRE_PTR(state, "state");
    REQUIRE_PTR(hit, "hit");
    REQUIRE_PTR(n_hit, "n_hit");
    REQUIRE_PTR(miss, "miss");
    REQUIRE_PTR(n_miss, "n_miss");
    return launch_status(fn, moe::launch_cache_plan(state, c->E, c->slots, c->pinned, c->policy, uniq, n_uniq, hit,
                                                    n_hit, miss, n_miss, (hipStream_t)stream));
}

int moe_cache_fetch(const moe_shape *s, const moe_cache_shape *c, const moe_qffn *host_tier, const moe_qffn *slots,
                    const void *state, const int32_t *miss, const int32_t *n_miss, void *stream) {
    const char *fn = "moe_cache_fetch";
    int rc = check_shape(fn, s);
    if (rc) return rc;
    rc = check_cache_shape(fn, c);
    if (rc) return rc;
    if (s->E != c->E) return fail(MOE_EINVAL, "%s: layer E=%d and cache E=%d differ", fn, s->E, c->E);
    rc = check_qffn(fn, host_tier, "host_tier");
    if (rc) return rc;
    rc = check_qffn(fn, slots, "slots");
    if (rc) return rc;
    REQUIRE_PTR(state, "state");
    REQUIRE_PTR(miss, "miss");
    REQUIRE_PTR(n_miss, "n_miss");
    const void *hp[9] = {host_tier->q_gate, host_tier->q_up, host_tier->q_down, host_tier->s_gate, host_tier->s_up,
                         host_tier->s_down, host_tier->z_gate, host_tier->z_up, host_tier->z_down};
    static const char *names[9] = {"q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down"};
    const void *dv[9];
    for (int j = 0; j < 9; j++) {
        rc = tier_address(fn, hp[j], names[j], &dv[j]);
        if (rc) return rc;
    }
    moe_qffn src = {dv[0], dv[1], dv[2], (const float *)dv[3], (const float *)dv[4], (const float *)dv[5],
                    dv[6], dv[7], dv[8]};
    long bytes[9];
    expert_tensor_bytes(s, bytes);
    return launch_status(fn, moe::launch_cache_fetch(to_qw(&src), to_qw(slots), bytes, miss, n_miss, state, c->E,
                                                     c->slots, kFetchWorkgroups, (hipStream_t)stream));
}

int moe_forward_cached(const moe_shape *s, const moe_cache_shape *c, const void *x, const moe_qffn *slots,
                       const void *state, const moe_qffn *shared, const int32_t *offsets, const int32_t *perm,
                       const int32_t *list, const int32_t *n_list, float *y_perm, float *y_shared, uint32_t *diag,
                       void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_forward_cached";
    int rc = check_cache_shape(fn, c);
    if (rc) return rc;
    rc = check_forward(fn, s, x, slots, shared, offsets, perm, list, n_list, y_perm, y_shared, diag, true);
    if (rc) return rc;
    if (s->E != c->E) return fail(MOE_EINVAL, "%s: layer E=%d and cache E=%d differ", fn, s->E, c->E);
    REQUIRE_PTR(state, "state");
    rc = check_ws(fn, s, ws, ws_bytes);
    if (rc) return rc;
    return run_forward(fn, s, x, slots, shared, offsets, perm, list, n_list, y_perm, y_shared, diag, ws, stream,
                       moe::cache_slot_map(state, c->E, c->slots), c->slots);
}

int moe_cache_stats(const moe_cache_shape *c, const void *state, int64_t out[5], int32_t *slot_expert, void *stream) {
    const char *fn = "moe_cache_stats";
    int rc = check_cache_shape(fn, c);
    if (rc) return rc;
    REQUIRE_PTR(state, "state");
    if (!out) return fail(MOE_EINVAL, "%s: out is NULL", fn);
    hipError_t err = hipMemcpyAsync(out, state, 5 * sizeof(int64_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (err == hipSuccess && slot_expert)
        err = hipMemcpyAsync(slot_expert, (const uint8_t *)state + 64, sizeof(int32_t) * (size_t)c->slots,
                             hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (err == hipSuccess) err = hipStreamSynchronize((hipStream_t)stream);
    return launch_status(fn, err);
}

}  // extern "C"
