// Drives the host side of the C ABI (argument checks, workspace sizing, path choice) over many shapes, for a
// build whose host code runs under AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure).  No
// call here reaches the GPU: every shape given to a compute call fails validation, or has T = 0.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/moe.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}

int main() {
    int fails = 0;
    char *FAKE = (char *)(uintptr_t)0x10000;
    int32_t *I32 = (int32_t *)FAKE;
    float *F32 = (float *)FAKE;
    moe_qffn q;
    void **qp = (void **)&q;
    for (int i = 0; i < 9; i++) qp[i] = FAKE;
    // workspace sizes over random shapes, valid and not
    for (int it = 0; it < 20000; it++) {
        moe_shape s;
        s.T = (int)(rnd() % 20000) - 10;
        s.d = 32 * (int)(rnd() % 5000);
        s.E = (int)(rnd() % 1100);
        s.k = (int)(rnd() % 40);
        s.I = 32 * (int)(rnd() % 4500);
        s.I_shared = (rnd() & 1) ? 0 : 32 * (int)(rnd() % 4500);
        s.routed_scale = 2.5f;
        s.act_dtype = (int)(rnd() % 3);
        s.wbits = (rnd() & 1) ? 4 : ((rnd() & 1) ? 8 : 2);
        s.path = (int)(rnd() % 4);
        s.flags = (int)(rnd() % 3);
        const size_t ws = moe_workspace_size(&s);
        // a compute call with a NULL required pointer: fails validation whatever the shape
        int rc = moe_route(&s, FAKE, NULL, F32, I32, F32, NULL, FAKE, ws, NULL);
        if (rc == MOE_OK && s.T != 0) fails++;
        rc = moe_forward(&s, FAKE, &q, &q, NULL, I32, I32, I32, F32, F32, NULL, FAKE, ws, NULL);
        if (rc == MOE_OK && s.T != 0) fails++;
        rc = moe_forward_static(&s, FAKE, &q, &q, I32, I32, NULL, I32, F32, F32, NULL, NULL);
        if (rc == MOE_OK && s.T != 0) fails++;
        if (strlen(moe_last_error()) >= 512) fails++;
    }
    // T = 0 on valid shapes: every call returns OK without touching the device
    moe_shape s0 = {0, 7168, 256, 8, 2048, 2048, 2.5f, MOE_ACT_BF16, 4, MOE_PATH_AUTO, 0};
    const size_t ws0 = moe_workspace_size(&s0);
    if (moe_route(&s0, NULL, (float *)FAKE, (float *)FAKE, NULL, NULL, NULL, FAKE, ws0, NULL) != MOE_OK) fails++;
    if (moe_forward(&s0, NULL, &q, &q, I32, NULL, I32, I32, NULL, NULL, NULL, FAKE, ws0, NULL) != MOE_OK) fails++;
    if (moe_forward_static(&s0, NULL, &q, &q, I32, NULL, I32, I32, NULL, NULL, NULL, NULL) != MOE_OK) fails++;
    if (moe_combine(&s0, NULL, NULL, NULL, NULL, NULL, NULL) != MOE_OK) fails++;
    if (moe_abi_version() < 3) fails++;
    printf(fails ? "abi driver: %d unexpected results\n" : "abi driver ok\n", fails);
    return fails != 0;
}
