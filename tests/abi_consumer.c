/*
 * A plain C consumer of the library's C ABI (compiled with gcc by test_abi.py, no GPU needed): it includes
 * moe2bit.h, links libmoe2bit.so, and checks the host-side behaviour every caller can rely on before any device
 * work -- the ABI version, the weight sizes, and that bad arguments return MOE_ERR_INVALID_ARG with a message and
 * launch nothing.  Prints "ok" and exits 0 on success.
 */
#include <stdio.h>
#include <string.h>

#include "moe2bit.h"

static int fails = 0;

static void expect(int cond, const char *what) {
    if (!cond) {
        printf("FAIL: %s (last error: %s)\n", what, moe_last_error());
        ++fails;
    }
}

int main(void) {
    expect(moe_abi_version() == MOE_ABI_VERSION, "ABI version matches the header");
    expect(moe_weight_bytes(MOE_FMT_IQ2X, 256, 2048, 4096) == (size_t)256 * 2048 * 16 * 66, "iq2x bytes");
    expect(moe_weight_bytes(MOE_FMT_Q2K, 1, 4096, 2048) == (size_t)4096 * 8 * 84, "q2k bytes");
    expect(moe_weight_bytes(MOE_FMT_Q4K, 1, 256, 256) == 144 * 256, "q4k bytes");
    expect(moe_weight_bytes(7, 1, 256, 256) == 0, "unknown format has no size");

    void *p = (void *)0x1000;   /* never dereferenced: every call below must fail its host checks */
    int32_t *ip = (int32_t *)0x1000;
    float *fp = (float *)0x1000;
    expect(moe_route(NULL, MOE_DT_BF16, 1, 4096, p, MOE_DT_BF16, 256, NULL, 8, ip, fp, NULL, ip, ip, ip, p,
                     1 << 20, NULL) == MOE_ERR_INVALID_ARG, "moe_route rejects a null x");
    expect(strlen(moe_last_error()) > 0, "a failure leaves a message");
    expect(moe_route(p, MOE_DT_BF16, 1, 4096, p, MOE_DT_BF16, 256, NULL, 0, ip, fp, NULL, ip, ip, ip, p, 1 << 20,
                     NULL) == MOE_ERR_INVALID_ARG, "moe_route rejects top_k = 0");

    moe_layer_desc L;
    memset(&L, 0, sizeof L);
    L.hidden = 4096; L.inter = 2048; L.n_experts = 256; L.top_k = 8;
    L.gate_up_fmt = MOE_FMT_IQ2X; L.down_fmt = MOE_FMT_Q2K;
    L.gate = L.up = L.down = p; L.codebook = (const uint8_t *)p;
    L.top_k = 300;
    expect(moe_expert_ffn_workspace(&L, 1) == 0, "no workspace size for top_k > n_experts");
    L.top_k = 8;
    expect(moe_expert_ffn_workspace(&L, 1) > 0, "workspace size of a valid layer");
    expect(moe_expert_ffn(&L, p, MOE_DT_BF16, 1, ip, ip, ip, ip, fp, NULL, p, 16, NULL) == MOE_ERR_INVALID_ARG,
           "moe_expert_ffn rejects a workspace that is too small");

    expect(moe_combine(NULL, fp, NULL, 1, 8, 4096, fp, NULL) == MOE_ERR_INVALID_ARG, "moe_combine null input");
    expect(moe_combine_steer(fp, fp, NULL, 1, 8, 4096, NULL, 1.0f, fp, NULL) == MOE_ERR_INVALID_ARG,
           "moe_combine_steer needs a direction");
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
