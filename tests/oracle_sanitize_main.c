/*
 * Drives every exported function of the CPU oracle (oracle/moe_oracle.c) over
 * small, ragged layers so that the test suite can run the oracle under the
 * address and undefined-behaviour sanitizers and compare it bit for bit with
 * the ordinary build.  Test infrastructure only.
 *
 * Inputs come from splitmix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), seeded per case.  Each stage
 * prints one line "<case> <stage> <FNV-1a 64 of its output bytes>"; the
 * caller compares the lines of the two builds.
 *
 * Cases cover: T = 0 and T = 1, k = 1 and k = E, experts that receive no
 * token, H not a multiple of 64 (the router's partial sums), the three weight
 * formats, fp32 and bf16 activations, a router bias, and quantizer inputs with
 * zero, tiny and huge blocks.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_block_bytes(int fmt);
void oracle_dequant(int fmt, const uint8_t *blocks, int64_t nblocks, const uint8_t *codebook, double *out);
void oracle_quantize(int fmt, const float *w, int64_t nblocks, const uint8_t *codebook, uint8_t *out);
void oracle_route(const void *x, int x_dt, int T, int H, const void *w, int w_dt, int E, const float *bias, int k,
                  float *logits, int32_t *topk_idx, double *topk_w);
void oracle_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *offsets, int32_t *perm, int32_t *active);
void oracle_expert_ffn(const void *x, int x_dt, int T, int H, int I, int E, int k, const int32_t *topk_idx,
                       int fmt_gu, const uint8_t *Wg, const uint8_t *Wu, int fmt_d, const uint8_t *Wd,
                       const uint8_t *codebook, double *out);
void oracle_shared_ffn(const void *x, int x_dt, int T, int H, int Is, const uint16_t *Wg, const uint16_t *Wu,
                       const uint16_t *Wd, double *out);
void oracle_combine(const double *slot_out, const double *topk_w, const double *shared_out, int T, int k, int H,
                    double *y);
void oracle_steer(const double *y, const double *v, double F, int T, int H, double *out);
double oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16(double x);
double oracle_bf16_to_f64(uint16_t b);

static uint64_t sm_state;

static uint64_t sm_next(void) {
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* uniform in [-1, 1) from the top 53 bits */
static double sm_sym(void) { return (double)(sm_next() >> 11) * 0x1.0p-52 - 1.0; }

static uint64_t fnv(const void *p, size_t n) {
    const uint8_t *b = (const uint8_t *)p;
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; i++) h = (h ^ b[i]) * 0x100000001b3ull;
    return h;
}

static void report(const char *name, const char *stage, const void *p, size_t n) {
    printf("%s %s %016llx\n", name, stage, (unsigned long long)fnv(p, n));
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* bf16 by truncation of an fp32 bit pattern: any bf16 value is a valid input */
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint8_t *random_blocks(int fmt, int64_t nblocks, const uint8_t *cb, float wscale) {
    /* quantize random weights, so that every field holds what the quantizer writes */
    float *w = (float *)xmalloc(sizeof(float) * (size_t)nblocks * 256);
    for (int64_t i = 0; i < nblocks * 256; i++) w[i] = (float)(wscale * sm_sym());
    uint8_t *b = (uint8_t *)xmalloc((size_t)nblocks * oracle_block_bytes(fmt));
    oracle_quantize(fmt, w, nblocks, cb, b);
    free(w);
    return b;
}

static void layer_case(const char *name, uint64_t seed, int T, int H, int I, int Is, int E, int k, int fmt_gu,
                       int fmt_d, int x_bf16, int with_bias) {
    sm_state = seed;
    uint8_t cb[256 * 8];
    for (int i = 0; i < 256 * 8; i++) cb[i] = (uint8_t)(1 + sm_next() % 3);

    size_t nx = (size_t)T * H;
    float *xf = (float *)xmalloc(sizeof(float) * nx);
    uint16_t *xb = (uint16_t *)xmalloc(sizeof(uint16_t) * nx);
    for (size_t i = 0; i < nx; i++) { xf[i] = (float)sm_sym(); xb[i] = bf16_of(xf[i]); }
    const void *x = x_bf16 ? (const void *)xb : (const void *)xf;
    int x_dt = x_bf16 ? 1 : 0;

    uint16_t *wr = (uint16_t *)xmalloc(sizeof(uint16_t) * (size_t)E * H);
    for (int64_t i = 0; i < (int64_t)E * H; i++) wr[i] = bf16_of((float)(0.05 * sm_sym()));
    float *bias = (float *)xmalloc(sizeof(float) * (size_t)E);
    for (int e = 0; e < E; e++) bias[e] = (float)(0.01 * sm_sym());

    float *logits = (float *)xmalloc(sizeof(float) * (size_t)T * E);
    int32_t *idx = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)T * k);
    double *tw = (double *)xmalloc(sizeof(double) * (size_t)T * k);
    oracle_route(x, x_dt, T, H, wr, 1, E, with_bias ? bias : NULL, k, logits, idx, tw);
    report(name, "logits", logits, sizeof(float) * (size_t)T * E);
    report(name, "topk_idx", idx, sizeof(int32_t) * (size_t)T * k);
    report(name, "topk_w", tw, sizeof(double) * (size_t)T * k);

    int64_t S = (int64_t)T * k;
    int32_t *off = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *perm = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)S);
    int32_t *act = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)(E + 1));
    oracle_permute(idx, T, k, E, off, perm, act);
    report(name, "offsets", off, sizeof(int32_t) * (size_t)(E + 1));
    report(name, "perm", perm, sizeof(int32_t) * (size_t)S);
    report(name, "active", act, sizeof(int32_t) * (size_t)(1 + act[0]));

    int64_t gu_blocks = (int64_t)I * H / 256, d_blocks = (int64_t)H * I / 256;
    uint8_t *Wg = random_blocks(fmt_gu, E * gu_blocks, cb, 0.03f);
    uint8_t *Wu = random_blocks(fmt_gu, E * gu_blocks, cb, 0.03f);
    uint8_t *Wd = random_blocks(fmt_d, E * d_blocks, cb, 0.03f);
    double *deq = (double *)xmalloc(sizeof(double) * (size_t)gu_blocks * 256);
    oracle_dequant(fmt_gu, Wg, gu_blocks, cb, deq);
    report(name, "dequant_gu", deq, sizeof(double) * (size_t)gu_blocks * 256);
    free(deq);
    deq = (double *)xmalloc(sizeof(double) * (size_t)d_blocks * 256);
    oracle_dequant(fmt_d, Wd, d_blocks, cb, deq);
    report(name, "dequant_d", deq, sizeof(double) * (size_t)d_blocks * 256);
    free(deq);

    double *slot = (double *)xmalloc(sizeof(double) * (size_t)S * H);
    oracle_expert_ffn(x, x_dt, T, H, I, E, k, idx, fmt_gu, Wg, Wu, fmt_d, Wd, cb, slot);
    report(name, "slot_out", slot, sizeof(double) * (size_t)S * H);

    uint16_t *sg = (uint16_t *)xmalloc(sizeof(uint16_t) * (size_t)Is * H);
    uint16_t *su = (uint16_t *)xmalloc(sizeof(uint16_t) * (size_t)Is * H);
    uint16_t *sd = (uint16_t *)xmalloc(sizeof(uint16_t) * (size_t)H * Is);
    for (int64_t i = 0; i < (int64_t)Is * H; i++) {
        sg[i] = bf16_of((float)(0.05 * sm_sym()));
        su[i] = bf16_of((float)(0.05 * sm_sym()));
        sd[i] = bf16_of((float)(0.05 * sm_sym()));
    }
    double *sh = (double *)xmalloc(sizeof(double) * (size_t)T * H);
    oracle_shared_ffn(x, x_dt, T, H, Is, sg, su, sd, sh);
    report(name, "shared_out", sh, sizeof(double) * (size_t)T * H);

    double *y = (double *)xmalloc(sizeof(double) * (size_t)T * H);
    oracle_combine(slot, tw, sh, T, k, H, y);
    report(name, "y", y, sizeof(double) * (size_t)T * H);
    oracle_combine(slot, tw, NULL, T, k, H, y);
    report(name, "y_routed", y, sizeof(double) * (size_t)T * H);

    double *v = (double *)xmalloc(sizeof(double) * (size_t)H);
    for (int c = 0; c < H; c++) v[c] = sm_sym();
    oracle_steer(y, v, 0.75, T, H, y); /* in place, as the oracle allows */
    report(name, "steer", y, sizeof(double) * (size_t)T * H);

    free(v); free(y); free(sh); free(sg); free(su); free(sd); free(slot);
    free(Wg); free(Wu); free(Wd); free(off); free(perm); free(act);
    free(logits); free(idx); free(tw); free(bias); free(wr); free(xf); free(xb);
}

static void quant_edge_case(void) {
    /* blocks of zeros, of tiny and of huge weights, and of one spike */
    sm_state = 99;
    uint8_t cb[256 * 8];
    for (int i = 0; i < 256 * 8; i++) cb[i] = (uint8_t)(1 + sm_next() % 3);
    const int nb = 5;
    float *w = (float *)xmalloc(sizeof(float) * nb * 256);
    for (int i = 0; i < 256; i++) {
        w[i] = 0.0f;
        w[256 + i] = (float)(1e-7 * sm_sym());
        w[512 + i] = (float)(6.0e4 * sm_sym());
        w[768 + i] = (i == 77) ? 1.0f : 0.0f;
        w[1024 + i] = (float)sm_sym();
    }
    for (int fmt = 1; fmt <= 3; fmt++) {
        uint8_t *b = (uint8_t *)xmalloc((size_t)nb * oracle_block_bytes(fmt));
        double *d = (double *)xmalloc(sizeof(double) * nb * 256);
        oracle_quantize(fmt, w, nb, cb, b);
        oracle_dequant(fmt, b, nb, cb, d);
        char stage[32];
        snprintf(stage, sizeof stage, "quant_fmt%d", fmt);
        report("edges", stage, b, (size_t)nb * oracle_block_bytes(fmt));
        snprintf(stage, sizeof stage, "dequant_fmt%d", fmt);
        report("edges", stage, d, sizeof(double) * nb * 256);
        free(b); free(d);
    }
    free(w);
    /* every fp16 and bf16 bit pattern through the conversions */
    double acc[3] = {0.0, 0.0, 0.0};
    uint64_t h = 0xcbf29ce484222325ull;
    for (uint32_t u = 0; u < 65536; u++) {
        double a = oracle_f16_to_f64((uint16_t)u), b = oracle_bf16_to_f64((uint16_t)u);
        uint16_t r = oracle_f64_to_f16(a);
        h = (h ^ r) * 0x100000001b3ull;
        if (isfinite(a)) acc[0] += a;
        if (isfinite(b)) acc[1] += fabs(b) > 1e30 ? 0.0 : b;
        acc[2] += (double)oracle_f64_to_f16(sm_sym() * 7e4);
    }
    printf("edges conversions %016llx\n", (unsigned long long)(h ^ fnv(acc, sizeof acc)));
}

int main(void) {
    /* name, seed, T, H, I, Is, E, k, fmt_gu, fmt_d, x_bf16, bias */
    layer_case("empty", 1, 0, 256, 64, 32, 8, 2, 1, 2, 1, 0);
    layer_case("one_token", 2, 1, 256, 64, 32, 16, 4, 1, 2, 1, 1);
    layer_case("ragged_h", 3, 7, 96, 32, 16, 5, 2, 1, 2, 0, 0);
    layer_case("k_eq_e", 4, 5, 128, 64, 32, 4, 4, 3, 3, 1, 1);
    layer_case("k_one", 5, 9, 256, 32, 24, 12, 1, 1, 3, 0, 1);
    layer_case("many", 6, 37, 320, 64, 48, 24, 6, 3, 2, 1, 0);
    quant_edge_case();
    return 0;
}
