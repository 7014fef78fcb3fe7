/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for the routed
 * 2-bit Mixture-of-Experts FFN layer.  TEST INFRASTRUCTURE ONLY: it is loaded
 * by the test suite, by the smoke check and by the CPU-baseline leg of the
 * benchmark, never by the GPU library.  It shares no code, header, table or
 * constant with the GPU path.
 *
 * What the method is (source pages):
 *   - "antirez가 만든 DeepSeek V4 Flash 전용 로컬 추론 엔진 ds4" (jeff.news), summary
 *     bullets on the 2-bit quantization: only the routed MoE experts are
 *     quantized; up/gate use IQ2_XXS, down uses Q2_K; shared experts,
 *     projections and routing stay at full precision.
 *   - "antirez/ds4 — Metal용 DeepSeek V4 Flash 로컬 추론 엔진 완벽 가이드"
 *     (sigco.tistory.com), section "ds4의 혁신적 설계 철학": the same policy, and
 *     that the routed experts hold most of the model's bytes; a q4 variant
 *     exists (section "설치 및 사용법").
 * The pages name the formats only.  Field layouts, the codebook alphabet, the
 * quantizers and the router arithmetic below are this project's readings; every
 * one is listed with its justification in the design notes.
 *
 * Arithmetic: every value is carried in IEEE binary64.  Dequantized weights are
 * exact (each is a product of small integers and an fp16 scale), products of
 * bf16/fp32 inputs are exact in binary64, and only sums round.
 *
 * Formats (canonical, little-endian, 256 weights per block, blocks run along
 * the flattened row-major [out][in] matrix):
 *   iq2x (66 B):  d:fp16 | 8 group records of 8 B: idx[4] (one codebook row per
 *                 8 weights) then aux:u32 = signs (7 bits per 8 weights, bit
 *                 7j+i -> weight 8j+i negative, i<7; the 8th sign makes the
 *                 number of negatives even) | s (bits 28..31).
 *                 w = d * (2s+1) * C[idx][i] * sign
 *   q2k  (84 B):  d:fp16 | dmin:fp16 | 16 bytes (sc | m<<4) per 16-weight
 *                 sub-block | 64 bytes of 2-bit q (weight n at byte n/4, bits
 *                 2(n%4)).  w = d*sc*q - dmin*m
 *   q4k (144 B):  d:fp16 | dmin:fp16 | 12 bytes = 16 six-bit fields (field f at
 *                 bits 6f; f<8: sc_f, f>=8: m_(f-8)) for 8 sub-blocks of 32 |
 *                 128 bytes of 4-bit q (weight n at byte n/2, low nibble when n
 *                 even).  w = d*sc*q - dmin*m
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256

/* ------------------------------------------------------------------------ */
/* IEEE 754 conversions, written from the encoding definitions.              */
/* ------------------------------------------------------------------------ */

/* binary16 -> binary64 (exact). */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* binary64 -> binary16, round to nearest, ties to even; overflow -> inf. */
uint16_t oracle_f64_to_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = M * 2^-24; M == 1024 encodes 2^-14 */
        double M = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)M;
    }
    int e;
    (void)frexp(a, &e);                            /* a in [2^(e-1), 2^e) */
    double M = nearbyint(ldexp(a, 11 - e));        /* 11 significant bits */
    int E = e - 1;
    if (M >= 2048.0) { M = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)M - 1024));
}

/* bfloat16 -> binary64 (exact). */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Dequantization (exact).                                                  */
/* ------------------------------------------------------------------------ */

static uint32_t rd_u32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static int popcount7(uint32_t v) {
    int c = 0;
    for (int i = 0; i < 7; i++) c += (v >> i) & 1;
    return c;
}

/* one iq2x block -> 256 weights */
static void dequant_iq2x_block(const uint8_t *blk, const uint8_t *codebook, double *out) {
    double d = oracle_f16_to_f64(rd_u16(blk));
    for (int g = 0; g < 8; g++) {
        const uint8_t *rec = blk + 2 + 8 * g;
        uint32_t aux = rd_u32(rec + 4);
        int s = (int)(aux >> 28);
        double S = d * (double)(2 * s + 1);
        for (int j = 0; j < 4; j++) {
            int idx = rec[j];
            uint32_t sbits = (aux >> (7 * j)) & 0x7f;
            int neg8 = popcount7(sbits) & 1;       /* even number of negatives */
            for (int i = 0; i < 8; i++) {
                int neg = (i < 7) ? (int)((sbits >> i) & 1) : neg8;
                double v = S * (double)codebook[8 * idx + i];
                out[32 * g + 8 * j + i] = neg ? -v : v;
            }
        }
    }
}

static void dequant_q2k_block(const uint8_t *blk, double *out) {
    double d = oracle_f16_to_f64(rd_u16(blk));
    double dmin = oracle_f16_to_f64(rd_u16(blk + 2));
    for (int n = 0; n < QK; n++) {
        int j = n / 16;
        int sc = blk[4 + j] & 0xf;
        int m = blk[4 + j] >> 4;
        int q = (blk[20 + n / 4] >> (2 * (n % 4))) & 3;
        out[n] = d * (double)(sc * q) - dmin * (double)m;
    }
}

static int q4k_field(const uint8_t *f12, int f) {
    /* 96-bit little-endian string of 6-bit fields */
    int bit = 6 * f, v = 0;
    for (int b = 0; b < 6; b++) {
        int pos = bit + b;
        v |= ((f12[pos / 8] >> (pos % 8)) & 1) << b;
    }
    return v;
}

static void dequant_q4k_block(const uint8_t *blk, double *out) {
    double d = oracle_f16_to_f64(rd_u16(blk));
    double dmin = oracle_f16_to_f64(rd_u16(blk + 2));
    for (int n = 0; n < QK; n++) {
        int j = n / 32;
        int sc = q4k_field(blk + 4, j);
        int m = q4k_field(blk + 4, 8 + j);
        int q = (blk[16 + n / 2] >> (4 * (n % 2))) & 0xf;
        out[n] = d * (double)(sc * q) - dmin * (double)m;
    }
}

int oracle_block_bytes(int fmt) {
    switch (fmt) { case 1: return 66; case 2: return 84; case 3: return 144; default: return 0; }
}

/* fmt: 1 = iq2x, 2 = q2k, 3 = q4k.  Writes nblocks*256 doubles. */
void oracle_dequant(int fmt, const uint8_t *blocks, int64_t nblocks, const uint8_t *codebook, double *out) {
    int bb = oracle_block_bytes(fmt);
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; b++) {
        const uint8_t *blk = blocks + b * bb;
        if (fmt == 1) dequant_iq2x_block(blk, codebook, out + b * QK);
        else if (fmt == 2) dequant_q2k_block(blk, out + b * QK);
        else dequant_q4k_block(blk, out + b * QK);
    }
}

/* ------------------------------------------------------------------------ */
/* Quantizers (reference encoders; offline, not on the layer's hot path).    */
/* Rounding is round-half-even in binary64 (nearbyint).                      */
/* ------------------------------------------------------------------------ */

static double clampd(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

static void quant_iq2x_block(const float *w, const uint8_t *codebook, uint8_t *blk) {
    double G[8], Gmax = 0.0;
    for (int g = 0; g < 8; g++) {
        double mx = 0.0;
        for (int i = 0; i < 32; i++) { double a = fabs((double)w[32 * g + i]); if (a > mx) mx = a; }
        G[g] = mx / 3.0;
        if (G[g] > Gmax) Gmax = G[g];
    }
    memset(blk, 0, 66);
    uint16_t dh = oracle_f64_to_f16(Gmax / 31.0);
    double d = oracle_f16_to_f64(dh);
    if (d == 0.0) return;                            /* all-zero block */
    blk[0] = dh & 0xff; blk[1] = dh >> 8;
    for (int g = 0; g < 8; g++) {
        int s = (int)clampd(nearbyint((G[g] / d - 1.0) / 2.0), 0.0, 15.0);
        double S = d * (double)(2 * s + 1);
        uint8_t *rec = blk + 2 + 8 * g;
        uint32_t aux = (uint32_t)s << 28;
        for (int j = 0; j < 4; j++) {
            const float *x = w + 32 * g + 8 * j;
            /* brute-force nearest codebook row for the magnitudes; ties -> lowest row */
            int best = 0; double best_err = INFINITY;
            for (int e = 0; e < 256; e++) {
                double err = 0.0;
                for (int i = 0; i < 8; i++) {
                    double r = fabs((double)x[i]) - S * (double)codebook[8 * e + i];
                    err += r * r;
                }
                if (err < best_err) { best_err = err; best = e; }
            }
            rec[j] = (uint8_t)best;
            int neg[8], nneg = 0;
            for (int i = 0; i < 8; i++) { neg[i] = x[i] < 0.0f; nneg += neg[i]; }
            if (nneg & 1) {
                /* make the count even: flip the cheapest sign; ties -> lowest i */
                int fi = 0; double fc = INFINITY;
                for (int i = 0; i < 8; i++) {
                    double c = fabs((double)x[i]) * (double)codebook[8 * best + i];
                    if (c < fc) { fc = c; fi = i; }
                }
                neg[fi] ^= 1;
            }
            for (int i = 0; i < 7; i++) aux |= (uint32_t)neg[i] << (7 * j + i);
        }
        for (int b = 0; b < 4; b++) rec[4 + b] = (aux >> (8 * b)) & 0xff;
    }
}

/* q2k (nsub = 16, qmax = 3, smax = 15) and q4k (nsub = 8, qmax = 15, smax = 63). */
static void quant_kq_block(const float *w, int nsub, int qmax, int smax, uint8_t *sc_out, uint8_t *m_out,
                           uint16_t *d_out, uint16_t *dmin_out, uint8_t *q_out) {
    int L = QK / nsub;
    double step[16], off[16], max_step = 0.0, max_off = 0.0;
    for (int j = 0; j < nsub; j++) {
        double lo = 0.0, hi = 0.0;
        for (int i = 0; i < L; i++) {
            double v = (double)w[L * j + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        step[j] = (hi - lo) / (double)qmax;
        off[j] = -lo;
        if (step[j] > max_step) max_step = step[j];
        if (off[j] > max_off) max_off = off[j];
    }
    uint16_t dh = oracle_f64_to_f16(max_step / (double)smax);
    uint16_t mh = oracle_f64_to_f16(max_off / (double)smax);
    double d = oracle_f16_to_f64(dh), dmin = oracle_f16_to_f64(mh);
    *d_out = dh; *dmin_out = mh;
    for (int j = 0; j < nsub; j++) {
        int sc = d > 0.0 ? (int)clampd(nearbyint(step[j] / d), 0.0, (double)smax) : 0;
        int m = dmin > 0.0 ? (int)clampd(nearbyint(off[j] / dmin), 0.0, (double)smax) : 0;
        sc_out[j] = (uint8_t)sc; m_out[j] = (uint8_t)m;
        double unit = d * (double)sc;
        for (int i = 0; i < L; i++) {
            int q = 0;
            if (unit > 0.0)
                q = (int)clampd(nearbyint(((double)w[L * j + i] + dmin * (double)m) / unit), 0.0, (double)qmax);
            q_out[L * j + i] = (uint8_t)q;
        }
    }
}

static void quant_q2k_block(const float *w, uint8_t *blk) {
    uint8_t sc[16], m[16], q[QK];
    uint16_t dh, mh;
    quant_kq_block(w, 16, 3, 15, sc, m, &dh, &mh, q);
    memset(blk, 0, 84);
    blk[0] = dh & 0xff; blk[1] = dh >> 8; blk[2] = mh & 0xff; blk[3] = mh >> 8;
    for (int j = 0; j < 16; j++) blk[4 + j] = (uint8_t)(sc[j] | (m[j] << 4));
    for (int n = 0; n < QK; n++) blk[20 + n / 4] |= (uint8_t)(q[n] << (2 * (n % 4)));
}

static void quant_q4k_block(const float *w, uint8_t *blk) {
    uint8_t sc[16], m[16], q[QK];
    uint16_t dh, mh;
    quant_kq_block(w, 8, 15, 63, sc, m, &dh, &mh, q);
    memset(blk, 0, 144);
    blk[0] = dh & 0xff; blk[1] = dh >> 8; blk[2] = mh & 0xff; blk[3] = mh >> 8;
    for (int f = 0; f < 16; f++) {
        int v = f < 8 ? sc[f] : m[f - 8];
        for (int b = 0; b < 6; b++) {
            int pos = 6 * f + b;
            blk[4 + pos / 8] |= (uint8_t)(((v >> b) & 1) << (pos % 8));
        }
    }
    for (int n = 0; n < QK; n++) blk[16 + n / 2] |= (uint8_t)(q[n] << (4 * (n % 2)));
}

void oracle_quantize(int fmt, const float *w, int64_t nblocks, const uint8_t *codebook, uint8_t *out) {
    int bb = oracle_block_bytes(fmt);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t b = 0; b < nblocks; b++) {
        if (fmt == 1) quant_iq2x_block(w + b * QK, codebook, out + b * bb);
        else if (fmt == 2) quant_q2k_block(w + b * QK, out + b * bb);
        else quant_q4k_block(w + b * QK, out + b * bb);
    }
}

/* ------------------------------------------------------------------------ */
/* Routing: router logits, top-k, renormalised softmax.                     */
/* ------------------------------------------------------------------------ */

/* x and w elements as binary64: dt 0 = fp32, 1 = bf16 */
static double load_elem(const void *p, int dt, int64_t i) {
    if (dt == 1) return oracle_bf16_to_f64(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/*
 * Router logit l[t][e] = sum_h W[e][h] * x[t][h] (+ bias[e]).
 * Reading (the pages say only that routing stays at full precision): products
 * are exact in binary64; the sum is taken in a fixed order so that the fp32
 * logit is reproducible bit-for-bit: 64 partial sums, partial p accumulating
 * h = p, p+64, p+128, ... in increasing h; then p[i] += p[i+s] for
 * s = 32, 16, 8, 4, 2, 1 and i < s.  The logit is the binary64 total rounded
 * once to fp32; with a bias it is fp32(logit + bias) computed in binary64.
 */
static float router_logit(const void *x, int x_dt, const void *w, int w_dt, int64_t t, int64_t e, int H,
                          const float *bias) {
    double p[64];
    for (int i = 0; i < 64; i++) p[i] = 0.0;
    for (int h = 0; h < H; h++)
        p[h % 64] += load_elem(w, w_dt, e * (int64_t)H + h) * load_elem(x, x_dt, t * (int64_t)H + h);
    for (int s = 32; s >= 1; s /= 2)
        for (int i = 0; i < s; i++) p[i] += p[i + s];
    float l = (float)p[0];
    if (bias) l = (float)((double)l + (double)bias[e]);
    return l;
}

/*
 * Top-k with ties broken toward the lower expert index: experts ordered by
 * (-logit, index), the first k kept, in that order.  Weights: softmax over the
 * k selected logits, w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), binary64.
 */
void oracle_route(const void *x, int x_dt, int T, int H, const void *w, int w_dt, int E, const float *bias, int k,
                  float *logits, int32_t *topk_idx, double *topk_w) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; t++) {
        float *l = logits + (int64_t)t * E;
        for (int e = 0; e < E; e++) l[e] = router_logit(x, x_dt, w, w_dt, t, e, H, bias);
        int *taken = (int *)calloc((size_t)E, sizeof(int));
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict '>' keeps the lower index on ties */
            }
            taken[best] = 1;
            topk_idx[(int64_t)t * k + j] = best;
        }
        free(taken);
        double l0 = (double)l[topk_idx[(int64_t)t * k]], den = 0.0;
        for (int j = 0; j < k; j++) den += exp((double)l[topk_idx[(int64_t)t * k + j]] - l0);
        for (int j = 0; j < k; j++)
            topk_w[(int64_t)t * k + j] = exp((double)l[topk_idx[(int64_t)t * k + j]] - l0) / den;
    }
}

/*
 * Token-to-expert permutation: slot s = t*k + j carries expert topk_idx[s].
 * perm lists the slots grouped by expert in ascending expert order, keeping
 * slot order inside an expert (a stable counting sort); offsets[e] is where
 * expert e's group starts (offsets[E] = T*k); active[0] is the number of
 * experts with at least one slot, followed by those experts in ascending order.
 */
void oracle_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *offsets, int32_t *perm, int32_t *active) {
    int64_t S = (int64_t)T * k;
    int32_t *count = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t s = 0; s < S; s++) count[topk_idx[s]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + count[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t s = 0; s < S; s++) {
        int e = topk_idx[s];
        perm[offsets[e] + fill[e]] = (int32_t)s;
        fill[e]++;
    }
    int na = 0;
    for (int e = 0; e < E; e++)
        if (count[e] > 0) active[1 + na++] = e;
    active[0] = na;
    free(count);
    free(fill);
}

/* ------------------------------------------------------------------------ */
/* Expert FFN (SwiGLU) and combine.                                         */
/* ------------------------------------------------------------------------ */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* Dequantize row r of a [R][C] matrix stored as a sequence of blocks along the
 * flattened matrix; row r covers weights r*C .. r*C+C-1. */
static void dequant_row(int fmt, const uint8_t *mat, const uint8_t *codebook, int64_t r, int C, double *row,
                        double *scratch) {
    int bb = oracle_block_bytes(fmt);
    int64_t first = r * (int64_t)C, last = first + C;           /* [first, last) */
    for (int64_t b = first / QK; b * QK < last; b++) {
        const uint8_t *blk = mat + b * bb;
        if (fmt == 1) dequant_iq2x_block(blk, codebook, scratch);
        else if (fmt == 2) dequant_q2k_block(blk, scratch);
        else dequant_q4k_block(blk, scratch);
        for (int i = 0; i < QK; i++) {
            int64_t n = b * QK + i;
            if (n >= first && n < last) row[n - first] = scratch[i];
        }
    }
}

/*
 * Routed expert FFN for every slot: with e = topk_idx[s] and t = s / k,
 *   g = Wg_e x_t, u = Wu_e x_t, h = silu(g) * u, o_s = Wd_e h      (binary64)
 * Wg, Wu: n_experts x [I][H], Wd: n_experts x [H][I], canonical blocks.
 * Processes experts in ascending order, each over its slots (the permutation
 * groups the slots); results land in slot order in out[s][H].
 */
void oracle_expert_ffn(const void *x, int x_dt, int T, int H, int I, int E, int k, const int32_t *topk_idx,
                       int fmt_gu, const uint8_t *Wg, const uint8_t *Wu, int fmt_d, const uint8_t *Wd,
                       const uint8_t *codebook, double *out) {
    int64_t S = (int64_t)T * k;
    int64_t gu_bytes = (int64_t)I * H / QK * oracle_block_bytes(fmt_gu);
    int64_t d_bytes = (int64_t)H * I / QK * oracle_block_bytes(fmt_d);
    double *xs = (double *)malloc(sizeof(double) * (size_t)T * H);
    for (int64_t i = 0; i < (int64_t)T * H; i++) xs[i] = load_elem(x, x_dt, i);
    int32_t *slots = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1) * I);
    for (int e = 0; e < E; e++) {
        int64_t n = 0;
        for (int64_t s = 0; s < S; s++)
            if (topk_idx[s] == e) slots[n++] = (int32_t)s;
        if (n == 0) continue;
        const uint8_t *g_e = Wg + e * gu_bytes, *u_e = Wu + e * gu_bytes, *d_e = Wd + e * d_bytes;
        #pragma omp parallel
        {
            double *rg = (double *)malloc(sizeof(double) * (size_t)H);
            double *ru = (double *)malloc(sizeof(double) * (size_t)H);
            double *rd = (double *)malloc(sizeof(double) * (size_t)I);
            double *scr = (double *)malloc(sizeof(double) * QK);
            #pragma omp for schedule(static)
            for (int r = 0; r < I; r++) {
                dequant_row(fmt_gu, g_e, codebook, r, H, rg, scr);
                dequant_row(fmt_gu, u_e, codebook, r, H, ru, scr);
                for (int64_t a = 0; a < n; a++) {
                    const double *xt = xs + (int64_t)(slots[a] / k) * H;
                    double g = 0.0, u = 0.0;
                    for (int c = 0; c < H; c++) { g += rg[c] * xt[c]; u += ru[c] * xt[c]; }
                    h[a * I + r] = silu(g) * u;
                }
            }
            #pragma omp for schedule(static)
            for (int r = 0; r < H; r++) {
                dequant_row(fmt_d, d_e, codebook, r, I, rd, scr);
                for (int64_t a = 0; a < n; a++) {
                    double o = 0.0;
                    for (int c = 0; c < I; c++) o += rd[c] * h[a * I + c];
                    out[(int64_t)slots[a] * H + r] = o;
                }
            }
            free(rg); free(ru); free(rd); free(scr);
        }
    }
    free(xs); free(slots); free(h);
}

/*
 * Shared expert at full precision (bf16 weights): s_t = Wd (silu(Wg x_t) * (Wu x_t)).
 * Wg, Wu: [Is][H] bf16, Wd: [H][Is] bf16.
 */
void oracle_shared_ffn(const void *x, int x_dt, int T, int H, int Is, const uint16_t *Wg, const uint16_t *Wu,
                       const uint16_t *Wd, double *out) {
    double *h = (double *)malloc(sizeof(double) * (size_t)T * Is);
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < Is; r++) {
        for (int t = 0; t < T; t++) {
            double g = 0.0, u = 0.0;
            for (int c = 0; c < H; c++) {
                double xv = load_elem(x, x_dt, (int64_t)t * H + c);
                g += oracle_bf16_to_f64(Wg[(int64_t)r * H + c]) * xv;
                u += oracle_bf16_to_f64(Wu[(int64_t)r * H + c]) * xv;
            }
            h[(int64_t)t * Is + r] = silu(g) * u;
        }
    }
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < H; r++) {
        for (int t = 0; t < T; t++) {
            double o = 0.0;
            for (int c = 0; c < Is; c++) o += oracle_bf16_to_f64(Wd[(int64_t)r * Is + c]) * h[(int64_t)t * Is + c];
            out[(int64_t)t * H + r] = o;
        }
    }
    free(h);
}

/* y[t] = sum_{j<k} w[t][j] * o[t*k+j] + s[t] (s may be NULL), j in order, binary64. */
void oracle_combine(const double *slot_out, const double *topk_w, const double *shared_out, int T, int k, int H,
                    double *y) {
    for (int t = 0; t < T; t++)
        for (int c = 0; c < H; c++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) acc += topk_w[(int64_t)t * k + j] * slot_out[((int64_t)t * k + j) * H + c];
            if (shared_out) acc += shared_out[(int64_t)t * H + c];
            y[(int64_t)t * H + c] = acc;
        }
}

/*
 * Directional steering of the FFN output ("DwarfStar4 / ds4.c" user report on
 * modu-print.com, the ds4-server option listing, the FFN steering option): with
 * one direction v per layer and a strength F, every token's FFN output y loses
 * F times its component along v, y' = y - F * v * dot(v, y).  v is taken as
 * given (not normalised); dot(v, y) runs over c in increasing order, binary64.
 * y and out may be the same array.
 */
void oracle_steer(const double *y, const double *v, double F, int T, int H, double *out) {
    for (int t = 0; t < T; t++) {
        const double *yt = y + (int64_t)t * H;
        double d = 0.0;
        for (int c = 0; c < H; c++) d += v[c] * yt[c];
        for (int c = 0; c < H; c++) out[(int64_t)t * H + c] = yt[c] - F * v[c] * d;
    }
}
