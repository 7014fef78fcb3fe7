// Decode / verify expert FFN: GEMV kernels for at most 8 tokens per call.
//
// Each selected expert's weights are streamed once per call with 16-byte
// lane loads.  A lane always covers the same columns, so the activations (x
// for gate/up, h for down) are loaded once into registers and reused for every
// row; only the 2-bit fields move per row.  Weights are decoded in registers:
// an iq2x sub-group (8 weights) is one LDS lookup of its codebook row as eight
// fp4 codes, OR-ed with its spread sign word, then converted two at a time to
// bf16 pairs (magnitudes 1..3, exact) and dotted with bf16 activation pairs;
// the group scale (2s+1) and block scale d multiply the partial sums in fp32.
// q2k codes are fp4 codes already (value q/2) and dot with fp16 h pairs; the
// sub-block mins use per-sub-block sums of h.  Rows reduce across their lanes.
//
// The routed experts and the shared expert run in the same launch (different
// workgroups), so the HBM-heavy bf16 shared rows and the VALU-heavy 2-bit rows
// share the machine.
#include "common.h"
#include "internal.h"

using namespace moe;

namespace {

constexpr int WAVES = 4;

// rows per wave for bf16 rows with CPL 16-byte chunks per lane
template <int CPL> constexpr int shared_nr() { return CPL >= 4 ? 1 : 4 / CPL; }

// Down projection for one token: twice the rows per wave (routed and shared),
// so that the routed workgroups leave room for shared ones from the start.
template <int MAXM> constexpr int nr_down() { return MAXM == 1 ? 8 : 4; }
template <int CPL, int MAXM> constexpr int shared_nr_down() { return MAXM == 1 ? 2 * shared_nr<CPL>() : shared_nr<CPL>(); }

template <int LPR> __device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ void tables(const uint8_t *codebook, uint32_t *cb4, uint32_t *sgn) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb4[i] = codebook_row_fp4(codebook, i);
    for (int i = threadIdx.x; i < 128; i += blockDim.x) sgn[i] = sign_spread(i);
}

// Tokens of work item: routed expert (slots from the permutation) or all T (shared).
template <int MAXM> struct Tokens {
    int n;
    int slot[MAXM];
    int tok[MAXM];
};

// ---------------------------------------------------------------------------
// iq2x: one 16-byte chunk = groups c and c+4 of one block (64 weights)
// ---------------------------------------------------------------------------
template <int MAXM>
__device__ __forceinline__ void iq2x_chunk(uint4 q, float d, const uint32_t (&xr)[MAXM][32], const uint32_t *cb4,
                                           const uint32_t *sgn, float (&acc)[MAXM]) {
    float racc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) racc[m] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
        const uint32_t lo = grp ? q.z : q.x, hi = grp ? q.w : q.y;
        const uint32_t s = ((lo >> 15) & 1u) | ((lo >> 30) & 2u) | ((hi >> 13) & 4u) | ((hi >> 28) & 8u);
        float gacc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) gacc[m] = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t f = ((p < 2 ? lo : hi) >> (16 * (p & 1))) & 0xFFFFu;
            const uint32_t word = cb4[f & 0xFFu] | sgn[(f >> 8) & 0x7Fu];
            const bf16x2_t w0 = fp4x2_bf16<0>(word), w1 = fp4x2_bf16<1>(word);
            const bf16x2_t w2 = fp4x2_bf16<2>(word), w3 = fp4x2_bf16<3>(word);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                const uint32_t *xp = &xr[m][grp * 16 + p * 4];
                float g = gacc[m];
                g = dot2_bf16(w0, __builtin_bit_cast(bf16x2_t, xp[0]), g);
                g = dot2_bf16(w1, __builtin_bit_cast(bf16x2_t, xp[1]), g);
                g = dot2_bf16(w2, __builtin_bit_cast(bf16x2_t, xp[2]), g);
                g = dot2_bf16(w3, __builtin_bit_cast(bf16x2_t, xp[3]), g);
                gacc[m] = g;
            }
        }
        const float mult = (float)(2 * s + 1);
#pragma unroll
        for (int m = 0; m < MAXM; ++m) racc[m] = __fmaf_rn(mult, gacc[m], racc[m]);
    }
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = __fmaf_rn(d, racc[m], acc[m]);
}

// Routed gate/up for one expert and a tile of rows.  Row length H = 64*LPR*CPL.
template <int LPR, int CPL, int MAXM, int NR>
__device__ void routed_gateup(const FfnArgs &a, int e, const Tokens<MAXM> &tk, int row0, const uint32_t *cb4,
                              const uint32_t *sgn, _Float16 *__restrict__ h) {
    constexpr int RPI = 64 / LPR;                 // rows per wave iteration
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, I = a.I;
    const int64_t nb_row = H / MOE_QK, nb_mat = (int64_t)I * nb_row, NB = nb_mat * a.E;
    // activations for this lane's chunks, bf16 pairs
    uint32_t xr[CPL][MAXM][32];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = cp + LPR * i, b = ch >> 2, c = ch & 3;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int t = tk.tok[m < tk.n ? m : 0];
            const uint4 *xa = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + (int64_t)t * H +
                                                              MOE_QK * b + 32 * c);
            const uint4 *xb = xa + 16;            // +128 bf16: group c+4
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                uint4 u = xa[v];
                xr[i][m][4 * v + 0] = u.x; xr[i][m][4 * v + 1] = u.y; xr[i][m][4 * v + 2] = u.z; xr[i][m][4 * v + 3] = u.w;
                u = xb[v];
                xr[i][m][16 + 4 * v + 0] = u.x; xr[i][m][16 + 4 * v + 1] = u.y;
                xr[i][m][16 + 4 * v + 2] = u.z; xr[i][m][16 + 4 * v + 3] = u.w;
            }
        }
    }
    const uint8_t *Gq = a.gate, *Uq = a.up;
    const uint16_t *Gd = reinterpret_cast<const uint16_t *>(a.gate + NB * 64);
    const uint16_t *Ud = reinterpret_cast<const uint16_t *>(a.up + NB * 64);
    uint4 gq[NR][CPL], uq[NR][CPL];
    uint16_t gd[NR][CPL], ud[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, I - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = cp + LPR * i;
            const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (ch >> 2);
            gq[j][i] = *reinterpret_cast<const uint4 *>(Gq + bl * 64 + (ch & 3) * 16);
            uq[j][i] = *reinterpret_cast<const uint4 *>(Uq + bl * 64 + (ch & 3) * 16);
            gd[j][i] = Gd[bl];
            ud[j][i] = Ud[bl];
        }
    }
    // h scale exponent per token: the largest |x| over the row (the LPR lanes of a row cover it), after the
    // weight requests
    int sig[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        uint32_t mx = 0u;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int v = 0; v < 32; ++v) mx = bf16x2_absmax_acc(mx, xr[i][m][v]);
        sig[m] = h_sigma(wave_max_f32(bf16x2_absmax_value(mx)));  // the lanes of a wave cover the whole row
    }
    if (row0 == 0 && wv == 0 && lane == 0)
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
            if (m < tk.n) a.hsig[tk.tok[m]] = sig[m];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        float ga[MAXM], ua[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) { ga[m] = 0.f; ua[m] = 0.f; }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            iq2x_chunk<MAXM>(gq[j][i], f16_bits_to_f32(gd[j][i]), xr[i], cb4, sgn, ga);
            iq2x_chunk<MAXM>(uq[j][i], f16_bits_to_f32(ud[j][i]), xr[i], cb4, sgn, ua);
        }
        const int r = row0 + (wv * NR + j) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float g = row_sum<LPR>(ga[m]), u = row_sum<LPR>(ua[m]);
            if (m < tk.n && cp == 0 && r < I) h[(int64_t)tk.slot[m] * I + r] = (_Float16)ldexpf(silu_mul(g, u), -sig[m]);
        }
    }
}

// q4k chunk: 16 B = the 32 codes of sub-block j of a block (meta: the block's
// d | dmin and packed 6-bit fields).  Codes enter the dot products as bf16
// 128 + q (pattern 0x4300 | q; pairs sit in the two halves of a prepared word),
// so per sub-block  sum w x = d sc P - (128 d sc + dmin m) X  with P the dot
// of the offset codes and X the sum of the 32 activations.
template <int MAXM>
__device__ __forceinline__ void q4k_chunk_bf16(uint4 q, uint4 meta, int j, const uint32_t (&xr)[MAXM][16],
                                               const float (&xs)[MAXM], float (&acc)[MAXM]) {
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    float P[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) P[m] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t t = __builtin_bit_cast(bf16x2_t, ((qw[w] >> (4 * i)) & 0x000F000Fu) | 0x43004300u);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) P[m] = dot2_bf16(t, __builtin_bit_cast(bf16x2_t, xr[m][4 * w + i]), P[m]);
        }
    const float sc = f16_bits_to_f32(meta.x & 0xFFFFu) * (float)q4k_field(meta.y, meta.z, meta.w, j);
    const float off = __fmaf_rn(f16_bits_to_f32(meta.x >> 16), (float)q4k_field(meta.y, meta.z, meta.w, 8 + j),
                                128.f * sc);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] += __fmaf_rn(sc, P[m], -off * xs[m]);
}

// Routed q4k gate/up: a lane covers chunks cp + LPR*i (32 weights each) of a row of H = 32*LPR*CPL.
template <int LPR, int CPL, int MAXM, int NR>
__device__ void routed_gateup_q4k(const FfnArgs &a, int e, const Tokens<MAXM> &tk, int row0,
                                  _Float16 *__restrict__ h) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, I = a.I;
    const int64_t nb_row = H / MOE_QK, nb_mat = (int64_t)I * nb_row, NB = nb_mat * a.E;
    uint32_t xr[CPL][MAXM][16];
    float xs[CPL][MAXM];
    uint32_t xmax[MAXM];                                      // largest |x| of the lane's chunks, two bf16 fields
#pragma unroll
    for (int m = 0; m < MAXM; ++m) xmax[m] = 0u;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = cp + LPR * i;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int t = tk.tok[m < tk.n ? m : 0];
            const uint4 *xa = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + (int64_t)t * H + 32 * ch);
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 u = xa[v];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xr[i][m][4 * v + k] = w4[k];
                    sum += __uint_as_float(w4[k] << 16) + __uint_as_float(w4[k] & 0xFFFF0000u);
                    xmax[m] = bf16x2_absmax_acc(xmax[m], w4[k]);
                }
            }
            xs[i][m] = sum;
        }
    }
    uint4 gq[NR][CPL], uq[NR][CPL], gm[NR][CPL], um[NR][CPL];
#pragma unroll
    for (int jr = 0; jr < NR; ++jr) {
        const int r = min(row0 + (wv * NR + jr) * RPI + rsub, I - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = cp + LPR * i;
            const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (ch >> 3);
            gq[jr][i] = *reinterpret_cast<const uint4 *>(a.gate + bl * 128 + (ch & 7) * 16);
            uq[jr][i] = *reinterpret_cast<const uint4 *>(a.up + bl * 128 + (ch & 7) * 16);
            gm[jr][i] = *reinterpret_cast<const uint4 *>(a.gate + NB * 128 + bl * 16);
            um[jr][i] = *reinterpret_cast<const uint4 *>(a.up + NB * 128 + bl * 16);
        }
    }
    int sig[MAXM];                                            // h scale exponent per token (largest |x| of the row)
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        sig[m] = h_sigma(wave_max_f32(bf16x2_absmax_value(xmax[m])));  // the lanes of a wave cover the whole row
    }
#pragma unroll
    for (int jr = 0; jr < NR; ++jr) {
        float ga[MAXM], ua[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) { ga[m] = 0.f; ua[m] = 0.f; }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int j = (cp + LPR * i) & 7;
            q4k_chunk_bf16<MAXM>(gq[jr][i], gm[jr][i], j, xr[i], xs[i], ga);
            q4k_chunk_bf16<MAXM>(uq[jr][i], um[jr][i], j, xr[i], xs[i], ua);
        }
        const int r = row0 + (wv * NR + jr) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float g = row_sum<LPR>(ga[m]), u = row_sum<LPR>(ua[m]);
            if (m < tk.n && cp == 0 && r < I) h[(int64_t)tk.slot[m] * I + r] = (_Float16)ldexpf(silu_mul(g, u), -sig[m]);
        }
    }
    if (row0 == 0 && wv == 0 && lane == 0)
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
            if (m < tk.n) a.hsig[tk.tok[m]] = sig[m];
}

// Shared gate/up (bf16 rows of H = 8*LPR*CPL).
template <int LPR, int CPL, int MAXM, int NR>
__device__ void shared_gateup(const FfnArgs &a, const Tokens<MAXM> &tk, int row0, float *__restrict__ hs) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, Is = a.Is;
    uint32_t xr[CPL][MAXM][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int t = tk.tok[m < tk.n ? m : 0];
            const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + (int64_t)t * H +
                                                            8 * (cp + LPR * i));
            xr[i][m][0] = u.x; xr[i][m][1] = u.y; xr[i][m][2] = u.z; xr[i][m][3] = u.w;
        }
    uint4 gq[NR][CPL], uq[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, Is - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            gq[j][i] = *reinterpret_cast<const uint4 *>(a.sg + (int64_t)r * H + 8 * (cp + LPR * i));
            uq[j][i] = *reinterpret_cast<const uint4 *>(a.su + (int64_t)r * H + 8 * (cp + LPR * i));
        }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        float ga[MAXM], ua[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) { ga[m] = 0.f; ua[m] = 0.f; }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t g4[4] = {gq[j][i].x, gq[j][i].y, gq[j][i].z, gq[j][i].w};
            const uint32_t u4[4] = {uq[j][i].x, uq[j][i].y, uq[j][i].z, uq[j][i].w};
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, xr[i][m][v]);
                    ga[m] = dot2_bf16(__builtin_bit_cast(bf16x2_t, g4[v]), xv, ga[m]);
                    ua[m] = dot2_bf16(__builtin_bit_cast(bf16x2_t, u4[v]), xv, ua[m]);
                }
        }
        const int r = row0 + (wv * NR + j) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float g = row_sum<LPR>(ga[m]), u = row_sum<LPR>(ua[m]);
            if (m < tk.n && cp == 0 && r < Is) hs[(int64_t)tk.tok[m] * Is + r] = silu_mul(g, u);
        }
    }
}

// Expert ai (0 <= ai < k) of a one-token call, in selection order.  With a.sel_logits the calling wave selects
// the token's experts from its E logits itself (every lane gets the same result): k rounds of a wave-wide maximum
// of the selection keys, the order moe_route's selection defines.  With `write` the wave also writes the routing
// outputs of the call: topk_idx, the softmax over the selected logits (binary64, summed in selection order, as
// moe_route computes it), the expert offsets, the permutation and the active list.  Without a.sel_logits the
// routing is already in topk_idx.
__device__ __forceinline__ int one_token_expert(const FfnArgs &a, int ai, bool write) {
    if (!a.sel_logits) return a.topk_idx[min(ai, a.k - 1)];
    const int lane = threadIdx.x & 63, E = a.E, k = a.k;
    write = write && (threadIdx.x >> 6) == 0;                // one wave writes
    unsigned long long kk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        kk[i] = e < E ? logit_key(a.sel_logits[e], e) : 0ull;
    }
    int mine = 0, sel[SEL_MAXK];
#pragma unroll
    for (int j = 0; j < SEL_MAXK; ++j) {
        sel[j] = 0;
        if (j < k) {
            const unsigned long long m1 = kk[0] > kk[1] ? kk[0] : kk[1];
            const unsigned long long m2 = kk[2] > kk[3] ? kk[2] : kk[3];
            const unsigned long long m = wave_max_u64(m1 > m2 ? m1 : m2);
            sel[j] = key_expert(m);
            if (j == ai) mine = sel[j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kk[i] == m) kk[i] = 0ull;                       // keys are distinct: one owner
        }
    }
    if (write) {
        double ex[SEL_MAXK], den = 0.0;
        const double l0 = (double)a.sel_logits[sel[0]];
#pragma unroll
        for (int j = 0; j < SEL_MAXK; ++j) {
            ex[j] = 0.0;
            if (j < k) {
                ex[j] = exp((double)a.sel_logits[sel[j]] - l0);
                den += ex[j];
            }
        }
        // lane j < k: slot j = (token 0, rank j); its place among the selected experts in ascending order
        int rank = 0, my_e = 0;
        double my_ex = 0.0;
#pragma unroll
        for (int j = 0; j < SEL_MAXK; ++j) {
            if (j < k && j == lane) { my_e = sel[j]; my_ex = ex[j]; }
        }
#pragma unroll
        for (int j = 0; j < SEL_MAXK; ++j) rank += (j < k && sel[j] < my_e) ? 1 : 0;
        if (lane < k) {
            a.sel_idx[lane] = my_e;
            a.sel_w[lane] = (float)(my_ex / den);
            a.sel_perm[rank] = lane;
            a.sel_active[1 + rank] = my_e;
        }
        if (lane == 0) a.sel_active[0] = k;
        for (int e = lane; e <= E; e += 64) {
            int c = 0;
#pragma unroll
            for (int j = 0; j < SEL_MAXK; ++j) c += (j < k && sel[j] < e) ? 1 : 0;
            a.sel_offsets[e] = c;
        }
    }
    return mine;
}

template <int MAXM>
__device__ __forceinline__ bool routed_tokens(const FfnArgs &a, int ai, int &e, Tokens<MAXM> &tk,
                                              bool writer = false) {
    if (a.T == 1) {                              // one token: expert ai in selection order, slot ai
        if (ai >= a.k) return false;
        e = one_token_expert(a, ai, writer);
        tk.n = 1;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            tk.slot[m] = ai;
            tk.tok[m] = 0;
        }
        return true;
    }
    if (ai >= a.active[0]) return false;
    e = a.active[1 + ai];
    const int o0 = a.offsets[e];
    tk.n = min(a.offsets[e + 1] - o0, MAXM);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int s = a.perm[o0 + (m < tk.n ? m : 0)];
        tk.slot[m] = s;
        tk.tok[m] = s / a.k;
    }
    return true;
}

template <int MAXM> __device__ __forceinline__ void all_tokens(const FfnArgs &a, Tokens<MAXM> &tk) {
    tk.n = min(a.T, MAXM);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        tk.tok[m] = m < tk.n ? m : 0;
        tk.slot[m] = tk.tok[m];
    }
}

// ---------------------------------------------------------------------------
// iq2x gate/up on the matrix cores (T <= 4 tokens per expert).
//
// gfx950's v_mfma_f32_16x16x128_f8f6f4 with mixed operand formats: B = the
// weights in fp4 (E2M1), A = the activations in fp8 (E4M3).  Codebook
// magnitudes 1, 2, 3 and their signs are exact E2M1 codes, so an 8-weight
// sub-group is two 4-byte LDS lookups and an OR (codebook row as eight fp4
// codes, 7-bit sign index spread onto the code sign bits with the parity
// sign), fed to the instruction with no conversion.  Activations are split
// into two e4m3 pieces per 32-value group, hi = e4m3(x') and lo =
// e4m3(x' - hi) with x' = x * 2^s, 2^s the power of two that brings the
// group's max|x| into [128, 256); for |x'| >= 2^-2 the two pieces hold all
// eight significant bits of the bf16 value, and the group's sums pick up 2^-s
// with the weight scales.
//
// Operand layouts of the instruction (one 128-wide K step, lane = 16 g + i):
//   B (fp4): lane holds column i, K 32g .. 32g+31 (nibble j of register p = K 32g + 8p + j);
//   A (fp8): lane holds row i, K 16g .. 16g+15 (bytes 0..15) and 64 + 16g .. 64 + 16g + 15 (bytes 16..31);
//   D:       lane holds column i, rows 4g .. 4g+3.
// Lane (n, q) (n = lane % 16, q = lane / 16) decodes row n; in every
// 256-weight block it takes 16-byte chunk q (groups q and q + 4), and K step
// h (h = 0, 1: block columns 128h .. 128h+127) pairs its group q + 4h with
// B lane group q.  The pieces of token t sit in A row 4q' + 2t + p (p: 0 hi,
// 1 lo, t < 2 per product), non-zero only for K in group q' of the step, so
// group q' of every row lands in D rows 4q' .. 4q'+3 -- held by the lanes
// that own that group's 4-bit scale.  Each step is a fresh product, added to
// the lane's running sums times (2s+1) * d * 2^-s(x); the A operands depend
// on the tokens only, so they are built once and serve every row.
// A workgroup of H/512 waves takes one expert and MF_RB*16 rows, wave w the
// K slice [512w, 512w+512); the slices and quarters are summed in LDS.
// ---------------------------------------------------------------------------
constexpr int MF_KW = 512;
constexpr int MF_RB = 2;
constexpr int MF_MAXH = 4096;

typedef __attribute__((ext_vector_type(4))) float mf_acc_t;
typedef __attribute__((ext_vector_type(8))) int mf_ab_t;

// D = A (fp8 e4m3, 32 bytes per lane) x B (fp4 e2m1, 16 bytes per lane), unscaled
__device__ __forceinline__ mf_acc_t mfma_f8f4(const mf_ab_t &a, uint4 b) {
    const mf_ab_t bb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const mf_acc_t zero = {};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, zero, 0, 4, 0, 0, 0, 0);
}

// Activation pieces of one token: thread tid converts x[8 tid .. 8 tid + 7]
// (bf16 pairs in xv) into e4m3 hi and lo pieces at xhi/xlo[8 tid ..]; the four
// threads of a 32-value group share the scale 2^-s, stored at xsc[tid / 4].
__device__ __forceinline__ float x_to_pieces(uint4 xv, int tid, uint8_t *xhi, uint8_t *xlo, float *xsc) {
    const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(w4[k] << 16)), fabsf(__uint_as_float(w4[k] & 0xFFFF0000u))));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    const int sh = mx > 0.f ? 7 - ilogbf(mx) : 0;
    if ((tid & 3) == 0) xsc[tid >> 2] = ldexpf(1.f, -sh);
    uint32_t hi2[2], lo2[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float v0 = ldexpf(__uint_as_float(w4[k] << 16), sh);
        const float v1 = ldexpf(__uint_as_float(w4[k] & 0xFFFF0000u), sh);
        const uint32_t hp = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        const float r0 = v0 - __builtin_amdgcn_cvt_f32_fp8(hp, 0);
        const float r1 = v1 - __builtin_amdgcn_cvt_f32_fp8(hp, 1);
        const uint32_t lp = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
        if (k & 1) { hi2[k >> 1] |= (hp & 0xFFFFu) << 16; lo2[k >> 1] |= (lp & 0xFFFFu) << 16; }
        else { hi2[k >> 1] = hp & 0xFFFFu; lo2[k >> 1] = lp & 0xFFFFu; }
    }
    *reinterpret_cast<uint2 *>(xhi + 8 * tid) = make_uint2(hi2[0], hi2[1]);
    *reinterpret_cast<uint2 *>(xlo + 8 * tid) = make_uint2(lo2[0], lo2[1]);
    return mx;                                                // the group's largest |x|
}

// Largest |x| of a token over the workgroup: each wave's maximum into xmx[wave]; read back after a barrier.
__device__ __forceinline__ void wave_max_to(float mx, float *xmx) {
    mx = wave_max_f32(mx);
    if ((threadIdx.x & 63) == 0) xmx[threadIdx.x >> 6] = mx;
}

__device__ __forceinline__ int sigma_from(const float *xmx, int nw) {
    float mx = 0.f;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, xmx[w]);
    return h_sigma(mx);
}

// active: the active-expert list, read-only here; with uniform indices it is
// read through the scalar cache, whose wait counter is separate from the
// weight loads in flight.  The expert's slots come from topk_idx (T*k <= 64
// entries, one per lane), requested before the weights and used at the end.
template <int MAXM>
__device__ __forceinline__ void routed_gateup_mfma(const FfnArgs &a, const int32_t *__restrict__ active, int ai,
                                                   int row0,
                                                   _Float16 *__restrict__ h, uint32_t *cb4, uint32_t *sgn,
                                                   uint8_t (*xq)[2][MF_MAXH], float (*xsc)[MF_MAXH / 32], float *red,
                                                   float (*xmx)[MF_MAXH / MF_KW]) {
    constexpr int NP = (MAXM + 1) / 2;                       // products per K step (two tokens each)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const int H = a.H, I = a.I;
    const int k0w = wv * MF_KW;
    // --- expert id (scalar); slot experts, codebook rows and activations are
    // requested by every wave (unconditional loads, clamped indices) before
    // any wave requests weights, and the tables and activation pieces are
    // built while the weights stream in.
    // one token (MAXM == 1): expert ai in selection order (selected here from the logits when the launch
    // routes), slot ai; several tokens: the ai-th active expert, slots found by a ballot at the end
    const int n_active = MAXM == 1 ? a.k : active[0];
    const int n_slots = a.T * a.k;
    const int sel_raw = MAXM == 1 ? 0 : a.topk_idx[min(lane, n_slots - 1)];
    uint2 cbrow[4];                                          // rows tid + i * blockDim (blockDim >= 64)
#pragma unroll
    for (int i = 0; i < 4; ++i) cbrow[i] = reinterpret_cast<const uint2 *>(a.codebook)[min(tid + i * (int)blockDim.x, 255)];
    uint4 xv[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
        xv[m] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + (int64_t)min(m, a.T - 1) * H + 8 * tid);
    __builtin_amdgcn_sched_barrier(0);
    const int e = min(max(MAXM == 1 ? one_token_expert(a, ai, ai == 0 && row0 == 0) : active[1 + ai], 0), a.E - 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // whole workgroup, fewer experts than launched: leave before the weight requests (their address waits for
    // the same scalar load as this count)
    if (ai >= n_active) return;
    // --- all weights of this wave: units u = (row block u / 2, K block u % 2)
    const int64_t nb_row = H / MOE_QK, nb_mat = (int64_t)I * nb_row, NB = nb_mat * a.E;
    uint4 wq[2 * MF_RB][2];                                  // [unit][matrix]: chunk qd of the block
    uint32_t wd[2 * MF_RB];                                   // fp16 block scales of gate | up << 16
#pragma unroll
    for (int u = 0; u < 2 * MF_RB; ++u) {
        const int r = min(row0 + 16 * (u >> 1) + n, I - 1);
        const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (k0w >> 8) + (u & 1);
        wq[u][0] = reinterpret_cast<const uint4 *>(a.gate + bl * 64)[qd];
        wq[u][1] = reinterpret_cast<const uint4 *>(a.up + bl * 64)[qd];
        wd[u] = (uint32_t)reinterpret_cast<const uint16_t *>(a.gate + NB * 64)[bl] |
                ((uint32_t)reinterpret_cast<const uint16_t *>(a.up + NB * 64)[bl] << 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int sel = lane < n_slots ? sel_raw : -1;           // slot `lane`'s expert
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = tid + i * (int)blockDim.x;
        if (row < 256) cb4[row] = cbrow_fp4(cbrow[i].x, cbrow[i].y);
        if (row < 256) sgn[row] = sign_spread(row & 0x7F);   // indexed by a field's whole high byte
    }
    // --- activation pieces of every token of the call: thread tid converts
    // x[t][8 tid .. 8 tid + 7]; the four threads of a 32-value group share 2^s
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        if (m >= a.T) {                                      // no token: zero scale, pieces never read
            if ((tid & 3) == 0) xsc[m][tid >> 2] = 0.f;
            continue;
        }
        wave_max_to(x_to_pieces(xv[m], tid, xq[m][0], xq[m][1], xsc[m]), xmx[m]);
    }
    // --- every token of the call is multiplied (the products hold MAXM
    // tokens whichever are routed here); the expert's own tokens are picked
    // in the epilogue, so no routing load waits behind the weight stream.
    const int nt = min(a.T, MAXM);
    __syncthreads();
    // --- A operands [K block][K step][product]: A row n = 4 qa + 2 t + p holds
    // token (2 pr + t), piece p, for the K values of group qa of the step; this
    // lane holds 16 of them when lane group qd covers half of that group.
    const int qa = n >> 2, at0 = (n >> 1) & 1, ap = n & 1;
    const bool arow = (qd >> 1) == (qa & 1);
    mf_ab_t A[2][2][NP];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
        const int tt = min(2 * pr + at0, MAXM - 1);
        const bool val = arow && 2 * pr + at0 < nt;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (val) v = *reinterpret_cast<const uint4 *>(&xq[tt][ap][k0w + 256 * b + 128 * hs + 32 * qa + 16 * (qd & 1)]);
                const uint4 lo = qa < 2 ? v : make_uint4(0u, 0u, 0u, 0u), hi = qa < 2 ? make_uint4(0u, 0u, 0u, 0u) : v;
                A[b][hs][pr] = mf_ab_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
    }
    float tot[2][MAXM];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int m = 0; m < MAXM; ++m) tot[f][m] = 0.f;
#pragma unroll
    for (int u = 0; u < 2 * MF_RB; ++u) {
        const int b = u & 1;
        const float dsc[2] = {f16_bits_to_f32(wd[u] & 0xFFFFu), f16_bits_to_f32(wd[u] >> 16)};
        // all four products of the unit first (K steps hs = 0, 1: this lane's
        // groups qd and qd + 4), then their scales, so that no scale waits
        // on the product just issued
        mf_acc_t acc[2][2][NP];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const uint4 c = wq[u][f];
                const uint32_t lo = hs ? c.z : c.x, hi = hs ? c.w : c.y;
                uint4 bw;
                bw.x = cb4[lo & 0xFFu] | sgn[(lo >> 8) & 0xFFu];
                bw.y = cb4[(lo >> 16) & 0xFFu] | sgn[lo >> 24];
                bw.z = cb4[hi & 0xFFu] | sgn[(hi >> 8) & 0xFFu];
                bw.w = cb4[(hi >> 16) & 0xFFu] | sgn[hi >> 24];
#pragma unroll
                for (int pr = 0; pr < NP; ++pr) acc[hs][f][pr] = mfma_f8f4(A[b][hs][pr], bw);
            }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int g = (k0w + 256 * b) / 32 + qd + 4 * hs;       // this lane's group
            float xs[MAXM];
#pragma unroll
            for (int m = 0; m < MAXM; ++m) xs[m] = xsc[m][g];          // zero for tokens past T
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const uint4 c = wq[u][f];
                const uint32_t lo = hs ? c.z : c.x, hi = hs ? c.w : c.y;
                const float S = dsc[f] * (float)iq2x_gscale(lo, hi);
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    const mf_acc_t &d = acc[hs][f][m >> 1];
                    const float v = (m & 1) ? d[2] + d[3] : d[0] + d[1];
                    tot[f][m] = __fmaf_rn(S * xs[m], v, tot[f][m]);
                }
            }
        }
        if (b == 1) {                                                 // row block done: sum the quarters, to LDS
            const int rb = u >> 1;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    float v = tot[f][m];
                    v += __shfl_xor(v, 16, 64);
                    v += __shfl_xor(v, 32, 64);
                    if (qd == 0) red[(((wv * MF_RB + rb) * 2 + f) * MAXM + m) * 16 + n] = v;
                    tot[f][m] = 0.f;
                }
        }
    }
    __syncthreads();
    // --- token m's slot for this expert: m*k + j where topk_idx[m][j] == e (at most one j); one token: slot ai
    const uint64_t hit = MAXM == 1 ? (1ull << ai) : __ballot(sel == e);
    const uint64_t kmask = a.k >= 64 ? ~0ull : (1ull << a.k) - 1ull;
    for (int i = tid; i < MF_RB * MAXM * 16; i += blockDim.x) {
        const int nn = i & 15, m = (i >> 4) % MAXM, rb = (i >> 4) / MAXM;
        const int r = row0 + 16 * rb + nn;
        const uint64_t hm = m < a.T ? (hit >> (m * a.k)) & kmask : 0ull;
        if (hm == 0ull || r >= I) continue;
        const int sl = m * a.k + (__builtin_ffsll((long long)hm) - 1);
        float g = 0.f, u = 0.f;
        for (int w = 0; w < nw; ++w) {
            g += red[(((w * MF_RB + rb) * 2 + 0) * MAXM + m) * 16 + nn];
            u += red[(((w * MF_RB + rb) * 2 + 1) * MAXM + m) * 16 + nn];
        }
        h[(int64_t)sl * I + r] = (_Float16)ldexpf(silu_mul(g, u), -sigma_from(xmx[m], nw));
    }
    if (row0 == 0 && tid < nt) a.hsig[tid] = sigma_from(xmx[tid], nw);
}

// ---------------------------------------------------------------------------
// Several tokens per call (2 <= T <= MT_MAX, T*k <= 64: the speculative
// verifier's micro-batch).  Every selected expert is still read once per call,
// but a workgroup multiplies only the tokens routed to its expert, found from
// topk_idx by a ballot, two per pass (one product per K step, as for one
// token); experts with more tokens take more passes over the weights already
// in registers.  The shared rows loop over the tokens the same way, so register
// use does not grow with T.
// ---------------------------------------------------------------------------
// Makes a register value opaque to the optimizer (an empty asm that "modifies" it), so that work derived from
// weights held across a token loop is redone per token instead of being hoisted out of the loop, which would
// hold every decoded weight in registers at once.
__device__ __forceinline__ void opaque(uint32_t &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint4 &v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

constexpr int MT_MAX = 8;

__device__ __forceinline__ void routed_gateup_mt(const FfnArgs &a, const int32_t *__restrict__ active, int ai,
                                                 int row0, _Float16 *__restrict__ h, uint32_t *cb4, uint32_t *sgn,
                                                 uint8_t (*xq)[2][MF_MAXH], float (*xsc)[MF_MAXH / 32],
                                                 float *red, float (*xmx)[MF_MAXH / MF_KW]) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const int H = a.H, I = a.I;
    const int k0w = wv * MF_KW;
    const int n_active = active[0];
    const int e = min(max(active[1 + ai], 0), a.E - 1);
    const int n_slots = a.T * a.k;
    const int sel_raw = a.topk_idx[min(lane, n_slots - 1)];
    uint2 cbrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cbrow[i] = reinterpret_cast<const uint2 *>(a.codebook)[min(tid + i * (int)blockDim.x, 255)];
    // this expert's slots, ascending (so its tokens ascending; at most one slot per token).  They are
    // resolved before the weights are requested, so that the first pass's activations are requested ahead
    // of the weights and arrive first.
    uint64_t rest = __ballot(lane < n_slots && sel_raw == e);
    const uint16_t *xb = static_cast<const uint16_t *>(a.x);
    int s0 = rest ? __builtin_ffsll((long long)rest) - 1 : 0;
    int s1 = -1;
    {
        const uint64_t r1 = rest & (rest - 1);
        if (r1) s1 = __builtin_ffsll((long long)r1) - 1;
    }
    const uint4 xv0 = *reinterpret_cast<const uint4 *>(xb + (int64_t)(s0 / a.k) * H + 8 * tid);
    const uint4 xv1 = *reinterpret_cast<const uint4 *>(xb + (int64_t)((s1 >= 0 ? s1 : s0) / a.k) * H + 8 * tid);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (ai >= n_active) return;                               // whole workgroup, before the weight requests
    const int64_t nb_row = H / MOE_QK, nb_mat = (int64_t)I * nb_row, NB = nb_mat * a.E;
    uint4 wq[2 * MF_RB][2];
    uint32_t wd[2 * MF_RB];
#pragma unroll
    for (int u = 0; u < 2 * MF_RB; ++u) {
        const int r = min(row0 + 16 * (u >> 1) + n, I - 1);
        const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (k0w >> 8) + (u & 1);
        wq[u][0] = reinterpret_cast<const uint4 *>(a.gate + bl * 64)[qd];
        wq[u][1] = reinterpret_cast<const uint4 *>(a.up + bl * 64)[qd];
        wd[u] = (uint32_t)reinterpret_cast<const uint16_t *>(a.gate + NB * 64)[bl] |
                ((uint32_t)reinterpret_cast<const uint16_t *>(a.up + NB * 64)[bl] << 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = tid + i * (int)blockDim.x;
        if (row < 256) cb4[row] = cbrow_fp4(cbrow[i].x, cbrow[i].y);
        if (row < 256) sgn[row] = sign_spread(row & 0x7F);
    }
    wave_max_to(x_to_pieces(xv0, tid, xq[0][0], xq[0][1], xsc[0]), xmx[0]);
    if (s1 >= 0) wave_max_to(x_to_pieces(xv1, tid, xq[1][0], xq[1][1], xsc[1]), xmx[1]);
    else if ((tid & 3) == 0) xsc[1][tid >> 2] = 0.f;
    const int qa = n >> 2, at = (n >> 1) & 1, ap = n & 1;
    const bool arow = (qd >> 1) == (qa & 1);
    bool first = true;
    while (rest) {                                            // uniform: one pass per two tokens
#pragma unroll
        for (int u = 0; u < 2 * MF_RB; ++u) {
            opaque(wq[u][0]);
            opaque(wq[u][1]);
            opaque(wd[u]);
        }
        s0 = __builtin_ffsll((long long)rest) - 1;
        rest &= rest - 1;
        s1 = rest ? __builtin_ffsll((long long)rest) - 1 : -1;
        if (rest) rest &= rest - 1;
        // pieces of the pass's tokens: token s0 / k in position 0, s1 / k (or nothing) in position 1 (the
        // first pass's were made above, while the weights streamed in)
        if (!first) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(xb + (int64_t)(s0 / a.k) * H + 8 * tid);
            wave_max_to(x_to_pieces(v0, tid, xq[0][0], xq[0][1], xsc[0]), xmx[0]);
            if (s1 >= 0) {
                const uint4 v1 = *reinterpret_cast<const uint4 *>(xb + (int64_t)(s1 / a.k) * H + 8 * tid);
                wave_max_to(x_to_pieces(v1, tid, xq[1][0], xq[1][1], xsc[1]), xmx[1]);
            } else if ((tid & 3) == 0) {
                xsc[1][tid >> 2] = 0.f;
            }
        }
        first = false;
        __syncthreads();
        // A operands [K block][K step]: row n = 4 qa + 2 at + ap holds position at, piece ap
        const bool val = arow && (at == 0 || s1 >= 0);
        mf_ab_t A[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (val) v = *reinterpret_cast<const uint4 *>(&xq[at][ap][k0w + 256 * b + 128 * hs + 32 * qa + 16 * (qd & 1)]);
                const uint4 lo = qa < 2 ? v : make_uint4(0u, 0u, 0u, 0u), hi = qa < 2 ? make_uint4(0u, 0u, 0u, 0u) : v;
                A[b][hs] = mf_ab_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
        float tot[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
        for (int u = 0; u < 2 * MF_RB; ++u) {
            const int b = u & 1;
            const float dsc[2] = {f16_bits_to_f32(wd[u] & 0xFFFFu), f16_bits_to_f32(wd[u] >> 16)};
            mf_acc_t acc[2][2];
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const uint4 c = wq[u][f];
                    const uint32_t lo = hs ? c.z : c.x, hi = hs ? c.w : c.y;
                    uint4 bw;
                    bw.x = cb4[lo & 0xFFu] | sgn[(lo >> 8) & 0xFFu];
                    bw.y = cb4[(lo >> 16) & 0xFFu] | sgn[lo >> 24];
                    bw.z = cb4[hi & 0xFFu] | sgn[(hi >> 8) & 0xFFu];
                    bw.w = cb4[(hi >> 16) & 0xFFu] | sgn[hi >> 24];
                    acc[hs][f] = mfma_f8f4(A[b][hs], bw);
                }
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const int g = (k0w + 256 * b) / 32 + qd + 4 * hs;
                const float xs[2] = {xsc[0][g], xsc[1][g]};
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const uint4 c = wq[u][f];
                    const uint32_t lo = hs ? c.z : c.x, hi = hs ? c.w : c.y;
                    const float S = dsc[f] * (float)iq2x_gscale(lo, hi);
                    const mf_acc_t &d = acc[hs][f];
                    tot[f][0] = __fmaf_rn(S * xs[0], d[0] + d[1], tot[f][0]);
                    tot[f][1] = __fmaf_rn(S * xs[1], d[2] + d[3], tot[f][1]);
                }
            }
            if (b == 1) {
                const int rb = u >> 1;
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        float v = tot[f][m];
                        v += __shfl_xor(v, 16, 64);
                        v += __shfl_xor(v, 32, 64);
                        if (qd == 0) red[(((wv * MF_RB + rb) * 2 + f) * 2 + m) * 16 + n] = v;
                        tot[f][m] = 0.f;
                    }
            }
        }
        __syncthreads();
        for (int i = tid; i < MF_RB * 2 * 16; i += blockDim.x) {
            const int nn = i & 15, m = (i >> 4) & 1, rb = i >> 5;
            const int r = row0 + 16 * rb + nn, sl = m ? s1 : s0;
            if (sl < 0 || r >= I) continue;
            float g = 0.f, u = 0.f;
            for (int w = 0; w < nw; ++w) {
                g += red[(((w * MF_RB + rb) * 2 + 0) * 2 + m) * 16 + nn];
                u += red[(((w * MF_RB + rb) * 2 + 1) * 2 + m) * 16 + nn];
            }
            h[(int64_t)sl * I + r] = (_Float16)ldexpf(silu_mul(g, u), -sigma_from(xmx[m], nw));
        }
        if (row0 == 0 && tid < 2 && (tid == 0 || s1 >= 0)) a.hsig[(tid ? s1 : s0) / a.k] = sigma_from(xmx[tid], nw);
        __syncthreads();                                       // LDS pieces and sums are reused by the next pass
    }
}

// Shared gate/up rows on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) for
// every token of the call: A = the tokens' activations (rows; rows past T are
// zero), B = 16 weight rows.  Lane 16 g + i supplies the same 8 consecutive K
// values of A row i and of B column i, so the instruction's own K order inside
// a step does not matter.  A workgroup takes 16 rows; wave w the K slice
// [512 w, 512 w + 512) in four quarters of four steps; the slices are summed in
// LDS and SwiGLU is applied per (token, row).
typedef __attribute__((ext_vector_type(8))) __bf16 mf_bf16x8_t;

__device__ __forceinline__ mf_acc_t mfma_bf16(uint4 a, uint4 b, mf_acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8_t, a),
                                                   __builtin_bit_cast(mf_bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ void shared_gateup_mfma(const FfnArgs &a, int row0, float *__restrict__ hs,
                                                   float *red /* LDS [waves][2][16][16] */) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const int H = a.H, Is = a.Is, T = a.T;
    const int r = min(row0 + n, Is - 1);
    const uint16_t *wg = a.sg + (int64_t)r * H, *wu = a.su + (int64_t)r * H;
    const bool tok = n < T;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x) + (int64_t)min(n, T - 1) * H;
    mf_acc_t accg = {}, accu = {};
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
        uint4 bg[4], bu[4], av[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int k = wv * 512 + 128 * qt + 32 * st + 8 * g4;
            bg[st] = *reinterpret_cast<const uint4 *>(wg + k);
            bu[st] = *reinterpret_cast<const uint4 *>(wu + k);
            av[st] = tok ? *reinterpret_cast<const uint4 *>(xr + k) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            accg = mfma_bf16(av[st], bg[st], accg);
            accu = mfma_bf16(av[st], bu[st], accu);
        }
    }
    // D: lane (g4, n) holds row row0 + n for tokens 4 g4 .. 4 g4 + 3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * g4 + j;
        if (t < T) {
            red[((wv * 2 + 0) * 16 + t) * 16 + n] = accg[j];
            red[((wv * 2 + 1) * 16 + t) * 16 + n] = accu[j];
        }
    }
    __syncthreads();
    for (int i = tid; i < T * 16; i += blockDim.x) {
        const int t = i >> 4, nn = i & 15, rr = row0 + nn;
        if (rr >= Is) continue;
        float g = 0.f, u = 0.f;
        for (int w = 0; w < nw; ++w) {
            g += red[((w * 2 + 0) * 16 + t) * 16 + nn];
            u += red[((w * 2 + 1) * 16 + t) * 16 + nn];
        }
        hs[(int64_t)t * Is + rr] = silu_mul(g, u);
    }
}

// Shared workgroups first (16 rows each, the longest work items), then the routed ones.  Four waves per SIMD
// (at most 128 VGPRs) matter more here than the two registers the bound spills.
__global__ __launch_bounds__(512, 4) void k_gemv_gateup_mt(FfnArgs a, const int32_t *__restrict__ active,
                                                         int wgs_per_expert, int n_shared_wgs,
                                                         _Float16 *__restrict__ h, float *__restrict__ hs) {
    __shared__ uint32_t cb4[256], sgn[256];
    __shared__ __attribute__((aligned(16))) uint8_t xq[2][2][MF_MAXH];     // shared rows: their slice sums
    __shared__ float xsc[2][MF_MAXH / 32];
    __shared__ float red[(MF_MAXH / MF_KW) * MF_RB * 2 * 2 * 16];
    __shared__ float xmx[2][MF_MAXH / MF_KW];
    static_assert(sizeof(xq) >= (MF_MAXH / MF_KW) * 2 * 16 * 16 * sizeof(float), "shared slice sums");
    const int bid = blockIdx.x;
    if (bid < n_shared_wgs) {
        shared_gateup_mfma(a, bid * 16, hs, reinterpret_cast<float *>(&xq[0][0][0]));
    } else {
        const int rb = bid - n_shared_wgs;
        routed_gateup_mt(a, active, rb / wgs_per_expert, (rb % wgs_per_expert) * (16 * MF_RB), h, cb4, sgn, xq, xsc,
                         red, xmx);
    }
}

// Routed iq2x rows on the matrix cores, shared bf16 rows as in k_gemv_gateup.
template <int SLPR, int SCPL, int MAXM>
__global__ __launch_bounds__(512) void k_gemv_gateup_mfma(FfnArgs a, const int32_t *__restrict__ active,
                                                           int wgs_per_expert, int n_routed_wgs,
                                                           _Float16 *__restrict__ h, float *__restrict__ hs) {
    __shared__ uint32_t cb4[256], sgn[256];
    __shared__ __attribute__((aligned(16))) uint8_t xq[MAXM][2][MF_MAXH];
    __shared__ float xsc[MAXM][MF_MAXH / 32];
    __shared__ float red[(MF_MAXH / MF_KW) * MF_RB * 2 * MAXM * 16];
    __shared__ float xmx[MAXM][MF_MAXH / MF_KW];
    const int bid = blockIdx.x;
    if (bid < n_routed_wgs) {
        const int ai = bid / wgs_per_expert;
        routed_gateup_mfma<MAXM>(a, active, ai, (bid % wgs_per_expert) * (16 * MF_RB), h, cb4, sgn, xq, xsc, red,
                                 xmx);
    } else {
        Tokens<MAXM> tk;
        all_tokens<MAXM>(a, tk);
        constexpr int SNR = shared_nr<SCPL>();
        const int rows = (int)(blockDim.x >> 6) * SNR * (64 / SLPR);
        shared_gateup<SLPR, SCPL, MAXM, SNR>(a, tk, (bid - n_routed_wgs) * rows, hs);
    }
}

// FG: routed gate/up format (iq2x or q4k); LPR, CPL describe its routed rows.
template <int FG, int LPR, int CPL, int SLPR, int SCPL, int MAXM, int NR>
__global__ __launch_bounds__(256) void k_gemv_gateup(FfnArgs a, int wgs_per_expert, int n_routed_wgs,
                                                      _Float16 *__restrict__ h, float *__restrict__ hs) {
    __shared__ uint32_t cb4[256], sgn[128];
    const int bid = blockIdx.x;
    if (bid < n_routed_wgs) {
        if constexpr (FG == FMT_IQ2X) {
            tables(a.codebook, cb4, sgn);
            __syncthreads();
        }
        int e;
        Tokens<MAXM> tk;
        if (!routed_tokens<MAXM>(a, bid / wgs_per_expert, e, tk, bid == 0)) return;
        constexpr int ROWS = WAVES * NR * (64 / LPR);
        if constexpr (FG == FMT_Q4K) routed_gateup_q4k<LPR, CPL, MAXM, NR>(a, e, tk, (bid % wgs_per_expert) * ROWS, h);
        else routed_gateup<LPR, CPL, MAXM, NR>(a, e, tk, (bid % wgs_per_expert) * ROWS, cb4, sgn, h);
    } else {
        Tokens<MAXM> tk;
        all_tokens<MAXM>(a, tk);
        constexpr int SNR = shared_nr<SCPL>();
        constexpr int ROWS = WAVES * SNR * (64 / SLPR);
        shared_gateup<SLPR, SCPL, MAXM, SNR>(a, tk, (bid - n_routed_wgs) * ROWS, hs);
    }
}

// ---------------------------------------------------------------------------
// down projection
// ---------------------------------------------------------------------------
// q2k chunk (16 B = sub-blocks 4c..4c+3, 64 weights) against fp16 h pairs.
template <int MAXM>
__device__ __forceinline__ void q2k_chunk(uint4 q, uint32_t sm4, uint32_t dd, const uint32_t (&hr)[MAXM][32],
                                          const float (&hsum)[MAXM][4], float (&acc)[MAXM]) {
    float sacc[MAXM], macc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) { sacc[m] = 0.f; macc[m] = 0.f; }
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const uint32_t lo = qw[jj] & 0x33333333u, hi = (qw[jj] >> 2) & 0x33333333u;
        const f16x2_t w0 = fp4x2_f16<0>(lo), w1 = fp4x2_f16<1>(lo), w2 = fp4x2_f16<2>(lo), w3 = fp4x2_f16<3>(lo);
        const f16x2_t w4 = fp4x2_f16<0>(hi), w5 = fp4x2_f16<1>(hi), w6 = fp4x2_f16<2>(hi), w7 = fp4x2_f16<3>(hi);
        const float sc = (float)((sm4 >> (8 * jj)) & 15u), mn = (float)((sm4 >> (8 * jj + 4)) & 15u);
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const uint32_t *hp = &hr[m][8 * jj];
            float p = 0.f;
            p = dot2_f16(w0, __builtin_bit_cast(f16x2_t, hp[0]), p);
            p = dot2_f16(w1, __builtin_bit_cast(f16x2_t, hp[1]), p);
            p = dot2_f16(w2, __builtin_bit_cast(f16x2_t, hp[2]), p);
            p = dot2_f16(w3, __builtin_bit_cast(f16x2_t, hp[3]), p);
            p = dot2_f16(w4, __builtin_bit_cast(f16x2_t, hp[4]), p);
            p = dot2_f16(w5, __builtin_bit_cast(f16x2_t, hp[5]), p);
            p = dot2_f16(w6, __builtin_bit_cast(f16x2_t, hp[6]), p);
            p = dot2_f16(w7, __builtin_bit_cast(f16x2_t, hp[7]), p);
            sacc[m] = __fmaf_rn(sc, p, sacc[m]);
            macc[m] = __fmaf_rn(mn, hsum[m][jj], macc[m]);
        }
    }
    const float d2 = 2.0f * f16_bits_to_f32(dd & 0xFFFFu), dmin = f16_bits_to_f32(dd >> 16);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] += d2 * sacc[m] - dmin * macc[m];
}

// Loads this lane's 64 h values of chunk ch (f16) in the order q2k_chunk uses:
// sub-block jj pairs: (i, i+1) for i = 0,2,4,6 then (8+i, 9+i).
template <int MAXM>
__device__ __forceinline__ void load_h_chunk(const _Float16 *h, int I, const Tokens<MAXM> &tk, int ch,
                                             uint32_t (&hr)[MAXM][32], float (&hsum)[MAXM][4]) {
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const int s = tk.slot[m < tk.n ? m : 0];
        const uint4 *hp = reinterpret_cast<const uint4 *>(h + (int64_t)s * I + 64 * ch);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const uint4 u = hp[v];
            hr[m][4 * v + 0] = u.x; hr[m][4 * v + 1] = u.y; hr[m][4 * v + 2] = u.z; hr[m][4 * v + 3] = u.w;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const f16x2_t p = __builtin_bit_cast(f16x2_t, hr[m][8 * jj + v]);
                sum += (float)p.x + (float)p.y;
            }
            hsum[m][jj] = sum;
        }
    }
}

template <int LPR, int CPL, int MAXM, int NR>
__device__ void routed_down(const FfnArgs &a, int e, const Tokens<MAXM> &tk, int row0, const _Float16 *__restrict__ h) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, I = a.I;
    const int64_t nb_row = I / MOE_QK, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
    int sig[MAXM];                                            // h of token t was stored as h * 2^-sig[t]
#pragma unroll
    for (int m = 0; m < MAXM; ++m) sig[m] = a.hsig[tk.tok[m < tk.n ? m : 0]];
    uint32_t hr[CPL][MAXM][32];
    float hsum[CPL][MAXM][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i) load_h_chunk<MAXM>(h, I, tk, cp + LPR * i, hr[i], hsum[i]);
    const uint8_t *Q = a.down;
    const uint8_t *S = a.down + NB * 64;
    const uint32_t *D = reinterpret_cast<const uint32_t *>(a.down + NB * 80);
    uint4 q[NR][CPL];
    uint32_t sm[NR][CPL], dd[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, H - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = cp + LPR * i;
            const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (ch >> 2);
            q[j][i] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + (ch & 3) * 16);
            sm[j][i] = *reinterpret_cast<const uint32_t *>(S + bl * 16 + (ch & 3) * 4);
            dd[j][i] = D[bl];
        }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) q2k_chunk<MAXM>(q[j][i], sm[j][i], dd[j][i], hr[i], hsum[i], acc);
        const int r = row0 + (wv * NR + j) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float o = ldexpf(row_sum<LPR>(acc[m]), sig[m]);
            if (m < tk.n && cp == 0 && r < H) a.slot_out[(int64_t)tk.slot[m] * H + r] = o;
        }
    }
}

// q4k chunk against fp16 h pairs: codes enter as fp16 1024 + q (pattern
// 0x6400 | q), and  sum w h = d sc P - (1024 d sc + dmin m) S  per sub-block,
// S the sum of its 32 h values.
template <int MAXM>
__device__ __forceinline__ void q4k_chunk_f16(uint4 q, uint4 meta, int j, const uint32_t (&hr)[MAXM][16],
                                              const float (&hsum)[MAXM], float (&acc)[MAXM]) {
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    float P[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) P[m] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2_t t = __builtin_bit_cast(f16x2_t, ((qw[w] >> (4 * i)) & 0x000F000Fu) | 0x64006400u);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) P[m] = dot2_f16(t, __builtin_bit_cast(f16x2_t, hr[m][4 * w + i]), P[m]);
        }
    const float sc = f16_bits_to_f32(meta.x & 0xFFFFu) * (float)q4k_field(meta.y, meta.z, meta.w, j);
    const float off = __fmaf_rn(f16_bits_to_f32(meta.x >> 16), (float)q4k_field(meta.y, meta.z, meta.w, 8 + j),
                                1024.f * sc);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] += __fmaf_rn(sc, P[m], -off * hsum[m]);
}

// Routed q4k down: rows of I = 32*LPR*CPL, a lane covers chunks cp + LPR*i.
template <int LPR, int CPL, int MAXM, int NR>
__device__ void routed_down_q4k(const FfnArgs &a, int e, const Tokens<MAXM> &tk, int row0,
                                const _Float16 *__restrict__ h) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, I = a.I;
    const int64_t nb_row = I / MOE_QK, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
    int sig[MAXM];                                            // h of token t was stored as h * 2^-sig[t]
#pragma unroll
    for (int m = 0; m < MAXM; ++m) sig[m] = a.hsig[tk.tok[m < tk.n ? m : 0]];
    uint32_t hr[CPL][MAXM][16];
    float hsum[CPL][MAXM];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = cp + LPR * i;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int s = tk.slot[m < tk.n ? m : 0];
            const uint4 *hp = reinterpret_cast<const uint4 *>(h + (int64_t)s * I + 32 * ch);
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 u = hp[v];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    hr[i][m][4 * v + k] = w4[k];
                    const f16x2_t p = __builtin_bit_cast(f16x2_t, w4[k]);
                    sum += (float)p.x + (float)p.y;
                }
            }
            hsum[i][m] = sum;
        }
    }
    uint4 q[NR][CPL], mt[NR][CPL];
#pragma unroll
    for (int jr = 0; jr < NR; ++jr) {
        const int r = min(row0 + (wv * NR + jr) * RPI + rsub, H - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = cp + LPR * i;
            const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (ch >> 3);
            q[jr][i] = *reinterpret_cast<const uint4 *>(a.down + bl * 128 + (ch & 7) * 16);
            mt[jr][i] = *reinterpret_cast<const uint4 *>(a.down + NB * 128 + bl * 16);
        }
    }
#pragma unroll
    for (int jr = 0; jr < NR; ++jr) {
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) q4k_chunk_f16<MAXM>(q[jr][i], mt[jr][i], (cp + LPR * i) & 7, hr[i], hsum[i], acc);
        const int r = row0 + (wv * NR + jr) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float o = ldexpf(row_sum<LPR>(acc[m]), sig[m]);
            if (m < tk.n && cp == 0 && r < H) a.slot_out[(int64_t)tk.slot[m] * H + r] = o;
        }
    }
}

// Shared down: bf16 rows of Is = 8*LPR*CPL against fp32 h.
template <int LPR, int CPL, int MAXM, int NR>
__device__ void shared_down(const FfnArgs &a, const Tokens<MAXM> &tk, int row0, const float *__restrict__ hs) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, Is = a.Is;
    float hr[CPL][MAXM][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float4 *p = reinterpret_cast<const float4 *>(hs + (int64_t)tk.tok[m < tk.n ? m : 0] * Is +
                                                               8 * (cp + LPR * i));
            const float4 u = p[0], v = p[1];
            hr[i][m][0] = u.x; hr[i][m][1] = u.y; hr[i][m][2] = u.z; hr[i][m][3] = u.w;
            hr[i][m][4] = v.x; hr[i][m][5] = v.y; hr[i][m][6] = v.z; hr[i][m][7] = v.w;
        }
    uint4 q[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, H - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            q[j][i] = *reinterpret_cast<const uint4 *>(a.sd + (int64_t)r * Is + 8 * (cp + LPR * i));
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        float acc[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t w4[4] = {q[j][i].x, q[j][i].y, q[j][i].z, q[j][i].w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float wl = __uint_as_float(w4[v] << 16), wh = __uint_as_float(w4[v] & 0xFFFF0000u);
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    acc[m] = __fmaf_rn(wl, hr[i][m][2 * v], acc[m]);
                    acc[m] = __fmaf_rn(wh, hr[i][m][2 * v + 1], acc[m]);
                }
            }
        }
        const int r = row0 + (wv * NR + j) * RPI + rsub;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float o = row_sum<LPR>(acc[m]);
            if (m < tk.n && cp == 0 && r < H) a.shared_out[(int64_t)tk.tok[m] * H + r] = o;
        }
    }
}

// FD: routed down format (q2k or q4k); LPR, CPL describe its routed rows.
template <int FD, int LPR, int CPL, int SLPR, int SCPL, int MAXM, int NR>
__global__ __launch_bounds__(256) void k_gemv_down(FfnArgs a, int wgs_per_expert, int n_routed_wgs,
                                                    const _Float16 *__restrict__ h, const float *__restrict__ hs) {
    const int bid = blockIdx.x;
    if (bid < n_routed_wgs) {
        int e;
        Tokens<MAXM> tk;
        if (!routed_tokens<MAXM>(a, bid / wgs_per_expert, e, tk)) return;
        constexpr int ROWS = WAVES * NR * (64 / LPR);
        if constexpr (FD == FMT_Q4K) routed_down_q4k<LPR, CPL, MAXM, NR>(a, e, tk, (bid % wgs_per_expert) * ROWS, h);
        else routed_down<LPR, CPL, MAXM, NR>(a, e, tk, (bid % wgs_per_expert) * ROWS, h);
    } else {
        Tokens<MAXM> tk;
        all_tokens<MAXM>(a, tk);
        constexpr int SNR = shared_nr_down<SCPL, MAXM>();
        constexpr int ROWS = WAVES * SNR * (64 / SLPR);
        shared_down<SLPR, SCPL, MAXM, SNR>(a, tk, (bid - n_routed_wgs) * ROWS, hs);
    }
}

// Several tokens per call: the expert's rows stay in registers and its tokens
// (from the permutation) are taken one at a time; the shared rows loop over
// every token of the call the same way.
// NR rows of one routed expert (decoded weights q, sm, dd) against one slot's h.
template <int LPR, int CPL, int NR>
__device__ __forceinline__ void down_rows_one(const FfnArgs &a, const uint4 (&q)[NR][CPL],
                                              const uint32_t (&sm)[NR][CPL], const uint32_t (&dd)[NR][CPL],
                                              const uint32_t (&hr)[CPL][1][32], const float (&hsum)[CPL][1][4],
                                              int slot, int sig, int row0) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        float acc[1] = {0.f};
#pragma unroll
        for (int i = 0; i < CPL; ++i) q2k_chunk<1>(q[j][i], sm[j][i], dd[j][i], hr[i], hsum[i], acc);
        const float o = ldexpf(row_sum<LPR>(acc[0]), sig);
        const int r = row0 + (wv * NR + j) * RPI + rsub;
        if (cp == 0 && r < a.H) a.slot_out[(int64_t)slot * a.H + r] = o;
    }
}

template <int LPR, int CPL, int NR>
__device__ void routed_down_mt(const FfnArgs &a, int e, int o0, int ne, int row0, const _Float16 *__restrict__ h) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, I = a.I;
    const int64_t nb_row = I / MOE_QK, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
    // the first token's h is requested ahead of the weights, so that it arrives first
    Tokens<1> tk;
    tk.n = 1;
    tk.slot[0] = a.perm[o0];
    tk.tok[0] = tk.slot[0] / a.k;
    uint32_t hr[CPL][1][32];
    float hsum[CPL][1][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i) load_h_chunk<1>(h, I, tk, cp + LPR * i, hr[i], hsum[i]);
    const uint8_t *Q = a.down;
    const uint8_t *S = a.down + NB * 64;
    const uint32_t *D = reinterpret_cast<const uint32_t *>(a.down + NB * 80);
    uint4 q[NR][CPL];
    uint32_t sm[NR][CPL], dd[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, H - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = cp + LPR * i;
            const int64_t bl = (int64_t)e * nb_mat + (int64_t)r * nb_row + (ch >> 2);
            q[j][i] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + (ch & 3) * 16);
            sm[j][i] = *reinterpret_cast<const uint32_t *>(S + bl * 16 + (ch & 3) * 4);
            dd[j][i] = D[bl];
        }
    }
    down_rows_one<LPR, CPL, NR>(a, q, sm, dd, hr, hsum, tk.slot[0], a.hsig[tk.tok[0]], row0);
#pragma unroll 1
    for (int m = 1; m < ne; ++m) {
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                opaque(q[j][i]);
                opaque(sm[j][i]);
                opaque(dd[j][i]);
            }
        Tokens<1> tm;
        tm.n = 1;
        tm.slot[0] = a.perm[o0 + m];
        tm.tok[0] = tm.slot[0] / a.k;
        uint32_t hm[CPL][1][32];
        float sm_h[CPL][1][4];
#pragma unroll
        for (int i = 0; i < CPL; ++i) load_h_chunk<1>(h, I, tm, cp + LPR * i, hm[i], sm_h[i]);
        down_rows_one<LPR, CPL, NR>(a, q, sm, dd, hm, sm_h, tm.slot[0], a.hsig[tm.tok[0]], row0);
    }
}

template <int LPR, int CPL, int NR>
__device__ void shared_down_mt(const FfnArgs &a, int row0, const float *__restrict__ hs) {
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cp = lane % LPR, rsub = lane / LPR;
    const int H = a.H, Is = a.Is;
    uint4 q[NR][CPL];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int r = min(row0 + (wv * NR + j) * RPI + rsub, H - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            q[j][i] = *reinterpret_cast<const uint4 *>(a.sd + (int64_t)r * Is + 8 * (cp + LPR * i));
    }
#pragma unroll 1
    for (int t = 0; t < a.T; ++t) {
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i) opaque(q[j][i]);
        float hr[CPL][8];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const float4 *p = reinterpret_cast<const float4 *>(hs + (int64_t)t * Is + 8 * (cp + LPR * i));
            const float4 u = p[0], v = p[1];
            hr[i][0] = u.x; hr[i][1] = u.y; hr[i][2] = u.z; hr[i][3] = u.w;
            hr[i][4] = v.x; hr[i][5] = v.y; hr[i][6] = v.z; hr[i][7] = v.w;
        }
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t w4[4] = {q[j][i].x, q[j][i].y, q[j][i].z, q[j][i].w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc = __fmaf_rn(__uint_as_float(w4[v] << 16), hr[i][2 * v], acc);
                    acc = __fmaf_rn(__uint_as_float(w4[v] & 0xFFFF0000u), hr[i][2 * v + 1], acc);
                }
            }
            const float o = row_sum<LPR>(acc);
            const int r = row0 + (wv * NR + j) * RPI + rsub;
            if (cp == 0 && r < H) a.shared_out[(int64_t)t * H + r] = o;
        }
    }
}

template <int LPR, int CPL, int SLPR, int SCPL, int NR, int SNR>
__global__ __launch_bounds__(256) void k_gemv_down_mt(FfnArgs a, int wgs_per_expert, int n_routed_wgs,
                                                       const _Float16 *__restrict__ h, const float *__restrict__ hs) {
    const int bid = blockIdx.x;
    if (bid < n_routed_wgs) {
        const int ai = bid / wgs_per_expert;
        if (ai >= a.active[0]) return;
        const int e = a.active[1 + ai];
        const int o0 = a.offsets[e];
        constexpr int ROWS = WAVES * NR * (64 / LPR);
        routed_down_mt<LPR, CPL, NR>(a, e, o0, a.offsets[e + 1] - o0, (bid % wgs_per_expert) * ROWS, h);
    } else {
        constexpr int ROWS = WAVES * SNR * (64 / SLPR);
        shared_down_mt<SLPR, SCPL, SNR>(a, (bid - n_routed_wgs) * ROWS, hs);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// (lanes per row, chunks per lane) for a row of `len` elements in chunks of `per_chunk`.
bool split(int len, int per_chunk, int max_cpl, int &lpr, int &cpl) {
    if (len % per_chunk) return false;
    const int nch = len / per_chunk;
    if (nch <= 64) {
        if (64 % nch) return false;
        lpr = nch; cpl = 1;
        return nch >= 2;
    }
    if (nch % 64) return false;
    lpr = 64; cpl = nch / 64;
    return cpl <= max_cpl;
}

constexpr int NR = 4;

template <int FG, int MAXM, int LPR, int CPL, int SLPR, int SCPL>
hipError_t run_gateup(const FfnArgs &a, int max_active, _Float16 *h, float *hs, hipStream_t st) {
    // one q4k token over two chunks per lane: 3 rows per wave keep the kernel at 3 waves per SIMD
    constexpr int NRG = (FG == FMT_Q4K && CPL == 2 && MAXM == 1) ? 3 : NR;
    const int rows = WAVES * NRG * (64 / LPR);
    const int wpe = (a.I + rows - 1) / rows;
    const int nr = max_active * wpe;
    int ns = 0;
    if (a.Is > 0) {
        const int srows = WAVES * shared_nr<SCPL>() * (64 / SLPR);
        ns = (a.Is + srows - 1) / srows;
    }
    hipLaunchKernelGGL((k_gemv_gateup<FG, LPR, CPL, SLPR, SCPL, MAXM, NRG>), dim3(nr + ns), dim3(256), 0, st, a, wpe, nr,
                       h, hs);
    return hipGetLastError();
}

template <int MAXM, int SLPR, int SCPL>
hipError_t run_gateup_mfma(const FfnArgs &a, int max_active, _Float16 *h, float *hs, hipStream_t st) {
    const int threads = a.H / 8;                                  // H/512 waves
    const int wpe = a.I / (16 * MF_RB);
    const int nr = max_active * wpe;
    int ns = 0;
    if (a.Is > 0) {
        const int srows = (threads / 64) * shared_nr<SCPL>() * (64 / SLPR);
        ns = (a.Is + srows - 1) / srows;
    }
    hipLaunchKernelGGL((k_gemv_gateup_mfma<SLPR, SCPL, MAXM>), dim3(nr + ns), dim3(threads), 0, st, a, a.active,
                       wpe, nr, h, hs);
    return hipGetLastError();
}

bool gateup_mfma_ok(const FfnArgs &a) {
    return a.fmt_gu == FMT_IQ2X && a.H % MF_KW == 0 && a.H >= MF_KW && a.H <= MF_MAXH && a.I % (16 * MF_RB) == 0 &&
           a.T * a.k <= 64;
}

template <int FD, int MAXM, int LPR, int CPL, int SLPR, int SCPL>
hipError_t run_down(const FfnArgs &a, int max_active, const _Float16 *h, const float *hs, hipStream_t st) {
    constexpr int NRD = nr_down<MAXM>();
    const int rows = WAVES * NRD * (64 / LPR);
    const int wpe = (a.H + rows - 1) / rows;
    const int nr = max_active * wpe;
    int ns = 0;
    if (a.Is > 0) {
        const int srows = WAVES * shared_nr_down<SCPL, MAXM>() * (64 / SLPR);
        ns = (a.H + srows - 1) / srows;
    }
    hipLaunchKernelGGL((k_gemv_down<FD, LPR, CPL, SLPR, SCPL, MAXM, NRD>), dim3(nr + ns), dim3(256), 0, st, a, wpe,
                       nr, h, hs);
    return hipGetLastError();
}

hipError_t run_gateup_mt(const FfnArgs &a, int max_active, _Float16 *h, float *hs, hipStream_t st) {
    const int threads = a.H / 8;                                  // H/512 waves, one 512-wide K slice each
    const int wpe = a.I / (16 * MF_RB);
    const int nr = max_active * wpe;
    const int ns = (a.Is + 15) / 16;
    hipLaunchKernelGGL(k_gemv_gateup_mt, dim3(nr + ns), dim3(threads), 0, st, a, a.active, wpe, ns, h, hs);
    return hipGetLastError();
}

template <int LPR, int SLPR, int SCPL>
hipError_t run_down_mt(const FfnArgs &a, int max_active, const _Float16 *h, const float *hs, hipStream_t st) {
    constexpr int NRD = nr_down<1>(), SNR = shared_nr_down<SCPL, 1>();
    const int rows = WAVES * NRD * (64 / LPR);
    const int wpe = (a.H + rows - 1) / rows;
    const int nr = max_active * wpe;
    int ns = 0;
    if (a.Is > 0) {
        const int srows = WAVES * SNR * (64 / SLPR);
        ns = (a.H + srows - 1) / srows;
    }
    hipLaunchKernelGGL((k_gemv_down_mt<LPR, 1, SLPR, SCPL, NRD, SNR>), dim3(nr + ns), dim3(256), 0, st, a, wpe, nr, h,
                       hs);
    return hipGetLastError();
}

// iq2x gate/up and q2k down, a shared expert of the routed size or none, 2 <= T <= MT_MAX, T*k <= 64
bool mt_ok(const FfnArgs &a) {
    return a.T >= 2 && a.T <= MT_MAX && a.fmt_d == FMT_Q2K && gateup_mfma_ok(a) && (a.Is == a.I || a.Is == 0);
}

hipError_t dispatch_mt(const FfnArgs &a, _Float16 *h, float *hs, hipStream_t st) {
    const int max_active = min(a.T * a.k, a.E);
    hipError_t e = hipErrorInvalidValue;
    if (a.stages & STAGE_GATE_UP) {
        e = run_gateup_mt(a, max_active, h, hs, st);
        if (e != hipSuccess) return e;
    }
    if (!(a.stages & STAGE_DOWN)) return hipSuccess;
    if (a.I == 2048) return run_down_mt<32, 64, 4>(a, max_active, h, hs, st);
    if (a.I == 1024) return run_down_mt<16, 64, 2>(a, max_active, h, hs, st);
    if (a.I == 512) return run_down_mt<8, 64, 1>(a, max_active, h, hs, st);
    if (a.I == 256) return run_down_mt<4, 32, 1>(a, max_active, h, hs, st);
    return hipErrorInvalidValue;
}

template <int MAXM>
hipError_t dispatch(const FfnArgs &a, _Float16 *h, float *hs, hipStream_t st) {
    const int max_active = min(a.T * a.k, a.E);
    hipError_t e = hipErrorInvalidValue;
    if (a.stages & STAGE_GATE_UP) {
        // routed rows of H (iq2x: 64 weights per lane chunk, q4k: 32), shared rows of H (8 per chunk)
#define MOE_GU(H_, LPR2_, CPL2_, LPR4_, CPL4_, SCPL_)                                                        \
    if (a.H == H_) {                                                                                          \
        if (a.fmt_gu == FMT_Q4K) e = run_gateup<FMT_Q4K, MAXM, LPR4_, CPL4_, 64, SCPL_>(a, max_active, h, hs, st); \
        else if (gateup_mfma_ok(a)) e = run_gateup_mfma<MAXM, 64, SCPL_>(a, max_active, h, hs, st);          \
        else e = run_gateup<FMT_IQ2X, MAXM, LPR2_, CPL2_, 64, SCPL_>(a, max_active, h, hs, st);             \
    }
        MOE_GU(4096, 64, 1, 64, 2, 8)
        MOE_GU(2048, 32, 1, 64, 1, 4)
        MOE_GU(1024, 16, 1, 32, 1, 2)
        MOE_GU(512, 8, 1, 16, 1, 1)
#undef MOE_GU
        if (e != hipSuccess) return e;
    }
    if (!(a.stages & STAGE_DOWN)) return hipSuccess;
    // down: routed rows of I (q2k: 64 weights per lane chunk, q4k: 32), shared rows of Is (8 per chunk)
    const int Is = a.Is > 0 ? a.Is : a.I;
#define MOE_DOWN(I_, LPR2_, LPR4_, SI_, SLPR_, SCPL_)                                                         \
    if (a.I == I_ && Is == SI_) {                                                                             \
        if (a.fmt_d == FMT_Q4K) return run_down<FMT_Q4K, MAXM, LPR4_, 1, SLPR_, SCPL_>(a, max_active, h, hs, st); \
        return run_down<FMT_Q2K, MAXM, LPR2_, 1, SLPR_, SCPL_>(a, max_active, h, hs, st);                   \
    }
    MOE_DOWN(2048, 32, 64, 2048, 64, 4)
    MOE_DOWN(1024, 16, 32, 1024, 64, 2)
    MOE_DOWN(512, 8, 16, 512, 64, 1)
    MOE_DOWN(256, 4, 8, 256, 32, 1)
    MOE_DOWN(2048, 32, 64, 1024, 64, 2)
    MOE_DOWN(1024, 16, 32, 2048, 64, 4)
#undef MOE_DOWN
    return hipErrorInvalidValue;
}

}  // namespace

namespace moe {

bool ffn_gemv_supported(const FfnArgs &a) {
    if (!a.x_bf16 || a.T > MT_MAX) return false;
    if (a.T > 4 && !mt_ok(a)) return false;
    if (a.fmt_gu != FMT_IQ2X && a.fmt_gu != FMT_Q4K) return false;
    if (a.fmt_d != FMT_Q2K && a.fmt_d != FMT_Q4K) return false;
    if (!(a.H == 4096 || a.H == 2048 || a.H == 1024 || a.H == 512)) return false;
    const int Is = a.Is > 0 ? a.Is : a.I;
    const int pairs[6][2] = {{2048, 2048}, {1024, 1024}, {512, 512}, {256, 256}, {2048, 1024}, {1024, 2048}};
    for (auto &p : pairs)
        if (a.I == p[0] && Is == p[1]) return true;
    return false;
}

// workspace: h [T*k][I] fp16 | hs [T][Is] fp32 | hsig [T] int32, each 256-byte aligned
static size_t gemv_h_bytes(int I, int k, int T) { return ((size_t)T * k * I * sizeof(_Float16) + 255) / 256 * 256; }
static size_t gemv_hs_bytes(int Is, int T) { return ((size_t)T * Is * sizeof(float) + 255) / 256 * 256; }

size_t ffn_workspace_gemv(int H, int I, int E, int k, int Is, int T) {
    (void)H; (void)E;
    return gemv_h_bytes(I, k, T) + gemv_hs_bytes(Is, T) + ((size_t)T * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_ffn_gemv(const FfnArgs &args, hipStream_t st) {
    FfnArgs a = args;
    char *ws = static_cast<char *>(a.ws);
    _Float16 *h = reinterpret_cast<_Float16 *>(ws);
    float *hs = reinterpret_cast<float *>(ws + gemv_h_bytes(a.I, a.k, a.T));
    a.hsig = reinterpret_cast<int32_t *>(ws + gemv_h_bytes(a.I, a.k, a.T) + gemv_hs_bytes(a.Is, a.T));
    if (a.T == 1) return dispatch<1>(a, h, hs, st);
    if (mt_ok(a)) return dispatch_mt(a, h, hs, st);
    return dispatch<4>(a, h, hs, st);
}

}  // namespace moe
