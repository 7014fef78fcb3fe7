// Grouped-GEMM expert FFN for many tokens per expert (prefill).
//
// Tokens are grouped by expert through the permutation (expert_offsets /
// perm); a work item is (expert, tile of 256 weight rows, tile of 64 of the
// expert's tokens).  Per item the matrix cores compute D[token][row] with
// v_mfma_f32_32x32x16: A = activations (64 tokens x 256-wide K block, staged in
// LDS), B = weights decoded in registers straight from the 16-byte lane loads.
//
// Exactness: the decoded B values are small integers, exact in fp16 --
// iq2x: sign * C * (2s+1) <= 93 (fp4 convert, then a packed fp16 multiply);
// q2k: sc * q <= 45.  The fp16 block scale d is applied by keeping each
// accumulator in units of the current block's d: before block b it is
// multiplied by d_{b-1}/d_b, after the last block by d_last.  q2k's mins use a
// second accumulator over per-16 sums of h (A = sums split into fp16 hi + lo,
// B = the 4-bit mins), scaled the same way by dmin.  The shared expert runs in
// the same launches with bf16 operands (x as is; h kept as bf16 hi + lo).
//
// Activations: the routed gate/up GEMM takes x converted to fp16 (exact for
// 2^-14 <= |x| <= 65504; smaller magnitudes round to fp16 subnormals); h is
// written in fp16.
//
// Work mapping: workgroups are dealt round-robin to the 8 XCDs; items are
// renumbered so that each XCD gets a contiguous run of items, and items are
// ordered (expert, row tile, token tile): the workgroups that share an
// expert's activation tile or weight tile run together on one XCD and share
// its L2.
#include "common.h"
#include "internal.h"

using namespace moe;

namespace {

constexpr int TOK = 64;          // tokens per tile (2 MFMA A fragments of 32)
constexpr int ROWS = 256;        // weight rows per workgroup (4 waves x 64)
constexpr int KB = 256;          // K per block (one quant block)
constexpr int XPITCH = KB + 8;   // LDS row pitch in halves (breaks bank alignment)

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

struct GemmArgs {
    FfnArgs a;
    const _Float16 *x16;         // [T][H] fp16 copy of x
    _Float16 *h;                 // [T*k][I] SwiGLU output by permutation position
    uint16_t *hs_hi, *hs_lo;     // [T][Is] shared-expert SwiGLU output, bf16 hi + lo
};

__device__ __forceinline__ f32x16_t mfma_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// work items
// ---------------------------------------------------------------------------
struct Item {
    int shared;     // 0 routed, 1 shared expert
    int e;          // expert
    int r;          // row tile
    int p0;         // first permutation position (routed) or first token (shared)
    int n;          // valid tokens in the tile
};

// Per-expert token-tile offsets (exclusive scan of ceil(n_e / TOK)), by wave 0.
__device__ void tile_scan(const int32_t *offsets, int E, int *tile_off) {
    const int lane = threadIdx.x;
    if (lane < 64) {
        int c[4], s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = e < E ? (offsets[e + 1] - offsets[e] + TOK - 1) / TOK : 0;
            s += c[i];
        }
        int inc = s;
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(inc, o, 64);
            if (lane >= o) inc += u;
        }
        int pre = inc - s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e <= E) tile_off[e] = pre;
            pre += c[i];
        }
        if (lane == 63 && E == 256) tile_off[256] = inc;
    }
}

// Workgroup id -> item index: each XCD (ids dealt round-robin over 8) gets a
// contiguous range of item indices.
__device__ __forceinline__ int xcd_remap(int p, int G) {
    const int x = p & 7, slot = p >> 3, q = G >> 3, r = G & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
}

// rows: weight rows of the routed matrix (I for gate/up, H for down);
// srows: rows of the shared matrix (Is for gate/up, H for down).
__device__ bool get_item(const FfnArgs &a, int rows, int srows, int *tile_off, Item &it) {
    tile_scan(a.offsets, a.E, tile_off);
    __syncthreads();
    const int RT = rows / ROWS;
    const int NT = tile_off[a.E];
    const int routed = NT * RT;
    const int RS = a.Is > 0 ? srows / ROWS : 0;
    const int st_tiles = (a.T + TOK - 1) / TOK;
    const int G = routed + RS * st_tiles;
    if ((int)blockIdx.x >= G) return false;
    const int q = xcd_remap(blockIdx.x, G);
    if (q < routed) {
        const int tq = q / RT;                 // global token-tile index if row tiles were innermost
        // find expert: largest e with RT*tile_off[e] <= q
        int lo = 0, hi = a.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_off[mid] * RT <= q) lo = mid; else hi = mid - 1;
        }
        (void)tq;
        const int e = lo, nt = tile_off[e + 1] - tile_off[e];
        const int local = q - tile_off[e] * RT;
        const int r = local / nt, t = local % nt;
        const int n_e = a.offsets[e + 1] - a.offsets[e];
        it.shared = 0; it.e = e; it.r = r;
        it.p0 = a.offsets[e] + t * TOK;
        it.n = min(TOK, n_e - t * TOK);
    } else {
        const int local = q - routed;
        const int r = local / st_tiles, t = local % st_tiles;
        it.shared = 1; it.e = -1; it.r = r;
        it.p0 = t * TOK;
        it.n = min(TOK, a.T - t * TOK);
    }
    return true;
}

// ---------------------------------------------------------------------------
// A-tile staging: 64 rows x 256 halves of K block kb into LDS (row pitch XPITCH)
// src_row[m] = pointer to the start of row m (or nullptr: zeros)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_rows(const uint16_t *const *src_row, int kb, uint16_t *lds) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + tid;
        const int m = idx >> 5, c = idx & 31;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        const uint16_t *s = src_row[m];
        if (s) v = *reinterpret_cast<const uint4 *>(s + (int64_t)kb * KB + 8 * c);
        *reinterpret_cast<uint4 *>(lds + m * XPITCH + 8 * c) = v;
    }
}

__device__ __forceinline__ f16x8_t lds_frag16(const uint16_t *lds, int m, int col) {
    return *reinterpret_cast<const f16x8_t *>(lds + m * XPITCH + col);
}
__device__ __forceinline__ bf16x8_t lds_fragbf(const uint16_t *lds, int m, int col) {
    return *reinterpret_cast<const bf16x8_t *>(lds + m * XPITCH + col);
}

// eight fp4 codes (word) -> eight fp16 values times the packed fp16 pair mul
__device__ __forceinline__ f16x8_t fp4x8_f16_mul(uint32_t word, f16x2_t mul) {
    f16x2_t p0 = fp4x2_f16<0>(word) * mul, p1 = fp4x2_f16<1>(word) * mul;
    f16x2_t p2 = fp4x2_f16<2>(word) * mul, p3 = fp4x2_f16<3>(word) * mul;
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// q2k codes (value q/2) -> q * sc: scale 2.0 is a power of two, applied exactly by the convert
__device__ __forceinline__ f16x8_t q2k_f16_mul(uint32_t codes, f16x2_t sc2) {
    f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 0) * sc2;
    f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 1) * sc2;
    f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 2) * sc2;
    f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 3) * sc2;
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ void scale_acc(f32x16_t &acc, float s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= s;
}

// D layout of v_mfma_f32_32x32x16: lane l holds column l % 32 and rows
// 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
__device__ __forceinline__ int drow(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_gemm_gateup(GemmArgs g) {
    const FfnArgs &a = g.a;
    __shared__ int tile_off[257];
    __shared__ uint32_t cb4[256], sgn[128];
    __shared__ const uint16_t *src[TOK];
    __shared__ int dst[TOK];
    __shared__ __attribute__((aligned(16))) uint16_t xs[TOK * XPITCH];
    Item it;
    if (!get_item(a, a.I, a.Is, tile_off, it)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int H = a.H;
    if (!it.shared) {
        for (int i = tid; i < 256; i += 256) cb4[i] = codebook_row_fp4(a.codebook, i);
        for (int i = tid; i < 128; i += 256) sgn[i] = sign_spread(i);
    }
    if (tid < TOK) {
        const uint16_t *s = nullptr;
        int d = -1;
        if (tid < it.n) {
            if (!it.shared) {
                const int p = it.p0 + tid;
                s = reinterpret_cast<const uint16_t *>(g.x16) + (int64_t)(a.perm[p] / a.k) * H;
                d = p;
            } else {
                s = static_cast<const uint16_t *>(a.x) + (int64_t)(it.p0 + tid) * H;
                d = it.p0 + tid;
            }
        }
        src[tid] = s;
        dst[tid] = d;
    }
    __syncthreads();

    f32x16_t acc[2][4];          // [token frag][gate rt0, gate rt1, up rt0, up rt1]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    const int row_base = it.r * ROWS + wv * 64;          // this wave's 64 rows
    const int nkb = H / KB;

    if (!it.shared) {
        const int64_t nb_row = H / KB, nb_mat = (int64_t)a.I * nb_row, NB = nb_mat * a.E;
        const uint8_t *W[2] = {a.gate, a.up};
        float dprev[4] = {1.f, 1.f, 1.f, 1.f};
        for (int kb = 0; kb < nkb; ++kb) {
            // this lane's 32 bytes of fields for its 4 rows (chunks 2hh, 2hh+1) and the block scales
            uint4 q[4][2];
            float dcur[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int row = row_base + (f & 1) * 32 + n;
                const int64_t bl = (int64_t)it.e * nb_mat + (int64_t)row * nb_row + kb;
                const uint8_t *base = W[f >> 1] + bl * 64 + hh * 32;
                q[f][0] = *reinterpret_cast<const uint4 *>(base);
                q[f][1] = *reinterpret_cast<const uint4 *>(base + 16);
                dcur[f] = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(W[f >> 1] + NB * 64)[bl]);
            }
            __syncthreads();                                   // previous block's readers are done
            stage_rows(src, kb, xs);
            // rescale accumulators into units of this block's d (d == 0: the block adds nothing)
            bool zero[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                zero[f] = dcur[f] == 0.f;
                const float dn = zero[f] ? dprev[f] : dcur[f];
                const float s = dprev[f] / dn;
                scale_acc(acc[0][f], s);
                scale_acc(acc[1][f], s);
                dprev[f] = dn;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int chunk = j >> 3, fld = j & 7;                        // within this lane's 32 B
                const int grp = 2 * hh + chunk + 4 * (fld >> 2), p = fld & 3;
                const int col = 32 * grp + 8 * p;
                const f16x8_t a0 = lds_frag16(xs, n, col);
                const f16x8_t a1 = lds_frag16(xs, 32 + n, col);
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const uint4 qq = q[f][chunk];
                    const uint32_t lo = (fld >> 2) ? qq.z : qq.x, hi = (fld >> 2) ? qq.w : qq.y;
                    const uint32_t s = ((lo >> 15) & 1u) | ((lo >> 30) & 2u) | ((hi >> 13) & 4u) | ((hi >> 28) & 8u);
                    const _Float16 m1 = zero[f] ? (_Float16)0.0f : (_Float16)(float)(2 * s + 1);
                    const uint32_t fw = ((p < 2 ? lo : hi) >> (16 * (p & 1))) & 0xFFFFu;
                    const uint32_t word = cb4[fw & 0xFFu] | sgn[(fw >> 8) & 0x7Fu];
                    const f16x8_t b = fp4x8_f16_mul(word, f16x2_t{m1, m1});
                    acc[0][f] = mfma_f16(a0, b, acc[0][f]);
                    acc[1][f] = mfma_f16(a1, b, acc[1][f]);
                }
            }
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            scale_acc(acc[0][f], dprev[f]);
            scale_acc(acc[1][f], dprev[f]);
        }
        // SwiGLU epilogue: h[position][row] in fp16
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * tf + drow(v, lane);
                    const int d = dst[m];
                    if (d >= 0)
                        g.h[(int64_t)d * a.I + row_base + 32 * rt + n] =
                            (_Float16)silu_mul(acc[tf][rt][v], acc[tf][2 + rt][v]);
                }
    } else {
        const uint16_t *W[2] = {a.sg, a.su};
        for (int kb = 0; kb < nkb; ++kb) {
            __syncthreads();
            stage_rows(src, kb, xs);
            __syncthreads();
#pragma unroll 4
            for (int j = 0; j < 16; ++j) {
                const int col = 16 * j + 8 * hh;
                const bf16x8_t a0 = lds_fragbf(xs, n, col);
                const bf16x8_t a1 = lds_fragbf(xs, 32 + n, col);
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int row = row_base + (f & 1) * 32 + n;
                    const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(W[f >> 1] + (int64_t)row * H + kb * KB + col);
                    acc[0][f] = mfma_bf16(a0, b, acc[0][f]);
                    acc[1][f] = mfma_bf16(a1, b, acc[1][f]);
                }
            }
        }
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * tf + drow(v, lane);
                    const int d = dst[m];
                    if (d >= 0) {
                        const float hv = silu_mul(acc[tf][rt][v], acc[tf][2 + rt][v]);
                        const uint32_t hb = __float_as_uint(hv);
                        const uint32_t hi = (hb + 0x7FFFu + ((hb >> 16) & 1u)) >> 16;   // bf16, nearest even
                        const float rest = hv - __uint_as_float(hi << 16);
                        const uint32_t rb = __float_as_uint(rest);
                        const uint32_t lo = (rb + 0x7FFFu + ((rb >> 16) & 1u)) >> 16;
                        const int64_t o = (int64_t)d * a.Is + row_base + 32 * rt + n;
                        g.hs_hi[o] = (uint16_t)hi;
                        g.hs_lo[o] = (uint16_t)lo;
                    }
                }
    }
}

// ---------------------------------------------------------------------------
// down projection
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_gemm_down(GemmArgs g) {
    const FfnArgs &a = g.a;
    __shared__ int tile_off[257];
    __shared__ const uint16_t *src[TOK];
    __shared__ const uint16_t *src_lo[TOK];
    __shared__ int dst[TOK];
    __shared__ __attribute__((aligned(16))) uint16_t xs[TOK * XPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t xs2[TOK * XPITCH];      // shared: lo plane
    __shared__ __attribute__((aligned(16))) uint16_t hsum[2][TOK * 24];      // routed: per-16 sums, hi/lo
    Item it;
    if (!get_item(a, a.H, a.H, tile_off, it)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int I = a.I, H = a.H;
    if (tid < TOK) {
        const uint16_t *s = nullptr, *s2 = nullptr;
        int d = -1;
        if (tid < it.n) {
            if (!it.shared) {
                const int p = it.p0 + tid;
                s = reinterpret_cast<const uint16_t *>(g.h) + (int64_t)p * I;
                d = a.perm[p];                                   // output slot
            } else {
                s = g.hs_hi + (int64_t)(it.p0 + tid) * a.Is;
                s2 = g.hs_lo + (int64_t)(it.p0 + tid) * a.Is;
                d = it.p0 + tid;
            }
        }
        src[tid] = s;
        src_lo[tid] = s2;
        dst[tid] = d;
    }
    __syncthreads();

    const int row_base = it.r * ROWS + wv * 64;
    if (!it.shared) {
        f32x16_t acc[2][2], accm[2][2];      // [token frag][row tile]
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) { acc[i][j] = f32x16_t{}; accm[i][j] = f32x16_t{}; }
        const int64_t nb_row = I / KB, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
        const uint8_t *Q = a.down, *S = a.down + NB * 64;
        const uint32_t *D = reinterpret_cast<const uint32_t *>(a.down + NB * 80);
        float dprev[2] = {1.f, 1.f}, mprev[2] = {1.f, 1.f};
        const int nkb = I / KB;
        for (int kb = 0; kb < nkb; ++kb) {
            uint4 q[2][2];
            uint2 sm[2];
            float dcur[2], mcur[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int row = row_base + 32 * rt + n;
                const int64_t bl = (int64_t)it.e * nb_mat + (int64_t)row * nb_row + kb;
                q[rt][0] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + hh * 32);
                q[rt][1] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + hh * 32 + 16);
                sm[rt] = *reinterpret_cast<const uint2 *>(S + bl * 16 + hh * 8);
                const uint32_t dd = D[bl];
                dcur[rt] = f16_bits_to_f32(dd & 0xFFFFu);
                mcur[rt] = f16_bits_to_f32(dd >> 16);
            }
            __syncthreads();
            stage_rows(src, kb, xs);
            // per-16 sums of the staged h rows: 256 threads = 64 rows x 4 quarters of 64 columns
            {
                const int m = tid >> 2, qd = tid & 3;
                const uint16_t *row = src[m];
#pragma unroll
                for (int sbq = 0; sbq < 4; ++sbq) {
                    float s = 0.f;
                    if (row) {
                        const uint4 u0 = *reinterpret_cast<const uint4 *>(row + (int64_t)kb * KB + 64 * qd + 16 * sbq);
                        const uint4 u1 = *reinterpret_cast<const uint4 *>(row + (int64_t)kb * KB + 64 * qd + 16 * sbq + 8);
                        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const f16x2_t pr = __builtin_bit_cast(f16x2_t, w[i]);
                            s += (float)pr.x + (float)pr.y;
                        }
                    }
                    const _Float16 shi = (_Float16)s;
                    const _Float16 slo = (_Float16)(s - (float)shi);
                    hsum[0][m * 24 + 4 * qd + sbq] = __builtin_bit_cast(uint16_t, shi);
                    hsum[1][m * 24 + 4 * qd + sbq] = __builtin_bit_cast(uint16_t, slo);
                }
            }
            bool zq[2], zm[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                zq[rt] = dcur[rt] == 0.f;
                zm[rt] = mcur[rt] == 0.f;
                const float dn = zq[rt] ? dprev[rt] : dcur[rt];
                const float mn = zm[rt] ? mprev[rt] : mcur[rt];
                const float s1 = dprev[rt] / dn, s2 = mprev[rt] / mn;
                scale_acc(acc[0][rt], s1);
                scale_acc(acc[1][rt], s1);
                scale_acc(accm[0][rt], s2);
                scale_acc(accm[1][rt], s2);
                dprev[rt] = dn;
                mprev[rt] = mn;
            }
            __syncthreads();
            // main term: K-step j covers sub-block 8*hh + j/2, half j%2
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int sbl = j >> 1, half = j & 1;
                const int col = 16 * (8 * hh + sbl) + 8 * half;
                const f16x8_t a0 = lds_frag16(xs, n, col);
                const f16x8_t a1 = lds_frag16(xs, 32 + n, col);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const uint4 qq = q[rt][sbl >> 2];
                    const uint32_t dw = (sbl & 3) == 0 ? qq.x : ((sbl & 3) == 1 ? qq.y : ((sbl & 3) == 2 ? qq.z : qq.w));
                    const uint32_t codes = half ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u);
                    const uint32_t scb = (sbl < 4 ? sm[rt].x >> (8 * sbl) : sm[rt].y >> (8 * (sbl - 4))) & 15u;
                    const _Float16 sc = zq[rt] ? (_Float16)0.0f : (_Float16)(float)scb;
                    const f16x8_t b = q2k_f16_mul(codes, f16x2_t{sc, sc});
                    acc[0][rt] = mfma_f16(a0, b, acc[0][rt]);
                    acc[1][rt] = mfma_f16(a1, b, acc[1][rt]);
                }
            }
            // min term: K = the 16 sub-blocks; A = per-16 sums (hi, lo), B = mins
            {
                const f16x8_t ah0 = *reinterpret_cast<const f16x8_t *>(&hsum[0][n * 24 + 8 * hh]);
                const f16x8_t ah1 = *reinterpret_cast<const f16x8_t *>(&hsum[0][(32 + n) * 24 + 8 * hh]);
                const f16x8_t al0 = *reinterpret_cast<const f16x8_t *>(&hsum[1][n * 24 + 8 * hh]);
                const f16x8_t al1 = *reinterpret_cast<const f16x8_t *>(&hsum[1][(32 + n) * 24 + 8 * hh]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    f16x8_t b;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t byte = (i < 4 ? sm[rt].x >> (8 * i) : sm[rt].y >> (8 * (i - 4))) & 0xFFu;
                        b[i] = zm[rt] ? (_Float16)0.0f : (_Float16)(float)(byte >> 4);
                    }
                    accm[0][rt] = mfma_f16(ah0, b, accm[0][rt]);
                    accm[0][rt] = mfma_f16(al0, b, accm[0][rt]);
                    accm[1][rt] = mfma_f16(ah1, b, accm[1][rt]);
                    accm[1][rt] = mfma_f16(al1, b, accm[1][rt]);
                }
            }
        }
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * tf + drow(v, lane);
                    const int d = dst[m];
                    if (d >= 0)
                        a.slot_out[(int64_t)d * H + row_base + 32 * rt + n] =
                            acc[tf][rt][v] * dprev[rt] - accm[tf][rt][v] * mprev[rt];
                }
    } else {
        f32x16_t acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
        const int Is = a.Is, nkb = Is / KB;
        for (int kb = 0; kb < nkb; ++kb) {
            __syncthreads();
            stage_rows(src, kb, xs);
            stage_rows(src_lo, kb, xs2);
            __syncthreads();
#pragma unroll 4
            for (int j = 0; j < 16; ++j) {
                const int col = 16 * j + 8 * hh;
                const bf16x8_t h0 = lds_fragbf(xs, n, col), h1 = lds_fragbf(xs, 32 + n, col);
                const bf16x8_t l0 = lds_fragbf(xs2, n, col), l1 = lds_fragbf(xs2, 32 + n, col);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int row = row_base + 32 * rt + n;
                    const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(a.sd + (int64_t)row * Is + kb * KB + col);
                    acc[0][rt] = mfma_bf16(h0, b, acc[0][rt]);
                    acc[0][rt] = mfma_bf16(l0, b, acc[0][rt]);
                    acc[1][rt] = mfma_bf16(h1, b, acc[1][rt]);
                    acc[1][rt] = mfma_bf16(l1, b, acc[1][rt]);
                }
            }
        }
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = 32 * tf + drow(v, lane);
                    const int d = dst[m];
                    if (d >= 0) a.shared_out[(int64_t)d * H + row_base + 32 * rt + n] = acc[tf][rt][v];
                }
    }
}

// x (bf16) -> fp16 copy, 8 elements per thread
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t *__restrict__ x, _Float16 *__restrict__ y,
                                                  int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const uint4 v = reinterpret_cast<const uint4 *>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    f16x8_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = (_Float16)__uint_as_float(w[j] << 16);
        o[2 * j + 1] = (_Float16)__uint_as_float(w[j] & 0xFFFF0000u);
    }
    reinterpret_cast<f16x8_t *>(y)[i] = o;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct Layout {
    size_t x16, h, hs_hi, hs_lo, total;
};
Layout layout(int H, int I, int k, int Is, int T) {
    Layout L;
    L.x16 = 0;
    L.h = L.x16 + align256((size_t)T * H * 2);
    L.hs_hi = L.h + align256((size_t)T * k * I * 2);
    L.hs_lo = L.hs_hi + align256((size_t)T * Is * 2);
    L.total = L.hs_lo + align256((size_t)T * Is * 2);
    return L;
}

}  // namespace

namespace moe {

bool ffn_gemm_supported(const FfnArgs &a) {
    if (!a.x_bf16 || a.fmt_gu != FMT_IQ2X || a.fmt_d != FMT_Q2K) return false;
    if (a.H % 256 || a.I % 256 || (a.Is > 0 && a.Is % 256)) return false;
    if (a.E > 256) return false;
    return true;
}

size_t ffn_workspace_gemm(int H, int I, int E, int k, int Is, int T) {
    (void)E;
    return layout(H, I, k, Is, T).total + 256;
}

hipError_t launch_ffn_gemm(const FfnArgs &a, hipStream_t st) {
    const Layout L = layout(a.H, a.I, a.k, a.Is, a.T);
    GemmArgs g;
    g.a = a;
    char *ws = static_cast<char *>(a.ws);
    g.x16 = reinterpret_cast<const _Float16 *>(ws + L.x16);
    g.h = reinterpret_cast<_Float16 *>(ws + L.h);
    g.hs_hi = reinterpret_cast<uint16_t *>(ws + L.hs_hi);
    g.hs_lo = reinterpret_cast<uint16_t *>(ws + L.hs_lo);
    const int S = a.T * a.k;
    const int max_tiles = (S + TOK - 1) / TOK + (S < a.E ? S : a.E);   // sum_e ceil(n_e / TOK) bound
    const int st_tiles = (a.T + TOK - 1) / TOK;
    hipError_t e = hipSuccess;
    if (a.stages & STAGE_GATE_UP) {
        const int64_t n8 = (int64_t)a.T * a.H / 8;
        hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint16_t *>(a.x), const_cast<_Float16 *>(g.x16), n8);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int G = max_tiles * (a.I / ROWS) + (a.Is > 0 ? st_tiles * (a.Is / ROWS) : 0);
        hipLaunchKernelGGL(k_gemm_gateup, dim3(G), dim3(256), 0, st, g);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.stages & STAGE_DOWN) {
        const int G = max_tiles * (a.H / ROWS) + (a.Is > 0 ? st_tiles * (a.H / ROWS) : 0);
        hipLaunchKernelGGL(k_gemm_down, dim3(G), dim3(256), 0, st, g);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace moe
