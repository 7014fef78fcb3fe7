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
// Activations: the routed gate/up GEMM takes x converted to fp16 after a
// per-token power-of-two prescale, x16 = x * 2^-e(t) with e(t) = ilogb(max_c
// |x[t][c]|) - 1 (clamped to [-50, 50]), so every row's largest magnitude
// lies in [2, 4) and no finite bf16 row overflows fp16; the epilogue
// multiplies the gate and up sums by 2^e(t) before the SwiGLU (exact).  h is
// written in fp16 as h * 2^-2e(t), and the down projection multiplies its
// sums by 2^2e(t).
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
constexpr int ROWS = 256;        // weight rows per workgroup (8 waves x 32)
constexpr int NTHR = 512;        // threads per workgroup
constexpr int KB = 256;          // K per block (one quant block)

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

// Workgroup id -> item.  Workgroups are dealt round-robin to the 8 XCDs (id % 8);
// XCD x runs q_x = G/8 (+1) of them.  Each XCD first takes its even share of the
// S shared-expert items (the longest ones), then a contiguous run of routed items,
// so that workgroups sharing an expert's tiles sit on one XCD's L2.
struct XcdSplit {
    bool shared;
    int index;      // into the shared or the routed item list
};
__device__ __forceinline__ XcdSplit xcd_remap(int p, int G, int S) {
    const int x = p & 7, slot = p >> 3;
    const int gq = G >> 3, gr = G & 7, sq = S >> 3, sr = S & 7;
    const int s_x = sq + (x < sr ? 1 : 0);
    if (slot < s_x) return {true, (x < sr ? x * (sq + 1) : sr * (sq + 1) + (x - sr) * sq) + slot};
    const int pre_q = x < gr ? x * (gq + 1) : gr * (gq + 1) + (x - gr) * gq;
    const int pre_s = x < sr ? x * (sq + 1) : sr * (sq + 1) + (x - sr) * sq;
    return {false, pre_q - pre_s + (slot - s_x)};
}

// rows: weight rows of the routed matrix (I for gate/up, H for down), cut
// into items of rpi rows; srows: rows of the shared matrix (Is for gate/up, H
// for down), cut into items of ROWS rows.
__device__ bool get_item(const FfnArgs &a, int rows, int rpi, int srows, int *tile_off, Item &it) {
    tile_scan(a.offsets, a.E, tile_off);
    __syncthreads();
    const int RT = rows / rpi;
    const int NT = tile_off[a.E];
    const int routed = NT * RT;
    const int RS = a.Is > 0 ? srows / ROWS : 0;
    const int st_tiles = (a.T + TOK - 1) / TOK;
    const int S = RS * st_tiles;
    const int G = routed + S;
    if ((int)blockIdx.x >= G) return false;
    const XcdSplit xs = xcd_remap(blockIdx.x, G, S);
    if (!xs.shared) {
        const int q = xs.index;
        // find the expert: largest e with RT*tile_off[e] <= q
        int lo = 0, hi = a.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_off[mid] * RT <= q) lo = mid; else hi = mid - 1;
        }
        const int e = lo, nt = tile_off[e + 1] - tile_off[e];
        const int local = q - tile_off[e] * RT;
        const int r = local / nt, t = local % nt;
        const int n_e = a.offsets[e + 1] - a.offsets[e];
        it.shared = 0; it.e = e; it.r = r;
        it.p0 = a.offsets[e] + t * TOK;
        it.n = min(TOK, n_e - t * TOK);
    } else {
        const int local = xs.index;
        const int r = local / st_tiles, t = local % st_tiles;
        it.shared = 1; it.e = -1; it.r = r;
        it.p0 = t * TOK;
        it.n = min(TOK, a.T - t * TOK);
    }
    return true;
}

// ---------------------------------------------------------------------------
// A tiles in LDS: 64 rows x 256 16-bit values (32 chunks of 16 B per row),
// chunk c of row m stored at position c ^ (m & 15) so that the 32 lanes of a
// fragment read (rows 0..31, one chunk) hit distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tpos(int m, int c) { return m * 32 + (c ^ (m & 15)); }

// Tiles are staged through registers: x_fetch issues the global loads of a
// tile (4 x 16 B per thread, 32 consecutive threads per 512-byte row), the
// compute of the current tile runs, then x_store writes the registers to LDS.
template <int NV> struct XStageN {
    uint4 v[NV];                 // NV x 16 B per thread: the first 16 * NV rows of a tile
};
using XStage = XStageN<4>;

// Row pointers are read back from LDS, so the compiler cannot tell they point
// to global memory; loading through a flat pointer would tie the loads to the
// LDS wait counter.  Load through an explicit global pointer instead.
typedef __attribute__((address_space(1))) const u32x4_t gbl_u32x4;

__device__ __forceinline__ uint4 gload16(const uint16_t *p) {
    const u32x4_t v = *(gbl_u32x4 *)(reinterpret_cast<uintptr_t>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// src_row[m]: start of row m (rows past the tile's tokens alias row 0); k0: first column
template <int NV>
__device__ __forceinline__ void x_fetch(const uint16_t *const *src_row, int k0, XStageN<NV> &xs) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + NTHR * i, m = idx >> 5, c = idx & 31;
        xs.v[i] = gload16(src_row[m] + k0 + 8 * c);
    }
}

// 128-wide K stage of two planes: chunks 0..15 from hi, 16..31 from lo
__device__ __forceinline__ void x_fetch_hilo(const uint16_t *const *hi, const uint16_t *const *lo, int k0,
                                             XStage &xs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = threadIdx.x + NTHR * i, m = idx >> 5, c = idx & 31;
        const uint16_t *row = c < 16 ? hi[m] : lo[m];
        xs.v[i] = gload16(row + k0 + 8 * (c & 15));
    }
}

template <int NV> __device__ __forceinline__ void x_store(const XStageN<NV> &xs, uint4 *tile) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + NTHR * i, m = idx >> 5, c = idx & 31;
        tile[tpos(m, c)] = xs.v[i];
    }
}



__device__ __forceinline__ f16x8_t frag16(const uint4 *tile, int m, int c) {
    return __builtin_bit_cast(f16x8_t, tile[tpos(m, c)]);
}
__device__ __forceinline__ bf16x8_t fragbf(const uint4 *tile, int m, int c) {
    return __builtin_bit_cast(bf16x8_t, tile[tpos(m, c)]);
}

// eight fp4 codes (word) -> eight fp16 values times a packed fp16 pair
__device__ __forceinline__ f16x8_t fp4x8_f16_mul(uint32_t word, f16x2_t mul) {
    const f16x2_t p0 = fp4x2_f16<0>(word) * mul, p1 = fp4x2_f16<1>(word) * mul;
    const f16x2_t p2 = fp4x2_f16<2>(word) * mul, p3 = fp4x2_f16<3>(word) * mul;
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// q2k codes (value q/2) -> q * sc: the convert's scale 2.0 is a power of two, applied exactly
__device__ __forceinline__ f16x8_t q2k_f16_mul(uint32_t codes, f16x2_t sc2) {
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 0) * sc2;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 1) * sc2;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 2) * sc2;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 3) * sc2;
    return f16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ f16x2_t f16pair(uint32_t v) {
    const _Float16 h = (_Float16)(float)v;
    return f16x2_t{h, h};
}

__device__ __forceinline__ void scale_acc(f32x16_t &acc, float s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= s;
}

// New unit for an accumulator kept in units of the previous block scale:
// returns the factor to apply and updates prev; a zero scale keeps the unit.
__device__ __forceinline__ float rescale(float cur, float &prev) {
    const float dn = cur == 0.f ? prev : cur;
    const float s = prev * __builtin_amdgcn_rcpf(dn);
    prev = dn;
    return s;
}

// D layout of v_mfma_f32_32x32x16: lane l holds column l % 32 and rows
// 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
__device__ __forceinline__ int drow(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Wave w owns weight rows row_base .. row_base+31 of both
// gate and up (B fragments 0 and 1) for the tile's 64 tokens (A fragments 0, 1).
// ---------------------------------------------------------------------------
struct GuW {
    uint4 q[2][2];      // [gate/up][chunk]: this lane's 32 bytes of sub-group fields
    float d[2];         // block scales
};

__device__ __forceinline__ void gu_load(const FfnArgs &a, int e, int row, int kb, int hh, int64_t nb_row,
                                        int64_t nb_mat, int64_t NB, GuW &w) {
    const int64_t bl = (int64_t)e * nb_mat + (int64_t)row * nb_row + kb;
    const uint8_t *W[2] = {a.gate, a.up};
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const uint8_t *base = W[f] + bl * 64 + hh * 32;
        w.q[f][0] = *reinterpret_cast<const uint4 *>(base);
        w.q[f][1] = *reinterpret_cast<const uint4 *>(base + 16);
        w.d[f] = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(W[f] + NB * 64)[bl]);
    }
}

// 4 * byte B of v in one instruction (sub-dword operand select): the byte offset of a 32-bit table entry
template <int B> __device__ __forceinline__ uint32_t byte_x4(uint32_t v) {
    uint32_t r;
    if constexpr (B == 0) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(v));
    else if constexpr (B == 1) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(v));
    else if constexpr (B == 2) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(v));
    else asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ uint32_t lds_at(const uint32_t *tab, uint32_t byte_off) {
    return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(tab) + byte_off);
}

// One 256-wide K block: 16 K-steps x 2 B fragments x (1 or 2) token fragments.
template <bool two>
__device__ __forceinline__ void gu_block(const GuW &w, const uint4 *tile, const uint32_t *cb4, const uint32_t *sgn,
                                         int n, int hh, float (&dprev)[2], f32x16_t (&acc)[2][2]) {
    f16x2_t mul[2][4];                                   // [gate/up][group]: (2s+1), or 0 for a zero block
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const float sf = rescale(w.d[f], dprev[f]);
        scale_acc(acc[0][f], sf);
        if constexpr (two) scale_acc(acc[1][f], sf);
        const uint32_t keep = w.d[f] == 0.f ? 0u : 0xFFFFFFFFu;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const uint4 qq = w.q[f][gi >> 1];
            const uint32_t lo = (gi & 1) ? qq.z : qq.x, hi = (gi & 1) ? qq.w : qq.y;
            mul[f][gi] = f16pair(iq2x_gscale(lo, hi) & keep);
        }
    }
    // phase 1: all 32 codebook/sign lookups of the block at once (one LDS round trip); a field is the 16-bit
    // half of a word: byte 0 the codebook row, byte 1 the sign index, each turned into a table byte offset by one
    // sub-dword shift
    uint32_t words[2][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int chunk = j >> 3, fld = j & 7, p = fld & 3;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const uint4 qq = w.q[f][chunk];
            const uint32_t dw = (fld >> 2) ? ((p < 2) ? qq.z : qq.w) : ((p < 2) ? qq.x : qq.y);
            words[f][j] = (p & 1) ? (lds_at(cb4, byte_x4<2>(dw)) | lds_at(sgn, byte_x4<3>(dw)))
                                  : (lds_at(cb4, byte_x4<0>(dw)) | lds_at(sgn, byte_x4<1>(dw)));
        }
    }
    // phase 2: convert and multiply on the matrix cores; A fragments read one K-step ahead
    auto col_chunk = [&](int j) {
        const int chunk = j >> 3, fld = j & 7;
        return 4 * (2 * hh + chunk + 4 * (fld >> 2)) + (fld & 3);   // 16-B chunk of column 32*grp + 8p
    };
    f16x8_t a0 = frag16(tile, n, col_chunk(0)), a1;
    if constexpr (two) a1 = frag16(tile, 32 + n, col_chunk(0));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        f16x8_t na0, na1;
        if (j + 1 < 16) {
            na0 = frag16(tile, n, col_chunk(j + 1));
            if constexpr (two) na1 = frag16(tile, 32 + n, col_chunk(j + 1));
        }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const f16x8_t b = fp4x8_f16_mul(words[f][j], mul[f][j >> 2]);
            acc[0][f] = mfma_f16(a0, b, acc[0][f]);
            if constexpr (two) acc[1][f] = mfma_f16(a1, b, acc[1][f]);
        }
        if (j + 1 < 16) {
            a0 = na0;
            if constexpr (two) a1 = na1;
        }
    }
}

template <bool two>
__device__ __forceinline__ void gu_loop(const FfnArgs &a, int e, int row, int hh, int n, const uint16_t *const *src,
                                        uint4 (*tiles)[TOK * 32], const uint32_t *cb4, const uint32_t *sgn,
                                        float (&dprev)[2], f32x16_t (&acc)[2][2]) {
    const int H = a.H, nkb = H / KB;
    const int64_t nb_row = H / KB, nb_mat = (int64_t)a.I * nb_row, NB = nb_mat * a.E;
    GuW w0, w1;
    XStageN<two ? 4 : 2> xs;                             // a one-fragment tile needs its first 32 rows only
    x_fetch(src, 0, xs);
    gu_load(a, e, row, 0, hh, nb_row, nb_mat, NB, w0);
    x_store(xs, tiles[0]);
    __syncthreads();
    // every iteration prefetches block min(kb + 1, nkb - 1): no conditional loads
    for (int kb = 0; kb < nkb; kb += 2) {
        const int k1 = min(kb + 1, nkb - 1), k2 = min(kb + 2, nkb - 1);
        x_fetch(src, k1 * KB, xs);
        gu_load(a, e, row, k1, hh, nb_row, nb_mat, NB, w1);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        gu_block<two>(w0, tiles[0], cb4, sgn, n, hh, dprev, acc);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store(xs, tiles[1]);
        __syncthreads();
        if (kb + 1 >= nkb) break;
        x_fetch(src, k2 * KB, xs);
        gu_load(a, e, row, k2, hh, nb_row, nb_mat, NB, w0);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        gu_block<two>(w1, tiles[1], cb4, sgn, n, hh, dprev, acc);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store(xs, tiles[0]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// q4k routed rows (gate, up or down).  A wave owns 32 rows of ONE matrix; lane
// (n, hh) holds half hh of row n's block: sub-blocks 4hh .. 4hh+3, 64 bytes of
// codes, one u32 per K-step.  Codes become exact fp16 integers sc*q through
// (1024 + q) * sc - 1024 * sc in one fused multiply-add (1024 + q is the fp16
// pattern 0x6400 | q).  The mins use per-32 sums of the activation tile, kept
// as fp16 hi + lo and fed to one MFMA per block: lane hh supplies
// {hi of sub-blocks 4hh..4hh+3, lo of the same} against {m, m}.
// ---------------------------------------------------------------------------
struct Q4W {
    uint4 q[4];
    uint4 meta;         // d | dmin, low nibbles of sc0..7, low nibbles of m0..7, top bits
};

__device__ __forceinline__ void q4_load(const uint8_t *W, int64_t NB, int64_t bl, int hh, Q4W &w) {
    const uint4 *Q = reinterpret_cast<const uint4 *>(W + bl * 128 + hh * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.q[i] = Q[i];
    w.meta = *reinterpret_cast<const uint4 *>(W + NB * 128 + bl * 16);
}

// (v & m) | c in one instruction
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(m), "v"(c));
    return r;
}

__device__ __forceinline__ f16x8_t q4_f16(uint32_t word, f16x2_t sc2, f16x2_t nsc2) {
    f16x8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = and_or(word >> (4 * i), 0x000F000Fu, 0x64006400u);
        const f16x2_t p = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, t), sc2, nsc2);
        r[2 * i] = p.x;
        r[2 * i + 1] = p.y;
    }
    return r;
}

// Store a fetched tile to LDS and its per-32 sums to hs (hs[m] = {hi 0..3,
// lo 0..3, hi 4..7, lo 4..7}).  The four chunks of a sub-block sit in four
// consecutive lanes; they reduce with two cross-lane steps.
template <int NV>
__device__ __forceinline__ void x_store_sums32(const XStageN<NV> &xs, uint4 *tile, _Float16 (*hs)[16]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + NTHR * i, m = idx >> 5, c = idx & 31;
        tile[tpos(m, c)] = xs.v[i];
        const uint32_t wds[4] = {xs.v[i].x, xs.v[i].y, xs.v[i].z, xs.v[i].w};
        float sm = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f16x2_t pr = __builtin_bit_cast(f16x2_t, wds[k]);
            sm += (float)pr.x + (float)pr.y;
        }
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        if ((c & 3) == 0) {
            const int sb = c >> 2;
            const _Float16 hi = (_Float16)sm;
            hs[m][8 * (sb >> 2) + (sb & 3)] = hi;
            hs[m][8 * (sb >> 2) + 4 + (sb & 3)] = (_Float16)(sm - (float)hi);
        }
    }
}

template <bool two>
__device__ __forceinline__ void q4_block(const Q4W &w, const uint4 *tile, const _Float16 (*hs)[16], int n, int hh,
                                         float &dprev, float &mprev, f32x16_t (&acc)[2], f32x16_t (&accm)[2]) {
    const float d = f16_bits_to_f32(w.meta.x & 0xFFFFu), dm = f16_bits_to_f32(w.meta.x >> 16);
    const float s1 = rescale(d, dprev), s2 = rescale(dm, mprev);
    scale_acc(acc[0], s1);
    scale_acc(accm[0], s2);
    if constexpr (two) {
        scale_acc(acc[1], s1);
        scale_acc(accm[1], s2);
    }
    const uint32_t kq = d == 0.f ? 0u : 0xFFu, km = dm == 0.f ? 0u : 0xFFu;
    f16x2_t scp[4], nsc[4];
    f16x8_t mins;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int sb = 4 * hh + jj;
        const uint32_t sc = q4k_field(w.meta.y, w.meta.z, w.meta.w, sb) & kq;
        const uint32_t m = q4k_field(w.meta.y, w.meta.z, w.meta.w, 8 + sb) & km;
        scp[jj] = f16pair(sc);
        const _Float16 ns = (_Float16)(-1024.f * (float)sc);
        nsc[jj] = f16x2_t{ns, ns};
        mins[jj] = mins[4 + jj] = (_Float16)(float)m;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int c = 16 * hh + j;
        const uint4 qq = w.q[j >> 2];
        const uint32_t word = (j & 3) == 0 ? qq.x : ((j & 3) == 1 ? qq.y : ((j & 3) == 2 ? qq.z : qq.w));
        const f16x8_t b = q4_f16(word, scp[j >> 2], nsc[j >> 2]);
        acc[0] = mfma_f16(frag16(tile, n, c), b, acc[0]);
        if constexpr (two) acc[1] = mfma_f16(frag16(tile, 32 + n, c), b, acc[1]);
    }
    accm[0] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[n][8 * hh]), mins, accm[0]);
    if constexpr (two) accm[1] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[32 + n][8 * hh]), mins, accm[1]);
}

// W: prepared q4k stack (NB blocks); bl0: first block of this lane's row; nkb: blocks per row.
template <bool two>
__device__ __forceinline__ void q4_loop(const uint8_t *W, int64_t NB, int64_t bl0, int nkb, int n, int hh,
                                        const uint16_t *const *src, uint4 (*tiles)[TOK * 32],
                                        _Float16 (*hs)[TOK][16], float &dprev, float &mprev, f32x16_t (&acc)[2],
                                        f32x16_t (&accm)[2]) {
    Q4W w0, w1;
    XStageN<two ? 4 : 2> xs;                             // a one-fragment tile needs its first 32 rows only
    x_fetch(src, 0, xs);
    q4_load(W, NB, bl0, hh, w0);
    x_store_sums32(xs, tiles[0], hs[0]);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
        const int k1 = min(kb + 1, nkb - 1), k2 = min(kb + 2, nkb - 1);
        x_fetch(src, k1 * KB, xs);
        q4_load(W, NB, bl0 + k1, hh, w1);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        q4_block<two>(w0, tiles[0], hs[0], n, hh, dprev, mprev, acc, accm);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store_sums32(xs, tiles[1], hs[1]);
        __syncthreads();
        if (kb + 1 >= nkb) break;
        x_fetch(src, k2 * KB, xs);
        q4_load(W, NB, bl0 + k2, hh, w0);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        q4_block<two>(w1, tiles[1], hs[1], n, hh, dprev, mprev, acc, accm);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store_sums32(xs, tiles[0], hs[0]);
        __syncthreads();
    }
}

// Shared expert gate/up: bf16 B fragments straight from the weight rows, read
// one 64-wide K stage (4 K-steps) ahead into registers; x tiles double-buffered
// in LDS as for the routed experts.
typedef bf16x8_t BStage[2][4];       // [gate/up][K-step of the stage]

__device__ __forceinline__ void sg_stage_load(const FfnArgs &a, int row, int hh, int st, BStage &b) {
    const int kb = st >> 2, j0 = 4 * (st & 3);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int c = 2 * (j0 + jj) + hh;
        b[0][jj] = *reinterpret_cast<const bf16x8_t *>(a.sg + (int64_t)row * a.H + kb * KB + 8 * c);
        b[1][jj] = *reinterpret_cast<const bf16x8_t *>(a.su + (int64_t)row * a.H + kb * KB + 8 * c);
    }
}

template <bool two>
__device__ __forceinline__ void sg_stage(const BStage &b, const uint4 *tile, int st, int n, int hh,
                                         f32x16_t (&acc)[2][2]) {
    const int j0 = 4 * (st & 3);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int c = 2 * (j0 + jj) + hh;                 // columns 16j + 8hh
        const bf16x8_t a0 = fragbf(tile, n, c);
        bf16x8_t a1;
        if constexpr (two) a1 = fragbf(tile, 32 + n, c);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            acc[0][f] = mfma_bf16(a0, b[f][jj], acc[0][f]);
            if constexpr (two) acc[1][f] = mfma_bf16(a1, b[f][jj], acc[1][f]);
        }
    }
}

template <bool two>
__device__ __forceinline__ void sg_loop(const FfnArgs &a, int row, int hh, int n, const uint16_t *const *src,
                                        uint4 (*tiles)[TOK * 32], f32x16_t (&acc)[2][2]) {
    const int nkb = a.H / KB, nst = 4 * nkb;
    BStage b0, b1;
    XStage xs;
    x_fetch(src, 0, xs);
    sg_stage_load(a, row, hh, 0, b0);
    x_store(xs, tiles[0]);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {               // two 64-wide stages per iteration, four per block
        const int kb = st >> 2;
        const bool block_start = (st & 3) == 0;
        if (block_start) x_fetch(src, min(kb + 1, nkb - 1) * KB, xs);
        sg_stage_load(a, row, hh, st + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        sg_stage<two>(b0, tiles[kb & 1], st, n, hh, acc);
        sg_stage_load(a, row, hh, min(st + 2, nst - 1), b0);
        __builtin_amdgcn_sched_barrier(0);
        sg_stage<two>(b1, tiles[kb & 1], st + 1, n, hh, acc);
        if (!block_start) {                              // end of block kb: publish tile kb + 1
            __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
            x_store(xs, tiles[(kb + 1) & 1]);
            __syncthreads();
        }
    }
}

// FG: routed gate/up format.  iq2x: a wave owns 32 rows of gate AND up (256
// rows per item, SwiGLU in registers).  q4k: waves 0-3 own 32 gate rows each,
// waves 4-7 the same 128 rows of up (128 rows per item); the up values meet
// the gate values in LDS for the SwiGLU.
template <int FG, bool FAST>
__global__ __launch_bounds__(NTHR) void k_gemm_gateup(GemmArgs g) {
    const FfnArgs &a = g.a;
    constexpr int RPI = FG == FMT_Q4K ? ROWS / 2 : ROWS;
    __shared__ int tile_off[257];
    // the tables are laid out first (largest alignment), below 64 KiB, so that their base address folds into the
    // lookups' immediate offsets; sgn is indexed by a field's whole high byte (bit 7 is not a sign bit)
    __shared__ __attribute__((aligned(64))) uint32_t cb4[256];
    __shared__ __attribute__((aligned(64))) uint32_t sgn[256];
    __shared__ const uint16_t *src[TOK];
    __shared__ int dst[TOK];
    __shared__ float hfac[TOK];                                 // routed rows: 2^-sigma of the row's token
    __shared__ float xfac[TOK];                                 // routed rows: 2^(sigma/2), undoes the x16 prescale
    __shared__ uint4 tiles[2][TOK * 32];
    __shared__ __attribute__((aligned(16))) _Float16 hsum[2][TOK][16];
    Item it;
    if (!get_item(a, a.I, RPI, a.Is, tile_off, it)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int H = a.H;
    if (FG == FMT_IQ2X && !it.shared) {
        if (tid < 256) cb4[tid] = codebook_row_fp4(a.codebook, tid);
        else sgn[tid - 256] = sign_spread((tid - 256) & 0x7F);
    }
    if (tid < TOK) {
        const int m = tid < it.n ? tid : 0;                  // rows past the tile alias row 0
        const uint16_t *s;
        if (!it.shared) {
            const int tok = a.perm[it.p0 + m] / a.k;
            s = reinterpret_cast<const uint16_t *>(g.x16) + (int64_t)tok * H;
            const int sig = a.hsig[tok];
            hfac[tid] = ldexpf(1.f, -sig);
            xfac[tid] = ldexpf(1.f, sig / 2);
        } else {
            s = static_cast<const uint16_t *>(a.x) + (int64_t)(it.p0 + m) * H;
        }
        src[tid] = s;
        dst[tid] = tid < it.n ? it.p0 + tid : -1;
    }
    __syncthreads();
    const bool two = it.n > 32;
    f32x16_t acc[2][2];          // [token frag][gate, up]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
    const int row = it.r * ROWS + wv * 32 + n;           // this lane's weight row (iq2x, shared)

    if (FG == FMT_Q4K && !it.shared) {
        const bool up = wv >= 4;
        const int r4 = it.r * RPI + (wv & 3) * 32 + n;
        const int nkb = H / KB;
        const int64_t NB = (int64_t)a.E * a.I * nkb, bl0 = ((int64_t)it.e * a.I + r4) * nkb;
        f32x16_t accq[2] = {f32x16_t{}, f32x16_t{}}, accm[2] = {f32x16_t{}, f32x16_t{}};
        float dprev = 1.f, mprev = 1.f;
        if (two) q4_loop<true>(up ? a.up : a.gate, NB, bl0, nkb, n, hh, src, tiles, hsum, dprev, mprev, accq, accm);
        else q4_loop<false>(up ? a.up : a.gate, NB, bl0, nkb, n, hh, src, tiles, hsum, dprev, mprev, accq, accm);
        float *xch = reinterpret_cast<float *>(&tiles[0][0]);     // [4 waves][TOK][32] up values
        if (up) {
#pragma unroll
            for (int tf = 0; tf < 2; ++tf)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    xch[((wv & 3) * TOK + 32 * tf + drow(v, lane)) * 32 + n] =
                        (accq[tf][v] * dprev - accm[tf][v] * mprev) * xfac[32 * tf + drow(v, lane)];
        }
        __syncthreads();
        if (!up) {
#pragma unroll
            for (int tf = 0; tf < 2; ++tf)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int tt = 32 * tf + drow(v, lane), d = dst[tt];
                    if (d >= 0)
                        g.h[(int64_t)d * a.I + r4] =
                            (_Float16)(silu_mul((accq[tf][v] * dprev - accm[tf][v] * mprev) * xfac[tt],
                                                xch[((wv & 3) * TOK + tt) * 32 + n]) *
                                       hfac[tt]);
                }
        }
    } else if (!it.shared) {
        float dprev[2] = {1.f, 1.f};
        if (two) gu_loop<true>(a, it.e, row, hh, n, src, tiles, cb4, sgn, dprev, acc);
        else gu_loop<false>(a, it.e, row, hh, n, src, tiles, cb4, sgn, dprev, acc);
        // SwiGLU epilogue: h[position][row] in fp16
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tt = 32 * tf + drow(v, lane), d = dst[tt];
                if (d >= 0)
                    g.h[(int64_t)d * a.I + row] = (_Float16)(silu_mul(acc[tf][0][v] * dprev[0] * xfac[tt],
                                                                      acc[tf][1][v] * dprev[1] * xfac[tt]) *
                                                             hfac[tt]);
            }
    } else {
        if (two) sg_loop<true>(a, row, hh, n, src, tiles, acc);
        else sg_loop<false>(a, row, hh, n, src, tiles, acc);
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int d = dst[32 * tf + drow(v, lane)];
                if (d >= 0) {
                    const float hv = silu_mul(acc[tf][0][v], acc[tf][1][v]);
                    const uint32_t hb = __float_as_uint(hv);
                    const uint32_t hi = (hb + 0x7FFFu + ((hb >> 16) & 1u)) >> 16;   // bf16, nearest even
                    const float rest = hv - __uint_as_float(hi << 16);
                    const uint32_t rb = __float_as_uint(rest);
                    const uint32_t lo = (rb + 0x7FFFu + ((rb >> 16) & 1u)) >> 16;
                    const int64_t o = (int64_t)d * a.Is + row;
                    g.hs_hi[o] = (uint16_t)hi;
                    if constexpr (!FAST) g.hs_lo[o] = (uint16_t)lo;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// down projection.  Wave w owns output rows row_base .. row_base+31.
// ---------------------------------------------------------------------------
struct DnW {
    uint4 q[2];         // [chunk]: 32 bytes = sub-blocks 8hh .. 8hh+7
    uint2 sm;           // their (sc | m << 4) bytes
    float d, dm;
};

__device__ __forceinline__ void dn_load(const FfnArgs &a, int e, int row, int kb, int hh, int64_t nb_row,
                                        int64_t nb_mat, int64_t NB, DnW &w) {
    const uint8_t *Q = a.down, *S = a.down + NB * 64;
    const uint32_t *D = reinterpret_cast<const uint32_t *>(a.down + NB * 80);
    const int64_t bl = (int64_t)e * nb_mat + (int64_t)row * nb_row + kb;
    w.q[0] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + hh * 32);
    w.q[1] = *reinterpret_cast<const uint4 *>(Q + bl * 64 + hh * 32 + 16);
    w.sm = *reinterpret_cast<const uint2 *>(S + bl * 16 + hh * 8);
    const uint32_t dd = D[bl];
    w.d = f16_bits_to_f32(dd & 0xFFFFu);
    w.dm = f16_bits_to_f32(dd >> 16);
}

// x_store for an h tile, plus its per-16 sums: the two threads that hold a 16-wide sub-block (chunks 2 sb and
// 2 sb + 1 of a row) add their halves in fp32 and store the sum as fp16 hi (hs[m][sb]) + lo (hs[m][16 + sb]).
// The barrier that publishes the tile publishes the sums.
template <int NV>
__device__ __forceinline__ void x_store_sums16(const XStageN<NV> &xs, uint4 *tile, _Float16 (*hs)[32]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + NTHR * i, m = idx >> 5, c = idx & 31;
        tile[tpos(m, c)] = xs.v[i];
        const uint32_t wds[4] = {xs.v[i].x, xs.v[i].y, xs.v[i].z, xs.v[i].w};
        float sm = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f16x2_t pr = __builtin_bit_cast(f16x2_t, wds[k]);
            sm += (float)pr.x + (float)pr.y;
        }
        sm += __shfl_xor(sm, 1, 64);
        if ((c & 1) == 0) {
            const _Float16 hi = (_Float16)sm;
            hs[m][c >> 1] = hi;
            hs[m][16 + (c >> 1)] = (_Float16)(sm - (float)hi);
        }
    }
}

template <bool two>
__device__ __forceinline__ void dn_block(const DnW &w, const uint4 *tile, const _Float16 (*hs)[32], int n, int hh,
                                         float &dprev, float &mprev, f32x16_t (&acc)[2], f32x16_t (&accm)[2]) {
    const float s1 = rescale(w.d, dprev), s2 = rescale(w.dm, mprev);
    scale_acc(acc[0], s1);
    scale_acc(accm[0], s2);
    if constexpr (two) {
        scale_acc(acc[1], s1);
        scale_acc(accm[1], s2);
    }
    const uint32_t kq = w.d == 0.f ? 0u : 0xFFu, km = w.dm == 0.f ? 0u : 0xFFu;
    f16x2_t scp[8];
    f16x8_t mins;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t byte = (i < 4 ? w.sm.x >> (8 * i) : w.sm.y >> (8 * (i - 4))) & 0xFFu;
        scp[i] = f16pair(byte & 15u & kq);
        mins[i] = (_Float16)(float)((byte >> 4) & km);
    }
    // main term: K-step j covers sub-block 8hh + j/2, half j%2 (columns 16*(8hh+j/2) + 8*(j%2))
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int sbl = j >> 1, half = j & 1;
        const int c = 2 * (8 * hh + sbl) + half;
        const f16x8_t a0 = frag16(tile, n, c);
        const uint4 qq = w.q[sbl >> 2];
        const uint32_t dw = (sbl & 3) == 0 ? qq.x : ((sbl & 3) == 1 ? qq.y : ((sbl & 3) == 2 ? qq.z : qq.w));
        const uint32_t codes = half ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u);
        const f16x8_t b = q2k_f16_mul(codes, scp[sbl]);
        acc[0] = mfma_f16(a0, b, acc[0]);
        if constexpr (two) acc[1] = mfma_f16(frag16(tile, 32 + n, c), b, acc[1]);
    }
    // min term: K = the 16 sub-blocks; A = per-16 sums (hi, lo), B = mins
    accm[0] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[n][8 * hh]), mins, accm[0]);
    accm[0] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[n][16 + 8 * hh]), mins, accm[0]);
    if constexpr (two) {
        accm[1] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[32 + n][8 * hh]), mins, accm[1]);
        accm[1] = mfma_f16(*reinterpret_cast<const f16x8_t *>(&hs[32 + n][16 + 8 * hh]), mins, accm[1]);
    }
}

template <bool two>
__device__ __forceinline__ void dn_loop(const FfnArgs &a, int e, int row, int hh, int n, const uint16_t *const *src,
                                        uint4 (*tiles)[TOK * 32], _Float16 (*hsum)[TOK][32], float &dprev,
                                        float &mprev, f32x16_t (&acc)[2], f32x16_t (&accm)[2]) {
    const int I = a.I, H = a.H, nkb = I / KB;
    const int64_t nb_row = I / KB, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
    DnW w0, w1;
    XStageN<two ? 4 : 2> xs;                             // a one-fragment tile needs its first 32 rows only
    x_fetch(src, 0, xs);
    dn_load(a, e, row, 0, hh, nb_row, nb_mat, NB, w0);
    x_store_sums16(xs, tiles[0], hsum[0]);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
        const int k1 = min(kb + 1, nkb - 1), k2 = min(kb + 2, nkb - 1);
        x_fetch(src, k1 * KB, xs);
        dn_load(a, e, row, k1, hh, nb_row, nb_mat, NB, w1);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        dn_block<two>(w0, tiles[0], hsum[0], n, hh, dprev, mprev, acc, accm);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store_sums16(xs, tiles[1], hsum[1]);
        __syncthreads();
        if (kb + 1 >= nkb) break;
        x_fetch(src, k2 * KB, xs);
        dn_load(a, e, row, k2, hh, nb_row, nb_mat, NB, w0);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        dn_block<two>(w1, tiles[1], hsum[1], n, hh, dprev, mprev, acc, accm);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store_sums16(xs, tiles[0], hsum[0]);
        __syncthreads();
    }
}

// Fast mode (approximate, opt-in): every weight becomes one fp16 value, q * fp16(d sc) - fp16(dmin m) in a fused
// packed multiply-add, so neither the per-16 sums of h, nor the min products, nor rescaling between blocks remain.
template <bool two>
__device__ __forceinline__ void dn_block_fast(const DnW &w, const uint4 *tile, int n, int hh, f32x16_t (&acc)[2]) {
    f16x2_t dsc[8], nmn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t byte = (i < 4 ? w.sm.x >> (8 * i) : w.sm.y >> (8 * (i - 4))) & 0xFFu;
        const _Float16 a = (_Float16)(w.d * (float)(byte & 15u)), b = (_Float16)(-w.dm * (float)(byte >> 4));
        dsc[i] = f16x2_t{a, a};
        nmn[i] = f16x2_t{b, b};
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int sbl = j >> 1, half = j & 1;
        const int c = 2 * (8 * hh + sbl) + half;
        const f16x8_t a0 = frag16(tile, n, c);
        const uint4 qq = w.q[sbl >> 2];
        const uint32_t dw = (sbl & 3) == 0 ? qq.x : ((sbl & 3) == 1 ? qq.y : ((sbl & 3) == 2 ? qq.z : qq.w));
        const uint32_t codes = half ? ((dw >> 2) & 0x33333333u) : (dw & 0x33333333u);
        const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 0);   // q, exact
        const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 1);
        const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 2);
        const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 2.0f, 3);
        const f16x2_t w0 = __builtin_elementwise_fma(p0, dsc[sbl], nmn[sbl]);
        const f16x2_t w1 = __builtin_elementwise_fma(p1, dsc[sbl], nmn[sbl]);
        const f16x2_t w2 = __builtin_elementwise_fma(p2, dsc[sbl], nmn[sbl]);
        const f16x2_t w3 = __builtin_elementwise_fma(p3, dsc[sbl], nmn[sbl]);
        const f16x8_t b = f16x8_t{w0.x, w0.y, w1.x, w1.y, w2.x, w2.y, w3.x, w3.y};
        acc[0] = mfma_f16(a0, b, acc[0]);
        if constexpr (two) acc[1] = mfma_f16(frag16(tile, 32 + n, c), b, acc[1]);
    }
}

template <bool two>
__device__ __forceinline__ void dn_loop_fast(const FfnArgs &a, int e, int row, int hh, int n,
                                             const uint16_t *const *src, uint4 (*tiles)[TOK * 32],
                                             f32x16_t (&acc)[2]) {
    const int I = a.I, H = a.H, nkb = I / KB;
    const int64_t nb_row = I / KB, nb_mat = (int64_t)H * nb_row, NB = nb_mat * a.E;
    DnW w0, w1;
    XStageN<two ? 4 : 2> xs;
    x_fetch(src, 0, xs);
    dn_load(a, e, row, 0, hh, nb_row, nb_mat, NB, w0);
    x_store(xs, tiles[0]);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
        const int k1 = min(kb + 1, nkb - 1), k2 = min(kb + 2, nkb - 1);
        x_fetch(src, k1 * KB, xs);
        dn_load(a, e, row, k1, hh, nb_row, nb_mat, NB, w1);
        __builtin_amdgcn_sched_barrier(0);
        dn_block_fast<two>(w0, tiles[0], n, hh, acc);
        __builtin_amdgcn_sched_barrier(0);
        x_store(xs, tiles[1]);
        __syncthreads();
        if (kb + 1 >= nkb) break;
        x_fetch(src, k2 * KB, xs);
        dn_load(a, e, row, k2, hh, nb_row, nb_mat, NB, w0);
        __builtin_amdgcn_sched_barrier(0);
        dn_block_fast<two>(w1, tiles[1], n, hh, acc);
        __builtin_amdgcn_sched_barrier(0);
        x_store(xs, tiles[0]);
        __syncthreads();
    }
}

// Shared expert down in fast mode: A = h as one bf16 plane (256-wide K blocks), B = the bf16 rows, 8 K-steps of
// B read one half-block ahead.
template <bool two>
__device__ __forceinline__ void sd_half_fast(const bf16x8_t (&b)[8], const uint4 *tile, int half, int n, int hh,
                                             f32x16_t (&acc)[2]) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int c = 16 * half + 2 * jj + hh;            // columns 128 half + 16 jj + 8 hh
        acc[0] = mfma_bf16(fragbf(tile, n, c), b[jj], acc[0]);
        if constexpr (two) acc[1] = mfma_bf16(fragbf(tile, 32 + n, c), b[jj], acc[1]);
    }
}

template <bool two>
__device__ __forceinline__ void sd_loop_fast(const FfnArgs &a, int row, int hh, int n, const uint16_t *const *hi,
                                             uint4 (*tiles)[TOK * 32], f32x16_t (&acc)[2]) {
    const int nkb = a.Is / KB;
    bf16x8_t b0[8], b1[8];
    XStage xs;
    auto bload = [&](int st, bf16x8_t (&b)[8]) {         // K-steps of the 128-wide stage st
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            b[jj] = *reinterpret_cast<const bf16x8_t *>(a.sd + (int64_t)row * a.Is + st * 128 + 16 * jj + 8 * hh);
    };
    x_fetch(hi, 0, xs);
    bload(0, b0);
    x_store(xs, tiles[0]);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int k1 = min(kb + 1, nkb - 1);
        x_fetch(hi, k1 * KB, xs);
        bload(2 * kb + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        sd_half_fast<two>(b0, tiles[kb & 1], 0, n, hh, acc);
        bload(2 * k1, b0);
        __builtin_amdgcn_sched_barrier(0);
        sd_half_fast<two>(b1, tiles[kb & 1], 1, n, hh, acc);
        __builtin_amdgcn_sched_barrier(0);
        x_store(xs, tiles[(kb + 1) & 1]);
        __syncthreads();
    }
}

// Shared expert down: A = h as bf16 hi + lo.  One LDS tile holds a 128-wide K
// stage of both planes (chunks 0..15 = hi, 16..31 = lo), double-buffered; the
// bf16 B fragments of the stage (8 K-steps) are read into registers one stage
// ahead.
typedef bf16x8_t DStage[8];

__device__ __forceinline__ void sd_stage_load(const FfnArgs &a, int row, int hh, int st, DStage &b) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        b[jj] = *reinterpret_cast<const bf16x8_t *>(a.sd + (int64_t)row * a.Is + st * 128 + 16 * jj + 8 * hh);
}

template <bool two>
__device__ __forceinline__ void sd_stage(const DStage &b, const uint4 *tile, int n, int hh, f32x16_t (&acc)[2]) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int c = 2 * jj + hh;
        acc[0] = mfma_bf16(fragbf(tile, n, c), b[jj], acc[0]);
        acc[0] = mfma_bf16(fragbf(tile, n, 16 + c), b[jj], acc[0]);
        if constexpr (two) {
            acc[1] = mfma_bf16(fragbf(tile, 32 + n, c), b[jj], acc[1]);
            acc[1] = mfma_bf16(fragbf(tile, 32 + n, 16 + c), b[jj], acc[1]);
        }
    }
}

template <bool two>
__device__ __forceinline__ void sd_loop(const FfnArgs &a, int row, int hh, int n, const uint16_t *const *hi,
                                        const uint16_t *const *lo, uint4 (*tiles)[TOK * 32], f32x16_t (&acc)[2]) {
    const int nst = a.Is / 128;
    DStage b0, b1;
    XStage xs;
    x_fetch_hilo(hi, lo, 0, xs);
    sd_stage_load(a, row, hh, 0, b0);
    x_store(xs, tiles[0]);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        const int s1 = min(st + 1, nst - 1), s2 = min(st + 2, nst - 1);
        x_fetch_hilo(hi, lo, s1 * 128, xs);
        sd_stage_load(a, row, hh, s1, b1);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        sd_stage<two>(b0, tiles[0], n, hh, acc);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store(xs, tiles[1]);
        __syncthreads();
        if (st + 1 >= nst) break;
        x_fetch_hilo(hi, lo, s2 * 128, xs);
        sd_stage_load(a, row, hh, s2, b0);
        __builtin_amdgcn_sched_barrier(0);     // keep the prefetch above the compute
        sd_stage<two>(b1, tiles[1], n, hh, acc);
        __builtin_amdgcn_sched_barrier(0);     // store the next tile after the compute
        x_store(xs, tiles[0]);
        __syncthreads();
    }
}

// FD: routed down format (q2k or q4k).
template <int FD, bool FAST>
__global__ __launch_bounds__(NTHR) void k_gemm_down(GemmArgs g) {
    const FfnArgs &a = g.a;
    __shared__ int tile_off[257];
    __shared__ const uint16_t *src[TOK];
    __shared__ const uint16_t *src_lo[TOK];
    __shared__ int dst[TOK];
    __shared__ float hfac[TOK];                                 // routed rows: 2^sigma of the row's token
    __shared__ uint4 tiles[2][TOK * 32];
    __shared__ __attribute__((aligned(16))) _Float16 hsum_lds[2 * TOK * 32];   // two buffers of per-row sums
    _Float16 (*hsum)[TOK][16] = reinterpret_cast<_Float16 (*)[TOK][16]>(hsum_lds);      // q4k: per 32
    _Float16 (*hsum16)[TOK][32] = reinterpret_cast<_Float16 (*)[TOK][32]>(hsum_lds);    // q2k: per 16
    Item it;
    if (!get_item(a, a.H, ROWS, a.H, tile_off, it)) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int I = a.I, H = a.H;
    if (tid < TOK) {
        const int m = tid < it.n ? tid : 0;
        if (!it.shared) {
            src[tid] = reinterpret_cast<const uint16_t *>(g.h) + (int64_t)(it.p0 + m) * I;
            src_lo[tid] = nullptr;
            dst[tid] = tid < it.n ? a.perm[it.p0 + tid] : -1;          // output slot
            hfac[tid] = ldexpf(1.f, a.hsig[a.perm[it.p0 + m] / a.k]);
        } else {
            src[tid] = g.hs_hi + (int64_t)(it.p0 + m) * a.Is;
            src_lo[tid] = g.hs_lo + (int64_t)(it.p0 + m) * a.Is;
            dst[tid] = tid < it.n ? it.p0 + tid : -1;
        }
    }
    __syncthreads();
    const bool two = it.n > 32;
    const int row = it.r * ROWS + wv * 32 + n;           // this lane's output row
    f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
    if (!it.shared) {
        f32x16_t accm[2] = {f32x16_t{}, f32x16_t{}};
        float dprev = 1.f, mprev = 1.f;
        if constexpr (FD == FMT_Q4K) {
            const int nkb = I / KB;
            const int64_t NB = (int64_t)a.E * H * nkb, bl0 = ((int64_t)it.e * H + row) * nkb;
            if (two) q4_loop<true>(a.down, NB, bl0, nkb, n, hh, src, tiles, hsum, dprev, mprev, acc, accm);
            else q4_loop<false>(a.down, NB, bl0, nkb, n, hh, src, tiles, hsum, dprev, mprev, acc, accm);
        } else if constexpr (FAST) {
            if (two) dn_loop_fast<true>(a, it.e, row, hh, n, src, tiles, acc);
            else dn_loop_fast<false>(a, it.e, row, hh, n, src, tiles, acc);
        } else {
            if (two) dn_loop<true>(a, it.e, row, hh, n, src, tiles, hsum16, dprev, mprev, acc, accm);
            else dn_loop<false>(a, it.e, row, hh, n, src, tiles, hsum16, dprev, mprev, acc, accm);
        }
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tt = 32 * tf + drow(v, lane), d = dst[tt];
                if (d >= 0) a.slot_out[(int64_t)d * H + row] = (acc[tf][v] * dprev - accm[tf][v] * mprev) * hfac[tt];
            }
    } else {
        if constexpr (FAST) {
            if (two) sd_loop_fast<true>(a, row, hh, n, src, tiles, acc);
            else sd_loop_fast<false>(a, row, hh, n, src, tiles, acc);
        } else {
            if (two) sd_loop<true>(a, row, hh, n, src, src_lo, tiles, acc);
            else sd_loop<false>(a, row, hh, n, src, src_lo, tiles, acc);
        }
#pragma unroll
        for (int tf = 0; tf < 2; ++tf)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int d = dst[32 * tf + drow(v, lane)];
                if (d >= 0) a.shared_out[(int64_t)d * H + row] = acc[tf][v];
            }
    }
}

// x (bf16) -> fp16 copy, one workgroup per token row, 8 elements per thread and step: the row's largest |x|
// first, then x * 2^-e with e = sigma / 2, where sigma (the exponent of the token's routed h scale, written to
// hsig[token]) is 2 * (ilogb(max |x|) - 1) clamped to [-100, 100]
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t *__restrict__ x, _Float16 *__restrict__ y, int H,
                                                  int32_t *__restrict__ hsig) {
    __shared__ float wmax[4];
    const int t = blockIdx.x, n8 = H / 8;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (int64_t)t * H);
    f16x8_t *yr = reinterpret_cast<f16x8_t *>(y + (int64_t)t * H);
    float mx = 0.f;
    for (int i = threadIdx.x; i < n8; i += 256) {
        const uint4 v = xr[i];
        mx = fmaxf(fmaxf(mx, fmaxf(bf16x2_absmax(v.x), bf16x2_absmax(v.y))),
                   fmaxf(bf16x2_absmax(v.z), bf16x2_absmax(v.w)));
    }
    mx = wave_max_f32(mx);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    const int sig = h_sigma(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    if (threadIdx.x == 0) hsig[t] = sig;
    const int sh = -(sig / 2);
    for (int i = threadIdx.x; i < n8; i += 256) {
        const uint4 v = xr[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        f16x8_t o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = (_Float16)ldexpf(__uint_as_float(w[j] << 16), sh);
            o[2 * j + 1] = (_Float16)ldexpf(__uint_as_float(w[j] & 0xFFFF0000u), sh);
        }
        yr[i] = o;
    }
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct Layout {
    size_t x16, h, hs_hi, hs_lo, hsig, total;
};
Layout layout(int H, int I, int k, int Is, int T) {
    Layout L;
    L.x16 = 0;
    L.h = L.x16 + align256((size_t)T * H * 2);
    L.hs_hi = L.h + align256((size_t)T * k * I * 2);
    L.hs_lo = L.hs_hi + align256((size_t)T * Is * 2);
    L.hsig = L.hs_lo + align256((size_t)T * Is * 2);
    L.total = L.hsig + align256((size_t)T * 4);
    return L;
}

}  // namespace

namespace moe {

bool ffn_gemm_supported(const FfnArgs &a) {
    if (!a.x_bf16) return false;
    if (a.fmt_gu != FMT_IQ2X && a.fmt_gu != FMT_Q4K) return false;
    if (a.fmt_d != FMT_Q2K && a.fmt_d != FMT_Q4K) return false;
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
    g.a.hsig = reinterpret_cast<int32_t *>(ws + L.hsig);
    const int S = a.T * a.k;
    const int max_tiles = (S + TOK - 1) / TOK + (S < a.E ? S : a.E);   // sum_e ceil(n_e / TOK) bound
    const int st_tiles = (a.T + TOK - 1) / TOK;
    hipError_t e = hipSuccess;
    if (a.stages & STAGE_GATE_UP) {
        hipLaunchKernelGGL(k_x_to_f16, dim3(a.T), dim3(256), 0, st, static_cast<const uint16_t *>(a.x),
                           const_cast<_Float16 *>(g.x16), a.H, g.a.hsig);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int rpi = a.fmt_gu == FMT_Q4K ? ROWS / 2 : ROWS;
        const int G = max_tiles * (a.I / rpi) + (a.Is > 0 ? st_tiles * (a.Is / ROWS) : 0);
        // fast mode changes the shared expert's h planes here (one bf16 plane); the routed gate/up rows stay exact
        if (a.fmt_gu == FMT_Q4K && a.fast) hipLaunchKernelGGL((k_gemm_gateup<FMT_Q4K, true>), dim3(G), dim3(NTHR), 0, st, g);
        else if (a.fmt_gu == FMT_Q4K) hipLaunchKernelGGL((k_gemm_gateup<FMT_Q4K, false>), dim3(G), dim3(NTHR), 0, st, g);
        else if (a.fast) hipLaunchKernelGGL((k_gemm_gateup<FMT_IQ2X, true>), dim3(G), dim3(NTHR), 0, st, g);
        else hipLaunchKernelGGL((k_gemm_gateup<FMT_IQ2X, false>), dim3(G), dim3(NTHR), 0, st, g);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.stages & STAGE_DOWN) {
        const int G = max_tiles * (a.H / ROWS) + (a.Is > 0 ? st_tiles * (a.H / ROWS) : 0);
        if (a.fmt_d == FMT_Q4K && a.fast) hipLaunchKernelGGL((k_gemm_down<FMT_Q4K, true>), dim3(G), dim3(NTHR), 0, st, g);
        else if (a.fmt_d == FMT_Q4K) hipLaunchKernelGGL((k_gemm_down<FMT_Q4K, false>), dim3(G), dim3(NTHR), 0, st, g);
        else if (a.fast) hipLaunchKernelGGL((k_gemm_down<FMT_Q2K, true>), dim3(G), dim3(NTHR), 0, st, g);
        else hipLaunchKernelGGL((k_gemm_down<FMT_Q2K, false>), dim3(G), dim3(NTHR), 0, st, g);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace moe
