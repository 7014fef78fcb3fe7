// Device-side helpers shared by the kernels of libmoe2bit (gfx950 only).
//
// Prepared (device) layouts.  A stack of NB blocks (NB = n_mats*rows*cols/256)
// is stored as structure-of-arrays regions so that every 16-byte lane load
// lands on whole fields:
//
//  iq2x  Q: NB x 64 B, then D: NB x fp16.
//        Block b's 64 bytes are four 16-byte chunks; chunk c holds the eight
//        16-bit sub-group fields of groups c and c+4 (fields 0..3 = group c,
//        sub-groups 0..3; fields 4..7 = group c+4).  A sub-group field is
//          bits 0..7  codebook row, bits 8..14 the seven stored signs,
//          bit 15     bit p of the group's 4-bit scale s (p = sub-group).
//        A lane that loads one chunk therefore owns two complete groups.
//  q2k   Q: NB x 64 B, S: NB x 16 B, D: NB x u32 (d | dmin << 16).
//        Chunk c (16 B) = sub-blocks 4c..4c+3, one dword each; in the dword of
//        sub-block j, nibble i carries q[16j+i] in bits 0..1 and q[16j+8+i] in
//        bits 2..3, so (v & 0x33333333) and ((v >> 2) & 0x33333333) are eight
//        fp4 codes each.  S keeps the canonical (sc | m << 4) bytes.
//  q4k   Q: NB x 128 B, one u32 per 8 consecutive weights w0..w7 with the
//        code of w(2i+h) at bits 16h + 4i (so (word >> 4i) & 0x000F000F holds
//        the pair w(2i), w(2i+1) in its two 16-bit halves),
//        M: NB x 16 B = d | dmin | u32 low nibbles of fields 0..7 | u32 low
//        nibbles of fields 8..15 | u32 top two bits of field f at bits 2f.
//
// fp4 (E2M1) codes: a 2- or 4-bit unsigned integer code q placed in a nibble
// decodes to q/2 (codes 0..3: 0, 0.5, 1, 1.5); iq2x magnitudes 1, 2, 3 are the
// codes 0x2, 0x4, 0x5, and bit 3 is the sign.  The hardware converts two codes
// at a time to bf16/f16/f32 pairs (v_cvt_scalef32_pk_*_fp4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

#define MOE_QK 256

namespace moe {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

// fp4 code of an iq2x magnitude (1 -> 1.0, 2 -> 2.0, 3 -> 3.0).
__device__ __forceinline__ uint32_t mag_to_fp4(uint32_t c) { return c == 1 ? 0x2u : (c == 2 ? 0x4u : 0x5u); }

// Eight codebook magnitudes of row e as eight fp4 codes (nibble i = weight i).
__device__ __forceinline__ uint32_t codebook_row_fp4(const uint8_t *cb, int e) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= mag_to_fp4(cb[8 * e + i]) << (4 * i);
    return w;
}

// Sign bits of an 8-weight sub-group spread onto fp4 sign positions (bit 4i+3);
// the eighth sign is the parity of the seven stored ones.
__device__ __forceinline__ uint32_t sign_spread(uint32_t s7) {
    uint32_t x = s7 | ((uint32_t)(__builtin_popcount(s7) & 1) << 7);    // eight sign bits
    x = (x | (x << 12)) & 0x000F000Fu;                                   // bit i -> 4i in three doubling steps
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x << 3;
}

// A codebook row as two little-endian words of magnitude bytes (1, 2, 3) ->
// eight fp4 codes (2, 4, 5), nibble i = weight i.  Per byte 2m - [m == 3],
// then the bytes are packed into nibbles.
__device__ __forceinline__ uint32_t cbrow_fp4(uint32_t x, uint32_t y) {
    const uint32_t lo = (x << 1) - ((x >> 1) & x & 0x01010101u);
    const uint32_t hi = (y << 1) - ((y >> 1) & y & 0x01010101u);
    const uint32_t l2 = (lo | (lo >> 4)) & 0x00FF00FFu, h2 = (hi | (hi >> 4)) & 0x00FF00FFu;
    return ((l2 | (l2 >> 8)) & 0xFFFFu) | (((h2 | (h2 >> 8)) & 0xFFFFu) << 16);
}

// 2s + 1 for the 4-bit group scale s of an iq2x group held as the two words
// of its four prepared fields: scale bit i is bit 15 of field i.
__device__ __forceinline__ uint32_t iq2x_gscale(uint32_t lo, uint32_t hi) {
    uint32_t u = ((lo >> 14) & 0x00020002u) | 1u;          // s0 -> bit 1, s1 -> bit 17
    u |= (hi >> 12) & 0x00080008u;                         // s2 -> bit 3, s3 -> bit 19
    return (u | (u >> 15)) & 0x1Fu;
}

// Two fp4 codes (byte `sel` of v) -> bf16 / f16 / f32 pairs, unscaled.
template <int SEL> __device__ __forceinline__ bf16x2_t fp4x2_bf16(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL);
}
template <int SEL> __device__ __forceinline__ f16x2_t fp4x2_f16(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, SEL);
}
template <int SEL> __device__ __forceinline__ f32x2_t fp4x2_f32(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, SEL);
}

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ float dot2_f16(f16x2_t a, f16x2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Wave-wide (64 lanes) sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Code of weight i (0..7) in a prepared q4k word.
__device__ __forceinline__ uint32_t q4k_code(uint32_t word, int i) {
    return (word >> (16 * (i & 1) + 4 * (i >> 1))) & 15u;
}

// q4k field f (6 bits) from the prepared 16-byte meta record.
__device__ __forceinline__ uint32_t q4k_field(uint32_t lo8, uint32_t hi8, uint32_t top, int f) {
    uint32_t nib = f < 8 ? (lo8 >> (4 * f)) & 15u : (hi8 >> (4 * (f - 8))) & 15u;
    return nib | (((top >> (2 * f)) & 3u) << 4);
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Scalar-path decoders of the prepared layouts (used by the generic kernels).
// NB is the block count of the whole stack; bl a block index in the stack.
// cb4 / sgn are the fp4 codebook rows and spread sign words (LDS tables).
// ---------------------------------------------------------------------------

// Eight weights of sub-group sg (0..31) of iq2x block bl, exact.
__device__ __forceinline__ void iq2x_sub8(const uint8_t *prep, int64_t NB, int64_t bl, int sg, const uint32_t *cb4,
                                          const uint32_t *sgn, float w[8]) {
    const int g = sg >> 2, p = sg & 3;
    const uint16_t *F = reinterpret_cast<const uint16_t *>(prep + bl * 64) + (g & 3) * 8 + (g >> 2) * 4;
    uint32_t s = ((F[0] >> 15) & 1u) | (((F[1] >> 15) & 1u) << 1) | (((F[2] >> 15) & 1u) << 2) |
                 (((F[3] >> 15) & 1u) << 3);
    uint32_t f = F[p];
    float S = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(prep + NB * 64)[bl]) * (float)(2 * s + 1);
    uint32_t word = cb4[f & 0xFF] | sgn[(f >> 8) & 0x7F];
    f32x2_t a = fp4x2_f32<0>(word), b = fp4x2_f32<1>(word), c = fp4x2_f32<2>(word), d = fp4x2_f32<3>(word);
    w[0] = S * a.x; w[1] = S * a.y; w[2] = S * b.x; w[3] = S * b.y;
    w[4] = S * c.x; w[5] = S * c.y; w[6] = S * d.x; w[7] = S * d.y;
}

// Sixteen weights of sub-block j (0..15) of q2k block bl, exact.
__device__ __forceinline__ void q2k_sub16(const uint8_t *prep, int64_t NB, int64_t bl, int j, float w[16]) {
    uint32_t v = reinterpret_cast<const uint32_t *>(prep + bl * 64)[j];
    uint32_t sm = prep[NB * 64 + bl * 16 + j];
    uint32_t dd = reinterpret_cast<const uint32_t *>(prep + NB * 80)[bl];
    float sc = 2.0f * f16_bits_to_f32(dd & 0xFFFF) * (float)(sm & 15u);   // codes decode to q/2
    float mn = f16_bits_to_f32(dd >> 16) * (float)(sm >> 4);
    uint32_t lo = v & 0x33333333u, hi = (v >> 2) & 0x33333333u;
    f32x2_t a;
    a = fp4x2_f32<0>(lo); w[0] = sc * a.x - mn; w[1] = sc * a.y - mn;
    a = fp4x2_f32<1>(lo); w[2] = sc * a.x - mn; w[3] = sc * a.y - mn;
    a = fp4x2_f32<2>(lo); w[4] = sc * a.x - mn; w[5] = sc * a.y - mn;
    a = fp4x2_f32<3>(lo); w[6] = sc * a.x - mn; w[7] = sc * a.y - mn;
    a = fp4x2_f32<0>(hi); w[8] = sc * a.x - mn; w[9] = sc * a.y - mn;
    a = fp4x2_f32<1>(hi); w[10] = sc * a.x - mn; w[11] = sc * a.y - mn;
    a = fp4x2_f32<2>(hi); w[12] = sc * a.x - mn; w[13] = sc * a.y - mn;
    a = fp4x2_f32<3>(hi); w[14] = sc * a.x - mn; w[15] = sc * a.y - mn;
}

// Eight weights of 8-weight unit u (0..31) of q4k block bl, exact.
__device__ __forceinline__ void q4k_sub8(const uint8_t *prep, int64_t NB, int64_t bl, int u, float w[8]) {
    uint32_t v = reinterpret_cast<const uint32_t *>(prep + bl * 128)[u];
    const uint32_t *M = reinterpret_cast<const uint32_t *>(prep + NB * 128 + bl * 16);
    const int j = u >> 2;
    float sc = f16_bits_to_f32(M[0] & 0xFFFF) * (float)q4k_field(M[1], M[2], M[3], j);
    float mn = f16_bits_to_f32(M[0] >> 16) * (float)q4k_field(M[1], M[2], M[3], 8 + j);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = sc * (float)q4k_code(v, i) - mn;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Power-of-two exponent s of a token's routed SwiGLU output h, from the largest magnitude of its activations:
// h grows as |x|^2, so the fp16 copy of h carries h * 2^-s, which stays near unit scale whatever the input range
// (s = 0 for a largest |x| in [2, 4)); the down projection multiplies its sums by 2^s.  Every kernel derives s
// from the same bf16 x row, so all of them agree.
__device__ __forceinline__ int h_sigma(float max_abs_x) {
    if (!(max_abs_x > 0.f)) return 0;
    return min(max(2 * (ilogbf(max_abs_x) - 1), -100), 100);
}

// Wave-wide maximum of a non-negative float, the same in every lane: within each row of 16 lanes by DPP (quad
// swaps 1 and 2, half-row mirror, row mirror), then across the four rows from one lane of each.
template <int CTRL> __device__ __forceinline__ float fmax_dpp(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                               false)));
}
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmax_dpp<0xB1>(v);
    v = fmax_dpp<0x4E>(v);
    v = fmax_dpp<0x141>(v);
    v = fmax_dpp<0x140>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// largest magnitude of the two bf16 values in a word
__device__ __forceinline__ float bf16x2_absmax(uint32_t w) {
    return fmaxf(fabsf(__uint_as_float(w << 16)), fabsf(__uint_as_float(w & 0xFFFF0000u)));
}

// Running largest magnitude over bf16 pairs, kept as two 16-bit fields: with the sign bits cleared, bf16 bit
// patterns order as the magnitudes they encode, so one packed 16-bit integer maximum per word does the update.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_absmax_acc(uint32_t acc, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, acc),
                                                                  __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu)));
}
// the larger of the two fields, as a float
__device__ __forceinline__ float bf16x2_absmax_value(uint32_t acc) {
    return __uint_as_float(max(acc << 16, acc & 0xFFFF0000u));
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Top-k selection keys.  Expert e with logit l has the 64-bit key (orderable
// bits of l + 0, then 255 - e): a larger key is a larger logit, ties going to
// the lower index, and keys are distinct.  -0 compares equal to +0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long logit_key(float l, int e) {
    const uint32_t u = __float_as_uint(l + 0.0f);
    const uint32_t ord = u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
    return ((unsigned long long)ord << 32) | (uint32_t)(255 - e);
}
__device__ __forceinline__ int key_expert(unsigned long long m) { return 255 - (int)(uint32_t)m; }

// max(m, m of the lane that DPP control CTRL reads), 64-bit; every CTRL used here gives every lane a source
template <int CTRL> __device__ __forceinline__ unsigned long long max_dpp_u64(unsigned long long m) {
    const int lo = (int)(uint32_t)m, hi = (int)(uint32_t)(m >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
    const unsigned long long o = ((unsigned long long)ohi << 32) | olo;
    return o > m ? o : m;
}

__device__ __forceinline__ unsigned long long lane_u64(unsigned long long m, int l) {
    return ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(m >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, l);
}

// Wave-wide maximum of a 64-bit value: within each row of 16 lanes by DPP (quad swaps 1 and 2, half-row
// mirror, row mirror), then across the four rows from one lane of each.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long m) {
    m = max_dpp_u64<0xB1>(m);          // quad_perm [1,0,3,2]
    m = max_dpp_u64<0x4E>(m);          // quad_perm [2,3,0,1]
    m = max_dpp_u64<0x141>(m);         // row_half_mirror
    m = max_dpp_u64<0x140>(m);         // row_mirror
    const unsigned long long a = lane_u64(m, 0), b = lane_u64(m, 16), c = lane_u64(m, 32), d = lane_u64(m, 48);
    const unsigned long long ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

}  // namespace moe
