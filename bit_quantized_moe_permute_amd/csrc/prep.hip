// Weight preparation (canonical blocks -> device layout) and the exact fp32
// export of prepared weights.  Both run once per weight load, off the hot path.
#include "common.h"
#include "internal.h"

using namespace moe;

namespace {

__device__ __forceinline__ uint32_t rd32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

__global__ void k_prep_iq2x(const uint8_t *__restrict__ canon, uint8_t *__restrict__ prep, int64_t NB) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= NB) return;
    const uint8_t *c = canon + b * 66;
    uint16_t *Q = reinterpret_cast<uint16_t *>(prep + b * 64);
    uint16_t *D = reinterpret_cast<uint16_t *>(prep + NB * 64);
    D[b] = (uint16_t)(c[0] | (c[1] << 8));
    for (int g = 0; g < 8; ++g) {
        const uint8_t *rec = c + 2 + 8 * g;
        uint32_t aux = rd32(rec + 4);
        uint32_t s = aux >> 28;
        for (int p = 0; p < 4; ++p) {
            uint32_t f = rec[p] | (((aux >> (7 * p)) & 0x7Fu) << 8) | (((s >> p) & 1u) << 15);
            Q[(g & 3) * 8 + (g >> 2) * 4 + p] = (uint16_t)f;
        }
    }
}

__global__ void k_prep_q2k(const uint8_t *__restrict__ canon, uint8_t *__restrict__ prep, int64_t NB) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= NB) return;
    const uint8_t *c = canon + b * 84;
    uint32_t *Q = reinterpret_cast<uint32_t *>(prep + b * 64);
    uint8_t *S = prep + NB * 64 + b * 16;
    uint32_t *D = reinterpret_cast<uint32_t *>(prep + NB * 80);
    D[b] = rd32(c);
    for (int j = 0; j < 16; ++j) S[j] = c[4 + j];
    for (int j = 0; j < 16; ++j) {
        uint32_t v = 0;
        for (int i = 0; i < 8; ++i) {
            int n0 = 16 * j + i, n1 = 16 * j + 8 + i;
            uint32_t q0 = (c[20 + n0 / 4] >> (2 * (n0 % 4))) & 3u;
            uint32_t q1 = (c[20 + n1 / 4] >> (2 * (n1 % 4))) & 3u;
            v |= (q0 << (4 * i)) | (q1 << (4 * i + 2));
        }
        Q[j] = v;
    }
}

__global__ void k_prep_q4k(const uint8_t *__restrict__ canon, uint8_t *__restrict__ prep, int64_t NB) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= NB) return;
    const uint8_t *c = canon + b * 144;
    uint8_t *Q = prep + b * 128;
    uint32_t *M = reinterpret_cast<uint32_t *>(prep + NB * 128 + b * 16);
    for (int u = 0; u < 32; ++u) {                     // 8 weights per word, pairs in the two halves
        uint32_t v = 0;
        for (int i = 0; i < 8; ++i) {
            const int n = 8 * u + i;
            const uint32_t q = (c[16 + n / 2] >> (4 * (n % 2))) & 15u;
            v |= q << (16 * (i & 1) + 4 * (i >> 1));
        }
        reinterpret_cast<uint32_t *>(Q)[u] = v;
    }
    uint32_t lo8 = 0, hi8 = 0, top = 0;
    for (int f = 0; f < 16; ++f) {
        uint32_t v = 0;
        for (int bit = 0; bit < 6; ++bit) {
            int pos = 6 * f + bit;
            v |= ((uint32_t)(c[4 + pos / 8] >> (pos % 8)) & 1u) << bit;
        }
        if (f < 8) lo8 |= (v & 15u) << (4 * f);
        else hi8 |= (v & 15u) << (4 * (f - 8));
        top |= (v >> 4) << (2 * f);
    }
    M[0] = rd32(c);
    M[1] = lo8;
    M[2] = hi8;
    M[3] = top;
}

// ---------------------------------------------------------------------------
// exact export: one thread per 8 consecutive weights
// ---------------------------------------------------------------------------
__global__ void k_dequant_iq2x(const uint8_t *__restrict__ prep, int64_t NB, int64_t blk0, int64_t nblk,
                               const uint8_t *__restrict__ codebook, float *__restrict__ out) {
    __shared__ uint32_t cb4[256];
    __shared__ uint32_t sgn[128];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb4[i] = codebook_row_fp4(codebook, i);
    for (int i = threadIdx.x; i < 128; i += blockDim.x) sgn[i] = sign_spread(i);
    __syncthreads();
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // sub-group index within the range
    if (t >= nblk * 32) return;
    int64_t b = blk0 + (t >> 5);
    int sgi = (int)(t & 31), g = sgi >> 2, p = sgi & 3;
    const uint16_t *Q = reinterpret_cast<const uint16_t *>(prep + b * 64);
    uint32_t f = Q[(g & 3) * 8 + (g >> 2) * 4 + p];
    uint32_t s = 0;
    for (int pp = 0; pp < 4; ++pp) s |= ((uint32_t)(Q[(g & 3) * 8 + (g >> 2) * 4 + pp] >> 15) & 1u) << pp;
    float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(prep + NB * 64)[b]);
    float S = d * (float)(2 * s + 1);
    uint32_t word = cb4[f & 0xFF] | sgn[(f >> 8) & 0x7F];
    float *o = out + t * 8;
    f32x2_t v0 = fp4x2_f32<0>(word), v1 = fp4x2_f32<1>(word), v2 = fp4x2_f32<2>(word), v3 = fp4x2_f32<3>(word);
    o[0] = S * v0.x; o[1] = S * v0.y; o[2] = S * v1.x; o[3] = S * v1.y;
    o[4] = S * v2.x; o[5] = S * v2.y; o[6] = S * v3.x; o[7] = S * v3.y;
}

__global__ void k_dequant_q2k(const uint8_t *__restrict__ prep, int64_t NB, int64_t blk0, int64_t nblk,
                              float *__restrict__ out) {
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // sub-block index (16 weights) within the range
    if (t >= nblk * 16) return;
    int64_t b = blk0 + (t >> 4);
    int j = (int)(t & 15);
    uint32_t v = reinterpret_cast<const uint32_t *>(prep + b * 64)[j];
    uint32_t sm = prep[NB * 64 + b * 16 + j];
    uint32_t dd = reinterpret_cast<const uint32_t *>(prep + NB * 80)[b];
    float d2 = 2.0f * f16_bits_to_f32(dd & 0xFFFF);                  // codes decode to q/2
    float mn = f16_bits_to_f32(dd >> 16) * (float)(sm >> 4);
    float sc = d2 * (float)(sm & 15u);
    uint32_t lo = v & 0x33333333u, hi = (v >> 2) & 0x33333333u;
    float *o = out + t * 16;
    f32x2_t a;
    a = fp4x2_f32<0>(lo); o[0] = sc * a.x - mn; o[1] = sc * a.y - mn;
    a = fp4x2_f32<1>(lo); o[2] = sc * a.x - mn; o[3] = sc * a.y - mn;
    a = fp4x2_f32<2>(lo); o[4] = sc * a.x - mn; o[5] = sc * a.y - mn;
    a = fp4x2_f32<3>(lo); o[6] = sc * a.x - mn; o[7] = sc * a.y - mn;
    a = fp4x2_f32<0>(hi); o[8] = sc * a.x - mn; o[9] = sc * a.y - mn;
    a = fp4x2_f32<1>(hi); o[10] = sc * a.x - mn; o[11] = sc * a.y - mn;
    a = fp4x2_f32<2>(hi); o[12] = sc * a.x - mn; o[13] = sc * a.y - mn;
    a = fp4x2_f32<3>(hi); o[14] = sc * a.x - mn; o[15] = sc * a.y - mn;
}

__global__ void k_dequant_q4k(const uint8_t *__restrict__ prep, int64_t NB, int64_t blk0, int64_t nblk,
                              float *__restrict__ out) {
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-weight unit within the range
    if (t >= nblk * 32) return;
    int64_t b = blk0 + (t >> 5);
    int u = (int)(t & 31), j = u >> 2;
    uint32_t v = reinterpret_cast<const uint32_t *>(prep + b * 128)[u];
    const uint32_t *M = reinterpret_cast<const uint32_t *>(prep + NB * 128 + b * 16);
    float d = f16_bits_to_f32(M[0] & 0xFFFF), dmin = f16_bits_to_f32(M[0] >> 16);
    float sc = d * (float)q4k_field(M[1], M[2], M[3], j);
    float mn = dmin * (float)q4k_field(M[1], M[2], M[3], 8 + j);
    float *o = out + t * 8;
    for (int i = 0; i < 8; ++i) o[i] = sc * (float)q4k_code(v, i) - mn;
}

}  // namespace

namespace moe {

hipError_t launch_prepare(int fmt, int64_t NB, const void *canonical, void *prepared, hipStream_t st) {
    dim3 blk(256), grd((unsigned)((NB + 255) / 256));
    const uint8_t *c = static_cast<const uint8_t *>(canonical);
    uint8_t *p = static_cast<uint8_t *>(prepared);
    if (fmt == 1) hipLaunchKernelGGL(k_prep_iq2x, grd, blk, 0, st, c, p, NB);
    else if (fmt == 2) hipLaunchKernelGGL(k_prep_q2k, grd, blk, 0, st, c, p, NB);
    else hipLaunchKernelGGL(k_prep_q4k, grd, blk, 0, st, c, p, NB);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int64_t NB, int64_t blk0, int64_t nblk, const void *prepared,
                          const uint8_t *codebook, float *out, hipStream_t st) {
    const uint8_t *p = static_cast<const uint8_t *>(prepared);
    dim3 blk(256);
    if (fmt == 1) {
        dim3 grd((unsigned)((nblk * 32 + 255) / 256));
        hipLaunchKernelGGL(k_dequant_iq2x, grd, blk, 0, st, p, NB, blk0, nblk, codebook, out);
    } else if (fmt == 2) {
        dim3 grd((unsigned)((nblk * 16 + 255) / 256));
        hipLaunchKernelGGL(k_dequant_q2k, grd, blk, 0, st, p, NB, blk0, nblk, out);
    } else {
        dim3 grd((unsigned)((nblk * 32 + 255) / 256));
        hipLaunchKernelGGL(k_dequant_q4k, grd, blk, 0, st, p, NB, blk0, nblk, out);
    }
    return hipGetLastError();
}

}  // namespace moe
