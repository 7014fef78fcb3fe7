// Generic expert-FFN kernels: one thread per output row, weights decoded one
// sub-group at a time, fp32 accumulation.  They serve any shape the formats
// allow (e.g. the tiny layer whose down rows are shorter than a block) and fp32
// activations; the decode and grouped-GEMM kernels cover the large layers.
#include "common.h"
#include "internal.h"

using namespace moe;

namespace {

template <bool XB> __device__ __forceinline__ float ldx(const void *x, int64_t i) {
    if constexpr (XB) return bf16_bits_to_f32(static_cast<const uint16_t *>(x)[i]);
    else return static_cast<const float *>(x)[i];
}

__device__ __forceinline__ void build_tables(const uint8_t *codebook, uint32_t *cb4, uint32_t *sgn) {
    if (codebook)
        for (int i = threadIdx.x; i < 256; i += blockDim.x) cb4[i] = codebook_row_fp4(codebook, i);
    for (int i = threadIdx.x; i < 128; i += blockDim.x) sgn[i] = sign_spread(i);
    __syncthreads();
}

// dot of row r of matrix e (rows x cols, stacked) with v[0..cols)
template <bool XB>
__device__ float row_dot(int fmt, const uint8_t *prep, int64_t NB, int64_t nb_mat, int e, int r, int cols,
                         const void *v, int64_t voff, const uint32_t *cb4, const uint32_t *sgn) {
    float acc = 0.0f;
    const int64_t n0 = (int64_t)r * cols;
    if (fmt == FMT_IQ2X || fmt == FMT_Q4K) {
        for (int c = 0; c < cols; c += 8) {
            int64_t n = n0 + c, bl = (int64_t)e * nb_mat + n / MOE_QK;
            int sub = (int)((n % MOE_QK) / 8);
            float w[8];
            if (fmt == FMT_IQ2X) iq2x_sub8(prep, NB, bl, sub, cb4, sgn, w);
            else q4k_sub8(prep, NB, bl, sub, w);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = __fmaf_rn(w[i], ldx<XB>(v, voff + c + i), acc);
        }
    } else {
        for (int c = 0; c < cols; c += 16) {
            int64_t n = n0 + c, bl = (int64_t)e * nb_mat + n / MOE_QK;
            int sub = (int)((n % MOE_QK) / 16);
            float w[16];
            q2k_sub16(prep, NB, bl, sub, w);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc = __fmaf_rn(w[i], ldx<XB>(v, voff + c + i), acc);
        }
    }
    return acc;
}

template <bool XB> __global__ __launch_bounds__(256) void k_gateup_generic(FfnArgs a, float *__restrict__ h) {
    __shared__ uint32_t cb4[256], sgn[128];
    build_tables(a.codebook, cb4, sgn);
    const int nrt = (a.I + 255) / 256;
    const int r = (blockIdx.x % nrt) * 256 + threadIdx.x, s = blockIdx.x / nrt;
    if (r >= a.I) return;
    const int e = a.topk_idx[s], t = s / a.k;
    const int64_t nb_mat = (int64_t)a.I * a.H / MOE_QK, NB = nb_mat * a.E;
    float g = row_dot<XB>(a.fmt_gu, a.gate, NB, nb_mat, e, r, a.H, a.x, (int64_t)t * a.H, cb4, sgn);
    float u = row_dot<XB>(a.fmt_gu, a.up, NB, nb_mat, e, r, a.H, a.x, (int64_t)t * a.H, cb4, sgn);
    h[(int64_t)s * a.I + r] = silu_mul(g, u);
}

__global__ __launch_bounds__(256) void k_down_generic(FfnArgs a, const float *__restrict__ h) {
    __shared__ uint32_t cb4[256], sgn[128];
    build_tables(nullptr, cb4, sgn);
    const int nrt = (a.H + 255) / 256;
    const int r = (blockIdx.x % nrt) * 256 + threadIdx.x, s = blockIdx.x / nrt;
    if (r >= a.H) return;
    const int e = a.topk_idx[s];
    const int64_t nb_mat = (int64_t)a.H * a.I / MOE_QK, NB = nb_mat * a.E;
    a.slot_out[(int64_t)s * a.H + r] =
        row_dot<false>(a.fmt_d, a.down, NB, nb_mat, e, r, a.I, h, (int64_t)s * a.I, cb4, sgn);
}

template <bool XB> __global__ __launch_bounds__(256) void k_shared_gateup_generic(FfnArgs a, float *__restrict__ h) {
    const int nrt = (a.Is + 255) / 256;
    const int r = (blockIdx.x % nrt) * 256 + threadIdx.x, t = blockIdx.x / nrt;
    if (r >= a.Is) return;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < a.H; ++c) {
        float xv = ldx<XB>(a.x, (int64_t)t * a.H + c);
        g = __fmaf_rn(bf16_bits_to_f32(a.sg[(int64_t)r * a.H + c]), xv, g);
        u = __fmaf_rn(bf16_bits_to_f32(a.su[(int64_t)r * a.H + c]), xv, u);
    }
    h[(int64_t)t * a.Is + r] = silu_mul(g, u);
}

__global__ __launch_bounds__(256) void k_shared_down_generic(FfnArgs a, const float *__restrict__ h) {
    const int nrt = (a.H + 255) / 256;
    const int r = (blockIdx.x % nrt) * 256 + threadIdx.x, t = blockIdx.x / nrt;
    if (r >= a.H) return;
    float o = 0.f;
    for (int c = 0; c < a.Is; ++c) o = __fmaf_rn(bf16_bits_to_f32(a.sd[(int64_t)r * a.Is + c]), h[(int64_t)t * a.Is + c], o);
    a.shared_out[(int64_t)t * a.H + r] = o;
}

}  // namespace

namespace moe {

size_t ffn_workspace_generic(int H, int I, int E, int k, int Is, int T) {
    (void)H; (void)E;
    return sizeof(float) * ((size_t)T * k * I + (size_t)T * Is) + 256;
}

hipError_t launch_ffn_generic(const FfnArgs &a, hipStream_t st) {
    float *h = static_cast<float *>(a.ws);
    float *hs = h + (size_t)a.T * a.k * a.I;
    const int S = a.T * a.k;
    hipError_t e = hipSuccess;
    if (a.stages & STAGE_GATE_UP) {
        if (a.x_bf16) hipLaunchKernelGGL(k_gateup_generic<true>, dim3((a.I + 255) / 256 * S), dim3(256), 0, st, a, h);
        else hipLaunchKernelGGL(k_gateup_generic<false>, dim3((a.I + 255) / 256 * S), dim3(256), 0, st, a, h);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.Is > 0) {
            if (a.x_bf16)
                hipLaunchKernelGGL(k_shared_gateup_generic<true>, dim3((a.Is + 255) / 256 * a.T), dim3(256), 0, st, a, hs);
            else
                hipLaunchKernelGGL(k_shared_gateup_generic<false>, dim3((a.Is + 255) / 256 * a.T), dim3(256), 0, st, a,
                                   hs);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if (a.stages & STAGE_DOWN) {
        hipLaunchKernelGGL(k_down_generic, dim3((a.H + 255) / 256 * S), dim3(256), 0, st, a, h);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.Is > 0) {
            hipLaunchKernelGGL(k_shared_down_generic, dim3((a.H + 255) / 256 * a.T), dim3(256), 0, st, a, hs);
            e = hipGetLastError();
        }
    }
    return e;
}

}  // namespace moe
