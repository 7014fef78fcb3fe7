// Top-k weighted combine: y[t] = sum_{j<k} w[t][j] * o[t*k+j] (+ s[t]), j in order,
// optionally followed by directional steering y[t] -= F * v * dot(v, y[t]).
#include "common.h"
#include "internal.h"

namespace {

__device__ __forceinline__ float4 ld4(const float *p, int c) { return reinterpret_cast<const float4 *>(p)[c]; }

__device__ __forceinline__ void fma4(float a, const float4 &b, float4 &acc) {
    acc.x = __fmaf_rn(a, b.x, acc.x);
    acc.y = __fmaf_rn(a, b.y, acc.y);
    acc.z = __fmaf_rn(a, b.z, acc.z);
    acc.w = __fmaf_rn(a, b.w, acc.w);
}

// Four consecutive outputs c*4..c*4+3 of token t.  With the top-k known at compile time (KC > 0) every slot row is
// loaded before the first product, so one thread has all k + 1 loads in flight at once; the arithmetic is the same
// either way: acc starts at 0, one fused multiply-add per slot in slot order, then the shared row is added.
template <int KC>
__device__ __forceinline__ float4 combine4(const float *__restrict__ o, const float *__restrict__ w,
                                          const float *__restrict__ s, int t, int k, int H, int c) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (KC > 0) {
        float4 ov[KC];
        float wj[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            ov[j] = ld4(o + ((int64_t)t * KC + j) * H, c);
            wj[j] = w[(int64_t)t * KC + j];
        }
        const float4 sv = s ? ld4(s + (int64_t)t * H, c) : acc;
#pragma unroll
        for (int j = 0; j < KC; ++j) fma4(wj[j], ov[j], acc);
        if (s) { acc.x += sv.x; acc.y += sv.y; acc.z += sv.z; acc.w += sv.w; }
    } else {
        for (int j = 0; j < k; ++j) fma4(w[(int64_t)t * k + j], ld4(o + ((int64_t)t * k + j) * H, c), acc);
        if (s) {
            const float4 sv = ld4(s + (int64_t)t * H, c);
            acc.x += sv.x; acc.y += sv.y; acc.z += sv.z; acc.w += sv.w;
        }
    }
    return acc;
}

__device__ __forceinline__ float combine1(const float *__restrict__ o, const float *__restrict__ w,
                                          const float *__restrict__ s, int t, int k, int H, int c) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = __fmaf_rn(w[(int64_t)t * k + j], o[((int64_t)t * k + j) * H + c], acc);
    if (s) acc += s[(int64_t)t * H + c];
    return acc;
}

// One thread per 4 consecutive outputs (VEC: H % 4 == 0 and 16-byte aligned rows) or per output.
template <bool VEC, int KC>
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ o, const float *__restrict__ w,
                                                 const float *__restrict__ s, int T, int k, int H,
                                                 float *__restrict__ y) {
    const int per_t = VEC ? H / 4 : H;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * per_t) return;
    const int t = (int)(i / per_t), c = (int)(i % per_t);
    if constexpr (VEC) reinterpret_cast<float4 *>(y + (int64_t)t * H)[c] = combine4<KC>(o, w, s, t, k, H, c);
    else y[(int64_t)t * H + c] = combine1(o, w, s, t, k, H, c);
}

constexpr int ST_THREADS = 1024;

// Sum over the workgroup in a fixed order (lanes by xor butterfly, then the waves in index order); every thread
// gets the same value.
__device__ __forceinline__ float block_sum(float d, float *part) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = d;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += part[i];
    return tot;
}

// Combine + steering, one workgroup per token; each thread keeps RV groups of 4 outputs in registers between the
// dot product and the update.  Needs H % 4 == 0, 16-byte aligned rows and H / 4 <= ST_THREADS * RV.
template <int KC, int RV>
__global__ __launch_bounds__(ST_THREADS) void k_combine_steer(const float *__restrict__ o,
                                                              const float *__restrict__ w,
                                                              const float *__restrict__ s, int k, int H,
                                                              const float *__restrict__ v, float F,
                                                              float *__restrict__ y) {
    __shared__ float part[ST_THREADS / 64];
    const int t = blockIdx.x, n4 = H >> 2;
    float4 acc[RV], vv[RV];
    float d = 0.f;
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        const int c = (int)threadIdx.x + r * ST_THREADS;
        if (c < n4) {
            vv[r] = ld4(v, c);
            acc[r] = combine4<KC>(o, w, s, t, k, H, c);
            d = __fmaf_rn(vv[r].x, acc[r].x, d);
            d = __fmaf_rn(vv[r].y, acc[r].y, d);
            d = __fmaf_rn(vv[r].z, acc[r].z, d);
            d = __fmaf_rn(vv[r].w, acc[r].w, d);
        }
    }
    const float sf = -F * block_sum(d, part);
    float4 *yt = reinterpret_cast<float4 *>(y + (int64_t)t * H);
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        const int c = (int)threadIdx.x + r * ST_THREADS;
        if (c < n4) {
            float4 out = acc[r];
            fma4(sf, vv[r], out);
            yt[c] = out;
        }
    }
}

// Any H and alignment: the dot product in a first pass, then the combine is recomputed (same order, so the same
// values) and updated in a second pass.
__global__ __launch_bounds__(ST_THREADS) void k_combine_steer_any(const float *__restrict__ o,
                                                                  const float *__restrict__ w,
                                                                  const float *__restrict__ s, int k, int H,
                                                                  const float *__restrict__ v, float F,
                                                                  float *__restrict__ y) {
    __shared__ float part[ST_THREADS / 64];
    const int t = blockIdx.x;
    float d = 0.f;
    for (int c = threadIdx.x; c < H; c += ST_THREADS) d = __fmaf_rn(v[c], combine1(o, w, s, t, k, H, c), d);
    const float sf = -F * block_sum(d, part);
    for (int c = threadIdx.x; c < H; c += ST_THREADS)
        y[(int64_t)t * H + c] = __fmaf_rn(sf, v[c], combine1(o, w, s, t, k, H, c));
}

template <int KC>
hipError_t launch_steer_vec(int rv, const float *o, const float *w, const float *s, int T, int k, int H,
                            const float *v, float F, float *y, hipStream_t st) {
    if (rv == 1) hipLaunchKernelGGL((k_combine_steer<KC, 1>), dim3(T), dim3(ST_THREADS), 0, st, o, w, s, k, H, v, F, y);
    else hipLaunchKernelGGL((k_combine_steer<KC, 2>), dim3(T), dim3(ST_THREADS), 0, st, o, w, s, k, H, v, F, y);
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p % 16) == 0; }

}  // namespace

namespace moe {

hipError_t launch_combine(const float *slot_out, const float *topk_w, const float *shared_out, int T, int k, int H,
                          float *y, hipStream_t st) {
    const bool vec = (H % 4) == 0 && aligned16(slot_out) && aligned16(y) &&
                     (shared_out == nullptr || aligned16(shared_out));
    const int64_t n = (int64_t)T * (vec ? H / 4 : H);
    // small batches: 64-thread workgroups spread the rows over more compute units
    const int bs = n <= 16384 ? 64 : 256;
    dim3 grd((unsigned)((n + bs - 1) / bs)), blk(bs);
    if (!vec) hipLaunchKernelGGL((k_combine<false, 0>), grd, blk, 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    else if (k == 8) hipLaunchKernelGGL((k_combine<true, 8>), grd, blk, 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    else if (k == 4) hipLaunchKernelGGL((k_combine<true, 4>), grd, blk, 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    else hipLaunchKernelGGL((k_combine<true, 0>), grd, blk, 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    return hipGetLastError();
}

hipError_t launch_combine_steer(const float *slot_out, const float *topk_w, const float *shared_out, int T, int k,
                                int H, const float *v, float F, float *y, hipStream_t st) {
    const bool vec = (H % 4) == 0 && aligned16(slot_out) && aligned16(y) && aligned16(v) &&
                     (shared_out == nullptr || aligned16(shared_out)) && H / 4 <= 2 * ST_THREADS;
    if (!vec) {
        hipLaunchKernelGGL(k_combine_steer_any, dim3(T), dim3(ST_THREADS), 0, st, slot_out, topk_w, shared_out, k, H,
                           v, F, y);
        return hipGetLastError();
    }
    const int rv = H / 4 <= ST_THREADS ? 1 : 2;
    if (k == 8) return launch_steer_vec<8>(rv, slot_out, topk_w, shared_out, T, k, H, v, F, y, st);
    if (k == 4) return launch_steer_vec<4>(rv, slot_out, topk_w, shared_out, T, k, H, v, F, y, st);
    return launch_steer_vec<0>(rv, slot_out, topk_w, shared_out, T, k, H, v, F, y, st);
}

}  // namespace moe
