// Top-k weighted combine: y[t] = sum_{j<k} w[t][j] * o[t*k+j] (+ s[t]), j in order.
#include "common.h"
#include "internal.h"

namespace {

// One thread per 4 consecutive outputs (H % 4 == 0) or per output.
template <bool VEC>
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ o, const float *__restrict__ w,
                                                 const float *__restrict__ s, int T, int k, int H,
                                                 float *__restrict__ y) {
    const int per_t = VEC ? H / 4 : H;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * per_t) return;
    const int t = (int)(i / per_t), c = (int)(i % per_t);
    if constexpr (VEC) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const float wj = w[(int64_t)t * k + j];
            const float4 v = reinterpret_cast<const float4 *>(o + ((int64_t)t * k + j) * H)[c];
            acc.x = __fmaf_rn(wj, v.x, acc.x);
            acc.y = __fmaf_rn(wj, v.y, acc.y);
            acc.z = __fmaf_rn(wj, v.z, acc.z);
            acc.w = __fmaf_rn(wj, v.w, acc.w);
        }
        if (s) {
            const float4 v = reinterpret_cast<const float4 *>(s + (int64_t)t * H)[c];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        reinterpret_cast<float4 *>(y + (int64_t)t * H)[c] = acc;
    } else {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) acc = __fmaf_rn(w[(int64_t)t * k + j], o[((int64_t)t * k + j) * H + c], acc);
        if (s) acc += s[(int64_t)t * H + c];
        y[(int64_t)t * H + c] = acc;
    }
}

}  // namespace

namespace moe {

hipError_t launch_combine(const float *slot_out, const float *topk_w, const float *shared_out, int T, int k, int H,
                          float *y, hipStream_t st) {
    const bool vec = (H % 4) == 0 && ((uintptr_t)slot_out % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     (shared_out == nullptr || ((uintptr_t)shared_out % 16) == 0);
    const int64_t n = (int64_t)T * (vec ? H / 4 : H);
    dim3 grd((unsigned)((n + 255) / 256));
    if (vec) hipLaunchKernelGGL(k_combine<true>, grd, dim3(256), 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    else hipLaunchKernelGGL(k_combine<false>, grd, dim3(256), 0, st, slot_out, topk_w, shared_out, T, k, H, y);
    return hipGetLastError();
}

}  // namespace moe
