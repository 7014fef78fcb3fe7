// Routing: router logits, top-k with renormalised softmax weights, and the
// token-to-expert permutation.
//
// The pages keep the router at full precision ("antirez가 만든 DeepSeek V4 Flash 전용
// 로컬 추론 엔진 ds4", summary bullets on 2-bit quantization) and do not say how
// its sum is formed.  Reading used here (and by the reference implementation in
// the test suite): products are exact in binary64; the 64 lanes of a wave are
// the 64 partial sums (lane p takes h = p, p+64, ... in increasing h), folded by
// the tree p[i] += p[i+s], s = 32..1, and rounded once to fp32.  The selected
// experts are therefore bit-reproducible whatever the tiling.
#include "common.h"
#include "internal.h"

using namespace moe;

namespace {

template <bool BF16> __device__ __forceinline__ double ld(const void *p, int64_t i) {
    if constexpr (BF16) return (double)bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return (double)static_cast<const float *>(p)[i];
}

// One wave computes TT tokens x EE experts; lane = partial-sum index.
template <bool XB, bool WB, int TT, int EE>
__global__ __launch_bounds__(256) void k_router_logits(const void *__restrict__ x, const void *__restrict__ w,
                                                       const float *__restrict__ bias, int T, int H, int E,
                                                       float *__restrict__ logits, float *__restrict__ logits_copy) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e0 = (blockIdx.x * 4 + wv) * EE;
    const int t0 = blockIdx.y * TT;
    if (e0 >= E) return;
    double acc[TT][EE];
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < EE; ++b) acc[a][b] = 0.0;
    int tt[TT], ee[EE];
#pragma unroll
    for (int a = 0; a < TT; ++a) tt[a] = min(t0 + a, T - 1);       // ragged tail: recompute the last row, not stored
#pragma unroll
    for (int b = 0; b < EE; ++b) ee[b] = min(e0 + b, E - 1);
#pragma unroll 4
    for (int h = lane; h < H; h += 64) {
        double xv[TT], wv_[EE];
#pragma unroll
        for (int a = 0; a < TT; ++a) xv[a] = ld<XB>(x, (int64_t)tt[a] * H + h);
#pragma unroll
        for (int b = 0; b < EE; ++b) wv_[b] = ld<WB>(w, (int64_t)ee[b] * H + h);
#pragma unroll
        for (int a = 0; a < TT; ++a)
#pragma unroll
            for (int b = 0; b < EE; ++b) acc[a][b] = __fma_rn(wv_[b], xv[a], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < EE; ++b) {
            double v = acc[a][b];
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
            if (lane == 0 && t0 + a < T && e0 + b < E) {
                float l = (float)v;
                if (bias) l = (float)((double)l + (double)bias[e0 + b]);
                logits[(int64_t)(t0 + a) * E + e0 + b] = l;
                if (logits_copy) logits_copy[(int64_t)(t0 + a) * E + e0 + b] = l;
            }
        }
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);        // larger logit, then lower index
}

// One wave per token: k rounds of wave-wide argmax, then softmax over the
// selected logits in binary64 (selected logit j is kept by lane j % 64).
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E, int k,
                                              int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    float v[4], sel[4] = {0.f, 0.f, 0.f, 0.f};
    bool taken[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = lane + 64 * i;
        v[i] = e < E ? logits[(int64_t)t * E + e] : 0.0f;
        taken[i] = e >= E;
    }
    float l0 = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = lane + 64 * i;
            if (!taken[i] && (bi == 0x7fffffff || better(v[i], e, bv, bi))) { bv = v[i]; bi = e; }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (lane + 64 * i == bi) taken[i] = true;
            if ((j >> 6) == i && (j & 63) == lane) sel[i] = bv;
        }
        if (j == 0) l0 = bv;
        if (lane == 0) topk_idx[(int64_t)t * k + j] = bi;
    }
    double ex[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ex[i] = exp((double)sel[i] - (double)l0);
    double den = 0.0;
    for (int jj = 0; jj < k; ++jj) {
        int i = jj >> 6;
        double vv = i == 0 ? ex[0] : (i == 1 ? ex[1] : (i == 2 ? ex[2] : ex[3]));
        den += __shfl(vv, jj & 63, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int j = lane + 64 * i;
        if (j < k) topk_w[(int64_t)t * k + j] = (float)(ex[i] / den);
    }
}

// Stable counting sort of the T*k slots by expert (one workgroup).  Each token
// carries k distinct experts, so inside a tile of tokens the rank of slot
// (t, e) among expert e's slots is the number of tile tokens before t that
// chose e: a popcount over a per-expert token bitmap.
constexpr int PERM_TILE = 1024;                    // tokens per tile
constexpr int PERM_WORDS = PERM_TILE / 64;         // bitmap words per expert

__global__ __launch_bounds__(1024) void k_permute(const int32_t *__restrict__ topk_idx, int T, int k, int E,
                                                  int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                  int32_t *__restrict__ active) {
    __shared__ unsigned long long bm[256 * PERM_WORDS];
    __shared__ uint16_t wpre[256 * PERM_WORDS];
    __shared__ int cnt[256], base[256], tilecnt[256];
    const int tid = threadIdx.x;
    const int64_t S = (int64_t)T * k;
    if (tid < 256) cnt[tid] = 0;
    __syncthreads();
    for (int64_t s = tid; s < S; s += blockDim.x) atomicAdd(&cnt[topk_idx[s]], 1);
    __syncthreads();
    // exclusive scans of the counts and of the active flags (256 entries, one wave)
    if (tid < 64) {
        int c[4], a[4], cs = 0, as = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = 4 * tid + i;
            c[i] = e < E ? cnt[e] : 0;
            a[i] = c[i] > 0;
            cs += c[i];
            as += a[i];
        }
        int ci = cs, ai = as;                       // inclusive scan over lanes
        for (int o = 1; o < 64; o <<= 1) {
            int u = __shfl_up(ci, o, 64), v = __shfl_up(ai, o, 64);
            if (tid >= o) { ci += u; ai += v; }
        }
        int cpre = ci - cs, apre = ai - as;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = 4 * tid + i;
            if (e < E) {
                offsets[e] = cpre;
                base[e] = cpre;
                if (a[i]) active[1 + apre] = e;
            }
            cpre += c[i];
            apre += a[i];
        }
        if (tid == 63) {
            offsets[E] = ci;
            active[0] = ai;
        }
    }
    __syncthreads();
    for (int t0 = 0; t0 < T; t0 += PERM_TILE) {
        const int nt = min(PERM_TILE, T - t0);
        for (int i = tid; i < 256 * PERM_WORDS; i += blockDim.x) bm[i] = 0ull;
        __syncthreads();
        for (int i = tid; i < nt * k; i += blockDim.x) {
            int tt = i / k;
            int e = topk_idx[(int64_t)(t0 + tt) * k + (i % k)];
            atomicOr(&bm[e * PERM_WORDS + (tt >> 6)], 1ull << (tt & 63));
        }
        __syncthreads();
        if (tid < E) {
            int run = 0;
            for (int wd = 0; wd < PERM_WORDS; ++wd) {
                wpre[tid * PERM_WORDS + wd] = (uint16_t)run;
                run += __popcll(bm[tid * PERM_WORDS + wd]);
            }
            tilecnt[tid] = run;
        }
        __syncthreads();
        for (int i = tid; i < nt * k; i += blockDim.x) {
            int tt = i / k;
            int64_t s = (int64_t)(t0 + tt) * k + (i % k);
            int e = topk_idx[s];
            int wd = tt >> 6;
            unsigned long long below = bm[e * PERM_WORDS + wd] & ((1ull << (tt & 63)) - 1ull);
            perm[base[e] + wpre[e * PERM_WORDS + wd] + __popcll(below)] = (int32_t)s;
        }
        __syncthreads();
        if (tid < E) base[tid] += tilecnt[tid];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Small batches (T <= 8: decode and verify).  Two launches instead of three.
// ---------------------------------------------------------------------------
constexpr int SMALL_T = 8;

// One wave per (expert, token), grid (E/4, T).  Lane p holds partial p and
// issues all its H/64 loads before the first multiply, so the latency of the
// strided loads is paid once; the sum order is the same as k_router_logits.
template <bool XB, bool WB, int NJ>
__global__ __launch_bounds__(256) void k_router_logits_small(const void *__restrict__ x, const void *__restrict__ w,
                                                             const float *__restrict__ bias, int E,
                                                             float *__restrict__ logits,
                                                             float *__restrict__ logits_copy) {
    constexpr int H = 64 * NJ;
    const int lane = threadIdx.x & 63, e = blockIdx.x * 4 + (threadIdx.x >> 6), t = blockIdx.y;
    if (e >= E) return;
    float wv[NJ], xv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        wv[j] = (float)ld<WB>(w, (int64_t)e * H + lane + 64 * j);
        xv[j] = (float)ld<XB>(x, (int64_t)t * H + lane + 64 * j);
    }
    double v = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) v = __fma_rn((double)wv[j], (double)xv[j], v);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
    if (lane == 0) {
        float l = (float)v;
        if (bias) l = (float)((double)l + (double)bias[e]);
        logits[(int64_t)t * E + e] = l;
        if (logits_copy) logits_copy[(int64_t)t * E + e] = l;
    }
}

// max(m, m of the lane that DPP control CTRL reads), 64-bit; every CTRL used here gives every lane a source
template <int CTRL> __device__ __forceinline__ unsigned long long max_dpp(unsigned long long m) {
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
    m = max_dpp<0xB1>(m);          // quad_perm [1,0,3,2]
    m = max_dpp<0x4E>(m);          // quad_perm [2,3,0,1]
    m = max_dpp<0x141>(m);         // row_half_mirror
    m = max_dpp<0x140>(m);         // row_mirror
    const unsigned long long a = lane_u64(m, 0), b = lane_u64(m, 16), c = lane_u64(m, 32), d = lane_u64(m, 48);
    const unsigned long long ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

// Top-k, weights and permutation for T <= 8 tokens in one workgroup of 1024
// threads.  Expert e of token t carries the key (orderable logit bits, then
// 255 - e): a larger key is a larger logit, ties going to the lower index, and
// keys are distinct.  For one or two tokens the rank of e is the number of
// larger keys, counted in four quarters by four threads (all 16 waves busy);
// ranks below k are the selection, already in order.  For more tokens wave t
// selects token t's experts: k rounds of a wave-wide maximum over the
// remaining keys (each lane holds four), the winner leaving the set.  Slot
// s = t*k + j then goes to position offsets[e] + (the number of earlier slots
// with the same expert).
__global__ __launch_bounds__(1024) void k_select_small(const float *__restrict__ logits, int T, int E, int k,
                                                       int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ active) {
    constexpr int RANK_T = 2;
    __shared__ float lg[SMALL_T][256];
    __shared__ __attribute__((aligned(16))) unsigned long long key[RANK_T][256];
    __shared__ uint8_t part[4][RANK_T][256];                               // at most 64 larger keys per quarter
    __shared__ int sel[SMALL_T * 256];
    __shared__ double ex[SMALL_T][256];
    __shared__ int cnt[256];
    __shared__ uint32_t tmask[256];                                        // bit t: token t selected the expert
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid < 256) {
        cnt[tid] = 0;
        tmask[tid] = 0u;
    }
    if (T <= RANK_T) {
        const int e = tid & 255, q = tid >> 8;
        if (q < T) {
            const float l = e < E ? logits[q * E + e] : 0.f;
            lg[q][e] = l;
            const uint32_t u = __float_as_uint(l + 0.0f);                   // -0 compares equal to +0
            const uint32_t ord = u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
            key[q][e] = e < E ? (((unsigned long long)ord << 32) | (uint32_t)(255 - e)) : 0ull;
        }
        __syncthreads();
        for (int t = 0; t < T; ++t) {
            const unsigned long long me = key[t][e];
            const ulonglong2 *row = reinterpret_cast<const ulonglong2 *>(&key[t][64 * q]);
            int r = 0;
#pragma unroll
            for (int o2 = 0; o2 < 32; ++o2) {
                const ulonglong2 u = row[o2];
                r += (u.x > me ? 1 : 0) + (u.y > me ? 1 : 0);
            }
            part[q][t][e] = (uint8_t)r;
        }
        __syncthreads();
        if (q < T && e < E) {
            const int r = part[0][q][e] + part[1][q][e] + part[2][q][e] + part[3][q][e];
            if (r < k) sel[q * k + r] = e;
        }
    } else if (wv < T) {
        unsigned long long kk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            const float l = e < E ? logits[wv * E + e] : 0.f;
            lg[wv][e] = l;
            const uint32_t u = __float_as_uint(l + 0.0f);                   // -0 compares equal to +0
            const uint32_t ord = u ^ ((u >> 31) ? 0xFFFFFFFFu : 0x80000000u);
            kk[i] = e < E ? (((unsigned long long)ord << 32) | (uint32_t)(255 - e)) : 0ull;
        }
        for (int j = 0; j < k; ++j) {
            const unsigned long long m1 = kk[0] > kk[1] ? kk[0] : kk[1];
            const unsigned long long m2 = kk[2] > kk[3] ? kk[2] : kk[3];
            const unsigned long long m = wave_max_u64(m1 > m2 ? m1 : m2);
            if (lane == 0) sel[wv * k + j] = 255 - (int)(uint32_t)m;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kk[i] == m) kk[i] = 0ull;                               // keys are distinct: one owner
        }
    }
    __syncthreads();
    const int S = T * k;
    // softmax over the selected logits, binary64; per-expert slot counts and token sets
    for (int s = tid; s < S; s += 1024) {
        const int t = s / k, x = sel[s];
        ex[t][s % k] = exp((double)lg[t][x] - (double)lg[t][sel[t * k]]);
        atomicAdd(&cnt[x], 1);
        atomicOr(&tmask[x], 1u << t);
    }
    __syncthreads();
    for (int s = tid; s < S; s += 1024) {
        const int t = s / k;
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += ex[t][j];
        topk_idx[s] = sel[s];
        topk_w[s] = (float)(ex[t][s % k] / den);
    }
    // offsets and the active list: exclusive scans over the experts (one wave)
    if (tid < 64) {
        int c[4], a[4], cs = 0, as = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int x = 4 * tid + i;
            c[i] = x < E ? cnt[x] : 0;
            a[i] = c[i] > 0;
            cs += c[i];
            as += a[i];
        }
        int ci = cs, ai = as;
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(ci, o, 64), v = __shfl_up(ai, o, 64);
            if (tid >= o) { ci += u; ai += v; }
        }
        int cpre = ci - cs, apre = ai - as;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int x = 4 * tid + i;
            if (x < E) {
                offsets[x] = cpre;
                cnt[x] = cpre;                   // becomes the expert's base position
                if (a[i]) active[1 + apre] = x;
            }
            cpre += c[i];
            apre += a[i];
        }
        if (tid == 63) {
            offsets[E] = ci;
            active[0] = ai;
        }
    }
    __syncthreads();
    // slot s = t*k + j follows the expert's slots of earlier tokens (a token holds an expert at most once)
    for (int s = tid; s < S; s += 1024) {
        const int x = sel[s], t = s / k;
        perm[cnt[x] + __popc(tmask[x] & ((1u << t) - 1u))] = s;
    }
}

template <bool XB, bool WB>
hipError_t launch_logits(const RouteArgs &a, hipStream_t st) {
    if (a.T == 1) {
        dim3 grd((a.E + 3) / 4, 1);
        hipLaunchKernelGGL((k_router_logits<XB, WB, 1, 1>), grd, dim3(256), 0, st, a.x, a.w, a.bias, a.T, a.H, a.E,
                           a.logits_ws, a.logits_out);
    } else if (a.T <= 4) {
        dim3 grd((a.E + 3) / 4, 1);
        hipLaunchKernelGGL((k_router_logits<XB, WB, 4, 1>), grd, dim3(256), 0, st, a.x, a.w, a.bias, a.T, a.H, a.E,
                           a.logits_ws, a.logits_out);
    } else {
        dim3 grd((a.E + 15) / 16, (a.T + 3) / 4);
        hipLaunchKernelGGL((k_router_logits<XB, WB, 4, 4>), grd, dim3(256), 0, st, a.x, a.w, a.bias, a.T, a.H, a.E,
                           a.logits_ws, a.logits_out);
    }
    return hipGetLastError();
}

}  // namespace

namespace moe {

template <bool XB, bool WB>
hipError_t launch_logits_small(const RouteArgs &a, hipStream_t st) {
    const dim3 grd((a.E + 3) / 4, a.T);
#define MOE_LOGITS(NJ_)                                                                                      \
    case 64 * NJ_:                                                                                           \
        hipLaunchKernelGGL((k_router_logits_small<XB, WB, NJ_>), grd, dim3(256), 0, st, a.x, a.w, a.bias, a.E, \
                           a.logits_ws, a.logits_out);                                                       \
        break;
    switch (a.H) {
        MOE_LOGITS(64)
        MOE_LOGITS(32)
        MOE_LOGITS(16)
        MOE_LOGITS(8)
        MOE_LOGITS(4)
        default: return hipErrorInvalidValue;
    }
#undef MOE_LOGITS
    return hipGetLastError();
}

bool small_logits_shape(int H) { return H == 4096 || H == 2048 || H == 1024 || H == 512 || H == 256; }

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
    hipError_t e;
    if (a.T <= SMALL_T && small_logits_shape(a.H)) {
        if (a.x_bf16 && a.w_bf16) e = launch_logits_small<true, true>(a, st);
        else if (a.x_bf16) e = launch_logits_small<true, false>(a, st);
        else if (a.w_bf16) e = launch_logits_small<false, true>(a, st);
        else e = launch_logits_small<false, false>(a, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_select_small, dim3(1), dim3(1024), 0, st, a.logits_ws, a.T, a.E, a.k, a.topk_idx, a.topk_w,
                           a.offsets, a.perm, a.active);
        return hipGetLastError();
    }
    if (a.x_bf16 && a.w_bf16) e = launch_logits<true, true>(a, st);
    else if (a.x_bf16) e = launch_logits<true, false>(a, st);
    else if (a.w_bf16) e = launch_logits<false, true>(a, st);
    else e = launch_logits<false, false>(a, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_topk, dim3((a.T + 3) / 4), dim3(256), 0, st, a.logits_ws, a.T, a.E, a.k, a.topk_idx,
                       a.topk_w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, st, a.topk_idx, a.T, a.k, a.E, a.offsets, a.perm, a.active);
    return hipGetLastError();
}

}  // namespace moe
