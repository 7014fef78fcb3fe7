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

// Stable counting sort of the T*k slots by expert, one 256-thread workgroup per
// expert.  Slots are taken in blocks of PERM_BLK: wave w of the workgroup holds
// slots w*PERM_BLK/4 .. of a block in registers, 64 per lane (slot = block
// start + w*PERM_BLK/4 + 64 j + lane), all requested at once.  Every workgroup
// counts all slots per expert in LDS (the topk array is read from the cache by
// all of them) and takes its expert's offset and active position from the
// exclusive scans of the counts.  Then, per block, each wave counts its matches
// by ballot, the waves' counts give each wave its first position, and the
// matching slots are written in slot order (position = the ballot's lower-lane
// popcount).
constexpr int PERM_BLK = 4 * 64 * 64;              // slots per block: 4 waves x 64 lanes x 64 registers

__global__ __launch_bounds__(256) void k_permute(const int32_t *__restrict__ topk_idx, int T, int k, int E,
                                                 int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                 int32_t *__restrict__ active) {
    __shared__ int cnt[256];
    __shared__ int wsum[4];
    __shared__ int base_e, apre_e;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, e = blockIdx.x;
    const int S = T * k, nblk = (S + PERM_BLK - 1) / PERM_BLK;
    int v[64];
    auto load = [&](int b0) {
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const int sl = b0 + wv * (PERM_BLK / 4) + 64 * j + lane;
            v[j] = sl < S ? topk_idx[sl] : -1;
        }
    };
    cnt[tid] = 0;
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
        load(b * PERM_BLK);
#pragma unroll
        for (int j = 0; j < 64; ++j)
            if (v[j] >= 0) atomicAdd(&cnt[v[j]], 1);
    }
    __syncthreads();
    if (wv == 0) {                                           // exclusive scans of the counts and active flags
        int c[4], cs = 0, as = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ee = 4 * lane + i;
            c[i] = ee < E ? cnt[ee] : 0;
            cs += c[i];
            as += c[i] > 0;
        }
        int ci = cs, ai = as;
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(ci, o, 64), vv = __shfl_up(ai, o, 64);
            if (lane >= o) { ci += u; ai += vv; }
        }
        int cpre = ci - cs, apre = ai - as;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (4 * lane + i == e) { base_e = cpre; apre_e = apre; }
            cpre += c[i];
            apre += c[i] > 0;
        }
        if (e == 0 && lane == 63) {
            offsets[E] = ci;
            active[0] = ai;
        }
    }
    __syncthreads();
    if (tid == 0) {
        offsets[e] = base_e;
        if (cnt[e] > 0) active[1 + apre_e] = e;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    int run = base_e;                                        // this expert's next position
    for (int b = 0; b < nblk; ++b) {
        if (nblk > 1) load(b * PERM_BLK);                    // one block: still in registers
        int c = 0;
#pragma unroll
        for (int j = 0; j < 64; ++j) c += __popcll(__ballot(v[j] == e));
        if (lane == 0) wsum[wv] = c;
        __syncthreads();
        int pos = run;
        for (int q = 0; q < wv; ++q) pos += wsum[q];
        run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const bool m = v[j] == e;
            const unsigned long long ball = __ballot(m);
            if (m) perm[pos + __popcll(ball & below)] = b * PERM_BLK + wv * (PERM_BLK / 4) + 64 * j + lane;
            pos += __popcll(ball);
        }
        __syncthreads();                                     // wsum is reused by the next block
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

// bf16 x and W_r with H a multiple of 512: one wave per (expert, token), grid
// (E, T), so that the 2 MB of a 4096 x 256 router spread over every CU.  The
// wave reads the expert's row and the token's row with 16-byte loads (H/512
// per lane each) and passes them through LDS, from where lane p takes
// elements p, p+64, ... in increasing order: the same products and the same
// sum order as k_router_logits_small, with an eighth of the load instructions.
template <int NJ>
__global__ __launch_bounds__(64) void k_router_logits_vec(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w,
                                                          const float *__restrict__ bias, int E,
                                                          float *__restrict__ logits,
                                                          float *__restrict__ logits_copy) {
    constexpr int H = 64 * NJ, NV = H / 512;
    static_assert(NV >= 1, "H must be a multiple of 512");
    __shared__ __attribute__((aligned(16))) uint16_t ws[H], xs[H];
    const int lane = threadIdx.x, e = blockIdx.x, t = blockIdx.y;
    const uint4 *wr = reinterpret_cast<const uint4 *>(w + (int64_t)e * H);
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (int64_t)t * H);
    uint4 wv[NV], xv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        wv[j] = wr[64 * j + lane];
        xv[j] = xr[64 * j + lane];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        reinterpret_cast<uint4 *>(ws)[64 * j + lane] = wv[j];
        reinterpret_cast<uint4 *>(xs)[64 * j + lane] = xv[j];
    }
    __syncthreads();
    double v = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        v = __fma_rn((double)bf16_bits_to_f32(ws[lane + 64 * j]), (double)bf16_bits_to_f32(xs[lane + 64 * j]), v);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_down(v, s, 64);
    if (lane == 0) {
        float l = (float)v;
        if (bias) l = (float)((double)l + (double)bias[e]);
        logits[(int64_t)t * E + e] = l;
        if (logits_copy) logits_copy[(int64_t)t * E + e] = l;
    }
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
            key[q][e] = e < E ? logit_key(l, e) : 0ull;
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
            kk[i] = e < E ? logit_key(l, e) : 0ull;
        }
        for (int j = 0; j < k; ++j) {
            const unsigned long long m1 = kk[0] > kk[1] ? kk[0] : kk[1];
            const unsigned long long m2 = kk[2] > kk[3] ? kk[2] : kk[3];
            const unsigned long long m = wave_max_u64(m1 > m2 ? m1 : m2);
            if (lane == 0) sel[wv * k + j] = key_expert(m);
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


// ---------------------------------------------------------------------------
// Many tokens (prefill): bounded logits on the matrix cores, then the fixed-
// order binary64 sum only where it can change the selection.
//
// k_router_bounds computes every logit in fp32 with bf16 MFMA (x and W_r are
// bf16, so each product is exact) together with sum_h |w||x| (a second MFMA
// on the magnitudes), and turns them into an interval [lo, hi] that provably
// holds the fp32 logit the fixed-order binary64 sum gives (bias included):
// whatever order and rounding the matrix cores use inside an accumulation,
// each of its at most H + 8 roundings moves the result by at most 2^-23 of
// sum |p|; the binary64 sum is within 80 * 2^-53 of it, and the final fp32
// rounding within 2^-24 of its magnitude; products that underflow add at most
// H * 2^-126.  k_router_select then takes, per token, the experts whose upper
// bound reaches the k-th largest lower bound -- every other expert has k
// experts certainly above it, even after the fp32 rounding that could make
// logits tie -- recomputes exactly those logits with the fixed-order sum, and
// selects and weights among them: indices and weights are those of the full
// binary64 router, bit for bit.  Tokens or experts whose rows hold subnormal
// bf16 values (which matrix cores may flush) and non-finite sums take the
// exact sum for every expert.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float rb_acc_t;
typedef __attribute__((ext_vector_type(8))) __bf16 rb_bf16x8_t;

constexpr int RB_WAVES = 8;          // K slices per workgroup

__device__ __forceinline__ rb_acc_t rb_mfma(uint4 a, uint4 b, rb_acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rb_bf16x8_t, a),
                                                   __builtin_bit_cast(rb_bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint4 rb_abs(uint4 v) {
    return make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu);
}
// a nonzero bf16 with a zero exponent field in either half of the word
__device__ __forceinline__ bool has_subnormal(uint32_t v) {
    const uint32_t lo = v & 0x7FFFu, hi = (v >> 16) & 0x7FFFu;
    return (lo != 0u && lo < 0x80u) || (hi != 0u && hi < 0x80u);
}

// A 32-token x 32-expert tile of bounds per workgroup, wave w summing the K slice w (of RB_WAVES), the slices added
// in order; the workgroups of the first token tile also flag, in wflag, the expert rows that hold a subnormal value
// (from the router rows they load anyway).
__global__ __launch_bounds__(64 * RB_WAVES) void k_router_bounds(const uint16_t *__restrict__ x,
                                                                 const uint16_t *__restrict__ w,
                                                                 const float *__restrict__ bias, int T, int H, int E,
                                                                 float *__restrict__ lo, float *__restrict__ hi,
                                                                 int32_t *__restrict__ wflag) {
    __shared__ float red[2][RB_WAVES][16][64];
    __shared__ int sflag[RB_WAVES][64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nte = (E + 31) / 32;
    const int t0 = (blockIdx.x / nte) * 32, e0 = (blockIdx.x % nte) * 32;
    const bool flags = t0 == 0;                                // uniform
    const int r = lane & 31, hh = lane >> 5;
    const uint16_t *xr = x + (int64_t)min(t0 + r, T - 1) * H + 32 * hh;
    const uint16_t *wr = w + (int64_t)min(e0 + r, E - 1) * H + 32 * hh;
    const int kq = H / RB_WAVES, kb = wv * kq;
    rb_acc_t acc = {}, aac = {};
    uint4 av[4], bv[4], na[4], nb[4];
    bool sub = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        av[j] = *reinterpret_cast<const uint4 *>(xr + kb + 8 * j);
        bv[j] = *reinterpret_cast<const uint4 *>(wr + kb + 8 * j);
    }
    for (int k0 = kb; k0 < kb + kq; k0 += 64) {
        const int kn = min(k0 + 64, kb + kq - 64);             // next chunk (the last one reloads itself)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            na[j] = *reinterpret_cast<const uint4 *>(xr + kn + 8 * j);
            nb[j] = *reinterpret_cast<const uint4 *>(wr + kn + 8 * j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = rb_mfma(av[j], bv[j], acc);
            aac = rb_mfma(rb_abs(av[j]), rb_abs(bv[j]), aac);
        }
        if (flags)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sub = sub || has_subnormal(bv[j].x) || has_subnormal(bv[j].y) || has_subnormal(bv[j].z) ||
                      has_subnormal(bv[j].w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            av[j] = na[j];
            bv[j] = nb[j];
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        red[0][wv][v][lane] = acc[v];
        red[1][wv][v][lane] = aac[v];
    }
    if (flags) sflag[wv][lane] = sub ? 1 : 0;
    __syncthreads();
    if (flags && tid < 32 && e0 + tid < E) {
        int any = 0;
        for (int q = 0; q < RB_WAVES; ++q) any |= sflag[q][tid] | sflag[q][tid + 32];
        wflag[e0 + tid] = any;
    }
    // thread (wave q, lane l): outputs v = (16 / RB_WAVES) q + i of lane l's column
    const double nr = (double)(H + 8);
    const double eps = nr * 0x1p-23 * 1.0001;
#pragma unroll
    for (int i = 0; i < 16 / RB_WAVES; ++i) {
        const int v = (16 / RB_WAVES) * wv + i;
        float a = red[0][0][v][lane], s = red[1][0][v][lane];
#pragma unroll
        for (int q = 1; q < RB_WAVES; ++q) {
            a += red[0][q][v][lane];
            s += red[1][q][v][lane];
        }
        const int t = t0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), e = e0 + (lane & 31);
        if (t >= T || e >= E) continue;
        float l32 = -INFINITY, h32 = INFINITY;
        if (isfinite(a) && isfinite(s)) {
            const double sat = (double)s / (1.0 - eps) + (double)H * 0x1p-126;    // >= sum |p| exactly
            double b = eps * sat + (double)H * 0x1p-126 + nr * 0x1p-149 + 80.0 * 0x1p-53 * sat;
            b += 0x1p-24 * (fabs((double)a) + b);
            b *= 1.0 + 0x1p-40;
            l32 = __double2float_rd((double)a - b);
            h32 = __double2float_ru((double)a + b);
            if (bias) {
                l32 = (float)((double)l32 + (double)bias[e]);
                h32 = (float)((double)h32 + (double)bias[e]);
            }
        }
        lo[(int64_t)t * E + e] = l32;
        hi[(int64_t)t * E + e] = h32;
    }
}

// One wave per token: candidates from the bounds, their logits with the
// fixed-order binary64 sum (the same operations as k_router_logits), top-k by
// (descending logit, ascending index) among them, and the softmax over the
// selected logits as k_topk computes it.  A candidate's router row is read
// with 16-byte loads into the wave's LDS slice (the next candidate's row is
// requested while the current one is summed), then lane p reads its strided
// elements h = p + 64 j from there.
// H = 64 * NJ (a multiple of 512 up to 4096)
template <int NJ>
__global__ __launch_bounds__(256) void k_router_select(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                       const float *__restrict__ bias, int T, int E, int k,
                                                       const float *__restrict__ lo, const float *__restrict__ hi,
                                                       const int32_t *__restrict__ wflag,
                                                       int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
    constexpr int H = 64 * NJ, NV = H / 512;                 // 16-byte loads per lane and router row
    __shared__ uint4 wrow[4][2][H / 8];
    __shared__ int clist[4][256];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    uint32_t xb[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) xb[j] = x[(int64_t)t * H + lane + 64 * j];
    uint32_t xp[NJ / 2];                                      // x[lane + 64 j] for j = 2i (low) and 2i + 1 (high)
    bool xsub = false;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint32_t m7 = xb[j] & 0x7FFFu;
        xsub = xsub || (m7 != 0u && m7 < 0x80u);
    }
#pragma unroll
    for (int i = 0; i < NJ / 2; ++i) xp[i] = (xb[2 * i] & 0xFFFFu) | (xb[2 * i + 1] << 16);
    const bool all = __ballot(xsub) != 0ull;
    // the k-th largest lower bound (keys make equal bounds distinct)
    float lv[4], hv[4];
    unsigned long long kk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        lv[i] = e < E ? lo[(int64_t)t * E + e] : -INFINITY;
        hv[i] = e < E ? hi[(int64_t)t * E + e] : -INFINITY;
        kk[i] = e < E ? logit_key(lv[i], e) : 0ull;
    }
    unsigned long long m = 0ull;
    for (int j = 0; j < k; ++j) {
        const unsigned long long m1 = kk[0] > kk[1] ? kk[0] : kk[1];
        const unsigned long long m2 = kk[2] > kk[3] ? kk[2] : kk[3];
        m = wave_max_u64(m1 > m2 ? m1 : m2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (kk[i] == m) kk[i] = 0ull;
    }
    const float thr = lo[(int64_t)t * E + key_expert(m)];
    // the candidates, listed in ascending expert order in the wave's LDS slice
    bool cand[4];
    int n_cand = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        cand[i] = e < E && (all || hv[i] >= thr || wflag[e] != 0 || !(hv[i] >= lv[i]));
        const uint64_t bal = __ballot(cand[i]);
        if (cand[i]) clist[wv][n_cand + __popcll(bal & ((1ull << lane) - 1ull))] = e;
        n_cand += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    float lx[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4_t rv[NV];                                           // native vectors: kept in registers across the loop
    {
        const u32x4_t *row = reinterpret_cast<const u32x4_t *>(w + (int64_t)clist[wv][0] * H);
#pragma unroll
        for (int v = 0; v < NV; ++v) rv[v] = row[v * 64 + lane];
    }
    for (int c = 0; c < n_cand; ++c) {
        const int e = clist[wv][c];
        u32x4_t *slot = reinterpret_cast<u32x4_t *>(wrow[wv][c & 1]);
#pragma unroll
        for (int v = 0; v < NV; ++v) slot[v * 64 + lane] = rv[v];
        {                                                     // the next row is in flight while this one is summed
            const u32x4_t *row =
                reinterpret_cast<const u32x4_t *>(w + (int64_t)clist[wv][min(c + 1, n_cand - 1)] * H);
#pragma unroll
            for (int v = 0; v < NV; ++v) rv[v] = row[v * 64 + lane];
        }
        __builtin_amdgcn_wave_barrier();
        const uint16_t *wr = reinterpret_cast<const uint16_t *>(slot);
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float xj = __uint_as_float((j & 1) ? (xp[j >> 1] & 0xFFFF0000u) : (xp[j >> 1] << 16));
            s = __fma_rn((double)bf16_bits_to_f32(wr[lane + 64 * j]), (double)xj, s);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s = s + __shfl_down(s, o, 64);
        float l = (float)s;
        if (bias) l = (float)((double)l + (double)bias[e]);
        l = __shfl(l, 0, 64);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) lx[i] = l;
    }
    // top-k among the candidates, then the weights (as k_topk)
#pragma unroll
    for (int i = 0; i < 4; ++i) kk[i] = cand[i] ? logit_key(lx[i], lane + 64 * i) : 0ull;
    float sel[4] = {0.f, 0.f, 0.f, 0.f}, l0 = 0.f;
    for (int j = 0; j < k; ++j) {
        const unsigned long long m1 = kk[0] > kk[1] ? kk[0] : kk[1];
        const unsigned long long m2 = kk[2] > kk[3] ? kk[2] : kk[3];
        const unsigned long long mm = wave_max_u64(m1 > m2 ? m1 : m2);
        const int bi = key_expert(mm);
        float bv = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (kk[i] == mm) kk[i] = 0ull;
            if (lane + 64 * i == bi) bv = lx[i];
        }
        bv = __shfl(bv, bi & 63, 64);                      // the winner's logit, from the lane that holds it
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((j >> 6) == i && (j & 63) == lane) sel[i] = bv;
        if (j == 0) l0 = bv;
        if (lane == 0) topk_idx[(int64_t)t * k + j] = bi;
    }
    double ex[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ex[i] = exp((double)sel[i] - (double)l0);
    double den = 0.0;
    for (int jj = 0; jj < k; ++jj) {
        const int i = jj >> 6;
        const double vv = i == 0 ? ex[0] : (i == 1 ? ex[1] : (i == 2 ? ex[2] : ex[3]));
        den += __shfl(vv, jj & 63, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        if (j < k) topk_w[(int64_t)t * k + j] = (float)(ex[i] / den);
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
    if constexpr (XB && WB) {
        if (a.H % 512 == 0 && (((uintptr_t)a.x | (uintptr_t)a.w) & 15u) == 0) {   // 16-byte row loads
            const uint16_t *x = static_cast<const uint16_t *>(a.x), *w = static_cast<const uint16_t *>(a.w);
#define MOE_LOGITS_VEC(NJ_)                                                                                  \
    case 64 * NJ_:                                                                                           \
        hipLaunchKernelGGL(k_router_logits_vec<NJ_>, dim3(a.E, a.T), dim3(64), 0, st, x, w, a.bias, a.E,      \
                           a.logits_ws, a.logits_out);                                                       \
        break;
            switch (a.H) {
                MOE_LOGITS_VEC(64)
                MOE_LOGITS_VEC(32)
                MOE_LOGITS_VEC(16)
                MOE_LOGITS_VEC(8)
                default: return hipErrorInvalidValue;
            }
#undef MOE_LOGITS_VEC
            return hipGetLastError();
        }
    }
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

hipError_t launch_route_logits(const RouteArgs &a, hipStream_t st) {
    if (a.T <= SMALL_T && small_logits_shape(a.H)) {
        if (a.x_bf16 && a.w_bf16) return launch_logits_small<true, true>(a, st);
        if (a.x_bf16) return launch_logits_small<true, false>(a, st);
        if (a.w_bf16) return launch_logits_small<false, true>(a, st);
        return launch_logits_small<false, false>(a, st);
    }
    if (a.x_bf16 && a.w_bf16) return launch_logits<true, true>(a, st);
    if (a.x_bf16) return launch_logits<true, false>(a, st);
    if (a.w_bf16) return launch_logits<false, true>(a, st);
    return launch_logits<false, false>(a, st);
}

// The bounded matrix-core router applies to bf16 x and W_r, H a multiple of 512 up to 4096, many tokens, and no
// request for the logits themselves (those come from the full binary64 router).
bool bounded_route(const RouteArgs &a) {
    return a.x_bf16 && a.w_bf16 && a.T > SMALL_T && a.H % 512 == 0 && a.H <= 4096 && !a.logits_out &&
           a.bounds_ws != nullptr && (((uintptr_t)a.x | (uintptr_t)a.w) & 15u) == 0;   // 16-byte row loads
}

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
    hipError_t e;
    if (bounded_route(a)) {
        float *lo = a.bounds_ws, *hi = a.bounds_ws + (size_t)a.T * a.E;
        int32_t *wflag = reinterpret_cast<int32_t *>(hi + (size_t)a.T * a.E);
        const int n_tiles = ((a.T + 31) / 32) * ((a.E + 31) / 32);
        hipLaunchKernelGGL(k_router_bounds, dim3(n_tiles), dim3(64 * RB_WAVES), 0, st,
                           static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.w), a.bias, a.T, a.H,
                           a.E, lo, hi, wflag);
        if ((e = hipGetLastError()) != hipSuccess) return e;
#define MOE_SELECT(NJ_)                                                                                     \
    case 64 * NJ_:                                                                                          \
        hipLaunchKernelGGL(k_router_select<NJ_>, dim3((a.T + 3) / 4), dim3(256), 0, st,                    \
                           static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.w), a.bias, a.T,  \
                           a.E, a.k, lo, hi, wflag, a.topk_idx, a.topk_w);                                   \
        break;
        switch (a.H) {
            MOE_SELECT(64)
            MOE_SELECT(56)
            MOE_SELECT(48)
            MOE_SELECT(40)
            MOE_SELECT(32)
            MOE_SELECT(24)
            MOE_SELECT(16)
            MOE_SELECT(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_SELECT
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_permute, dim3(a.E), dim3(256), 0, st, a.topk_idx, a.T, a.k, a.E, a.offsets, a.perm,
                           a.active);
        return hipGetLastError();
    }
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
    hipLaunchKernelGGL(k_permute, dim3(a.E), dim3(256), 0, st, a.topk_idx, a.T, a.k, a.E, a.offsets, a.perm, a.active);
    return hipGetLastError();
}

}  // namespace moe
