// Internal launch interfaces between the C-ABI host code (api.cpp) and the
// kernel translation units.  Every launcher enqueues on `st` and returns the
// launch status; argument checking has already happened in api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { FMT_IQ2X = 1, FMT_Q2K = 2, FMT_Q4K = 3 };

// prep.hip
hipError_t launch_prepare(int fmt, int64_t NB, const void *canonical, void *prepared, hipStream_t st);
// Decodes blocks [blk0, blk0 + nblk) of a stack of NB prepared blocks.
hipError_t launch_dequant(int fmt, int64_t NB, int64_t blk0, int64_t nblk, const void *prepared,
                          const uint8_t *codebook, float *out, hipStream_t st);

// route.hip
struct RouteArgs {
    const void *x;
    int x_bf16;
    int T, H;
    const void *w;
    int w_bf16;
    int E;
    const float *bias;
    int k;
    int32_t *topk_idx;
    float *topk_w;
    float *logits_out;   // optional
    int32_t *offsets, *perm, *active;
    float *logits_ws;    // [T][E] scratch
    float *bounds_ws;    // [2][T][E] fp32 + [E] int32 scratch of the bounded router (NULL: full binary64 router)
};
hipError_t launch_route(const RouteArgs &a, hipStream_t st);
// the router logits alone (into a.logits_ws, and a.logits_out when set)
hipError_t launch_route_logits(const RouteArgs &a, hipStream_t st);

// ffn_*.hip
struct FfnArgs {
    int H, I, E, k, T;
    int fmt_gu, fmt_d;
    const uint8_t *gate, *up, *down;   // prepared stacks
    const uint8_t *codebook;
    int Is;
    const uint16_t *sg, *su, *sd;      // bf16
    const void *x;
    int x_bf16;
    const int32_t *topk_idx, *offsets, *perm, *active;
    float *slot_out, *shared_out;
    int32_t *hsig;                     // [T] exponent of the routed fp16 h per token (workspace; fp16-h kernels)
    void *ws;
    int stages;                        // bit 0: gate/up + SwiGLU, bit 1: down
    int fast;                          // approximate grouped-GEMM kernels (MOE_PRECISION_FAST)
    // One-token routing inside the gate/up launch (T == 1, k <= SEL_MAXK): when sel_logits is set, every routed
    // gate/up workgroup selects the token's experts from these E fp32 logits itself (topk_idx is not read), and
    // the workgroup of the first selected expert's first rows writes the routing outputs below, as moe_route does.
    const float *sel_logits;
    int32_t *sel_idx;
    float *sel_w;
    int32_t *sel_offsets, *sel_perm, *sel_active;
};
constexpr int SEL_MAXK = 16;
enum { STAGE_GATE_UP = 1, STAGE_DOWN = 2 };
size_t ffn_workspace_generic(int H, int I, int E, int k, int Is, int T);
hipError_t launch_ffn_generic(const FfnArgs &a, hipStream_t st);
size_t ffn_workspace_gemv(int H, int I, int E, int k, int Is, int T);
bool ffn_gemv_supported(const FfnArgs &a);
hipError_t launch_ffn_gemv(const FfnArgs &a, hipStream_t st);
size_t ffn_workspace_gemm(int H, int I, int E, int k, int Is, int T);
bool ffn_gemm_supported(const FfnArgs &a);
hipError_t launch_ffn_gemm(const FfnArgs &a, hipStream_t st);

// combine.hip
hipError_t launch_combine(const float *slot_out, const float *topk_w, const float *shared_out, int T, int k, int H,
                          float *y, hipStream_t st);
hipError_t launch_combine_steer(const float *slot_out, const float *topk_w, const float *shared_out, int T, int k,
                                int H, const float *v, float F, float *y, hipStream_t st);

// probe.hip: streaming-read ceiling (measurement only)
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int n_blocks, hipStream_t st);

}  // namespace moe
