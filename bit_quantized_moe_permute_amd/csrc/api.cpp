// C-ABI entry points of libmoe2bit: argument checking on the host, then kernel
// dispatch on the caller's stream.  Nothing here allocates device memory or
// synchronizes (unless MOE_SYNC_DEBUG asks for it); no C++ exception crosses
// the interface.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/moe2bit.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status ok() {
    g_err[0] = '\0';
    return MOE_OK;
}

// MOE_SYNC_DEBUG, read once per process: any value but "" or "0" turns it on.
bool sync_debug() {
    static const bool on = [] {
        const char *v = std::getenv("MOE_SYNC_DEBUG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// Result of a group of launches on stream s.  With the debug switch on, the call first waits for s (unless s is
// being captured into a graph, where waiting is not allowed) so that a fault in those kernels is reported by the
// entry point that launched them.
moe_status from_hip(hipError_t e, const char *what, hipStream_t s) {
    if (e == hipSuccess && sync_debug()) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(s, &cs);
        if (e == hipSuccess && cs == hipStreamCaptureStatusNone) {
            e = hipStreamSynchronize(s);
            if (e == hipSuccess) e = hipGetLastError();
        }
    }
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int block_bytes(int fmt) {
    switch (fmt) {
        case MOE_FMT_IQ2X: return 66;
        case MOE_FMT_Q2K: return 84;
        case MOE_FMT_Q4K: return 144;
        default: return 0;
    }
}

// Sub-blocks may not straddle rows.
int sub_len(int fmt) { return fmt == MOE_FMT_Q2K ? 16 : 32; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_matrix(int fmt, int64_t n_mats, int64_t rows, int64_t cols, const char *what) {
    if (!block_bytes(fmt)) return fail(MOE_ERR_INVALID_ARG, "%s: unknown format %d", what, fmt);
    if (n_mats < 1 || rows < 1 || cols < 1) return fail(MOE_ERR_INVALID_ARG, "%s: empty shape", what);
    if ((rows * cols) % 256) return fail(MOE_ERR_INVALID_ARG, "%s: rows*cols not a multiple of 256", what);
    if (cols % sub_len(fmt))
        return fail(MOE_ERR_INVALID_ARG, "%s: cols %% %d != 0 (sub-blocks would straddle rows)", what, sub_len(fmt));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_sync_debug(void) { return sync_debug() ? 1 : 0; }

const char *moe_last_error(void) { return g_err; }

size_t moe_weight_bytes(int32_t fmt, int64_t n_mats, int64_t rows, int64_t cols) {
    const int bb = block_bytes(fmt);
    if (!bb || n_mats < 1 || rows < 1 || cols < 1 || (rows * cols) % 256) return 0;
    return (size_t)(n_mats * rows * cols / 256) * (size_t)bb;
}

moe_status moe_prepare_weights(int32_t fmt, int64_t n_mats, int64_t rows, int64_t cols, const void *canonical,
                               void *prepared, void *stream) {
    moe_status st = check_matrix(fmt, n_mats, rows, cols, "moe_prepare_weights");
    if (st != MOE_OK) return st;
    if (!canonical || !prepared) return fail(MOE_ERR_INVALID_ARG, "moe_prepare_weights: null pointer");
    if (!aligned(prepared, 16)) return fail(MOE_ERR_INVALID_ARG, "moe_prepare_weights: prepared not 16-byte aligned");
    const size_t bytes = moe_weight_bytes(fmt, n_mats, rows, cols);
    const char *c = static_cast<const char *>(canonical), *p = static_cast<const char *>(prepared);
    if (c < p + bytes && p < c + bytes) return fail(MOE_ERR_INVALID_ARG, "moe_prepare_weights: buffers overlap");
    const int64_t NB = n_mats * rows * cols / 256;
    return from_hip(moe::launch_prepare(fmt, NB, canonical, prepared, (hipStream_t)stream), "moe_prepare_weights",
                    (hipStream_t)stream);
}

moe_status moe_dequantize(int32_t fmt, const void *prepared, int64_t n_mats, int64_t rows, int64_t cols,
                          int64_t mat_begin, int64_t mat_count, const uint8_t *codebook, float *out, void *stream) {
    moe_status st = check_matrix(fmt, n_mats, rows, cols, "moe_dequantize");
    if (st != MOE_OK) return st;
    if (!prepared || !out || (fmt == MOE_FMT_IQ2X && !codebook))
        return fail(MOE_ERR_INVALID_ARG, "moe_dequantize: null pointer");
    if (!aligned(prepared, 16) || !aligned(out, 4)) return fail(MOE_ERR_INVALID_ARG, "moe_dequantize: misaligned");
    if (mat_begin < 0 || mat_count < 1 || mat_begin + mat_count > n_mats)
        return fail(MOE_ERR_INVALID_ARG, "moe_dequantize: matrix range [%lld, +%lld) outside [0, %lld)",
                    (long long)mat_begin, (long long)mat_count, (long long)n_mats);
    if ((rows * cols) % 256) return fail(MOE_ERR_INVALID_ARG, "moe_dequantize: matrix not whole blocks");
    const int64_t per = rows * cols / 256;
    return from_hip(moe::launch_dequant(fmt, n_mats * per, mat_begin * per, mat_count * per, prepared, codebook, out,
                                        (hipStream_t)stream),
                    "moe_dequantize", (hipStream_t)stream);
}

// logits [T][E] fp32 | bounds of the matrix-core router: lo, hi [T][E] fp32, expert flags [E] int32
static size_t route_logits_bytes(int32_t T, int32_t E) { return ((size_t)T * E * sizeof(float) + 255) / 256 * 256; }

size_t moe_route_workspace(int32_t n_tokens, int32_t n_experts, int32_t top_k) {
    (void)top_k;
    if (n_tokens < 1 || n_experts < 1) return 0;
    return route_logits_bytes(n_tokens, n_experts) +
           ((2 * (size_t)n_tokens * n_experts + n_experts) * sizeof(float) + 255) / 256 * 256;
}

// Host checks of the routing arguments; fills `a` (logits scratch at ws).
static moe_status route_args(const char *fn, const void *x, int32_t x_dt, int32_t n_tokens, int32_t hidden,
                             const void *w_router, int32_t w_dt, int32_t n_experts, const float *bias, int32_t top_k,
                             int32_t *topk_idx, float *topk_w, float *logits, int32_t *expert_offsets, int32_t *perm,
                             int32_t *active, void *ws, size_t ws_bytes, moe::RouteArgs &a) {
    if (!x || !w_router || !topk_idx || !topk_w || !expert_offsets || !perm || !active || !ws)
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if ((x_dt != MOE_DT_F32 && x_dt != MOE_DT_BF16) || (w_dt != MOE_DT_F32 && w_dt != MOE_DT_BF16))
        return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    if (n_tokens < 1) return fail(MOE_ERR_INVALID_ARG, "%s: n_tokens < 1", fn);
    if (hidden < 64 || hidden % 64) return fail(MOE_ERR_INVALID_ARG, "%s: hidden %% 64 != 0", fn);
    if (n_experts < 1 || n_experts > 256) return fail(MOE_ERR_INVALID_ARG, "%s: n_experts outside [1, 256]", fn);
    if (top_k < 1 || top_k > n_experts) return fail(MOE_ERR_INVALID_ARG, "%s: top_k outside [1, n_experts]", fn);
    if ((int64_t)n_tokens * top_k > (int64_t)1 << 30) return fail(MOE_ERR_INVALID_ARG, "%s: too many slots", fn);
    if (ws_bytes < moe_route_workspace(n_tokens, n_experts, top_k))
        return fail(MOE_ERR_INVALID_ARG, "%s: workspace too small (%zu < %zu)", fn, ws_bytes,
                    moe_route_workspace(n_tokens, n_experts, top_k));
    if (!aligned(ws, 16) || !aligned(x, 4) || !aligned(w_router, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    a.x = x; a.x_bf16 = x_dt == MOE_DT_BF16; a.T = n_tokens; a.H = hidden;
    a.w = w_router; a.w_bf16 = w_dt == MOE_DT_BF16; a.E = n_experts; a.bias = bias; a.k = top_k;
    a.topk_idx = topk_idx; a.topk_w = topk_w; a.logits_out = logits;
    a.offsets = expert_offsets; a.perm = perm; a.active = active;
    a.logits_ws = static_cast<float *>(ws);
    a.bounds_ws = reinterpret_cast<float *>(static_cast<char *>(ws) + route_logits_bytes(n_tokens, n_experts));
    return MOE_OK;
}

moe_status moe_route(const void *x, int32_t x_dt, int32_t n_tokens, int32_t hidden, const void *w_router,
                     int32_t w_dt, int32_t n_experts, const float *bias, int32_t top_k, int32_t *topk_idx,
                     float *topk_w, float *logits, int32_t *expert_offsets, int32_t *perm, int32_t *active, void *ws,
                     size_t ws_bytes, void *stream) {
    moe::RouteArgs a;
    moe_status st = route_args("moe_route", x, x_dt, n_tokens, hidden, w_router, w_dt, n_experts, bias, top_k,
                               topk_idx, topk_w, logits, expert_offsets, perm, active, ws, ws_bytes, a);
    if (st != MOE_OK) return st;
    return from_hip(moe::launch_route(a, (hipStream_t)stream), "moe_route", (hipStream_t)stream);
}

static moe_status check_layer(const moe_layer_desc *L, const char *fn) {
    if (!L) return fail(MOE_ERR_INVALID_ARG, "%s: null layer", fn);
    if (L->hidden < 1 || L->inter < 1) return fail(MOE_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (L->n_experts < 1 || L->n_experts > 256) return fail(MOE_ERR_INVALID_ARG, "%s: n_experts outside [1, 256]", fn);
    if (L->top_k < 1 || L->top_k > L->n_experts) return fail(MOE_ERR_INVALID_ARG, "%s: top_k outside [1, E]", fn);
    if (L->gate_up_fmt != MOE_FMT_IQ2X && L->gate_up_fmt != MOE_FMT_Q4K)
        return fail(MOE_ERR_INVALID_ARG, "%s: gate/up format must be iq2x or q4k", fn);
    if (L->down_fmt != MOE_FMT_Q2K && L->down_fmt != MOE_FMT_Q4K)
        return fail(MOE_ERR_INVALID_ARG, "%s: down format must be q2k or q4k", fn);
    moe_status st = check_matrix(L->gate_up_fmt, L->n_experts, L->inter, L->hidden, fn);
    if (st != MOE_OK) return st;
    if ((st = check_matrix(L->down_fmt, L->n_experts, L->hidden, L->inter, fn)) != MOE_OK) return st;
    if (!L->gate || !L->up || !L->down) return fail(MOE_ERR_INVALID_ARG, "%s: null expert weights", fn);
    if (!aligned(L->gate, 16) || !aligned(L->up, 16) || !aligned(L->down, 16))
        return fail(MOE_ERR_INVALID_ARG, "%s: expert weights not 16-byte aligned", fn);
    if (L->gate_up_fmt == MOE_FMT_IQ2X && !L->codebook) return fail(MOE_ERR_INVALID_ARG, "%s: null codebook", fn);
    if (L->gate_up_fmt == MOE_FMT_IQ2X && !aligned(L->codebook, 8))
        return fail(MOE_ERR_INVALID_ARG, "%s: codebook not 8-byte aligned", fn);
    if (L->shared_inter < 0) return fail(MOE_ERR_INVALID_ARG, "%s: shared_inter < 0", fn);
    if (L->shared_inter > 0) {
        if (!L->shared_gate || !L->shared_up || !L->shared_down)
            return fail(MOE_ERR_INVALID_ARG, "%s: null shared expert weights", fn);
        if (!aligned(L->shared_gate, 16) || !aligned(L->shared_up, 16) || !aligned(L->shared_down, 16))
            return fail(MOE_ERR_INVALID_ARG, "%s: shared expert weights not 16-byte aligned", fn);
        if (L->hidden % 8 || L->shared_inter % 8)
            return fail(MOE_ERR_INVALID_ARG, "%s: shared expert dims must be multiples of 8", fn);
    }
    if (L->path < MOE_PATH_AUTO || L->path > MOE_PATH_GEMM) return fail(MOE_ERR_INVALID_ARG, "%s: unknown path", fn);
    if (L->precision != MOE_PRECISION_EXACT && L->precision != MOE_PRECISION_FAST)
        return fail(MOE_ERR_INVALID_ARG, "%s: unknown precision", fn);
    return MOE_OK;
}

static moe::FfnArgs make_args(const moe_layer_desc *L, const void *x, int x_dt, int T) {
    moe::FfnArgs a;
    memset(&a, 0, sizeof a);
    a.H = L->hidden; a.I = L->inter; a.E = L->n_experts; a.k = L->top_k; a.T = T;
    a.fmt_gu = L->gate_up_fmt; a.fmt_d = L->down_fmt;
    a.gate = static_cast<const uint8_t *>(L->gate);
    a.up = static_cast<const uint8_t *>(L->up);
    a.down = static_cast<const uint8_t *>(L->down);
    a.codebook = L->codebook;
    a.Is = L->shared_inter;
    a.sg = static_cast<const uint16_t *>(L->shared_gate);
    a.su = static_cast<const uint16_t *>(L->shared_up);
    a.sd = static_cast<const uint16_t *>(L->shared_down);
    a.x = x; a.x_bf16 = x_dt == MOE_DT_BF16;
    a.fast = L->precision == MOE_PRECISION_FAST;
    return a;
}

// Kernel family for this call: 1 generic, 2 gemv, 3 gemm.
static int choose_path(const moe_layer_desc *L, const moe::FfnArgs &a) {
    if (L->path != MOE_PATH_AUTO) return L->path;
    if (moe::ffn_gemv_supported(a)) return MOE_PATH_GEMV;
    if (a.T > 4 && moe::ffn_gemm_supported(a)) return MOE_PATH_GEMM;
    return MOE_PATH_GENERIC;
}

static size_t workspace_for(int path, const moe_layer_desc *L, int32_t T) {
    const int Is = L->shared_inter;
    switch (path) {
        case MOE_PATH_GEMV: return moe::ffn_workspace_gemv(L->hidden, L->inter, L->n_experts, L->top_k, Is, T);
        case MOE_PATH_GEMM: return moe::ffn_workspace_gemm(L->hidden, L->inter, L->n_experts, L->top_k, Is, T);
        default: return moe::ffn_workspace_generic(L->hidden, L->inter, L->n_experts, L->top_k, Is, T);
    }
}

size_t moe_expert_ffn_workspace(const moe_layer_desc *L, int32_t n_tokens) {
    if (n_tokens < 1 || check_layer(L, "moe_expert_ffn_workspace") != MOE_OK) return 0;
    size_t m = 0;
    for (int p = MOE_PATH_GENERIC; p <= MOE_PATH_GEMM; ++p) {
        size_t b = workspace_for(p, L, n_tokens);
        if (b > m) m = b;
    }
    return m;
}

// ---------------------------------------------------------------------------
// Static device scratch of moe_expert_ffn_noalloc: one copy per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; its device
// address is looked up per device with hipGetSymbolAddress and used instead.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first call on that device (with the device
// current).  The caller's stream must belong to the current device.
moe_status scratch_for(void *stream, const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
    if (stream) {
        int sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: hipStreamGetDevice: %s", fn, hipGetErrorString(e));
        if (sdev != dev)
            return fail(MOE_ERR_INVALID_ARG, "%s: the stream belongs to device %d, the current device is %d", fn,
                        sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_DEVICE, "%s: hipGetSymbolAddress of the static scratch: %s", fn,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

// Routing done inside the gate/up launch of a one-token call (moe_layer): the logits to select from and the
// routing outputs to write.
struct InKernelRoute {
    const float *logits;
    int32_t *idx;
    float *w;
    int32_t *offsets, *perm, *active;
};

// ws == nullptr with static_ws: the kernels' scratch is this device's static `scratch`.
static moe_status expert_call(const char *fn, int stages, const moe_layer_desc *L, const void *x, int32_t x_dt,
                              int32_t n_tokens, const int32_t *topk_idx, const int32_t *expert_offsets,
                              const int32_t *perm, const int32_t *active, float *slot_out, float *shared_out,
                              void *ws, size_t ws_bytes, void *stream, bool static_ws = false,
                              const InKernelRoute *route = nullptr) {
    moe_status st = check_layer(L, fn);
    if (st != MOE_OK) return st;
    if (!x || !topk_idx || !expert_offsets || !perm || !active || (!ws && !static_ws))
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if ((stages & moe::STAGE_DOWN) && !slot_out) return fail(MOE_ERR_INVALID_ARG, "%s: null slot_out", fn);
    if (x_dt != MOE_DT_F32 && x_dt != MOE_DT_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    if (n_tokens < 1) return fail(MOE_ERR_INVALID_ARG, "%s: n_tokens < 1", fn);
    if ((stages & moe::STAGE_DOWN) && (L->shared_inter > 0) != (shared_out != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "%s: shared_out must be given iff the layer has a shared expert", fn);
    if (!aligned(x, 16) || (slot_out && !aligned(slot_out, 16)) || (ws && !aligned(ws, 256)) ||
        (shared_out && !aligned(shared_out, 16)))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer (x/outputs 16 B, ws 256 B)", fn);
    moe::FfnArgs a = make_args(L, x, x_dt, n_tokens);
    a.topk_idx = topk_idx; a.offsets = expert_offsets; a.perm = perm; a.active = active;
    a.slot_out = slot_out; a.shared_out = shared_out; a.ws = ws; a.stages = stages;
    const int path = choose_path(L, a);
    if (path == MOE_PATH_GEMV && !(moe::ffn_gemv_supported(a)))
        return fail(MOE_ERR_UNSUPPORTED, "%s: decode kernels need bf16 x, T <= 4 (T <= 8 with iq2x gate/up, "
                                         "q2k down and T*k <= 64), hidden in {512..4096}, supported inter/shared "
                                         "sizes", fn);
    if (path == MOE_PATH_GEMM && !(moe::ffn_gemm_supported(a)))
        return fail(MOE_ERR_UNSUPPORTED, "%s: grouped-GEMM kernels need bf16 x and hidden, inter, "
                                         "shared_inter multiples of 256", fn);
    const size_t need = workspace_for(path, L, n_tokens);
    if (static_ws) {
        if (need > MOE_NOALLOC_SCRATCH_BYTES)
            return fail(MOE_ERR_INVALID_ARG, "%s: %d tokens need %zu bytes of scratch, the static scratch holds %zu; "
                                             "use moe_expert_ffn with a workspace", fn, n_tokens, need,
                        (size_t)MOE_NOALLOC_SCRATCH_BYTES);
        if ((st = scratch_for(stream, fn, &a.ws)) != MOE_OK) return st;
    } else if (ws_bytes < need) {
        return fail(MOE_ERR_INVALID_ARG, "%s: workspace too small (%zu < %zu)", fn, ws_bytes, need);
    }
    if (route) {
        a.sel_logits = route->logits;
        a.sel_idx = route->idx; a.sel_w = route->w;
        a.sel_offsets = route->offsets; a.sel_perm = route->perm; a.sel_active = route->active;
    }
    hipError_t e;
    if (path == MOE_PATH_GEMV) e = moe::launch_ffn_gemv(a, (hipStream_t)stream);
    else if (path == MOE_PATH_GEMM) e = moe::launch_ffn_gemm(a, (hipStream_t)stream);
    else e = moe::launch_ffn_generic(a, (hipStream_t)stream);
    return from_hip(e, fn, (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                          const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                          const int32_t *active, float *slot_out, float *shared_out, void *ws, size_t ws_bytes,
                          void *stream) {
    return expert_call("moe_expert_ffn", moe::STAGE_GATE_UP | moe::STAGE_DOWN, L, x, x_dt, n_tokens, topk_idx,
                       expert_offsets, perm, active, slot_out, shared_out, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_noalloc(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                                  const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                                  const int32_t *active, float *slot_out, float *shared_out, void *stream) {
    return expert_call("moe_expert_ffn_noalloc", moe::STAGE_GATE_UP | moe::STAGE_DOWN, L, x, x_dt, n_tokens,
                       topk_idx, expert_offsets, perm, active, slot_out, shared_out, nullptr, 0, stream, true);
}

moe_status moe_expert_gate_up(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                              const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                              const int32_t *active, void *ws, size_t ws_bytes, void *stream) {
    return expert_call("moe_expert_gate_up", moe::STAGE_GATE_UP, L, x, x_dt, n_tokens, topk_idx, expert_offsets,
                       perm, active, nullptr, nullptr, ws, ws_bytes, stream);
}

moe_status moe_expert_down(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                           const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                           const int32_t *active, float *slot_out, float *shared_out, void *ws, size_t ws_bytes,
                           void *stream) {
    return expert_call("moe_expert_down", moe::STAGE_DOWN, L, x, x_dt, n_tokens, topk_idx, expert_offsets, perm,
                       active, slot_out, shared_out, ws, ws_bytes, stream);
}

moe_status moe_combine(const float *slot_out, const float *topk_w, const float *shared_out, int32_t n_tokens,
                       int32_t top_k, int32_t hidden, float *y, void *stream) {
    if (!slot_out || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
    if (n_tokens < 1 || top_k < 1 || hidden < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine: bad shape");
    if (!aligned(slot_out, 4) || !aligned(y, 4) || !aligned(topk_w, 4) || (shared_out && !aligned(shared_out, 4)))
        return fail(MOE_ERR_INVALID_ARG, "moe_combine: misaligned pointer");
    return from_hip(moe::launch_combine(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, y, (hipStream_t)stream),
                    "moe_combine", (hipStream_t)stream);
}

moe_status moe_combine_steer(const float *slot_out, const float *topk_w, const float *shared_out, int32_t n_tokens,
                             int32_t top_k, int32_t hidden, const float *steer_v, float steer_f, float *y,
                             void *stream) {
    if (!slot_out || !topk_w || !y || !steer_v) return fail(MOE_ERR_INVALID_ARG, "moe_combine_steer: null pointer");
    if (n_tokens < 1 || top_k < 1 || hidden < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine_steer: bad shape");
    if (!aligned(slot_out, 4) || !aligned(y, 4) || !aligned(topk_w, 4) || !aligned(steer_v, 4) ||
        (shared_out && !aligned(shared_out, 4)))
        return fail(MOE_ERR_INVALID_ARG, "moe_combine_steer: misaligned pointer");
    if (!std::isfinite(steer_f)) return fail(MOE_ERR_INVALID_ARG, "moe_combine_steer: steering strength not finite");
    return from_hip(moe::launch_combine_steer(slot_out, topk_w, shared_out, n_tokens, top_k, hidden, steer_v, steer_f,
                                              y, (hipStream_t)stream),
                    "moe_combine_steer", (hipStream_t)stream);
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t moe_layer_workspace(const moe_layer_desc *L, int32_t n_tokens) {
    if (n_tokens < 1 || check_layer(L, "moe_layer_workspace") != MOE_OK) return 0;
    return align256(moe_route_workspace(n_tokens, L->n_experts, L->top_k)) + moe_expert_ffn_workspace(L, n_tokens);
}

moe_status moe_layer(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens, const void *w_router,
                     int32_t w_dt, const float *bias, int32_t *topk_idx, float *topk_w, float *logits,
                     int32_t *expert_offsets, int32_t *perm, int32_t *active, float *slot_out, float *shared_out,
                     const float *steer_v, float steer_f, float *y, void *ws, size_t ws_bytes, void *stream) {
    const char *fn = "moe_layer";
    moe_status st = check_layer(L, fn);
    if (st != MOE_OK) return st;
    if (!y || !slot_out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(y, 4) || (steer_v && !aligned(steer_v, 4)))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (steer_v && !std::isfinite(steer_f)) return fail(MOE_ERR_INVALID_ARG, "%s: steering strength not finite", fn);
    const size_t rws = align256(moe_route_workspace(n_tokens, L->n_experts, L->top_k));
    if (!ws || ws_bytes < rws) return fail(MOE_ERR_INVALID_ARG, "%s: workspace too small", fn);
    moe::RouteArgs ra;
    st = route_args(fn, x, x_dt, n_tokens, L->hidden, w_router, w_dt, L->n_experts, bias, L->top_k, topk_idx, topk_w,
                    logits, expert_offsets, perm, active, ws, rws, ra);
    if (st != MOE_OK) return st;
    void *fws = static_cast<char *>(ws) + rws;
    const size_t fbytes = ws_bytes - rws;
    // one token on the decode kernels: the routed gate/up workgroups select the token's experts from the logits
    // themselves, so routing takes one launch (the logits) instead of two
    moe::FfnArgs probe = make_args(L, x, x_dt, n_tokens);
    const bool in_kernel = n_tokens == 1 && L->top_k <= moe::SEL_MAXK && x_dt == MOE_DT_BF16 &&
                           choose_path(L, probe) == MOE_PATH_GEMV && moe::ffn_gemv_supported(probe);
    const hipStream_t hs = (hipStream_t)stream;
    if (in_kernel) {
        if ((st = from_hip(moe::launch_route_logits(ra, hs), fn, hs)) != MOE_OK) return st;
        const InKernelRoute r{ra.logits_ws, topk_idx, topk_w, expert_offsets, perm, active};
        st = expert_call(fn, moe::STAGE_GATE_UP, L, x, x_dt, n_tokens, topk_idx, expert_offsets, perm, active,
                         nullptr, nullptr, fws, fbytes, stream, false, &r);
        if (st != MOE_OK) return st;
        st = expert_call(fn, moe::STAGE_DOWN, L, x, x_dt, n_tokens, topk_idx, expert_offsets, perm, active, slot_out,
                         shared_out, fws, fbytes, stream);
    } else {
        if ((st = from_hip(moe::launch_route(ra, hs), fn, hs)) != MOE_OK) return st;
        st = expert_call(fn, moe::STAGE_GATE_UP | moe::STAGE_DOWN, L, x, x_dt, n_tokens, topk_idx, expert_offsets,
                         perm, active, slot_out, shared_out, fws, fbytes, stream);
    }
    if (st != MOE_OK) return st;
    const int T = n_tokens, k = L->top_k, H = L->hidden;
    if (steer_v)
        return from_hip(moe::launch_combine_steer(slot_out, topk_w, shared_out, T, k, H, steer_v, steer_f, y, hs), fn,
                        hs);
    return from_hip(moe::launch_combine(slot_out, topk_w, shared_out, T, k, H, y, hs), fn, hs);
}

moe_status moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_blocks, void *stream) {
    if (!buf || !sink) return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream_read: null pointer");
    if (bytes < 16 || bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4))
        return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream_read: need a 16-byte aligned, non-empty multiple of 16 bytes");
    if (n_blocks < 1 || n_blocks > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream_read: n_blocks outside [1, 2^20]");
    return from_hip(moe::launch_stream_read(buf, (int64_t)bytes, sink, n_blocks, (hipStream_t)stream),
                    "moe_probe_stream_read", (hipStream_t)stream);
}

}  // extern "C"
