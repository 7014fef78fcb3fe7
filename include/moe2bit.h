/*
 * moe2bit.h -- C ABI of the routed 2-bit Mixture-of-Experts FFN layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (source pages: "antirez가 만든 DeepSeek V4 Flash 전용 로컬 추론 엔진 ds4",
 * summary bullets on 2-bit quantization; "antirez/ds4 — Metal용 DeepSeek V4 Flash
 * 로컬 추론 엔진 완벽 가이드", section on the design philosophy): only the routed
 * experts are quantized -- up/gate in an IQ2_XXS-style codebook format ("iq2x"),
 * down in a Q2_K-style super-block format ("q2k"); a 4-bit Q4_K-style variant
 * ("q4k") exists.  The shared expert and the router stay at full precision.
 *
 *   y[t] = sum_{j<k} w[t][j] * FFN_{e[t][j]}(x[t]) + FFN_shared(x[t])
 *   FFN(x) = Wd (silu(Wg x) * (Wu x))
 *
 * and the work is split into three calls, all asynchronous on the caller's
 * HIP stream:
 *   moe_route       router logits, top-k + renormalised softmax weights, and
 *                   the token-to-expert permutation (counts, offsets, order);
 *   moe_expert_ffn  the routed experts (gate/up + SwiGLU + down, per slot) and
 *                   the shared expert;
 *   moe_combine     the top-k weighted sum of the slot outputs plus the shared
 *                   output (moe_combine_steer: the same, then directional
 *                   steering of the result).
 *
 * Conventions for every function below.
 *  - Pointers are DEVICE pointers unless the comment says "host".  The caller
 *    (e.g. PyTorch) allocates and owns all memory: weights, activations,
 *    outputs and workspaces.  The library allocates no device memory in the
 *    layer calls and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work; nothing synchronizes with the host.
 *  - Every argument is checked on the host before anything is launched.  A
 *    failed check returns MOE_ERR_INVALID_ARG and launches nothing; a valid but
 *    unimplemented combination returns MOE_ERR_UNSUPPORTED; a HIP launch error
 *    returns MOE_ERR_DEVICE.  moe_last_error() describes the last failure on
 *    the calling thread.  Faults inside kernels surface at the caller's next
 *    synchronization (at the faulting call itself when MOE_SYNC_DEBUG is set,
 *    see moe_sync_debug).  No C++ exception crosses this interface.
 *  - Non-finite inputs are outside the contract.
 *
 * Canonical block formats (256 weights per block; blocks run along the
 * flattened row-major [out][in] matrix; little-endian):
 *   iq2x  66 B: fp16 d | 8 x { idx[4] (codebook row per 8 weights),
 *               u32 aux: bits 7j..7j+6 = signs of weights 8j..8j+6 (set =
 *               negative), the 8th sign makes the count of negatives even,
 *               bits 28..31 = group scale s } ;  w = d * (2s+1) * C[idx][i] * sign
 *   q2k   84 B: fp16 d | fp16 dmin | 16 x (sc | m << 4) per 16 weights |
 *               64 B of 2-bit q (weight n: byte n/4, bits 2(n%4)) ;
 *               w = d * sc * q - dmin * m
 *   q4k  144 B: fp16 d | fp16 dmin | 12 B = sixteen 6-bit fields (sc0..sc7,
 *               m0..m7; field f at bits 6f) | 128 B of 4-bit q (weight n: byte
 *               n/2, low nibble when n even) ; w = d * sc * q - dmin * m
 * The codebook C is 256 x 8 magnitudes; its entries must be 1, 2 or 3.
 * These layouts are this library's reading of the format names on the pages.
 */
#ifndef MOE2BIT_H
#define MOE2BIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_DEVICE = 3
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

typedef enum { MOE_FMT_IQ2X = 1, MOE_FMT_Q2K = 2, MOE_FMT_Q4K = 3 } moe_format;

/* Expert-FFN kernel family; AUTO picks by token count and shapes. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GENERIC = 1, MOE_PATH_GEMV = 2, MOE_PATH_GEMM = 3 } moe_path;

/*
 * Precision of the expert FFN.  EXACT (default): decoded weights are exact and
 * every product accumulates in fp32 (the layer within 1e-3 relative L2 per
 * token of the binary64 reference).  FAST: the opt-in approximate mode, the
 * counterpart of the exact/approximate kernel choice the ds4-server option
 * listing offers ("DwarfStar4 / ds4.c" user report on modu-print.com, the
 * quality option): in the grouped-GEMM kernels (more than 8 tokens) every
 * q2k down weight is q * fp16(d sc) - fp16(dmin m) in one fp16 fused
 * multiply-add (no per-16 sums of h and no min products, no rescaling of the
 * accumulators between blocks), and the shared expert's SwiGLU output is one
 * bf16 plane instead of a hi + lo pair (half the shared down products);
 * gate/up and q4k rows stay exact.  The layer then lies within 5e-3 relative
 * L2 per token of the reference.  The decode and verify kernels (up to 8
 * tokens) are bound by the weight stream, gain nothing from an approximation,
 * and run exactly in both modes.
 */
typedef enum { MOE_PRECISION_EXACT = 0, MOE_PRECISION_FAST = 1 } moe_precision;

/*
 * Description of one layer (host struct; read during the call only).
 *   hidden (H), inter (I), n_experts (E), top_k (k): 1 <= k <= E <= 256.
 *   gate, up: E stacked [I][H] matrices, down: E stacked [H][I] matrices, each
 *     in the PREPARED layout written by moe_prepare_weights (same byte count
 *     as the canonical blocks).  gate_up_fmt is iq2x or q4k; down_fmt is q2k
 *     or q4k.
 *   codebook: device, 256 x 8 uint8 magnitudes in {1, 2, 3}, 8-byte aligned
 *     (iq2x only).
 *   shared_inter (Is): 0 = no shared expert; else shared_gate, shared_up
 *     [Is][H] and shared_down [H][Is], bf16 row-major.
 *   path: kernel family for moe_expert_ffn (MOE_PATH_AUTO normally).
 *   precision: MOE_PRECISION_EXACT (0, normally) or MOE_PRECISION_FAST.
 */
typedef struct {
    int32_t hidden, inter, n_experts, top_k;
    int32_t gate_up_fmt, down_fmt;
    const void *gate, *up, *down;
    const uint8_t *codebook;
    int32_t shared_inter;
    const void *shared_gate, *shared_up, *shared_down;
    int32_t path;
    int32_t precision;
} moe_layer_desc;

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* 1 if the library waits for the stream after each group of launches, else 0.
 * Set by the environment variable MOE_SYNC_DEBUG (any value but "" or "0"),
 * read once per process at the first call.  With it on, every entry point that
 * launches kernels synchronizes its stream before returning (not while the
 * stream is being captured into a graph) and returns MOE_ERR_DEVICE with the
 * device's error text if a kernel it launched failed, so that a fault is
 * reported by the call that caused it.  A debugging aid: it serializes the
 * host with the device. */
int moe_sync_debug(void);

/* Text for the last failure on the calling thread ("" if none). Host string,
 * owned by the library, valid until the next call on this thread. */
const char *moe_last_error(void);

/* Bytes of n_mats stacked [rows][cols] matrices in format fmt (canonical and
 * prepared layouts have the same size).  0 if the shape is not a whole number
 * of blocks or the format is unknown. */
size_t moe_weight_bytes(int32_t fmt, int64_t n_mats, int64_t rows, int64_t cols);

/*
 * Repack n_mats stacked [rows][cols] matrices from the canonical block layout
 * (`canonical`, device) into the device layout the kernels read (`prepared`,
 * device, moe_weight_bytes(...) bytes, 16-byte aligned, must not overlap
 * `canonical`).  rows*cols must be a multiple of 256, and sub-blocks may not
 * straddle rows: cols % 32 == 0 (iq2x, q4k) or cols % 16 == 0 (q2k).
 * Offline step (weight load), not part of the per-token path.  The formats are
 * the routed experts' storage on the pages (IQ2_XXS for up/gate, Q2_K for
 * down, a 4-bit Q4_K variant: "antirez가 만든 DeepSeek V4 Flash 전용 로컬 추론 엔진
 * ds4", summary bullets on 2-bit quantization and on the q4 model); the byte
 * layouts above are this library's reading of those names.  The prepared
 * layout holds the same bytes regrouped so one 16-byte lane load carries
 * whole fields; it is private to the library.  Errors: MOE_ERR_INVALID_ARG
 * for a bad shape, format, null, misaligned or overlapping buffer.
 */
moe_status moe_prepare_weights(int32_t fmt, int64_t n_mats, int64_t rows, int64_t cols, const void *canonical,
                               void *prepared, void *stream);

/*
 * Decode prepared weights to fp32 (parity/debug export).  `prepared` holds
 * n_mats stacked [rows][cols] matrices; matrices mat_begin .. mat_begin +
 * mat_count - 1 are written to out[mat_count*rows*cols] in row-major order,
 * every value exact.  codebook as in moe_layer_desc (iq2x only, else may be
 * NULL).  The dequantization formulas are the ones in the format table at the
 * top of this file (the block structure the pages name: 256-weight blocks,
 * fp16 block scale, per-32 group scale and per-8 codebook index with signs and
 * parity for iq2x; 16 sub-blocks with 4-bit scale and min and fp16 d, dmin for
 * q2k; 8 sub-blocks with 6-bit scale and min for q4k).  Every decoded weight
 * is a product of at most 21 significant bits, so fp32 holds it exactly.
 * Errors: MOE_ERR_INVALID_ARG for a bad shape, format, range, null or
 * misaligned pointer.
 */
moe_status moe_dequantize(int32_t fmt, const void *prepared, int64_t n_mats, int64_t rows, int64_t cols,
                          int64_t mat_begin, int64_t mat_count, const uint8_t *codebook, float *out, void *stream);

/* Workspace bytes moe_route needs for n_tokens tokens. */
size_t moe_route_workspace(int32_t n_tokens, int32_t n_experts, int32_t top_k);

/*
 * Routing for T tokens.  The router stays at full precision on the pages
 * ("antirez가 만든 DeepSeek V4 Flash 전용 로컬 추론 엔진 ds4", summary bullets on
 * 2-bit quantization: shared experts, projections and routing are not
 * quantized); they do not say how its dot products are summed, and this
 * library's reading is the fixed binary64 order below, so that the selected
 * experts are reproducible bit for bit whatever the tiling.  Selection is a
 * softmax top-k with ties to the lower expert index and weights renormalised
 * over the selected experts.
 *   x [T][H] (x_dt), w_router [E][H] (w_dt), bias [E] fp32 or NULL.
 *   logit[t][e] = fp32( sum_h w[e][h] * x[t][h] ) (+ bias[e], added in fp64 to
 *     the fp32 logit and rounded to fp32), where the sum takes exact products
 *     in binary64 in a fixed order: 64 partials, partial p holding h = p, p+64,
 *     ... in increasing h, then p[i] += p[i+s] for s = 32, 16, ..., 1.
 *   topk_idx [T][k] int32: experts ordered by (descending logit, ascending
 *     index); topk_w [T][k] fp32: softmax over the selected logits (binary64,
 *     rounded to fp32).
 *   logits [T][E] fp32 or NULL (optional copy of the logits).
 *   expert_offsets [E+1], perm [T*k], active [1+E] (int32): slot s = t*k + j
 *     carries expert topk_idx[t][j]; perm lists the slots grouped by expert in
 *     ascending expert order, in slot order within an expert (stable);
 *     expert_offsets is the exclusive scan of the per-expert counts;
 *     active[0] = number of experts with a slot, then those experts ascending.
 *   ws: workspace of at least moe_route_workspace(T, E, k) bytes.
 * Requires 1 <= T, H % 64 == 0, 1 <= k <= E <= 256.  Errors:
 * MOE_ERR_INVALID_ARG (null, misaligned, bad shape or dtype, workspace too
 * small), MOE_ERR_DEVICE (launch failure).  All outputs are caller-owned
 * device buffers; nothing is read back to the host.
 */
moe_status moe_route(const void *x, int32_t x_dt, int32_t n_tokens, int32_t hidden, const void *w_router,
                     int32_t w_dt, int32_t n_experts, const float *bias, int32_t top_k, int32_t *topk_idx,
                     float *topk_w, float *logits, int32_t *expert_offsets, int32_t *perm, int32_t *active, void *ws,
                     size_t ws_bytes, void *stream);

/* Workspace bytes moe_expert_ffn needs for n_tokens tokens of layer L. */
size_t moe_expert_ffn_workspace(const moe_layer_desc *L, int32_t n_tokens);

/*
 * Routed and shared experts for T tokens: for every slot s = t*k + j the
 * SwiGLU FFN of expert topk_idx[t][j] on x[t] with its 2-bit (or q4k) weights
 * decoded exactly, and the bf16 shared expert on every token ("antirez가 만든
 * DeepSeek V4 Flash 전용 로컬 추론 엔진 ds4", summary bullets on 2-bit
 * quantization: the routed experts are the quantized part, the shared expert
 * stays at full precision).  One token takes the decode kernels (each
 * selected expert's blocks streamed once), up to 8 tokens the verify kernels,
 * more the grouped-GEMM kernels over the token-to-expert permutation.
 *   x [T][H] (x_dt; fp32 activations take the generic kernels).
 *   topk_idx, expert_offsets, perm, active: as written by moe_route.
 *   slot_out [T*k][H] fp32: slot s = t*k + j gets FFN_{topk_idx[t][j]}(x[t]).
 *   shared_out [T][H] fp32: FFN_shared(x[t]); NULL iff L->shared_inter == 0.
 *   ws: workspace of at least moe_expert_ffn_workspace(L, T) bytes.
 * Numerics: decoded weights are exact; products accumulate in fp32.  The
 * SwiGLU output h of routed slots is kept in fp16 (decode kernels: T <= 4, or
 * T <= 8 for iq2x gate/up with q2k down and T*k <= 64; grouped-GEMM kernels
 * above that) or fp32 (generic kernels); the shared expert's
 * h in fp32 (decode, generic) or as a bf16 hi + lo pair (grouped GEMM).
 * Range: with s(t) = 2 * (ilogb(max_c |x[t][c]|) - 1), clamped to [-100, 100]
 * (0 for an all-zero row), the fp16 h of token t is stored as h * 2^-s(t) and
 * the down projection multiplies its sums by 2^s(t); the grouped-GEMM kernels
 * read x as fp16 after the same kind of prescale, x * 2^-s(t)/2 (the row's
 * largest magnitude then lies in [2, 4)), and multiply the gate and up sums by
 * 2^s(t)/2.  Powers of two scale exactly, so the results do not depend on the
 * input scale for rows whose largest |x| lies between 2^-48 and 2^48 (beyond
 * that the clamp lets fp16 h or x over- or underflow); the tests cover x scaled
 * by 2^-20 .. 2^16 around unit RMS.  Non-finite inputs give non-finite
 * outputs.  Errors: MOE_ERR_INVALID_ARG (bad layer, null, misaligned,
 * workspace too small), MOE_ERR_UNSUPPORTED (a forced kernel family that
 * cannot take the shapes), MOE_ERR_DEVICE (launch failure).
 */
moe_status moe_expert_ffn(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                          const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                          const int32_t *active, float *slot_out, float *shared_out, void *ws, size_t ws_bytes,
                          void *stream);

/* Bytes of the static device scratch moe_expert_ffn_noalloc uses (one copy per
 * GPU the library runs on, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * moe_expert_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments and kernels without `ws` -- their scratch (h, its
 * per-token scale exponents, the fp16 copy of x, the shared expert's h) lives
 * in a static device array of MOE_NOALLOC_SCRATCH_BYTES bytes, one per GPU.
 * Results are bit-identical to moe_expert_ffn's.  The call allocates nothing;
 * the first call on a device looks the array's address up (with that device
 * current).  Nothing in the array must start at zero, and it keeps the last
 * call's contents.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (several streams or threads) race and give
 * wrong results: serialize them on one stream.  Returns MOE_ERR_INVALID_ARG,
 * launching nothing, when the chosen kernel family needs more scratch than the
 * array holds -- decode and verify calls (up to 8 tokens) need at most 330 KB
 * at hidden 4096, intermediate 2048, top-8; the grouped-GEMM kernels about
 * 48 KiB per token at that shape, so up to about 340 tokens -- or when `stream`
 * belongs to another device than the current one.
 */
moe_status moe_expert_ffn_noalloc(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                                  const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                                  const int32_t *active, float *slot_out, float *shared_out, void *stream);

/*
 * The two halves of moe_expert_ffn, for callers that schedule them apart (or
 * time them): moe_expert_gate_up writes the SwiGLU activations h of every slot
 * and of the shared expert, with the per-token scale exponents of the fp16 h,
 * into `ws` (layout private to the library); moe_expert_down reads them from
 * the same `ws` and writes slot_out and shared_out.  Same arguments and checks
 * as moe_expert_ffn; both calls must see the same L, x, n_tokens, routing
 * arrays and ws, and ws must not be written in between.
 */
moe_status moe_expert_gate_up(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                              const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                              const int32_t *active, void *ws, size_t ws_bytes, void *stream);
moe_status moe_expert_down(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens,
                           const int32_t *topk_idx, const int32_t *expert_offsets, const int32_t *perm,
                           const int32_t *active, float *slot_out, float *shared_out, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * Top-k weighted combine that closes the layer (the sum in the formula at the
 * top of this file):
 *   y[t][c] = sum_{j<k} topk_w[t][j] * slot_out[t*k+j][c] (+ shared_out[t][c]),
 * fp32: fused multiply-adds from 0 in increasing j, the shared term added last.
 *   slot_out   [n_tokens*top_k][hidden] fp32 in slot order (moe_expert_ffn);
 *   topk_w     [n_tokens][top_k] fp32 (moe_route);
 *   shared_out [n_tokens][hidden] fp32, or NULL for a layer without one;
 *   y          [n_tokens][hidden] fp32, written; must not alias an input.
 * Rows with hidden % 4 == 0 and 16-byte aligned pointers take 16-byte loads;
 * the arithmetic is the same either way.  Returns MOE_ERR_INVALID_ARG for a
 * NULL slot_out, topk_w or y, a bad shape or a pointer not 4-byte aligned.
 */
moe_status moe_combine(const float *slot_out, const float *topk_w, const float *shared_out, int32_t n_tokens,
                       int32_t top_k, int32_t hidden, float *y, void *stream);

/*
 * The combine above followed by directional steering of the FFN output
 * ("DwarfStar4 / ds4.c" user report on modu-print.com, the ds4-server option
 * listing, the FFN steering option): with the layer's direction v and strength
 * F, every token's combined output y[t] loses F times its component along v,
 *
 *   y[t] <- y[t] - F * v * dot(v, y[t]).
 *
 * steer_v   [hidden] fp32, device; used as given (not normalised), read only.
 * steer_f   host scalar; F = 0 gives the plain combine (up to the sign of zero).
 * y         [n_tokens][hidden] fp32, written; must not alias any input.
 * dot(v, y[t]) is an fp32 sum whose order is fixed per launch shape, so
 * results are deterministic run to run.  One workgroup per token.  Returns
 * MOE_ERR_INVALID_ARG for a NULL input or output, a bad shape, a pointer not
 * 4-byte aligned or a non-finite steer_f.
 */
moe_status moe_combine_steer(const float *slot_out, const float *topk_w, const float *shared_out, int32_t n_tokens,
                             int32_t top_k, int32_t hidden, const float *steer_v, float steer_f, float *y,
                             void *stream);

/* Workspace bytes moe_layer needs for n_tokens tokens of layer L: the routing
 * workspace rounded up to 256 bytes, then the expert-FFN workspace. */
size_t moe_layer_workspace(const moe_layer_desc *L, int32_t n_tokens);

/*
 * The whole layer in one call: moe_route, moe_expert_ffn and moe_combine (or
 * moe_combine_steer when steer_v is not NULL) with the same arguments, the
 * same outputs, bit for bit, and the same checks -- w_router, w_dt and bias
 * as in moe_route (its E and k are L's), steer_v and steer_f as in
 * moe_combine_steer, y as in moe_combine.  ws (256-byte aligned, at least
 * moe_layer_workspace(L, T) bytes) holds the routing workspace, then the
 * expert-FFN workspace.  With one token on the decode kernels (bf16 x, k <= 16)
 * the routing costs one launch instead of two: the logits kernel runs alone,
 * and every routed gate/up workgroup selects the token's experts from the
 * logits itself (the top-k rule and softmax of moe_route, in the same
 * arithmetic), one of them writing topk_idx, topk_w, expert_offsets, perm and
 * active for the down projection and the combine.  The one-token routing of
 * moe_route is described in the route passage above: experts ordered by
 * (descending logit, ascending index), softmax over the selected logits.
 */
moe_status moe_layer(const moe_layer_desc *L, const void *x, int32_t x_dt, int32_t n_tokens, const void *w_router,
                     int32_t w_dt, const float *bias, int32_t *topk_idx, float *topk_w, float *logits,
                     int32_t *expert_offsets, int32_t *perm, int32_t *active, float *slot_out, float *shared_out,
                     const float *steer_v, float steer_f, float *y, void *ws, size_t ws_bytes, void *stream);

/*
 * Measurement helper, not part of the layer: reads `bytes` bytes of `buf`
 * (device, 16-byte aligned, a multiple of 16) once with 16-byte lane loads
 * in n_blocks workgroups of 256 threads, and XORs each workgroup's fold of the
 * words into sink[workgroup] (device, n_blocks uint32, contents meaningless).
 * Timing it gives the sustained HBM read rate at a given byte count, the
 * measured ceiling the layer's bandwidth-bound kernels are compared with.
 */
moe_status moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE2BIT_H */
