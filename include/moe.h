/*
 * moe.h - C ABI of libmoe.so, the MI355X (gfx950) sparse mixture-of-experts layer.
 *
 * What the layer computes, per token t (the small-T MoE router of the page
 * "feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8", ninfer-windows pull request
 * #8, commit message on the router; the expert FFN and weighted sum are the standard MoE layer
 * that router feeds):
 *   z[t][r]  = sum_h Wr[r][h] x[t][h] + b[r]    r = 0..E-1 expert logits; r = E, present when a
 *              shared expert exists, is the shared-expert gate logit (the page's S2 kernel keeps
 *              257 scores per token for 256 experts next to the shared-expert sigmoid).
 *   ids[t]   = the 8 experts ranked highest under the page's total order (larger logit first, the
 *              lower expert id first on equal logits; -0 and +0 are equal; a NaN ranks below
 *              every number), in rank order. The order is total, so ids are unique.
 *   w[t][k]  = softmax taken over the 8 chosen logits only (the tail of the page's select
 *              kernel), g[t] = sigmoid(z[t][E]) (the page's shared-expert sigmoid).
 *   y[t]     = sum_k w[t][k] FFN_{ids[t][k]}(x[t]) + g[t] FFN_shared(x[t]),
 *              FFN(x) = Wd (silu(Wg x) * (Wu x)), silu(a) = a / (1 + exp(-a)).
 * Arithmetic: products of the stored bf16 (or fp32) values accumulated in fp32; logits, weights,
 * the gate and y are fp32. The intermediate silu(a)*u is kept in fp32 (split into two bf16 terms
 * where it feeds a bf16 matrix instruction).
 *
 * Memory: every pointer argument is a DEVICE pointer owned by the caller, except the config,
 * weight and plan structs and the out-parameters of moe_create / moe_forward_plan, which are host
 * memory. The context BORROWS the weight pointers (nothing is copied); they must stay valid and
 * unchanged while the context is used. The library allocates no device memory: each call takes a
 * caller-provided workspace of at least moe_workspace_bytes(ctx, T) bytes, 256-byte aligned, that
 * the call owns until its kernels finish. A workspace must be zero-filled before its first use
 * (e.g. allocate it zeroed): its leading moe_workspace_state_bytes(ctx) bytes hold arrival
 * counters and work-queue words, and every call, whatever its T, leaves that region zero again,
 * so a workspace can be reused by later calls on any stream as long as two calls never use it
 * at the same time. The context is immutable after moe_create, so calls on different
 * streams are safe when each uses its own workspace and outputs.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a rejected call
 * enqueues nothing and returns a negative moe_status. Unsupported shapes are errors, never a
 * silent success. T == 0 returns MOE_OK and enqueues nothing. Work is asynchronous on `stream`;
 * a launch failure reported by the runtime is returned as MOE_ERR_HIP. Non-finite logits are
 * not an error: the order above still defines the selection (weights are then unspecified).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* NULL where a pointer is required, T out of range, bad enum */
    MOE_ERR_UNSUPPORTED = -2, /* a shape or parameter the library does not implement */
    MOE_ERR_WORKSPACE = -3,   /* workspace NULL, misaligned or smaller than required */
    MOE_ERR_HIP = -4          /* the HIP runtime reported an error */
} moe_status;

typedef enum {
    MOE_F32 = 0,      /* x and every weight stored as fp32 */
    MOE_BF16 = 1,     /* x and every weight stored as bf16 (raw 16-bit patterns) */
    MOE_FP8_E4M3 = 2, /* x and router_w bf16; the routed and shared expert weights stored as
                         OCP FP8 E4M3 codes (one byte each) with one fp32 scale per weight row:
                         weight = value(code) * scale[row]. The quantized expert formats the
                         pages name (groupwise integers, FP8, NVFP4) are not fixed by them; this
                         is the per-row-scaled FP8 reading (see the scale fields below). */
    MOE_MXFP4 = 3     /* x and router_w bf16; the expert weights in the Open Compute Project's
                         MXFP4 (Microscaling formats specification): FP4 E2M1 codes packed two
                         per byte along each row (the even column in the low nibble, so a row of
                         n weights is n/2 bytes) and one E8M0 scale byte per 32 consecutive
                         weights of a row: weight = value(code) * 2^(scale byte - 127), byte 0xFF
                         NaN. Exact while every product lies in bf16's finite range (scale bytes
                         up to 252 always do); a product beyond it becomes +-inf. The group-scaled
                         4-bit reading of the pages' quantized expert formats. */
} moe_dtype;

typedef struct {
    int32_t hidden;       /* H: 64..16384, a multiple of 64 (fp32), of 128 (bf16, FP8) or of
                             256 (MXFP4) */
    int32_t num_experts;  /* E: 8..256 */
    int32_t top_k;        /* must be 8 */
    int32_t inter;        /* I: expert intermediate size, 16..4096, a multiple of 16 (fp32), of
                             32 (bf16), of 128 (FP8) or of 256 (MXFP4) */
    int32_t shared_inter; /* I_s: 0 (no shared expert) or as I */
    int32_t max_tokens;   /* largest T any call on this context may pass, 1..65536 */
    int32_t dtype;        /* moe_dtype */
} moe_config;

/* Weight buffers, all row-major, element type = config.dtype (for MOE_FP8_E4M3: router_w bf16,
 * the four expert matrices FP8 E4M3 codes; for MOE_MXFP4: router_w bf16, the four expert
 * matrices packed E2M1 codes, so their last dimension is halved in bytes: [E][2I][H/2],
 * [E][H][I/2], [2 I_s][H/2], [H][I_s/2]). R = E + (I_s > 0 ? 1 : 0). */
typedef struct {
    const void *router_w;       /* [R][H]; row E is the shared-expert gate row when I_s > 0 */
    const float *router_bias;   /* [R] fp32, added to the logits, or NULL */
    const void *gate_up;        /* [E][2I][H]: rows 0..I-1 gate, rows I..2I-1 up */
    const void *down;           /* [E][H][I] */
    const void *shared_gate_up; /* [2 I_s][H] (gate rows first); NULL iff I_s == 0 */
    const void *shared_down;    /* [H][I_s]; NULL iff I_s == 0 */
    /* Scales of the quantized formats (NULL for MOE_F32 and MOE_BF16; the shared ones NULL iff
     * I_s == 0). MOE_FP8_E4M3: fp32, one per row of the matrix above, 16-byte aligned:
     * gate_up_scale [E][2I], down_scale [E][H], shared_gate_up_scale [2 I_s],
     * shared_down_scale [H]. MOE_MXFP4: E8M0 bytes, one per 32 weights of a row, any
     * alignment: [E][2I][H/32], [E][H][I/32], [2 I_s][H/32], [H][I_s/32]. */
    const void *gate_up_scale;
    const void *down_scale;
    const void *shared_gate_up_scale;
    const void *shared_down_scale;
} moe_weights;

typedef struct moe_ctx moe_ctx;

/* Validate the config and weights, query the current device, build an immutable context.
 * Returns MOE_OK and sets *out, or an error (then *out is NULL). */
int moe_create(const moe_config *cfg, const moe_weights *weights, moe_ctx **out);

/* Release a context (NULL is ignored). Does not free the borrowed weights. */
void moe_destroy(moe_ctx *ctx);

/* Bytes of workspace that serve every call with 1..T tokens (0 when T <= 0 or ctx is NULL): a
 * workspace sized for T can be reused for any smaller token count. */
size_t moe_workspace_bytes(const moe_ctx *ctx, int32_t T);

/* Size of the leading state region of every workspace of ctx (the same for every T; a multiple
 * of 256; 0 when ctx is NULL). It must be zero before a workspace's first use and every call
 * leaves it zero. It holds the arrival counters of the kernels whose last block to finish does
 * the final step of a pass (the routing kernel's selection, the down kernel's combine). */
size_t moe_workspace_state_bytes(const moe_ctx *ctx);

/* Router logits + top-8 selection + softmax weights + shared gate.
 * Exactly one of x ([T][H], config dtype) and logits_in ([T][R] fp32, final logits: no bias is
 * added) must be non-NULL. Outputs: logits_out [T][R] fp32 (may be NULL; when written it holds
 * exactly the values the selection ranked), topk_ids [T][8] int32, topk_w [T][8] fp32,
 * shared_gate [T] fp32 (required iff I_s > 0, else ignored). */
int moe_route(const moe_ctx *ctx, const void *x, const float *logits_in, int32_t T,
              float *logits_out, int32_t *topk_ids, float *topk_w, float *shared_gate,
              void *workspace, size_t ws_bytes, hipStream_t stream);

/* Stable counting sort of the T*8 (token, rank) pairs p = t*8 + k by expert id (the dispatch
 * step that feeds the experts; no atomics). ids_in [T][8] int32 with values in [0, E) (pairs
 * with other values are dropped). Outputs: counts [E], offsets [E+1] (exclusive prefix sums),
 * perm [T*8]: pair indices grouped by expert in increasing expert order, increasing p within an
 * expert; entries past offsets[E] are unspecified. */
int moe_bucket(const moe_ctx *ctx, const int32_t *ids_in, int32_t T, int32_t *counts,
               int32_t *offsets, int32_t *perm, void *workspace, size_t ws_bytes,
               hipStream_t stream);

/* The whole layer: y [T][H] fp32 from x [T][H].
 * Routing: ids_in, w_in, gate_in all NULL -> routed internally from x (as moe_route);
 * otherwise ids_in [T][8] (values in [0, E)) and w_in [T][8] are used as given (gate_in [T]
 * required iff I_s > 0), e.g. the output of moe_route called with logits_in. */
int moe_forward(const moe_ctx *ctx, const void *x, int32_t T, const int32_t *ids_in,
                const float *w_in, const float *gate_in, float *y, void *workspace,
                size_t ws_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and results, with the
 * workspace taken from a static device array of 8 MiB (8388608 bytes) that each GPU holds from
 * the library's load until the process ends, in place of a caller workspace. The caller still
 * passes x, y and the optional routing as in moe_forward. The call allocates nothing; it enqueues
 * a zero fill of the array's state region (a kernel, so that it can be captured) before the
 * layer's kernels. Calls whose workspace would exceed the array - moe_workspace_bytes(ctx, T)
 * > 8 MiB, e.g. T > 64 at H = 2048, I = 512 - return MOE_ERR_WORKSPACE and enqueue nothing.
 * Every call on one GPU shares that GPU's array (it keeps the last call's contents): calls that
 * overlap in time on one GPU, on any streams or contexts, race and give wrong results; serialize
 * them (one stream, or events). */
int moe_forward_noalloc(const moe_ctx *ctx, const void *x, int32_t T, const int32_t *ids_in,
                        const float *w_in, const float *gate_in, float *y, hipStream_t stream);

/* Kernel plan of moe_forward for T tokens (routing internal iff routing_given == 0): the number
 * of kernels it enqueues, in order, and their names (static strings; up to max_names written).
 * Host-only; enqueues nothing. */
int moe_forward_plan(const moe_ctx *ctx, int32_t T, int32_t routing_given, int32_t *n_kernels,
                     const char **names, int32_t max_names);

/* moe_forward whose kernel i of the plan records its own start time in events[2i] and its end
 * time in events[2i + 1] (timestamps of the kernel's dispatch, launch gaps excluded; n_events
 * must equal 2 * n_kernels; the events are created by the caller). For per-kernel timing:
 * hipEventElapsedTime(events[2i], events[2i + 1]) is kernel i's duration. */
int moe_forward_timed(const moe_ctx *ctx, const void *x, int32_t T, const int32_t *ids_in,
                      const float *w_in, const float *gate_in, float *y, void *workspace,
                      size_t ws_bytes, hipStream_t stream, hipEvent_t *events,
                      int32_t n_events);

/* Static description of a status code. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
