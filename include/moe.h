/*
 * libmoe: forward pass of one DeepSeek-V3-style mixture-of-experts block on an
 * AMD MI355X (gfx950), behind a plain C ABI.
 *
 * What is computed (the pages this follows):
 *   "DeepSeek-V3.2-Exp · Router" (atlas.klimoza.dev, router inspector), formula
 *   steps 1-4 and the Gate.forward excerpt: z = x W_r in fp32, s = sigmoid(z),
 *   selection on s + b (b only selects), expert groups scored by the sum of their
 *   two best selection scores, the best topk_groups groups kept, the topk best
 *   experts among them, weights = the unbiased s of those experts divided by
 *   their sum, times route_scale.
 *   "DeepSeek-V3.2-Exp · Mixture of experts" (open-model-atlas, MoE block), the
 *   MoE.forward excerpt and parameter table: tokens flattened to x[T, dim];
 *   per-expert token lists in token order; every routed expert and the shared
 *   expert a 3-matrix SwiGLU MLP dim -> inter -> dim; the routed outputs weighted
 *   and added in ascending expert order into an fp32 accumulator, then the shared
 *   expert's output; the result returned in x's dtype and shape.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer (memory of the current HIP
 *     device) owned by the caller, except `cfg`, `wts`, `bytes` and `layout`,
 *     which are host pointers read or written during the call only.
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work on it: they never allocate, free or synchronise, and return before
 *     the GPU has finished. Results are valid once the stream has reached them.
 *   - `ws` is caller-owned scratch of at least the size reported by
 *     moe_workspace_size(); its contents on entry do not matter and on return
 *     are unspecified (moe_workspace_layout() names the parts tests may read).
 *   - Argument and configuration errors are detected on the host before any
 *     launch and nothing is enqueued; launch failures return MOE_ERR_HIP.
 *     moe_last_error() then gives a message (thread-local, valid until the
 *     next call on that thread).
 *   - Non-finite inputs give unspecified values, never out-of-range indices:
 *     a NaN selection score ranks below every number, so each token still gets
 *     topk distinct experts in [0, n_experts). T = 0 is a valid no-op.
 *   - Two calls that share `ws` must be ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* null pointer, misalignment, negative size */
  MOE_ERR_CONFIG = -2,      /* inconsistent configuration (e.g. topk too large) */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes below moe_workspace_size() */
  MOE_ERR_HIP = -4,         /* a HIP launch failed */
  MOE_ERR_UNSUPPORTED = -5  /* valid but outside what the kernels handle */
} moe_status;

/* Storage and arithmetic types of a block.
 * MOE_F32:  x, out, router and expert weights fp32; expert activations fp32.
 * MOE_BF16: x, out, router and expert weights bf16; fp32 accumulation; the
 *           SwiGLU activation stored as bf16.
 * MOE_FP8:  x and out bf16; router weight bf16 (+ fp32 bias), computed in fp32;
 *           expert weights OCP e4m3fn with one fp32 scale per 128x128 block of
 *           the [out, in] matrix; expert inputs (x and the SwiGLU activation)
 *           quantised in the block to e4m3fn with one fp32 scale per token per
 *           128 columns (scale = amax / 448, or 1 when amax = 0). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype;

/* Router scoring (the Gate.forward excerpt's two branches):
 * MOE_SCORE_SIGMOID: s = sigmoid(z); weights = chosen s / their sum * route_scale
 *                    (DeepSeek-V3).
 * MOE_SCORE_SOFTMAX: s = softmax(z) over the token's experts; weights = chosen s
 *                    * route_scale, not renormalised. */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score_func;

/* Field names follow the Gate / MoE constructors on the pages. */
typedef struct {
  int32_t dim;          /* D: 7168 in DeepSeek-V3 */
  int32_t n_experts;    /* E routed experts: 256 */
  int32_t n_groups;     /* G expert groups: 8 (group g holds experts g*E/G .. (g+1)*E/G-1) */
  int32_t topk_groups;  /* groups kept per token: 4 */
  int32_t topk;         /* K experts per token: 8 */
  int32_t inter;        /* I, routed expert hidden size: 2048 */
  int32_t n_shared;     /* shared experts, fused into one MLP of hidden n_shared*I: 1 */
  float route_scale;    /* 2.5 */
  int32_t dtype;        /* moe_dtype */
  int32_t score_func;   /* moe_score_func: MOE_SCORE_SIGMOID in DeepSeek-V3 */
} moe_config;

/* Block weights, all device pointers, row-major, linear-layer [out, in] layout.
 *   w_gate [E, D]   (fp32 for MOE_F32, else bf16)
 *   bias   [E] fp32, selection only; NULL selects the excerpt's no-bias branch
 *          (group score = the group's maximum score)
 *   w1, w3 [E, I, D];  w2 [E, D, I]         routed experts (gate, up, down)
 *   ws1, ws3 [S, D];   ws2 [D, S]           shared expert, S = n_shared * I
 *   (element type fp32 / bf16 / e4m3fn per dtype)
 *   FP8 only, fp32 scales per 128x128 block:
 *   s1, s3 [E, I/128, D/128];  s2 [E, D/128, I/128];
 *   ss1, ss3 [S/128, D/128];   ss2 [D/128, S/128].  NULL for other dtypes. */
typedef struct {
  const void* w_gate;
  const float* bias;
  const void *w1, *w3, *w2;
  const void *ws1, *ws3, *ws2;
  const float *s1, *s3, *s2;
  const float *ss1, *ss3, *ss2;
} moe_weights;

/* Bytes of scratch moe_forward / moe_route / moe_dispatch need for T tokens.
 * Errors: MOE_ERR_ARG (null), MOE_ERR_CONFIG / MOE_ERR_UNSUPPORTED (as moe_forward). */
moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes);

/* The router (router page, steps 1-4).
 *   x     [T, D]  fp32 (MOE_F32) or bf16 (other dtypes)
 *   idx   [T, K]  int32 out: chosen experts, descending selection score s + b,
 *                 equal scores in ascending expert order
 *   w     [T, K]  fp32 out: routing weights aligned with idx
 * Logits are fp32 values of exact dot products (bf16 or fp32 products summed in
 * fp64 per 32-element chunk); sigmoid, or softmax over the token's experts, is
 * evaluated in fp64 and rounded once; the sigmoid weights' sum runs in rank
 * order. n_groups = 1 is plain top-k over all experts. A token with a NaN score
 * (NaN in its x, or a NaN bias) has that score ranked below every number; it
 * still receives topk distinct experts, its weights are then unspecified. */
moe_status moe_route(const moe_config* cfg, const void* w_gate, const float* bias, const void* x,
                     int64_t T, int32_t* idx, float* w, void* ws, size_t ws_bytes, void* stream);

/* Dispatch (MoE block page: bincount, then per expert the tokens that chose it,
 * in token order). Deterministic: no atomic decides an output position.
 *   idx       [T, K]  int32 in (values in [0, E), distinct per token)
 *   counts    [E]     out: tokens per expert
 *   offsets   [E + 1] out: exclusive prefix sum of counts (offsets[E] = T*K)
 *   row_token [T * K] out: rows grouped by expert ascending, tokens ascending
 *                     within an expert; row_token[r] = the token of row r
 *   row_of    [T, K]  out: the row of assignment (t, k)
 * An entry of idx outside [0, E) is not counted and gets row_of = -1 (the
 * forward's combine skips such entries); a token listing one expert twice gives
 * unspecified rows. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* idx, int64_t T, int32_t* counts,
                        int32_t* offsets, int32_t* row_token, int32_t* row_of, void* ws,
                        size_t ws_bytes, void* stream);

/* The whole block: out[T, D] = sum over the chosen experts e (ascending) of
 * w * SwiGLU_e(x) + SwiGLU_shared(x), accumulated in fp32, stored in x's dtype
 * (fp32 for MOE_F32, bf16 otherwise). x and out may not overlap. */
moe_status moe_forward(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T,
                       void* out, void* ws, size_t ws_bytes, void* stream);

/* moe_forward in a single launch, for decode-sized bf16 batches (1 to 32
 * tokens, at most 256 routed experts): router logits, selection, dispatch,
 * gate/up + SwiGLU, down projection and combine run as phases of one
 * cooperative grid separated by grid-wide barriers (hipLaunchCooperativeKernel:
 * every block of the grid is resident at once). Each phase runs the device code
 * of moe_forward's separate kernels, so the output equals moe_forward's bit for
 * bit, and the workspace is the same (moe_workspace_size, moe_workspace_layout).
 * The pages' MoE block and router as for moe_forward. Errors as moe_forward,
 * plus MOE_ERR_UNSUPPORTED for other dtypes or sizes (checked on the host before
 * any launch), and MOE_ERR_HIP when the cooperative launch is refused. */
moe_status moe_forward_fused(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T,
                             void* out, void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as moe_forward,
 * except that the workspace is the library's own static device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB; enough for about 380 tokens of the full
 * DeepSeek-V3 bf16 block), held on each device the library runs on until the
 * process ends. Nothing is allocated or freed by this call. Errors, besides
 * those of moe_forward: MOE_ERR_UNSUPPORTED when T needs a larger workspace
 * than that (checked on the host before any launch), MOE_ERR_HIP when the
 * array's device address cannot be found. Every call on one device uses the
 * same array: calls that overlap on one device (two streams, two host threads)
 * race and give undefined results; calls ordered on one stream are safe. The
 * array keeps the last call's intermediates; no call needs it cleared. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_static(const moe_config* cfg, const moe_weights* wts, const void* x, int64_t T,
                              void* out, void* stream);

/* Byte offsets inside the forward workspace of intermediates that tests read
 * after moe_forward has run (in stream order). Sizes: idx, w [T*K]; counts [E];
 * offsets [E+1]; row_token, row_of [T*K]; h_routed [T*K, I] and h_shared [T, S]
 * (fp32 / bf16 / e4m3 codes per dtype); h_scale [T*K, I/128] and
 * h_shared_scale [T, S/128] (fp8 only); o_routed [T*K, D] and o_shared [T, D]
 * (x's dtype); xq [T, D] and x_scale [T, D/128] (fp8 only). */
typedef struct {
  size_t idx, w, counts, offsets, row_token, row_of;
  size_t h_routed, h_shared, h_scale, h_shared_scale;
  size_t o_routed, o_shared, xq, x_scale;
  size_t total;
} moe_ws_layout;
moe_status moe_workspace_layout(const moe_config* cfg, int64_t T, moe_ws_layout* layout);

/* Dense SwiGLU feed-forward of the model's first three layers. "Hardware for
 * DeepSeek-V3 and R1: Why a 671B MoE Model Needs So Much Memory", section "Why
 * the dense layers and shared expert matter": those layers are ordinary dense
 * feed-forward blocks with an intermediate size of 18,432; their MLP has the
 * form the MoE block page gives its shared expert:
 *   out[T, D] = W2 (silu(W1 x) * (W3 x)) per token, no biases; the activation h
 *   is formed in fp32 and stored in the activation dtype (fp32, bf16, or e4m3
 *   with one fp32 scale per token per 128 columns, x quantised the same way);
 *   out is stored in x's dtype (fp32 for MOE_F32, bf16 otherwise).
 * The same GEMM kernels as the block's shared expert, with no router, dispatch
 * or combine. Conventions as above (device pointers, 16-byte aligned, ws of at
 * least moe_ffn_workspace_size() bytes, stream-ordered, host-side checks). */
typedef struct {
  int32_t dim;    /* D: 7168 in DeepSeek-V3 */
  int32_t inter;  /* I, the dense intermediate size: 18432 */
  int32_t dtype;  /* moe_dtype; bf16 needs dim % 128 == 0 and inter % 32 == 0,
                     fp8 dim and inter multiples of 128 */
} moe_ffn_config;

/* Dense FFN weights, device pointers, [out, in] row-major:
 *   w1, w3 [I, D];  w2 [D, I]   (fp32 / bf16 / e4m3fn per dtype)
 *   FP8 only, fp32 scales per 128x128 block: s1, s3 [I/128, D/128];
 *   s2 [D/128, I/128]. NULL for other dtypes. */
typedef struct {
  const void *w1, *w3, *w2;
  const float *s1, *s3, *s2;
} moe_ffn_weights;

/* Bytes of scratch moe_ffn needs for T tokens.
 * Errors: MOE_ERR_ARG (null, T < 0), MOE_ERR_CONFIG (sizes not positive, unknown
 * dtype), MOE_ERR_UNSUPPORTED (alignment of dim / inter for the dtype, too many
 * tokens). */
moe_status moe_ffn_workspace_size(const moe_ffn_config* cfg, int64_t T, size_t* bytes);

/* out[T, D] = the dense FFN of x[T, D] (fp32 for MOE_F32, bf16 otherwise).
 * x and out may not overlap. Errors as moe_ffn_workspace_size, plus
 * MOE_ERR_ARG for NULL or misaligned tensors (fp8 without its scales),
 * MOE_ERR_WORKSPACE for a short ws, MOE_ERR_HIP for a failed launch. */
moe_status moe_ffn(const moe_ffn_config* cfg, const moe_ffn_weights* wts, const void* x, int64_t T,
                   void* out, void* ws, size_t ws_bytes, void* stream);

/* Per-kernel GPU timing, for measurement only (the bench uses it; nothing else needs it).
 * While enabled (on != 0), every kernel the calls above launch is bracketed by a pair of HIP
 * events recorded on its stream; enabling or disabling drops any collected records. Enabling
 * creates HIP events (a host-side allocation), so do it outside code that must not allocate.
 * Errors: MOE_ERR_HIP if events cannot be created. Not thread-safe with concurrent launches. */
moe_status moe_timing_enable(int on);
/* Restrict the spans to kernels whose name contains name_part (NULL or "" = every kernel); the
 * events cost a few microseconds per launch, so a measurement can keep them on the kernel it
 * studies only. Persists across moe_timing_enable. Always MOE_OK. */
moe_status moe_timing_filter(const char* name_part);
/* Waits for the recorded events, then writes one line per kernel name,
 * "<name> <launches> <total milliseconds>\n", into buf (NUL-terminated, truncated to
 * bytes) and clears the records. Returns the number of lines, or a negative moe_status. */
int moe_timing_report(char* buf, size_t bytes);

/* Static description of a status code. */
const char* moe_status_str(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
