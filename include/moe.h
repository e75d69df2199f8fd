/* moe.h — C ABI of the MI355X (gfx950) DeepSeekMoE layer-forward library (libmoe.so).
 *
 * The layer is the one of the page "DeepSeek-V3 技術報告"
 * (xyznot.com/zh-tw/paper/2412.19437), section 方法 §2:
 *
 *   h'_t = u_t + sum_{i<=N_s} FFN^(s)_i(u_t) + sum_{i<=N_r} g_{i,t} FFN^(r)_i(u_t)
 *   s_{i,t} = Sigmoid(u_t^T e_i)
 *   g'_{i,t} = s_{i,t} if s_{i,t} + b_i is among the K_r largest {s_{j,t} + b_j}, else 0
 *   g_{i,t} = g'_{i,t} / sum_j g'_{j,t}
 *   end of step: b_i <- b_i - gamma if expert i is overloaded, + gamma if underloaded
 *
 * with every expert FFN a bias-free SwiGLU, FFN(x) = (SiLU(x Wg^T) * (x Wu^T)) Wd^T,
 * and, for MOE_DTYPE_FP8_B128, the FP8 scheme of the same page's 核心概念 list:
 * E4M3 values with one fp32 scale per 1x128 activation tile and per 128x128
 * weight block, accumulated in fp32.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates device memory and never synchronises: work is enqueued on
 *    `stream` (which must belong to the calling thread's current device) and
 *    results are valid once the stream has completed it.  Scratch memory is the
 *    caller's workspace.  Between calls the library keeps only per-device facts
 *    set up once per device (its CU count and the kernels' LDS limits), under
 *    std::call_once / a mutex, so host threads may call it concurrently.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and the outputs are untouched.  A failed launch
 *    returns MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Row-major layouts throughout.  Expert weights are stored like
 *    nn.Linear weights, [out_features, in_features]:
 *        gate/up projections  [N, I, d]   (row n of expert e = output feature n)
 *        down projection      [N, d, I]
 *  - Results are bit-reproducible run to run (no floating-point atomics).
 *  - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, K_r > N_r, ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle (see each call) */
  MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_dtype {
  MOE_DTYPE_F32 = 0,       /* u, weights, out: fp32 */
  MOE_DTYPE_BF16 = 1,      /* u, weights, out: bf16 */
  MOE_DTYPE_FP8_B128 = 2   /* u, out: bf16; weights E4M3 codes + fp32 128x128 block scales */
} moe_dtype;

/* Layer shape.  Limits: tokens >= 0; 1 <= n_routed <= 512; 1 <= top_k <= min(n_routed, 32);
 * 0 <= n_shared <= 64; hidden, inter >= 1 and multiples of 8 (bf16) or of 128 (fp8);
 * tokens * top_k < 2^31; fp8 also tokens * hidden, (padded permuted rows) * inter and
 * hidden * inter below 2^32 (the FP8 GEMMs' 32-bit byte offsets).  Outside them the calls
 * return MOE_ERR_INVALID_ARG (malformed) or MOE_ERR_UNSUPPORTED. */
typedef struct moe_shape {
  int32_t tokens;    /* T   */
  int32_t hidden;    /* d   */
  int32_t n_routed;  /* N_r */
  int32_t top_k;     /* K_r */
  int32_t n_shared;  /* N_s */
  int32_t inter;     /* I   */
  int32_t dtype;     /* moe_dtype */
} moe_shape;

/* Expert weights.  Element type: fp32 (F32), bf16 (BF16) or E4M3FN bytes (FP8_B128).
 * The shared pointers may be NULL when n_shared == 0.  The *_scale pointers are
 * read only for FP8_B128: one fp32 per 128x128 block of each stored matrix,
 * laid out [N, out/128, in/128] (as written by moe_quantize_weights). */
typedef struct moe_weights {
  const void* w_gate;       /* [N_r, I, d] */
  const void* w_up;         /* [N_r, I, d] */
  const void* w_down;       /* [N_r, d, I] */
  const void* sh_gate;      /* [N_s, I, d] */
  const void* sh_up;        /* [N_s, I, d] */
  const void* sh_down;      /* [N_s, d, I] */
  const float* w_gate_scale;   /* [N_r, I/128, d/128] */
  const float* w_up_scale;     /* [N_r, I/128, d/128] */
  const float* w_down_scale;   /* [N_r, d/128, I/128] */
  const float* sh_gate_scale;  /* [N_s, I/128, d/128] */
  const float* sh_up_scale;    /* [N_s, I/128, d/128] */
  const float* sh_down_scale;  /* [N_s, d/128, I/128] */
} moe_weights;

/* Number of stage boundaries moe_forward_profiled() records events at. */
#define MOE_FORWARD_EVENTS 6

/* Bytes of device workspace that moe_route and moe_forward need for `shape`
 * (one buffer serves both).  Never fails for a shape within the limits above. */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* Routing: sigmoid affinities, biased top-K_r selection, normalised gates, per-expert load
 * (方法 §2: the s_{i,t} and g'_{i,t} equations).
 *   u          [T, d]     fp32 (F32) or bf16 (BF16, FP8_B128)
 *   centroids  [N_r, d]   fp32 (e_i)
 *   bias       [N_r]      fp32 (b_i; only ranks experts, never enters a gate)
 *   topk_idx   [T, K_r]   int32 out: selected experts ordered by s+b descending, ties to the
 *                         lower index; NaN scores rank below every number
 *   topk_gate  [T, K_r]   fp32 out: s_{i,t} / sum of the selected s, in topk_idx order
 *   expert_load[N_r]      int32 out: number of (token, slot) picks of each expert
 * Affinities are computed fp32-accurately (the contraction over d is exact products
 * accumulated in fp32).  T == 0 writes expert_load = 0 and launches nothing else. */
moe_status moe_route(const moe_shape* shape, const void* u, const float* centroids,
                     const float* bias, int32_t* topk_idx, float* topk_gate,
                     int32_t* expert_load, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Size of the fixed device array that holds moe_route_noalloc's scratch (one per GPU). */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_route without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments,
 * outputs, errors and results as moe_route, bit for bit.  The routing's scratch lives in a
 * file-scope device array of MOE_ROUTE_NOALLOC_SCRATCH_BYTES (64 MiB): each GPU the library
 * runs on holds its own copy from the library's load until the process ends, and its address is
 * looked up once per device on the first call there.  The call allocates nothing.
 *   - A shape whose routing scratch exceeds the array (at d=7168, N_r=256 that is T > 52330)
 *     returns MOE_ERR_WORKSPACE before anything touches the GPU.
 *   - `stream` must belong to the calling thread's current device (else MOE_ERR_INVALID_ARG).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 *     two host threads, or a call overlapping a graph replay that contains one) race on it and
 *     must be ordered by the caller.  Nothing in the array needs clearing between calls. */
moe_status moe_route_noalloc(const moe_shape* shape, const void* u, const float* centroids,
                             const float* bias, int32_t* topk_idx, float* topk_gate,
                             int32_t* expert_load, hipStream_t stream);

/* moe_route with a per-token group limit.  The page's cross-node all-to-all section limits
 * every token to experts on at most 4 nodes and prints no rule for choosing them; the reading
 * here: the N_r experts form n_groups equal contiguous groups (expert i is in group
 * i / (N_r / n_groups)), a group's score is the highest s+b among its experts, the
 * topk_groups groups with the highest scores (ties to the lower group index; NaN below every
 * number) stay eligible, and the K_r experts are then picked among the eligible ones exactly as
 * in moe_route.  Gates and expert_load as in moe_route.  n_groups == 1 or
 * topk_groups == n_groups is moe_route.
 * Errors: MOE_ERR_INVALID_ARG unless 1 <= topk_groups <= n_groups <= 64, N_r % n_groups == 0 and
 * topk_groups * N_r / n_groups >= K_r (plus moe_route's checks); nothing is launched then. */
moe_status moe_route_grouped(const moe_shape* shape, int32_t n_groups, int32_t topk_groups,
                             const void* u, const float* centroids, const float* bias,
                             int32_t* topk_idx, float* topk_gate, int32_t* expert_load,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_route plus the sequence-wise balance statistic.  The page (方法 §2, last paragraph) adds
 * a tiny sequence-level balance loss (alpha = 0.0001) to the bias rule and prints no formula;
 * the reading here: for each of the T / seq_len sequences of consecutive tokens,
 *   f_i = N_r / (K_r seq_len) * (the sequence's picks of expert i),
 *   P_i = mean over the sequence's tokens of s_{i,t} / sum_j s_{j,t},
 *   seq_loss[q] = alpha * sum_i f_i P_i          (fp32 out, [T / seq_len]).
 * Routing outputs as in moe_route.  Errors: MOE_ERR_INVALID_ARG unless 1 <= seq_len <= 16384
 * divides T and seq_loss is non-null (plus moe_route's checks); nothing is launched then. */
moe_status moe_route_balance(const moe_shape* shape, int32_t seq_len, float alpha, const void* u,
                             const float* centroids, const float* bias, int32_t* topk_idx,
                             float* topk_gate, int32_t* expert_load, float* seq_loss,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Expert half of the layer (方法 §2, the h'_t equation): permutes tokens into per-expert
 * segments, runs every routed expert on its tokens and every shared expert on all tokens
 * (grouped SwiGLU GEMMs), and combines out_t = u_t + sum_s FFN_s(u_t) + sum_k gate FFN(u_t).
 *   u          [T, d]     fp32 (F32) or bf16 (BF16, FP8_B128; FP8 quantises it per 1x128 tile)
 *   topk_idx   [T, K_r]   int32 from moe_route (entries outside [0, N_r) are ignored)
 *   topk_gate  [T, K_r]   fp32 from moe_route
 *   out        [T, d]     fp32 (F32) or bf16 (BF16, FP8_B128); may not alias u
 * FP8_B128 needs d % 128 == 0 and I % 128 == 0 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_forward(const moe_shape* shape, const void* u, const moe_weights* weights,
                       const int32_t* topk_idx, const float* topk_gate, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_forward, recording events[0..MOE_FORWARD_EVENTS) on `stream` at its stage boundaries:
 * [0] start, [1] after the token->expert permutation, [2] after activation quantisation
 * (FP8 only; else right after [1]), [3] after the gate/up GEMM with SwiGLU, [4] after the
 * down GEMM, [5] after the combine.  events must hold MOE_FORWARD_EVENTS created events
 * (hipEvent_t); they are recorded, never created or destroyed, by the library. */
moe_status moe_forward_profiled(const moe_shape* shape, const void* u, const moe_weights* weights,
                                const int32_t* topk_idx, const float* topk_gate, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* events, int32_t n_events);

/* Weight gradients written by moe_backward: bf16, same layouts as the weights
 * (gate/up [N, I, d], down [N, d, I], N = N_r or N_s).  Owned by the caller. */
typedef struct {
  void* w_gate;
  void* w_up;
  void* w_down;
  void* sh_gate;
  void* sh_up;
  void* sh_down;
} moe_weight_grads;

/* Bytes of device workspace moe_backward needs for `shape` (BF16 or FP8_B128; d and I multiples
 * of 128).  MOE_ERR_UNSUPPORTED for other shapes. */
moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes);

/* Layer backward (方法 §2, the h'_t, s_{i,t} and g'_{i,t} equations): gradients of
 * L = <dout, h'> with the routing (topk_idx) held fixed — the Topk is piecewise constant — and
 * none for the bias, which never enters a gate.  With g_k = s_k / S (S = sum of the selected
 * s) the gate gradient flows through the unbiased s into u and the centroids.
 *   u, centroids, weights, topk_idx, topk_gate   as given to moe_route / moe_forward
 *   dout        [T, d]   bf16 dL/dh'
 *   du          [T, d]   bf16 out: dL/du (residual + every expert's input gradient + router term)
 *   d_centroids [N_r, d] fp32 out (rows of experts no token picked are zero)
 *   dw          bf16 out, every routed and shared expert's gate/up/down gradient (zero for
 *               experts no token picked)
 * FP8_B128 (section 方法, FP8 Mixed Precision Training: the forward and both backward GEMM
 * kinds in FP8; 核心概念, FP8 item: E4M3, 1x128 activation tiles, 128x128 weight blocks): the
 * weights are the E4M3 codes and block scales of moe_forward; every product runs on E4M3
 * operands with fp32 accumulation: dout and u in 1x128 tiles along d, [dA dB] along 2I, the
 * weights transposed per 128x128 block (codes and scales carry over), and for the weight
 * gradients the transposed activations in runs of 128 of each expert's rows (token order);
 * quantised from bf16 (u, dout, H, dA, dB) or fp32 (gate * dout).  Gates, router and residual
 * stay unquantised, and every output is bf16 / fp32 as for BF16.
 * Errors: MOE_ERR_UNSUPPORTED unless dtype is BF16 or FP8_B128, d % 128 == 0, I % 128 == 0;
 * MOE_ERR_INVALID_ARG for a null pointer (FP8_B128: also a null weight scale) or du aliasing
 * u or dout; MOE_ERR_WORKSPACE if workspace_bytes < moe_backward_workspace_size.  Nothing is
 * launched on an error. */
moe_status moe_backward(const moe_shape* shape, const void* u, const float* centroids,
                        const moe_weights* weights, const int32_t* topk_idx, const float* topk_gate,
                        const void* dout, void* du, float* d_centroids, const moe_weight_grads* dw,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Saved-input training pair (BF16 and FP8_B128).  The backward's gate/up step needs the SwiGLU inputs
 * a = x W_gate^T and b = x W_up^T of every (token, expert) row (方法 §2, the h'_t equation: the
 * expert FFN is SwiGLU).  moe_backward recomputes them with a second gate/up product; this pair
 * keeps them from the forward instead, trading [max_rows, 2I] bf16 of device memory for that
 * product.  The results equal moe_forward / moe_backward up to the rounding of a and b to bf16
 * before the backward's SwiGLU derivative (FP8_B128: a and b of the FP8 forward product, kept
 * in bf16; the backward's other FP8 products are unchanged).
 *
 * moe_saved_inputs_size: bytes of the saved buffer for `shape` (bf16 [max_rows, 2I] for both
 * dtypes).  Errors as for moe_backward_workspace_size. */
moe_status moe_saved_inputs_size(const moe_shape* shape, size_t* bytes);

/* moe_forward (same arguments, same workspace, same out) that also writes the SwiGLU inputs
 * [a b] of every row of the permuted token->expert layout to `saved` (bf16, row r at
 * saved + r * 2I: a then b; the layout is private to the library and fixed by topk_idx).  The
 * caller owns `saved` and passes it, unchanged, with the same topk_idx to moe_backward_saved.
 * Errors: those of moe_forward and moe_backward_workspace_size (so MOE_ERR_UNSUPPORTED for
 * F32); MOE_ERR_INVALID_ARG for a null `saved` (T > 0) or one aliasing u or out;
 * MOE_ERR_WORKSPACE if saved_bytes < moe_saved_inputs_size. */
moe_status moe_forward_train(const moe_shape* shape, const void* u, const moe_weights* weights,
                             const int32_t* topk_idx, const float* topk_gate, void* out, void* saved,
                             size_t saved_bytes, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_backward (same arguments and outputs, same workspace) reading the SwiGLU inputs that
 * moe_forward_train saved for the same shape, weights and topk_idx in place of recomputing
 * them.  Errors: those of moe_backward; MOE_ERR_INVALID_ARG for a null `saved` or one aliasing du; MOE_ERR_WORKSPACE if
 * saved_bytes < moe_saved_inputs_size. */
moe_status moe_backward_saved(const moe_shape* shape, const void* u, const float* centroids,
                              const moe_weights* weights, const int32_t* topk_idx, const float* topk_gate,
                              const void* saved, size_t saved_bytes, const void* dout, void* du,
                              float* d_centroids, const moe_weight_grads* dw, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Auxiliary-loss-free bias update (方法 §2, last paragraph), in place on bias[N_r] (fp32):
 * expert i is overloaded when load_i * N_r > total_assignments (= T * K_r, i.e. above the
 * step mean), underloaded when below; b_i <- b_i - gamma resp. b_i + gamma as one fp32 add;
 * equal to the mean: unchanged. */
moe_status moe_update_bias(int32_t n_routed, int64_t total_assignments, const int32_t* expert_load,
                           float* bias, float gamma, hipStream_t stream);

/* One-time weight preparation for moe_forward and moe_backward (untimed, outside the hot path).
 *   logical       the layer's weights as stored: bf16 for BF16 and FP8_B128, fp32 for F32
 *                 (scale pointers ignored; shared pointers may be NULL when n_shared == 0)
 *   packed        device buffer of *packed_bytes bytes owned by the caller (FP8_B128 only)
 *   prepared      out: the moe_weights to pass to moe_forward / moe_backward
 * With prepared == NULL the call only writes to *packed_bytes the size `packed` needs (0 for BF16
 * and F32) and touches nothing else.  BF16 and F32: the kernels read the weights as stored, so
 * `prepared` receives the logical pointers and nothing is launched.  FP8_B128 (核心概念, FP8 item:
 * E4M3 weights with one fp32 scale per 128x128 block): every stack is quantised as by
 * moe_quantize_weights into `packed` (the six code stacks, then the six scale stacks, each
 * 256-byte aligned), and `prepared` points into it.  `packed` must stay allocated while
 * `prepared` is in use and may not overlap the logical weights.
 * Errors: check_shape's; MOE_ERR_INVALID_ARG for a null logical, packed_bytes, needed weight
 * pointer or (FP8_B128) packed; MOE_ERR_WORKSPACE if *packed_bytes is too small.  Nothing is
 * launched on an error. */
moe_status moe_prepare_weights(const moe_shape* shape, const moe_weights* logical, void* packed,
                               size_t* packed_bytes, moe_weights* prepared, hipStream_t stream);

/* FP8 weight preparation (核心概念, FP8 item: 128x128 block scaling): quantises a stack of
 * n_mats bf16 matrices [rows, cols] into E4M3FN codes [n_mats, rows, cols] and fp32 scales
 * [n_mats, rows/128, cols/128]: scale = amax/448 (1 for an all-zero block), code =
 * round-to-nearest-even E4M3FN of fp32(x / scale), saturating at 448.
 * rows and cols must be multiples of 128. */
moe_status moe_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, const void* w_bf16,
                                uint8_t* codes, float* scales, hipStream_t stream);

/* FP8 activation quantisation (核心概念, FP8 item: 1x128 tile scaling), the step moe_forward
 * runs on u for FP8_B128: x [rows, cols] bf16 -> codes [rows, cols] E4M3FN and scales
 * [rows, cols/128] fp32, same rounding rule as moe_quantize_weights.  cols % 128 == 0. */
moe_status moe_quantize_act(int32_t rows, int32_t cols, const void* x_bf16, uint8_t* codes,
                            float* scales, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
