// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, and the ordered launch of the kernels of each call.
#include <mutex>
#include <new>

#include "moe_internal.h"

namespace moe {

hipError_t launch_gemm_bf16_swiglu(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_bf16_swiglu_save(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_bf16_down(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_f32_swiglu(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_f32_down(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_swiglu(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_swiglu_save(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_down(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_bf16_swiglu_bwd(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_bf16_wgrad(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_bf16_dgrad(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_swiglu_bwd(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_wgrad(const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_fp8_dgrad(const GemmOperands& g, hipStream_t st);

hipError_t launch_gemm_swiglu(int dtype, const GemmOperands& g, hipStream_t st) {
  if (dtype == MOE_DTYPE_F32) return launch_gemm_f32_swiglu(g, st);
  if (dtype == MOE_DTYPE_BF16) return launch_gemm_bf16_swiglu(g, st);
  return launch_gemm_fp8_swiglu(g, st);
}
hipError_t launch_gemm_down(int dtype, const GemmOperands& g, hipStream_t st) {
  if (dtype == MOE_DTYPE_F32) return launch_gemm_f32_down(g, st);
  if (dtype == MOE_DTYPE_BF16) return launch_gemm_bf16_down(g, st);
  return launch_gemm_fp8_down(g, st);
}

static size_t elem_bytes(int dtype) { return dtype == MOE_DTYPE_F32 ? 4 : 2; }

WorkspacePlan plan_workspace(const moe_shape& s) {
  WorkspacePlan p{};
  const int64_t T = s.tokens, d = s.hidden, N = s.n_routed, K = s.top_k, Ns = s.n_shared, I = s.inter;
  const bool fp8 = s.dtype == MOE_DTYPE_FP8_B128;
  p.route_blocks = ceil_div(T, kRouteTokens);
  p.chunks = ceil_div(T, kChunkTokens);
  p.max_tiles = walk_max_tiles(T, K, N, Ns);
  p.max_rows = p.max_tiles * kTileM;
  const size_t A = 256;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, A);
    return at;
  };
  const bool mfma_route = route_uses_mfma(s);
  const int64_t route_rows = mfma_route ? route_mfma_blocks(s) : p.route_blocks;
  const int64_t n_pad = ceil_div(N, 128) * 128;
  p.route_partial = take((size_t)route_rows * N * 4);
  p.route_e_hi = take(mfma_route ? (size_t)n_pad * d * 2 : 0);
  p.route_e_mid = take(mfma_route ? (size_t)n_pad * d * 2 : 0);
  p.route_e_lo = take(mfma_route ? (size_t)n_pad * d * 2 : 0);
  p.route_scores = take((size_t)T * N * 4);   // the fp32 path writes it only for the balance statistic
  const int splits = route_logit_splits(s);
  p.route_zpart = take(splits > 1 ? (size_t)splits * T * N * 4 : 0);
  // sequences of L >= 64 tokens: T/L sequences of ceil(L/64) chunks, at most T/64 + T/L <= T/32
  p.route_bal_part = take((size_t)ceil_div(T, 32) * N * 4);
  p.route_bytes = o;
  o = 0;
  p.chunk_counts = take((size_t)p.chunks * N * 4);
  p.chunk_base = take((size_t)p.chunks * N * 4);
  p.seg_off = take((size_t)(N + Ns + 1) * 4);
  p.seg_rows = take((size_t)(N + Ns) * 4);
  p.tile_seg = take((size_t)p.max_tiles * 4);
  p.pair_seg = take((size_t)p.max_tiles * 4);
  p.pair_off = take((size_t)(N + Ns + 1) * 4);
  p.row_token = take((size_t)p.max_rows * 4);
  p.perm_row = take((size_t)T * K * 4);
  p.h = take((size_t)p.max_rows * I * (fp8 ? 1 : elem_bytes(s.dtype)));
  p.h_scale = take(fp8 ? (size_t)p.max_rows * (I / 128) * 4 : 0);
  p.y = take((size_t)p.max_rows * d * elem_bytes(s.dtype == MOE_DTYPE_F32 ? MOE_DTYPE_F32 : MOE_DTYPE_BF16));
  p.u_q = take(fp8 ? (size_t)T * d : 0);
  p.u_scale = take(fp8 ? (size_t)T * (d / 128) * 4 : 0);
  p.forward_bytes = o;
  p.total = p.route_bytes > p.forward_bytes ? p.route_bytes : p.forward_bytes;
  p.bwd_h = take((size_t)p.max_rows * I * 2);
  p.bwd_dab = take((size_t)p.max_rows * 2 * I * 2);
  p.bwd_row_gate = take((size_t)p.max_rows * 4);
  p.bwd_row_dz = take((size_t)p.max_rows * 4);
  p.bwd_dg_part = take((size_t)p.max_rows * (I / 128 > 0 ? I / 128 : 1) * 4);
  p.bwd_dc_part = take((size_t)p.max_tiles * d * 4);
  const size_t eb = fp8 ? 1 : 2;   // bytes per element of the transposed copies
  const int64_t P = p.max_rows, d8 = d / 128, i8 = I / 128, p8 = P / 128;

  p.bwd_dy_t = take((size_t)d * P * eb);
  p.bwd_h_t = take((size_t)I * P * eb);
  p.bwd_dab_t = take((size_t)2 * I * P * eb);
  p.bwd_x_t = take((size_t)d * P * eb);
  p.bwd_dhu = take(fp8 ? (size_t)P * I * 2 : 0);
  p.bwd_dy_ts = take(fp8 ? (size_t)d * p8 * 4 : 0);
  p.bwd_h_ts = take(fp8 ? (size_t)I * p8 * 4 : 0);
  p.bwd_dab_ts = take(fp8 ? (size_t)2 * I * p8 * 4 : 0);
  p.bwd_x_ts = take(fp8 ? (size_t)d * p8 * 4 : 0);
  p.bwd_dout_q = take(fp8 ? (size_t)T * d : 0);
  p.bwd_dout_s = take(fp8 ? (size_t)T * d8 * 4 : 0);
  p.bwd_dab_q = take(fp8 ? (size_t)P * 2 * I : 0);
  p.bwd_dab_s = take(fp8 ? (size_t)P * 2 * i8 * 4 : 0);
  p.backward_total = o;
  return p;
}

static moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->tokens < 0 || s->hidden < 1 || s->inter < 1 || s->n_routed < 1 || s->top_k < 1 || s->n_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_routed) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_DTYPE_F32 && s->dtype != MOE_DTYPE_BF16 && s->dtype != MOE_DTYPE_FP8_B128)
    return MOE_ERR_INVALID_ARG;
  if (s->n_routed > kMaxRouted || s->top_k > kMaxTopK || s->n_shared > kMaxShared) return MOE_ERR_UNSUPPORTED;
  if (s->hidden % 8 != 0 || s->inter % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->dtype == MOE_DTYPE_FP8_B128 && (s->hidden % 128 != 0 || s->inter % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  const int64_t T = s->tokens, K = s->top_k;
  if (T * K >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const int64_t max_tiles = walk_max_tiles(T, K, s->n_routed, s->n_shared);
  if (max_tiles * kTileM >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  // the FP8 GEMMs address u codes [T, d], H codes [rows, I] and one expert's weight codes with
  // 32-bit byte offsets (the bf16 GEMMs fall back to a 64-bit-addressed kernel instead)
  if (s->dtype == MOE_DTYPE_FP8_B128) {
    const int64_t lim = int64_t(1) << 32;
    if (T * s->hidden >= lim || max_tiles * kTileM * s->inter >= lim || (int64_t)s->hidden * s->inter >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

static moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// saved: null, or (BF16, FP8_B128) [max_rows, 2I] bf16 for the gate/up GEMM's SwiGLU inputs [a b]
static moe_status forward_impl(const moe_shape* shape, const void* u, const moe_weights* w, const int32_t* idx,
                               const float* gate, void* out, void* ws, size_t ws_bytes, hipStream_t st,
                               hipEvent_t* ev, int32_t n_ev, void* saved = nullptr) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_shape& s = *shape;
  if (ev && n_ev < MOE_FORWARD_EVENTS) return MOE_ERR_INVALID_ARG;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
  if (s.tokens == 0) {
    for (int i = 0; i < (ev ? MOE_FORWARD_EVENTS : 0); ++i)
      if (mark(i) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
  }
  if (!u || !w || !idx || !gate || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_ERR_INVALID_ARG;
  const bool fp8 = s.dtype == MOE_DTYPE_FP8_B128;
  if (fp8 && (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale)) return MOE_ERR_INVALID_ARG;
  if (fp8 && s.n_shared > 0 && (!w->sh_gate_scale || !w->sh_up_scale || !w->sh_down_scale))
    return MOE_ERR_INVALID_ARG;
  if (out == u) return MOE_ERR_INVALID_ARG;
  const WorkspacePlan p = plan_workspace(s);
  if (ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(ws);

  if (mark(0) != hipSuccess) return MOE_ERR_HIP;
  if ((rc = hip_status(launch_permute(s, idx, p, wsb, st))) != MOE_OK) return rc;
  if (mark(1) != hipSuccess) return MOE_ERR_HIP;
  const void* act = u;
  const float* act_scale = nullptr;
  if (fp8) {
    uint8_t* uq = reinterpret_cast<uint8_t*>(wsb + p.u_q);
    float* us = reinterpret_cast<float*>(wsb + p.u_scale);
    if ((rc = hip_status(launch_quantize_act(s.tokens, s.hidden, u, uq, us, st))) != MOE_OK) return rc;
    act = uq;
    act_scale = us;
  }
  if (mark(2) != hipSuccess) return MOE_ERR_HIP;

  GemmOperands g1{};
  g1.act = act;
  g1.act_scale = act_scale;
  g1.row_token = reinterpret_cast<const int32_t*>(wsb + p.row_token);
  g1.w_routed[0] = w->w_gate;
  g1.w_routed[1] = w->w_up;
  g1.w_shared[0] = w->sh_gate;
  g1.w_shared[1] = w->sh_up;
  g1.s_routed[0] = w->w_gate_scale;
  g1.s_routed[1] = w->w_up_scale;
  g1.s_shared[0] = w->sh_gate_scale;
  g1.s_shared[1] = w->sh_up_scale;
  g1.tile_seg = reinterpret_cast<const int32_t*>(wsb + p.tile_seg);
  g1.seg_off = reinterpret_cast<const int32_t*>(wsb + p.seg_off);
  g1.seg_rows = reinterpret_cast<const int32_t*>(wsb + p.seg_rows);
  g1.pair_seg = reinterpret_cast<const int32_t*>(wsb + p.pair_seg);
  g1.pair_off = reinterpret_cast<const int32_t*>(wsb + p.pair_off);
  g1.n_routed = s.n_routed;
  g1.n_seg = s.n_routed + s.n_shared;
  g1.K = s.hidden;
  g1.N = s.inter;
  g1.act_rows = s.tokens;
  g1.max_tiles = p.max_tiles;
  g1.max_pairs = walk_max_pairs(p.max_tiles, s.n_routed + s.n_shared);
  g1.small_segments = (int64_t)s.tokens * s.top_k < (int64_t)kTileM * s.n_routed;
  g1.out = wsb + p.h;
  g1.out_scale = fp8 ? reinterpret_cast<float*>(wsb + p.h_scale) : nullptr;
  if (saved) {
    g1.out2 = saved;
    if ((rc = hip_status(fp8 ? launch_gemm_fp8_swiglu_save(g1, st) : launch_gemm_bf16_swiglu_save(g1, st))) != MOE_OK)
      return rc;
  } else if ((rc = hip_status(launch_gemm_swiglu(s.dtype, g1, st))) != MOE_OK) {
    return rc;
  }
  if (mark(3) != hipSuccess) return MOE_ERR_HIP;

  GemmOperands g2{};
  g2.act = wsb + p.h;
  g2.act_scale = g1.out_scale;
  g2.row_token = nullptr;
  g2.w_routed[0] = w->w_down;
  g2.w_shared[0] = w->sh_down;
  g2.s_routed[0] = w->w_down_scale;
  g2.s_shared[0] = w->sh_down_scale;
  g2.tile_seg = g1.tile_seg;
  g2.seg_off = g1.seg_off;
  g2.seg_rows = g1.seg_rows;
  g2.pair_seg = g1.pair_seg;
  g2.pair_off = g1.pair_off;
  g2.n_routed = s.n_routed;
  g2.n_seg = g1.n_seg;
  g2.K = s.inter;
  g2.N = s.hidden;
  g2.act_rows = p.max_rows;
  g2.max_tiles = p.max_tiles;
  g2.max_pairs = g1.max_pairs;
  g2.small_segments = g1.small_segments;
  g2.out = wsb + p.y;
  if ((rc = hip_status(launch_gemm_down(s.dtype, g2, st))) != MOE_OK) return rc;
  if (mark(4) != hipSuccess) return MOE_ERR_HIP;

  if ((rc = hip_status(launch_combine(s, u, gate, p, wsb, out, st))) != MOE_OK) return rc;
  if (mark(5) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = plan_workspace(*shape).total;
  return MOE_OK;
}

// route_only: the workspace holds the routing's scratch only (moe_route_noalloc), not the
// forward's as well
static moe_status route_impl(const moe_shape* shape, GroupLimit gl, const void* u, const float* centroids,
                             const float* bias, int32_t* topk_idx, float* topk_gate, int32_t* expert_load,
                             void* workspace, size_t workspace_bytes, hipStream_t stream, bool keep_scores = false,
                             bool route_only = false) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!expert_load) return MOE_ERR_INVALID_ARG;
  if (shape->tokens > 0 && (!u || !centroids || !bias || !topk_idx || !topk_gate || !workspace))
    return MOE_ERR_INVALID_ARG;
  const WorkspacePlan p = plan_workspace(*shape);
  if (shape->tokens > 0 && workspace_bytes < (route_only ? p.route_bytes : p.total)) return MOE_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);
  RouteWorkspace rw{reinterpret_cast<int32_t*>(wsb + p.route_partial), reinterpret_cast<uint16_t*>(wsb + p.route_e_hi),
                    reinterpret_cast<uint16_t*>(wsb + p.route_e_mid), reinterpret_cast<uint16_t*>(wsb + p.route_e_lo),
                    reinterpret_cast<float*>(wsb + p.route_scores), reinterpret_cast<float*>(wsb + p.route_zpart)};
  // the MFMA path always stages the affinities there; the fp32 path only when asked
  if (!keep_scores && !route_uses_mfma(*shape)) rw.scores = nullptr;
  return hip_status(launch_route(*shape, u, centroids, bias, gl, topk_idx, topk_gate, expert_load, rw, stream));
}

moe_status moe_route(const moe_shape* shape, const void* u, const float* centroids, const float* bias,
                     int32_t* topk_idx, float* topk_gate, int32_t* expert_load, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return route_impl(shape, GroupLimit{1, 1}, u, centroids, bias, topk_idx, topk_gate, expert_load, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

// ---- moe_route_noalloc: the routing scratch in a fixed device array ----
//
// One copy of `scratch` exists on every GPU the library runs on, from module load until the
// process ends.  In host code its name is only a host-side stand-in: the device address of the
// current GPU's copy comes from hipGetSymbolAddress, looked up once per device and kept in
// g_scratch_ptr; only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

// The current device's copy of `scratch`; `stream` must belong to that device.
moe_status scratch_for(hipStream_t stream, void** ptr) {
  int dev = 0;
  if (current_device(&dev) != hipSuccess || dev >= kScratchDevices) return MOE_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if (sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return MOE_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_route_noalloc(const moe_shape* shape, const void* u, const float* centroids, const float* bias,
                             int32_t* topk_idx, float* topk_gate, int32_t* expert_load, hipStream_t stream) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!expert_load) return MOE_ERR_INVALID_ARG;
  if (shape->tokens > 0 && (!u || !centroids || !bias || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  // size check first, on the host: a shape beyond the array is refused before the GPU is touched
  if (plan_workspace(*shape).route_bytes > (size_t)MOE_ROUTE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ptr = nullptr;
  if ((rc = scratch_for(stream, &ptr)) != MOE_OK) return rc;
  // the routing kernels write every scratch element they later read (partial counts, split
  // centroids, affinities, split-K partial logits), so nothing has to be cleared between calls
  return route_impl(shape, GroupLimit{1, 1}, u, centroids, bias, topk_idx, topk_gate, expert_load, ptr,
                    MOE_ROUTE_NOALLOC_SCRATCH_BYTES, stream, false, true);
}

moe_status moe_route_grouped(const moe_shape* shape, int32_t n_groups, int32_t topk_groups, const void* u,
                             const float* centroids, const float* bias, int32_t* topk_idx, float* topk_gate,
                             int32_t* expert_load, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (n_groups < 1 || n_groups > 64 || topk_groups < 1 || topk_groups > n_groups) return MOE_ERR_INVALID_ARG;
  if (shape->n_routed % n_groups != 0) return MOE_ERR_INVALID_ARG;
  if ((int64_t)topk_groups * (shape->n_routed / n_groups) < shape->top_k) return MOE_ERR_INVALID_ARG;
  return route_impl(shape, GroupLimit{n_groups, topk_groups}, u, centroids, bias, topk_idx, topk_gate, expert_load,
                    workspace, workspace_bytes, stream);
}

moe_status moe_route_balance(const moe_shape* shape, int32_t seq_len, float alpha, const void* u,
                             const float* centroids, const float* bias, int32_t* topk_idx, float* topk_gate,
                             int32_t* expert_load, float* seq_loss, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (seq_len < 1 || seq_len > 16384 || shape->tokens % seq_len != 0) return MOE_ERR_INVALID_ARG;
  if (shape->tokens > 0 && !seq_loss) return MOE_ERR_INVALID_ARG;
  if ((rc = route_impl(shape, GroupLimit{1, 1}, u, centroids, bias, topk_idx, topk_gate, expert_load, workspace,
                       workspace_bytes, stream, true)) != MOE_OK)
    return rc;
  if (shape->tokens == 0) return MOE_OK;
  const WorkspacePlan p = plan_workspace(*shape);
  const float* scores = reinterpret_cast<const float*>(static_cast<char*>(workspace) + p.route_scores);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.route_bal_part);
  return hip_status(launch_seq_balance(*shape, seq_len, alpha, scores, topk_idx, part, seq_loss, stream));
}

moe_status moe_forward(const moe_shape* shape, const void* u, const moe_weights* weights, const int32_t* topk_idx,
                       const float* topk_gate, void* out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return forward_impl(shape, u, weights, topk_idx, topk_gate, out, workspace, workspace_bytes, stream, nullptr, 0);
}

moe_status moe_forward_profiled(const moe_shape* shape, const void* u, const moe_weights* weights,
                                const int32_t* topk_idx, const float* topk_gate, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events, int32_t n_events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  return forward_impl(shape, u, weights, topk_idx, topk_gate, out, workspace, workspace_bytes, stream, events,
                      n_events);
}

// FP8_B128 backward GEMMs (every product on E4M3 operands, fp32 accumulation): input gradients
// with the weights transposed per 128 x 128 block, the gate/up products recomputed from the
// quantised u, and weight gradients on activations transposed and quantised per run of 128 rows
// of each segment.  Runs after the permutation and the row gates; ends with du (router_bwd).
static moe_status fp8_backward(const moe_shape& s, const WorkspacePlan& p, char* wsb, const void* u,
                               const float* centroids, const moe_weights* w, const int32_t* topk_idx,
                               const void* dout, void* du, const moe_weight_grads* dw, hipStream_t stream,
                               const void* saved) {
  moe_status rc;
  const int64_t T = s.tokens, d = s.hidden, I = s.inter, Nr = s.n_routed, Ns = s.n_shared, P = p.max_rows;
  const int64_t p8 = P / 128;
  auto at = [&](size_t off) { return wsb + off; };
  const int32_t* row_token = reinterpret_cast<const int32_t*>(at(p.row_token));
  const int32_t* perm_row = reinterpret_cast<const int32_t*>(at(p.perm_row));
  const int32_t* seg_off = reinterpret_cast<const int32_t*>(at(p.seg_off));
  const float* row_gate = reinterpret_cast<const float*>(at(p.bwd_row_gate));
  float* row_dz = reinterpret_cast<float*>(at(p.bwd_row_dz));
  float* dg_part = reinterpret_cast<float*>(at(p.bwd_dg_part));
  uint8_t* u_q = reinterpret_cast<uint8_t*>(at(p.u_q));
  float* u_s = reinterpret_cast<float*>(at(p.u_scale));
  uint8_t* dout_q = reinterpret_cast<uint8_t*>(at(p.bwd_dout_q));
  float* dout_s = reinterpret_cast<float*>(at(p.bwd_dout_s));
  uint16_t* dhu = reinterpret_cast<uint16_t*>(at(p.bwd_dhu));
  uint16_t* hb = reinterpret_cast<uint16_t*>(at(p.bwd_h));
  uint16_t* dab = reinterpret_cast<uint16_t*>(at(p.bwd_dab));
  uint8_t* dab_q = reinterpret_cast<uint8_t*>(at(p.bwd_dab_q));
  float* dab_s = reinterpret_cast<float*>(at(p.bwd_dab_s));
  uint16_t* dx = reinterpret_cast<uint16_t*>(at(p.y));
  uint8_t* dy_t = reinterpret_cast<uint8_t*>(at(p.bwd_dy_t));
  float* dy_ts = reinterpret_cast<float*>(at(p.bwd_dy_ts));
  uint8_t* h_t = reinterpret_cast<uint8_t*>(at(p.bwd_h_t));
  float* h_ts = reinterpret_cast<float*>(at(p.bwd_h_ts));
  uint8_t* dab_t = reinterpret_cast<uint8_t*>(at(p.bwd_dab_t));
  float* dab_ts = reinterpret_cast<float*>(at(p.bwd_dab_ts));
  uint8_t* x_t = reinterpret_cast<uint8_t*>(at(p.bwd_x_t));
  float* x_ts = reinterpret_cast<float*>(at(p.bwd_x_ts));
  const int64_t max_pairs = walk_max_pairs(p.max_tiles, Nr + Ns);

  auto wgrad = [&](const uint8_t* a_t, const float* a_s, int M, const uint8_t* b_t, const float* b_s, int N,
                   void* out_r, void* out_s) {
    GemmOperands g{};
    g.act = a_t;
    g.act_scale = a_s;
    g.w_routed[0] = b_t;
    g.s_routed[0] = b_s;
    g.seg_off = seg_off;
    g.n_routed = s.n_routed;
    g.K = (int)P;
    g.N = N;
    g.lda = P;
    g.ldw = P;
    g.wg_m = M;
    g.n_seg = (int)(Nr + Ns);
    g.out = out_r;
    g.out2 = out_s;
    return hip_status(launch_gemm_fp8_wgrad(g, stream));
  };
  if (T > 0) {
    // E4M3 copies of u and dout (1 x 128 tiles along d)
    if (!saved && (rc = hip_status(launch_quantize_act(T, (int)d, u, u_q, u_s, stream))) != MOE_OK) return rc;
    if ((rc = hip_status(launch_quantize_act(T, (int)d, dout, dout_q, dout_s, stream))) != MOE_OK) return rc;
    GemmOperands g{};
    g.tile_seg = reinterpret_cast<const int32_t*>(at(p.tile_seg));
    g.seg_off = seg_off;
    g.pair_seg = reinterpret_cast<const int32_t*>(at(p.pair_seg));
    g.pair_off = reinterpret_cast<const int32_t*>(at(p.pair_off));
    g.n_routed = s.n_routed;
    g.n_seg = (int)(Nr + Ns);
    g.max_tiles = p.max_tiles;
    g.max_pairs = max_pairs;
    // dH (before the gate) = dout[token] W_down, the W_down codes [d][I] and scales read K-major
    GemmOperands g1 = g;
    g1.act = dout_q;
    g1.act_scale = dout_s;
    g1.row_token = row_token;
    g1.act_rows = T;
    g1.w_routed[0] = w->w_down;
    g1.w_shared[0] = w->sh_down;
    g1.s_routed[0] = w->w_down_scale;
    g1.s_shared[0] = w->sh_down_scale;
    g1.K = (int)d;
    g1.N = (int)I;
    g1.kn_split = (int)d;
    g1.out = dhu;
    if ((rc = hip_status(launch_gemm_fp8_dgrad(g1, stream))) != MOE_OK) return rc;
    if (saved) {
      // [dA dB], H and the gate-gradient partials from the forward's saved [a b]
      if ((rc = hip_status(launch_swiglu_bwd_saved(saved, dhu, row_gate, row_token, seg_off + Nr + Ns, P, (int)I, dab,
                                                   hb, dg_part, stream))) != MOE_OK)
        return rc;
    } else {
      // gate/up recomputed from the quantised u: [dA dB], H and the gate-gradient partials
      GemmOperands g2 = g;
      g2.act = u_q;
      g2.act_scale = u_s;
      g2.row_token = row_token;
      g2.act_rows = T;
      g2.w_routed[0] = w->w_gate;
      g2.w_routed[1] = w->w_up;
      g2.w_shared[0] = w->sh_gate;
      g2.w_shared[1] = w->sh_up;
      g2.s_routed[0] = w->w_gate_scale;
      g2.s_routed[1] = w->w_up_scale;
      g2.s_shared[0] = w->sh_gate_scale;
      g2.s_shared[1] = w->sh_up_scale;
      g2.K = (int)d;
      g2.N = (int)I;
      g2.dh = dhu;
      g2.row_gate = row_gate;
      g2.out = dab;
      g2.out2 = hb;
      g2.dg_part = dg_part;
      if ((rc = hip_status(launch_gemm_fp8_swiglu_bwd(g2, stream))) != MOE_OK) return rc;
    }
    // dX = [dA dB] [W_gate; W_up], [dA dB] in 1 x 128 tiles along 2I
    if ((rc = hip_status(launch_quantize_act(P, (int)(2 * I), dab, dab_q, dab_s, stream))) != MOE_OK) return rc;
    // K rows [0, I) from the W_gate codes [I][d], [I, 2I) from W_up, as stored
    GemmOperands g3 = g;
    g3.act = dab_q;
    g3.act_scale = dab_s;
    g3.act_rows = P;
    g3.w_routed[0] = w->w_gate;
    g3.w_routed[1] = w->w_up;
    g3.w_shared[0] = w->sh_gate;
    g3.w_shared[1] = w->sh_up;
    g3.s_routed[0] = w->w_gate_scale;
    g3.s_routed[1] = w->w_up_scale;
    g3.s_shared[0] = w->sh_gate_scale;
    g3.s_shared[1] = w->sh_up_scale;
    g3.K = (int)(2 * I);
    g3.N = (int)d;
    g3.kn_split = (int)I;
    g3.out = dx;
    if ((rc = hip_status(launch_gemm_fp8_dgrad(g3, stream))) != MOE_OK) return rc;
    if ((rc = hip_status(launch_router_bwd(s, u, centroids, topk_idx, perm_row, dg_part, seg_off, dout, dx, du,
                                           row_dz, stream))) != MOE_OK)
      return rc;
    // weight-gradient operands: (g dout)^T, H^T, [dA dB]^T, X^T, quantised per run of 128 rows
    auto tq = [&](const void* src, int64_t lds, bool gather, const float* scale, uint8_t* dst, float* ds, int64_t C) {
      TransposeQuantArgs a{static_cast<const uint16_t*>(src), lds, row_token, gather, scale, dst, ds, P, P, (int)C};
      return hip_status(launch_transpose_quant(a, stream));
    };
    if ((rc = tq(dout, d, true, row_gate, dy_t, dy_ts, d)) != MOE_OK) return rc;
    if ((rc = tq(hb, I, false, nullptr, h_t, h_ts, I)) != MOE_OK) return rc;
    if ((rc = tq(dab, 2 * I, false, nullptr, dab_t, dab_ts, 2 * I)) != MOE_OK) return rc;
    if ((rc = tq(u, d, true, nullptr, x_t, x_ts, d)) != MOE_OK) return rc;
  }
  // dW_down = (g dY)^T H, dW_gate = dA^T X, dW_up = dB^T X over each segment's rows (an empty
  // segment writes zeros)
  if ((rc = wgrad(dy_t, dy_ts, (int)d, h_t, h_ts, (int)I, dw->w_down, dw->sh_down)) != MOE_OK) return rc;
  if ((rc = wgrad(dab_t, dab_ts, (int)I, x_t, x_ts, (int)d, dw->w_gate, dw->sh_gate)) != MOE_OK) return rc;
  return wgrad(dab_t + I * P, dab_ts + I * p8, (int)I, x_t, x_ts, (int)d, dw->w_up, dw->sh_up);
}

static moe_status check_backward_shape(const moe_shape* s) {
  moe_status rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->dtype != MOE_DTYPE_BF16 && s->dtype != MOE_DTYPE_FP8_B128) return MOE_ERR_UNSUPPORTED;
  if (s->hidden % 128 != 0 || s->inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  // the streaming and backward GEMMs address their operands with 32-bit byte offsets
  const int64_t max_rows =
      ((int64_t)s->tokens * s->top_k + (int64_t)s->n_routed * (kTileM - 1)) / kTileM * kTileM +
      (int64_t)s->n_shared * ceil_div(s->tokens, kTileM) * kTileM;
  const int64_t widest = std::max<int64_t>(s->hidden, 2 * (int64_t)s->inter);
  const int64_t lim = int64_t(1) << 32;
  if (max_rows * widest * 2 >= lim || (int64_t)s->tokens * s->hidden * 2 >= lim)
    return MOE_ERR_UNSUPPORTED;
  // the input-gradient products read one expert's stacked weights [d, 2I] (bf16) at 32-bit offsets
  if ((int64_t)s->hidden * 2 * s->inter * 2 >= lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status rc = check_backward_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = plan_workspace(*shape).backward_total;
  return MOE_OK;
}

// bytes of the saved SwiGLU inputs [a b] of every permuted row: [max_rows, 2I] bf16
static size_t saved_bytes_for(const moe_shape& s) {
  return (size_t)plan_workspace(s).max_rows * 2 * (size_t)s.inter * 2;
}

moe_status moe_saved_inputs_size(const moe_shape* shape, size_t* bytes) {
  moe_status rc = check_backward_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = saved_bytes_for(*shape);
  return MOE_OK;
}

moe_status moe_forward_train(const moe_shape* shape, const void* u, const moe_weights* weights,
                             const int32_t* topk_idx, const float* topk_gate, void* out, void* saved,
                             size_t saved_bytes, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status rc = check_backward_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->tokens == 0) return MOE_OK;
  if (!saved) return MOE_ERR_INVALID_ARG;
  if (saved_bytes < saved_bytes_for(*shape)) return MOE_ERR_WORKSPACE;
  if (saved == u || saved == out) return MOE_ERR_INVALID_ARG;
  return forward_impl(shape, u, weights, topk_idx, topk_gate, out, workspace, workspace_bytes, stream, nullptr, 0,
                      saved);
}

static moe_status backward_impl(const moe_shape* shape, const void* u, const float* centroids, const moe_weights* w,
                                const int32_t* topk_idx, const float* topk_gate, const void* dout, void* du,
                                float* d_centroids, const moe_weight_grads* dw, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, const void* saved) {
  moe_status rc = check_backward_shape(shape);
  if (rc != MOE_OK) return rc;
  const moe_shape& s = *shape;
  if (!u || !centroids || !w || !dout || !du || !d_centroids || !dw || !workspace) return MOE_ERR_INVALID_ARG;
  if (s.tokens > 0 && (!topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down || !dw->w_gate || !dw->w_up || !dw->w_down) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down || !dw->sh_gate || !dw->sh_up || !dw->sh_down))
    return MOE_ERR_INVALID_ARG;
  if (du == u || du == dout) return MOE_ERR_INVALID_ARG;
  const bool fp8 = s.dtype == MOE_DTYPE_FP8_B128;
  if (fp8 && (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale)) return MOE_ERR_INVALID_ARG;
  if (fp8 && s.n_shared > 0 && (!w->sh_gate_scale || !w->sh_up_scale || !w->sh_down_scale))
    return MOE_ERR_INVALID_ARG;
  const WorkspacePlan p = plan_workspace(s);
  if (workspace_bytes < p.backward_total) return MOE_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);
  const int64_t T = s.tokens, d = s.hidden, I = s.inter;
  const int32_t* row_token = reinterpret_cast<const int32_t*>(wsb + p.row_token);
  const int32_t* perm_row = reinterpret_cast<const int32_t*>(wsb + p.perm_row);
  const int32_t* seg_off = reinterpret_cast<const int32_t*>(wsb + p.seg_off);
  const int32_t* tile_seg = reinterpret_cast<const int32_t*>(wsb + p.tile_seg);
  float* dc_part = reinterpret_cast<float*>(wsb + p.bwd_dc_part);
  float* row_gate = reinterpret_cast<float*>(wsb + p.bwd_row_gate);
  float* row_dz = reinterpret_cast<float*>(wsb + p.bwd_row_dz);
  float* dg_part = reinterpret_cast<float*>(wsb + p.bwd_dg_part);
  uint16_t* dhu = reinterpret_cast<uint16_t*>(wsb + p.h);          // dL/dH before the gate
  uint16_t* dx = reinterpret_cast<uint16_t*>(wsb + p.y);           // dL/dX of every permuted row
  uint16_t* hb = reinterpret_cast<uint16_t*>(wsb + p.bwd_h);
  uint16_t* dab = reinterpret_cast<uint16_t*>(wsb + p.bwd_dab);
  auto bf = [](const void* q) { return static_cast<const uint16_t*>(q); };

  if (T > 0) {
    if ((rc = hip_status(launch_permute(s, topk_idx, p, wsb, stream))) != MOE_OK) return rc;
  } else {
    // no tokens: every segment is empty, so the weight and centroid gradients are zero
    if ((rc = hip_status(launch_permute(s, nullptr, p, wsb, stream))) != MOE_OK) return rc;
  }
  if ((rc = hip_status(launch_row_gate(s, perm_row, topk_gate, seg_off, p.max_rows, row_gate, row_dz, stream))) !=
      MOE_OK)
    return rc;
  if (fp8) {
    if ((rc = fp8_backward(s, p, wsb, u, centroids, w, topk_idx, dout, du, dw, stream, saved)) != MOE_OK) return rc;
    return hip_status(launch_dcentroid(s, u, row_token, row_dz, seg_off, tile_seg, p.max_tiles, dc_part,
                                       d_centroids, stream));
  }
  const int64_t Nr = s.n_routed, Ns = s.n_shared, P = p.max_rows;
  uint16_t* dy_t = reinterpret_cast<uint16_t*>(wsb + p.bwd_dy_t);   // [d][P]
  uint16_t* h_t = reinterpret_cast<uint16_t*>(wsb + p.bwd_h_t);     // [I][P]
  uint16_t* dab_t = reinterpret_cast<uint16_t*>(wsb + p.bwd_dab_t); // [2I][P]
  uint16_t* x_t = reinterpret_cast<uint16_t*>(wsb + p.bwd_x_t);     // [d][P]
  auto transpose = [&](const void* src, int64_t lds, int64_t src_b, const int32_t* gather, const float* scale,
                       uint16_t* dst, int64_t ldd, int64_t off, int64_t dst_b, int64_t R, int64_t C, int64_t batch) {
    TransposeArgs t{bf(src), lds, src_b, gather, scale, dst, ldd, off, dst_b, (int)R, (int)C};
    return hip_status(launch_transpose(t, (int)batch, stream));
  };
  const int32_t* pair_seg = reinterpret_cast<const int32_t*>(wsb + p.pair_seg);
  const int32_t* pair_off = reinterpret_cast<const int32_t*>(wsb + p.pair_off);
  const int64_t max_pairs = walk_max_pairs(p.max_tiles, Nr + Ns);
  auto grouped = [&](const void* act, const int32_t* rt, int64_t act_rows, const uint16_t* w_r, const uint16_t* w_s,
                     int K, int N, void* out) {
    GemmOperands g{};
    g.act = act;
    g.row_token = rt;
    g.w_routed[0] = w_r;
    g.w_shared[0] = w_s;
    g.tile_seg = tile_seg;
    g.seg_off = seg_off;
    g.pair_seg = pair_seg;
    g.pair_off = pair_off;
    g.n_routed = s.n_routed;
    g.n_seg = (int)(Nr + Ns);
    g.K = K;
    g.N = N;
    g.act_rows = act_rows;
    g.max_tiles = p.max_tiles;
    g.max_pairs = max_pairs;
    g.out = out;
    return g;
  };
  auto wgrad = [&](const uint16_t* a_t, int M, const uint16_t* b_t, int N, void* out_r, void* out_s) {
    GemmOperands g{};
    g.act = a_t;
    g.w_routed[0] = b_t;
    g.seg_off = seg_off;
    g.n_routed = s.n_routed;
    g.N = N;
    g.lda = P;
    g.ldw = P;
    g.wg_m = M;
    g.n_seg = (int)(Nr + Ns);
    g.out = out_r;
    g.out2 = out_s;
    return hip_status(launch_gemm_bf16_wgrad(g, stream));
  };

  if (T > 0) {
    // dH (before the gate) = dout[token] W_down, W_down [d][I] read K-major as stored
    GemmOperands g1 = grouped(dout, row_token, T, bf(w->w_down), bf(w->sh_down), (int)d, (int)I, dhu);
    g1.kn_split = (int)d;
    if ((rc = hip_status(launch_gemm_bf16_dgrad(g1, stream))) != MOE_OK) return rc;
    if (saved) {
      // [dA dB], H and the gate-gradient partials from the forward's saved [a b]
      if ((rc = hip_status(launch_swiglu_bwd_saved(saved, dhu, row_gate, row_token, seg_off + Nr + Ns, P, (int)I, dab,
                                                   hb, dg_part, stream))) != MOE_OK)
        return rc;
    } else {
      // gate/up recomputed: [dA dB], H and the gate-gradient partials
      GemmOperands g2 = grouped(u, row_token, T, nullptr, nullptr, (int)d, (int)I, dab);
      g2.w_routed[0] = w->w_gate;
      g2.w_routed[1] = w->w_up;
      g2.w_shared[0] = w->sh_gate;
      g2.w_shared[1] = w->sh_up;
      g2.dh = dhu;
      g2.row_gate = row_gate;
      g2.out2 = hb;
      g2.dg_part = dg_part;
      if ((rc = hip_status(launch_gemm_bf16_swiglu_bwd(g2, stream))) != MOE_OK) return rc;
    }
    // dX = [dA dB] [W_gate; W_up]: K rows [0, I) from W_gate [I][d], [I, 2I) from W_up, as stored
    GemmOperands g3 = grouped(dab, nullptr, P, bf(w->w_gate), bf(w->sh_gate), (int)(2 * I), (int)d, dx);
    g3.w_routed[1] = w->w_up;
    g3.w_shared[1] = w->sh_up;
    g3.kn_split = (int)I;
    if ((rc = hip_status(launch_gemm_bf16_dgrad(g3, stream))) != MOE_OK) return rc;
    // router backward and du
    if ((rc = hip_status(launch_router_bwd(s, u, centroids, topk_idx, perm_row, dg_part, seg_off, dout, dx, du,
                                           row_dz, stream))) != MOE_OK)
      return rc;
    // K-contiguous (transposed) activations of every permuted row for the weight-gradient GEMMs:
    // (g dout)^T [d][P], H^T [I][P], [dA dB]^T [2I][P], X^T [d][P]; padding rows are zero
    if ((rc = transpose(dout, d, 0, row_token, row_gate, dy_t, P, 0, 0, P, d, 1)) != MOE_OK) return rc;
    if ((rc = transpose(hb, I, 0, nullptr, nullptr, h_t, P, 0, 0, P, I, 1)) != MOE_OK) return rc;
    if ((rc = transpose(dab, 2 * I, 0, nullptr, nullptr, dab_t, P, 0, 0, P, 2 * I, 1)) != MOE_OK) return rc;
    if ((rc = transpose(u, d, 0, row_token, nullptr, x_t, P, 0, 0, P, d, 1)) != MOE_OK) return rc;
  }
  // dW_down = (g dY)^T H, dW_gate = dA^T X, dW_up = dB^T X over each segment's rows (an empty
  // segment writes zeros)
  if ((rc = wgrad(dy_t, (int)d, h_t, (int)I, dw->w_down, dw->sh_down)) != MOE_OK) return rc;
  if ((rc = wgrad(dab_t, (int)I, x_t, (int)d, dw->w_gate, dw->sh_gate)) != MOE_OK) return rc;
  if ((rc = wgrad(dab_t + I * P, (int)I, x_t, (int)d, dw->w_up, dw->sh_up)) != MOE_OK) return rc;
  return hip_status(launch_dcentroid(s, u, row_token, row_dz, seg_off, tile_seg, p.max_tiles, dc_part,
                                     d_centroids, stream));
}

moe_status moe_backward(const moe_shape* shape, const void* u, const float* centroids, const moe_weights* w,
                        const int32_t* topk_idx, const float* topk_gate, const void* dout, void* du,
                        float* d_centroids, const moe_weight_grads* dw, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return backward_impl(shape, u, centroids, w, topk_idx, topk_gate, dout, du, d_centroids, dw, workspace,
                       workspace_bytes, stream, nullptr);
}

moe_status moe_backward_saved(const moe_shape* shape, const void* u, const float* centroids, const moe_weights* w,
                              const int32_t* topk_idx, const float* topk_gate, const void* saved, size_t saved_bytes,
                              const void* dout, void* du, float* d_centroids, const moe_weight_grads* dw,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status rc = check_backward_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!saved) return MOE_ERR_INVALID_ARG;
  if (saved_bytes < saved_bytes_for(*shape)) return MOE_ERR_WORKSPACE;
  if (saved == du) return MOE_ERR_INVALID_ARG;
  return backward_impl(shape, u, centroids, w, topk_idx, topk_gate, dout, du, d_centroids, dw, workspace,
                       workspace_bytes, stream, saved);
}

moe_status moe_update_bias(int32_t n_routed, int64_t total_assignments, const int32_t* expert_load, float* bias,
                           float gamma, hipStream_t stream) {
  if (n_routed < 1 || total_assignments < 0 || !expert_load || !bias) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_update_bias(n_routed, total_assignments, expert_load, bias, gamma, stream));
}

moe_status moe_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, const void* w_bf16, uint8_t* codes,
                                float* scales, hipStream_t stream) {
  if (n_mats < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (rows % 128 != 0 || cols % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)n_mats * rows * cols == 0) return MOE_OK;
  if (!w_bf16 || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_weights(n_mats, rows, cols, w_bf16, codes, scales, stream));
}

moe_status moe_prepare_weights(const moe_shape* shape, const moe_weights* logical, void* packed, size_t* packed_bytes,
                               moe_weights* prepared, hipStream_t stream) {
  moe_status rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!logical || !packed_bytes) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *shape;
  const int64_t N = s.n_routed, Ns = s.n_shared, d = s.hidden, I = s.inter;
  const bool fp8 = s.dtype == MOE_DTYPE_FP8_B128;
  // the six stacks in moe_weights order: routed gate, up, down, then shared gate, up, down
  const void* src[6] = {logical->w_gate, logical->w_up, logical->w_down, logical->sh_gate, logical->sh_up,
                        logical->sh_down};
  const int64_t n[6] = {N, N, N, Ns, Ns, Ns};
  const int64_t rows[6] = {I, I, d, I, I, d}, cols[6] = {d, d, I, d, d, I};
  // FP8 packing: the six E4M3 code stacks, then the six fp32 scale stacks, each 256-byte aligned
  size_t code_off[6], scale_off[6], o = 0;
  for (int i = 0; i < 6; ++i) {
    code_off[i] = o;
    o = align_up(o + (fp8 ? (size_t)(n[i] * rows[i] * cols[i]) : 0), 256);
  }
  for (int i = 0; i < 6; ++i) {
    scale_off[i] = o;
    o = align_up(o + (fp8 ? (size_t)(n[i] * (rows[i] / 128) * (cols[i] / 128)) * 4 : 0), 256);
  }
  if (!prepared) {   // size query
    *packed_bytes = o;
    return MOE_OK;
  }
  for (int i = 0; i < 6; ++i)
    if (n[i] > 0 && !src[i]) return MOE_ERR_INVALID_ARG;
  if (!fp8) {        // bf16 and fp32 weights are used as stored
    *prepared = moe_weights{};
    prepared->w_gate = logical->w_gate;
    prepared->w_up = logical->w_up;
    prepared->w_down = logical->w_down;
    prepared->sh_gate = Ns > 0 ? logical->sh_gate : nullptr;
    prepared->sh_up = Ns > 0 ? logical->sh_up : nullptr;
    prepared->sh_down = Ns > 0 ? logical->sh_down : nullptr;
    return MOE_OK;
  }
  if (*packed_bytes < o) return MOE_ERR_WORKSPACE;
  if (!packed) return MOE_ERR_INVALID_ARG;
  char* base = static_cast<char*>(packed);
  const void* codes[6];
  const float* scales[6];
  for (int i = 0; i < 6; ++i) {
    codes[i] = n[i] > 0 ? base + code_off[i] : nullptr;
    scales[i] = n[i] > 0 ? reinterpret_cast<const float*>(base + scale_off[i]) : nullptr;
    if (n[i] == 0) continue;
    hipError_t e = launch_quantize_weights((int32_t)n[i], (int32_t)rows[i], (int32_t)cols[i], src[i],
                                           reinterpret_cast<uint8_t*>(base + code_off[i]),
                                           reinterpret_cast<float*>(base + scale_off[i]), stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  *prepared = moe_weights{codes[0], codes[1], codes[2], codes[3], codes[4], codes[5],
                          scales[0], scales[1], scales[2], scales[3], scales[4], scales[5]};
  return MOE_OK;
}

moe_status moe_quantize_act(int32_t rows, int32_t cols, const void* x_bf16, uint8_t* codes, float* scales,
                            hipStream_t stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (cols % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)rows * cols == 0) return MOE_OK;
  if (!x_bf16 || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_act(rows, cols, x_bf16, codes, scales, stream));
}

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
