// Internal declarations shared by the host API (moe_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "tile_walk.h"
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Rows per M-tile of the grouped GEMMs.  Every expert segment of the permuted
// layout starts on a multiple of kTileM rows.
constexpr int kTileM = 128;
static_assert(kTileM == kWalkTileM, "the tile walk's M-tile");
// Tokens per routing workgroup, and per permutation chunk.
constexpr int kRouteTokens = 32;
constexpr int kChunkTokens = 256;
constexpr int kMaxRouted = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Byte offsets of every buffer inside the caller's workspace.
struct WorkspacePlan {
  // routing
  size_t route_partial;     // int32 [route_blocks, N_r]  per-workgroup pick counts
  size_t route_e_hi, route_e_mid, route_e_lo;  // bf16 [N_pad, d]  exact 3-way split of the centroids
  size_t route_scores;      // fp32 [T, N_r]  affinities s (MFMA path)
  size_t route_zpart;       // fp32 [splits, T, N_r]  partial logits of a split contraction (small T)
  size_t route_bal_part;    // fp32 [ceil(T / 32), N_r] balance-statistic partials per chunk of 64 tokens
  // forward
  size_t chunk_counts;      // int32 [chunks, N_r]
  size_t chunk_base;        // int32 [chunks, N_r]
  size_t seg_off;           // int32 [N_r + N_s + 1]   first padded row of each segment
  size_t seg_rows;          // int32 [N_r + N_s]       real rows of each segment
  size_t tile_seg;          // int32 [max_tiles]       segment of each M-tile, -1 past the end
  size_t pair_seg;          // int32 [max_tiles]       segment of each pair of M-tiles (256-row tiles), -1 past the end
  size_t pair_off;          // int32 [N_r + N_s + 1]   first pair of each segment
  size_t row_token;         // int32 [max_rows]        token of each permuted row, -1 for padding
  size_t perm_row;          // int32 [T, K_r]          permuted row of each (token, slot), -1 if skipped
  size_t h;                 // [max_rows, I]  bf16 / fp32 / e4m3
  size_t h_scale;           // fp32 [max_rows, I/128]  (fp8)
  size_t y;                 // [max_rows, d]  bf16 / fp32
  size_t u_q;               // e4m3 [T, d]             (fp8)
  size_t u_scale;           // fp32 [T, d/128]         (fp8)
  size_t route_bytes, forward_bytes, total;
  // backward only (after the forward section): H, [dA dB], row gates, row dz, gate-gradient partials
  size_t bwd_h;             // bf16 [max_rows, I]
  size_t bwd_dab;           // bf16 [max_rows, 2 I]
  size_t bwd_row_gate;      // fp32 [max_rows]
  size_t bwd_row_dz;        // fp32 [max_rows]
  size_t bwd_dg_part;       // fp32 [max_rows, I / 128]
  size_t bwd_dc_part;       // fp32 [max_tiles, d]  centroid-gradient partial sums per M-tile
  // transposed activations: bf16, or E4M3 codes for FP8_B128 (per run of 128 rows, with the
  // scales below)
  size_t bwd_dy_t;          // [d, max_rows]      (gate * dout of each row) transposed
  size_t bwd_h_t;           // [I, max_rows]
  size_t bwd_dab_t;         // [2 I, max_rows]
  size_t bwd_x_t;           // [d, max_rows]
  // FP8_B128 only
  size_t bwd_dhu;           // bf16 [max_rows, I]      dL/dH before the gate
  size_t bwd_dy_ts;         // fp32 [d, max_rows/128]
  size_t bwd_h_ts;          // fp32 [I, max_rows/128]
  size_t bwd_dab_ts;        // fp32 [2 I, max_rows/128]
  size_t bwd_x_ts;          // fp32 [d, max_rows/128]
  size_t bwd_dout_q;        // e4m3 [T, d]
  size_t bwd_dout_s;        // fp32 [T, d/128]
  size_t bwd_dab_q;         // e4m3 [max_rows, 2 I]
  size_t bwd_dab_s;         // fp32 [max_rows, 2I/128]
  size_t backward_total;
  int64_t route_blocks, chunks, max_tiles, max_rows;
};

WorkspacePlan plan_workspace(const moe_shape& s);

struct RouteWorkspace {
  int32_t* partial;
  uint16_t *e_hi, *e_mid, *e_lo;
  float* scores;
  float* zpart;
};

// ---- per-device state (device_state.hip): set up once per device, thread-safe ----
hipError_t current_device(int* dev);
// CU count of the current device
hipError_t device_cu_count(int* n_cu);
// raise `kernel`'s dynamic LDS limit to `bytes` on the current device (once per device)
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

// ---- launchers (return hipSuccess or the launch error) ----
bool route_uses_mfma(const moe_shape& s);
int64_t route_mfma_blocks(const moe_shape& s);
int route_logit_splits(const moe_shape& s);
// group-limited selection: n_groups equal contiguous expert groups, picks only from the
// topk_groups best groups (topk_groups >= n_groups: no limit)
struct GroupLimit {
  int n_groups;
  int topk_groups;
};

hipError_t launch_route(const moe_shape& s, const void* u, const float* centroids, const float* bias,
                        GroupLimit gl, int32_t* idx, float* gate, int32_t* load, const RouteWorkspace& w,
                        hipStream_t st);

// per-sequence balance statistic from the affinities the routing call wrote to the workspace
// part: fp32 [ceil(T / 32), N_r] chunk partials (sequences of 64 tokens or more)
hipError_t launch_seq_balance(const moe_shape& s, int seq_len, float alpha, const float* scores, const int32_t* idx,
                              float* part, float* loss, hipStream_t st);

hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const WorkspacePlan& p, char* ws,
                          hipStream_t st);

struct GemmOperands {
  const void* act;           // activation rows (gathered through row_token when non-null)
  const float* act_scale;    // fp8 only: [rows, K/128]
  const int32_t* row_token;  // gate/up GEMM: token of each permuted row; down GEMM: nullptr
  const void* w_routed[2];   // [N_r, N, K] gate & up (SwiGLU) or down
  const void* w_shared[2];   // [N_s, N, K]
  const float* s_routed[2];  // fp8 block scales [N_r, N/128, K/128]
  const float* s_shared[2];
  const int32_t* tile_seg;
  const int32_t* seg_off;    // [N_r + N_s + 1] first padded row of each segment
  // [N_r + N_s] real rows of each segment, or null.  When given, the one-tile bf16 kernel idles the
  // wavefronts whose rows all lie in a segment's padding, as it does the upper half of a half tile
  // (those output rows, which nothing reads, are then not written)
  const int32_t* seg_rows;
  const int32_t* pair_seg;   // [max_tiles] segment of each 256-row tile (pairs of M-tiles; a segment
                             // with an odd M-tile count ends in a half tile)
  const int32_t* pair_off;   // [N_r + N_s + 1] first 256-row tile of each segment
  int n_routed;
  int K, N;                  // contraction length, output features per expert
  int64_t act_rows;          // rows of act
  int64_t max_tiles;
  int64_t max_pairs;         // upper bound on the 256-row tiles: min(max_tiles, (max_tiles + N_r + N_s) / 2)
  void* out;                 // [max_rows, N]
  float* out_scale;          // fp8 SwiGLU output: [max_rows, N/128]
  // SwiGLU backward epilogue (bf16, FP8): reads dh (dL/dH before the gate, [max_rows, N]) and
  // row_gate, writes out = [dA dB] ([max_rows, 2N]), out2 = H ([max_rows, N]) and
  // dg_part[row, N-tile] = sum over the tile's features of dh * H
  const void* dh;
  const float* row_gate;
  void* out2;
  float* dg_part;
  // weight-gradient kernels (bf16, FP8): out_e[m, n] = sum over the columns k of segment e of
  // act[m, k] * w_routed[0][n, k] (transposed activations, row strides lda and ldw), m < wg_m;
  // routed segments write out + e M N, shared ones out2 + (e - N_r) M N
  int64_t lda, ldw;
  int wg_m;
  int n_seg;                 // segments (N_r + N_s): entries of seg_off / pair_off minus one
  // input-gradient products (bf16, FP8): the weights are read K-major, as stored ([K rows][N features] per
  // expert, the w_*[0] matrix for K rows [0, kn_split), the w_*[1] matrix for the rest)
  int kn_split;
  // expected routed rows per expert (T K_r / N_r) below one M-tile: the bf16 forward GEMMs take
  // 128-row tiles with more weight rows
  bool small_segments;
};

// layer backward helpers (backward.hip)
// dst[b][c * ldd + off + r] = scale[r] * src[b][gather[r] * lds + c], r < R, c < C (bf16); R and C
// multiples of 8; a row whose gather entry is negative is written as zeros
struct TransposeArgs {
  const uint16_t* src;
  int64_t lds, src_bstride;
  const int32_t* gather;
  const float* scale;
  uint16_t* dst;
  int64_t ldd, off, dst_bstride;
  int R, C;
};
hipError_t launch_transpose(const TransposeArgs& a, int batch, hipStream_t st);
// bf16 activations transposed and quantised per run of 128 rows: for j < rows, c < C,
// v = scale[j] * src[(gather ? row_token[j] : j) * lds + c] (0 where row_token[j] < 0);
// dst[c * ldd + j] = E4M3(v / s), dst_scale[c * (ldd / 128) + j / 128] = s = amax / 448 of the run
struct TransposeQuantArgs {
  const uint16_t* src;
  int64_t lds;
  const int32_t* row_token;
  bool gather;
  const float* scale;
  uint8_t* dst;
  float* dst_scale;
  int64_t ldd, rows;
  int C;
};
hipError_t launch_transpose_quant(const TransposeQuantArgs& a, hipStream_t st);
hipError_t launch_row_gate(const moe_shape& s, const int32_t* perm_row, const float* gate, const int32_t* seg_off,
                           int64_t max_rows, float* row_gate, float* row_dz, hipStream_t st);
hipError_t launch_router_bwd(const moe_shape& s, const void* u, const float* centroids, const int32_t* idx,
                             const int32_t* perm_row, const float* dg_part, const int32_t* seg_off, const void* dout,
                             const void* dX, void* du, float* row_dz, hipStream_t st);
// SwiGLU backward from saved inputs: ab [rows, 2I] (a then b), dhu [rows, I] -> dab [rows, 2I],
// h [rows, I], dg_part [rows, I / 128], for the rows [0, *seg_end) (padding rows: zeros)
hipError_t launch_swiglu_bwd_saved(const void* ab, const void* dhu, const float* row_gate, const int32_t* row_token,
                                  const int32_t* seg_end, int64_t max_rows, int I, void* dab, void* h, float* dg_part,
                                  hipStream_t st);
// part: fp32 [max_tiles, d] per-tile partial sums
hipError_t launch_dcentroid(const moe_shape& s, const void* u, const int32_t* row_token, const float* row_dz,
                            const int32_t* seg_off, const int32_t* tile_seg, int64_t max_tiles, float* part, float* de,
                            hipStream_t st);

hipError_t launch_gemm_swiglu(int dtype, const GemmOperands& g, hipStream_t st);
hipError_t launch_gemm_down(int dtype, const GemmOperands& g, hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* u, const float* gate, const WorkspacePlan& p,
                          const char* ws, void* out, hipStream_t st);

hipError_t launch_update_bias(int32_t n, int64_t total, const int32_t* load, float* bias, float gamma,
                              hipStream_t st);

hipError_t launch_quantize_act(int64_t rows, int32_t cols, const void* x, uint8_t* codes, float* scales,
                               hipStream_t st);
hipError_t launch_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, const void* w,
                                   uint8_t* codes, float* scales, hipStream_t st);

}  // namespace moe
