// Token -> expert permutation into a padded, contiguous per-expert layout.
//
// The h'_t equation of 方法 §2 ("DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437) applies expert FFN^(r)_i only to the tokens
// that picked expert i.  To run all experts as one grouped GEMM the picked
// (token, slot) pairs are laid out expert by expert: segment i holds the tokens
// that picked routed expert i, in increasing token order; segment N_r + s holds
// every token, in order, for shared expert s.  Each segment starts on a multiple
// of kTileM rows, so every M-tile of the grouped GEMM belongs to one expert.
//
// Three atomic-free passes:
//  count:    per chunk of kChunkTokens tokens, thread e counts the picks of expert e
//            by scanning the chunk's topk_idx from LDS;
//  segments: one workgroup turns the per-chunk counts into segment sizes, padded
//            segment offsets (block-wide exclusive scan), the row base of every
//            (chunk, expert) pair, the segment id of every M-tile, and the same for
//            256-row tiles (pairs of M-tiles, a second scan);
//  scatter:  per chunk, thread e walks the chunk's picks in (token, slot) order and
//            hands out consecutive rows of segment e; extra workgroups write the
//            identity rows of the shared segments and mark padding rows -1.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSegThreads = 1024;

__global__ void __launch_bounds__(kThreads) perm_count_kernel(const int32_t* __restrict__ idx, int T, int K, int N,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t picks[kChunkTokens * kMaxTopK];
  const int c = blockIdx.x;
  const int t0 = c * kChunkTokens;
  const int nt = min(kChunkTokens, T - t0);
  const int n = nt * K;
  for (int q = threadIdx.x; q < n; q += kThreads) picks[q] = idx[(int64_t)t0 * K + q];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += kThreads) {
    int cnt = 0;
    for (int q = 0; q < n; ++q) cnt += (picks[q] == e);
    counts[(int64_t)c * N + e] = cnt;
  }
}

__global__ void __launch_bounds__(kSegThreads) perm_segments_kernel(const int32_t* __restrict__ counts,
                                                                    int64_t chunks, int T, int N, int Ns,
                                                                    int64_t max_tiles, int32_t* __restrict__ base,
                                                                    int32_t* __restrict__ seg_off,
                                                                    int32_t* __restrict__ seg_rows,
                                                                    int32_t* __restrict__ tile_seg,
                                                                    int32_t* __restrict__ pair_seg,
                                                                    int32_t* __restrict__ pair_off) {
  __shared__ int32_t scan[kSegThreads];
  __shared__ int32_t total_rows, total_pairs;
  const int tid = threadIdx.x;
  const int nseg = N + Ns;
  int rows = 0;
  if (tid < N) {
    for (int64_t c = 0; c < chunks; ++c) rows += counts[c * N + tid];
  } else if (tid < nseg) {
    rows = T;
  }
  const int padded = (rows + kTileM - 1) / kTileM * kTileM;
  scan[tid] = padded;
  __syncthreads();
  // Hillis-Steele inclusive scan over the padded sizes
  for (int off = 1; off < kSegThreads; off <<= 1) {
    int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int start = scan[tid] - padded;
  if (tid == kSegThreads - 1) total_rows = scan[tid];
  if (tid < nseg) {
    seg_off[tid] = start;
    seg_rows[tid] = rows;
    for (int j = 0; j < padded / kTileM; ++j) tile_seg[start / kTileM + j] = tid;
  }
  if (tid < N) {
    int run = start;
    for (int64_t c = 0; c < chunks; ++c) {
      base[c * N + tid] = run;
      run += counts[c * N + tid];
    }
  }
  // second scan: 256-row tiles (pairs of M-tiles) per segment
  const int pairs = (padded / kTileM + 1) / 2;
  __syncthreads();
  scan[tid] = pairs;
  __syncthreads();
  for (int off = 1; off < kSegThreads; off <<= 1) {
    int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int pstart = scan[tid] - pairs;
  if (tid == kSegThreads - 1) total_pairs = scan[tid];
  if (tid < nseg) {
    pair_off[tid] = pstart;
    for (int j = 0; j < pairs; ++j) pair_seg[pstart + j] = tid;
  }
  __syncthreads();
  if (tid == 0) {
    seg_off[nseg] = total_rows;
    pair_off[nseg] = total_pairs;
  }
  for (int64_t j = total_rows / kTileM + tid; j < max_tiles; j += kSegThreads) tile_seg[j] = -1;
  for (int64_t j = total_pairs + tid; j < max_tiles; j += kSegThreads) pair_seg[j] = -1;
}

__global__ void __launch_bounds__(kThreads) perm_scatter_kernel(const int32_t* __restrict__ idx, int T, int K, int N,
                                                                int Ns, int64_t chunks,
                                                                const int32_t* __restrict__ base,
                                                                const int32_t* __restrict__ seg_off,
                                                                const int32_t* __restrict__ seg_rows,
                                                                int32_t* __restrict__ row_token,
                                                                int32_t* __restrict__ perm_row) {
  __shared__ int32_t picks[kChunkTokens * kMaxTopK];
  const int tid = threadIdx.x;
  if (blockIdx.x < chunks) {
    const int c = blockIdx.x;
    const int t0 = c * kChunkTokens;
    const int nt = min(kChunkTokens, T - t0);
    const int n = nt * K;
    for (int q = tid; q < n; q += kThreads) {
      int e = idx[(int64_t)t0 * K + q];
      picks[q] = e;
      if (e < 0 || e >= N) perm_row[(int64_t)t0 * K + q] = -1;   // ignored pick
    }
    __syncthreads();
    for (int e = tid; e < N; e += kThreads) {
      int row = base[(int64_t)c * N + e];
      for (int q = 0; q < n; ++q) {
        if (picks[q] == e) {
          row_token[row] = t0 + q / K;
          perm_row[(int64_t)t0 * K + q] = row;
          ++row;
        }
      }
    }
    return;
  }
  // one workgroup per segment: padding rows, and the identity rows of shared segments
  const int s = blockIdx.x - (int)chunks;
  const int start = seg_off[s];
  const int rows = seg_rows[s];
  const int end = seg_off[s + 1];
  if (s >= N) {
    for (int r = tid; r < rows; r += kThreads) row_token[start + r] = r;
  }
  for (int r = start + rows + tid; r < end; r += kThreads) row_token[r] = -1;
}

}  // namespace

hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const WorkspacePlan& p, char* ws,
                          hipStream_t st) {
  const int N = s.n_routed, Ns = s.n_shared, T = s.tokens, K = s.top_k;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.chunk_counts);
  int32_t* base = reinterpret_cast<int32_t*>(ws + p.chunk_base);
  int32_t* seg_off = reinterpret_cast<int32_t*>(ws + p.seg_off);
  int32_t* seg_rows = reinterpret_cast<int32_t*>(ws + p.seg_rows);
  int32_t* tile_seg = reinterpret_cast<int32_t*>(ws + p.tile_seg);
  int32_t* pair_seg = reinterpret_cast<int32_t*>(ws + p.pair_seg);
  int32_t* pair_off = reinterpret_cast<int32_t*>(ws + p.pair_off);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + p.row_token);
  int32_t* perm_row = reinterpret_cast<int32_t*>(ws + p.perm_row);
  if (p.chunks > 0) {
    hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)p.chunks), dim3(kThreads), 0, st, idx, T, K, N, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(perm_segments_kernel, dim3(1), dim3(kSegThreads), 0, st, counts, p.chunks, T, N, Ns,
                     p.max_tiles, base, seg_off, seg_rows, tile_seg, pair_seg, pair_off);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)(p.chunks + N + Ns)), dim3(kThreads), 0, st, idx, T, K,
                     N, Ns, p.chunks, base, seg_off, seg_rows, row_token, perm_row);
  return hipGetLastError();
}

}  // namespace moe
