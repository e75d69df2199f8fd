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
// Three passes, with no global atomics (the result is the same on every run):
//  count:    per chunk of kChunkTokens tokens, the picks of every expert (LDS counters);
//  segments: one workgroup turns the per-chunk counts into segment sizes, padded
//            segment offsets (block-wide exclusive scan), the row base of every
//            (chunk, expert) pair, the segment id of every M-tile, and the same for
//            256-row tiles (pairs of M-tiles, a second scan); rows past the last
//            segment get row_token -1;
//  scatter:  per chunk, every pick gets row base[chunk][e] + (picks of e before it in
//            (token, slot) order), ranked 64 picks at a time with ballots; extra
//            workgroups write the identity rows of the shared segments and mark padding
//            rows -1.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSegThreads = 1024;

// per chunk and expert: the number of picks, from LDS atomic increments (exact integers, so
// the result does not depend on their order)
__global__ void __launch_bounds__(kThreads) perm_count_kernel(const int32_t* __restrict__ idx, int T, int K, int N,
                                                              int32_t* __restrict__ counts) {
  __shared__ int32_t cnt[kMaxRouted];
  const int c = blockIdx.x;
  const int t0 = c * kChunkTokens;
  const int n = min(kChunkTokens, T - t0) * K;
  for (int e = threadIdx.x; e < N; e += kThreads) cnt[e] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < n; q += kThreads) {
    const int e = idx[(int64_t)t0 * K + q];
    if (e >= 0 && e < N) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += kThreads) counts[(int64_t)c * N + e] = cnt[e];
}

// lanes holding the same expert as this lane (among the lanes with ok set), from one ballot per
// bit of the expert index
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool ok, int nbits) {
  uint64_t m = __ballot(ok);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t bal = __ballot(ok && set);
    m &= set ? bal : ~bal;
  }
  return m;
}

__global__ void __launch_bounds__(kSegThreads) perm_segments_kernel(const int32_t* __restrict__ counts,
                                                                    int64_t chunks, int T, int N, int Ns,
                                                                    int64_t max_tiles, int32_t* __restrict__ base,
                                                                    int32_t* __restrict__ seg_off,
                                                                    int32_t* __restrict__ seg_rows,
                                                                    int32_t* __restrict__ tile_seg,
                                                                    int32_t* __restrict__ pair_seg,
                                                                    int32_t* __restrict__ pair_off,
                                                                    int32_t* __restrict__ row_token) {
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
  // rows past the last segment belong to no token (passes over all max_rows rows gather through
  // row_token)
  for (int64_t j = total_rows + tid; j < max_tiles * kTileM; j += kSegThreads) row_token[j] = -1;
}

__global__ void __launch_bounds__(kThreads) perm_scatter_kernel(const int32_t* __restrict__ idx, int T, int K, int N,
                                                                int Ns, int64_t chunks,
                                                                const int32_t* __restrict__ base,
                                                                const int32_t* __restrict__ seg_off,
                                                                const int32_t* __restrict__ seg_rows,
                                                                int32_t* __restrict__ row_token,
                                                                int32_t* __restrict__ perm_row) {
  constexpr int kWaves = kThreads / 64;
  __shared__ int32_t before[kWaves][kMaxRouted];   // picks of each expert ahead of the wave's position
  const int tid = threadIdx.x;
  if (blockIdx.x < chunks) {
    // The chunk's picks, in (token, slot) order, are split into kWaves contiguous runs, one per
    // wavefront.  A pick's row is base[chunk][e] + (picks of e in earlier runs) + (picks of e
    // earlier in its own run); the latter is counted 64 picks at a time: the lanes holding the
    // same expert are found by ballots, and the highest of them adds the group to the count.
    const int c = blockIdx.x;
    const int t0 = c * kChunkTokens;
    const int n = min(kChunkTokens, T - t0) * K;
    const int wave = tid >> 6, lane = tid & 63;
    const int per = (n + kWaves - 1) / kWaves;
    const int q0 = wave * per, q1 = min(n, q0 + per);
    const int nbits = N > 1 ? 32 - __clz(N - 1) : 1;
    const uint64_t below = (1ull << lane) - 1;
    const int32_t* cidx = idx + (int64_t)t0 * K;
    for (int i = tid; i < kWaves * N; i += kThreads) before[i / N][i % N] = 0;
    __syncthreads();
    // pass 1: picks of each expert in each run
    for (int q = q0 + lane; q - lane < q1; q += 64) {
      const bool valid = q < q1;
      const int e = valid ? cidx[q] : -1;
      const bool ok = valid && e >= 0 && e < N;
      const uint64_t m = same_expert_lanes(e, ok, nbits);
      if (ok && (m >> lane) == 1ull) before[wave][e] += __popcll(m);   // highest lane of its group
    }
    __syncthreads();
    // exclusive prefix over the runs, per expert
    for (int e = tid; e < N; e += kThreads) {
      int acc = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int v = before[w][e];
        before[w][e] = acc;
        acc += v;
      }
    }
    __syncthreads();
    // pass 2: rows
    for (int q = q0 + lane; q - lane < q1; q += 64) {
      const bool valid = q < q1;
      const int e = valid ? cidx[q] : -1;
      const bool ok = valid && e >= 0 && e < N;
      const uint64_t m = same_expert_lanes(e, ok, nbits);
      if (valid && !ok) perm_row[(int64_t)t0 * K + q] = -1;   // ignored pick
      if (ok) {
        const int row = base[(int64_t)c * N + e] + before[wave][e] + __popcll(m & below);
        row_token[row] = t0 + q / K;
        perm_row[(int64_t)t0 * K + q] = row;
      }
      // every lane has read its count above (same wavefront, LDS in program order)
      if (ok && (m >> lane) == 1ull) before[wave][e] += __popcll(m);
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
                     p.max_tiles, base, seg_off, seg_rows, tile_seg, pair_seg, pair_off, row_token);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)(p.chunks + N + Ns)), dim3(kThreads), 0, st, idx, T, K,
                     N, Ns, p.chunks, base, seg_off, seg_rows, row_token, perm_row);
  return hipGetLastError();
}

}  // namespace moe
