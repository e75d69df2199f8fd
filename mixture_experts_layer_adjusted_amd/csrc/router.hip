// Router: sigmoid affinities, biased top-K_r, normalised gates and per-expert loads.
//
// Implements the s_{i,t} and g'_{i,t} equations of 方法 §2 of the page
// "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437), with the bias
// entering the ranking only and the gate normalised over the selected unbiased
// affinities.
//
// One workgroup (256 threads) owns kRouteTokens tokens:
//  1. logits z = u . e_i for its tokens and all experts, fp32 FMAs over LDS-staged
//     32-wide slices of d; each slice is summed in a fresh register and then added
//     to the running total (blocked summation keeps the rounding error of the
//     7168-long contraction near 1e-7 relative);
//  2. s = 1 / (1 + exp(-z)) written to LDS;
//  3. one wavefront per token: each lane holds ceil(N_r/64) candidate keys
//     (orderable bits of s+b in the high word, bit-inverted expert index in the
//     low word, so the 64-bit maximum is the highest score and, among equal
//     scores, the lowest index; NaN maps to the lowest key), K_r rounds of a
//     wave-wide 64-bit max pick the experts in order;
//  4. the workgroup's picks are counted per expert by a plain scan of its LDS
//     copy (no atomics) and written as one row of partial counts; a second
//     kernel sums the partial rows in a fixed order into expert_load.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;        // contraction slice staged in LDS
constexpr int kExpertTile = 256;  // experts per logit pass
constexpr int kEsPitch = kExpertTile + 1;

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

__device__ __forceinline__ uint64_t score_key(float c, int e) {
  uint32_t b = __float_as_uint(c);
  uint32_t ord;
  if (c != c) {
    ord = 0u;                              // NaN ranks below every number
  } else {
    if (c == 0.0f) b = 0u;                 // -0 and +0 are the same score
    ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int CPL, typename TIn>
__global__ void __launch_bounds__(kThreads) route_kernel(const TIn* __restrict__ u, const float* __restrict__ E,
                                                         const float* __restrict__ bias, int T, int d, int N, int K,
                                                         int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
                                                         int32_t* __restrict__ partial) {
  __shared__ float Us[kSlice][kRouteTokens + 1];
  __shared__ float Es[kSlice][kEsPitch];
  __shared__ float S[kRouteTokens][CPL * 64];
  __shared__ int32_t picks[kRouteTokens * kMaxTopK];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  const int tx = tid & 31;   // experts tx + 32 j
  const int ty = tid >> 5;   // tokens 4 ty .. 4 ty + 3

  for (int e0 = 0; e0 < N; e0 += kExpertTile) {
    float total[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) total[i][j] = 0.0f;

    for (int k0 = 0; k0 < d; k0 += kSlice) {
      // stage u[t0 .. t0+32, k0 .. k0+32] transposed into Us[k][t]
      for (int q = tid; q < kRouteTokens * kSlice; q += kThreads) {
        int t = q / kSlice, k = q % kSlice;
        float v = 0.0f;
        if (t0 + t < T && k0 + k < d) v = load_elem(u, (int64_t)(t0 + t) * d + k0 + k);
        Us[k][t] = v;
      }
      // stage E[e0 .. e0+256, k0 .. k0+32] transposed into Es[k][e]
      for (int q = tid; q < kExpertTile * kSlice; q += kThreads) {
        int e = q / kSlice, k = q % kSlice;
        float v = 0.0f;
        if (e0 + e < N && k0 + k < d) v = E[(int64_t)(e0 + e) * d + k0 + k];
        Es[k][e] = v;
      }
      __syncthreads();
      float acc[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
#pragma unroll 8
      for (int k = 0; k < kSlice; ++k) {
        float a[4], b[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = Us[k][4 * ty + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Es[k][tx + 32 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) total[i][j] += acc[i][j];
      __syncthreads();
    }
    // sigmoid into S
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int e = e0 + tx + 32 * j;
        if (e < CPL * 64) S[4 * ty + i][e] = 1.0f / (1.0f + expf(-total[i][j]));
      }
  }
  for (int q = tid; q < kRouteTokens * kMaxTopK; q += kThreads) picks[q] = -1;
  __syncthreads();

  // top-K: one wavefront per token
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float bl[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int e = lane + 64 * j;
    bl[j] = e < N ? bias[e] : 0.0f;
  }
  for (int tt = wave; tt < kRouteTokens; tt += kThreads / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    uint64_t key[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int e = lane + 64 * j;
      key[j] = e < N ? score_key(S[tt][e] + bl[j], e) : 0ull;
    }
    uint32_t taken = 0;
    float mys = 0.0f, sum = 0.0f;
    int myidx = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
      int bj = -1;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int e = lane + 64 * j;
        if (e < N && !((taken >> j) & 1u) && (bj < 0 || key[j] > best)) {
          best = key[j];
          bj = j;
        }
      }
      uint64_t win = wave_max_u64(bj < 0 ? 0ull : best);
      int we = (int)(~(uint32_t)win);
      if (bj >= 0 && best == win) taken |= 1u << bj;
      float sw = S[tt][we];
      sum += sw;
      if (lane == k) {
        mys = sw;
        myidx = we;
      }
    }
    if (lane < K) {
      idx_out[(int64_t)t * K + lane] = myidx;
      gate_out[(int64_t)t * K + lane] = mys / sum;
      picks[tt * K + lane] = myidx;
    }
  }
  __syncthreads();
  // partial per-expert counts of this workgroup's picks (plain scan, no atomics)
  for (int e = tid; e < N; e += kThreads) {
    int c = 0;
    for (int q = 0; q < kRouteTokens * K; ++q) c += (picks[q] == e);
    partial[(int64_t)blockIdx.x * N + e] = c;
  }
}

__global__ void __launch_bounds__(kThreads) load_reduce_kernel(const int32_t* __restrict__ partial, int64_t blocks,
                                                               int N, int32_t* __restrict__ load) {
  int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= N) return;
  int32_t s = 0;
  for (int64_t b = 0; b < blocks; ++b) s += partial[b * N + e];
  load[e] = s;
}

__global__ void zero_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename TIn>
hipError_t launch_route_t(const moe_shape& s, const TIn* u, const float* centroids, const float* bias,
                          int32_t* idx, float* gate, int32_t* load, int32_t* partial, int64_t blocks,
                          hipStream_t st) {
  const int N = s.n_routed;
  dim3 grid((unsigned)blocks), block(kThreads);
#define MOE_ROUTE_CASE(C)                                                                                  \
  hipLaunchKernelGGL((route_kernel<C, TIn>), grid, block, 0, st, u, centroids, bias, s.tokens, s.hidden, N, \
                     s.top_k, idx, gate, partial)
  if (N <= 64) MOE_ROUTE_CASE(1);
  else if (N <= 128) MOE_ROUTE_CASE(2);
  else if (N <= 256) MOE_ROUTE_CASE(4);
  else MOE_ROUTE_CASE(8);
#undef MOE_ROUTE_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(load_reduce_kernel, dim3((unsigned)ceil_div(N, kThreads)), block, 0, st, partial, blocks, N,
                     load);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const void* u, const float* centroids, const float* bias,
                        int32_t* idx, float* gate, int32_t* load, int32_t* partial, int64_t blocks,
                        hipStream_t st) {
  if (s.tokens == 0) {
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)ceil_div(s.n_routed, 256)), dim3(256), 0, st, load, s.n_routed);
    return hipGetLastError();
  }
  if (s.dtype == MOE_DTYPE_F32)
    return launch_route_t(s, static_cast<const float*>(u), centroids, bias, idx, gate, load, partial, blocks, st);
  return launch_route_t(s, static_cast<const uint16_t*>(u), centroids, bias, idx, gate, load, partial, blocks, st);
}

}  // namespace moe
