// Grouped fp32 expert GEMMs (VALU FMA), for layers whose tensors are fp32.
//
// Same grouped structure as the bf16 MFMA kernels (one expert per 128-row
// M-tile of the padded permuted layout, token rows gathered through row_token):
//   gate/up:  H[r, n] = SiLU(x_r . Wg[e][n]) * (x_r . Wu[e][n])
//   down:     Y[r, n] = H[r] . Wd[e][n]
// (the expert FFNs of the h'_t equation, 方法 §2, "DeepSeek-V3 技術報告").
// Workgroup tile: 128 rows x 32 output features, K in steps of 16 through LDS;
// each of the 256 threads accumulates a 4 x 4 block (two for gate and up).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 16;
constexpr int kBN = 32;

template <bool SWIGLU>
__global__ void __launch_bounds__(kThreads) grouped_gemm_f32_kernel(GemmOperands g) {
  __shared__ float As[kBK][kTileM + 4];
  __shared__ float Bs[kBK][2 * kBN + 4];
  const int mt = blockIdx.x;
  const int seg = g.tile_seg[mt];
  if (seg < 0) return;
  const int tid = threadIdx.x;
  const int K = g.K, N = g.N;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int n0 = blockIdx.y * kBN;
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  const size_t wstride = (size_t)N * K;
  const float* W0 = static_cast<const float*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride;
  const float* W1 = SWIGLU ? static_cast<const float*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride
                           : nullptr;
  const float* act = static_cast<const float*>(g.act);
  const int ty = tid >> 3, tx = tid & 7;

  float acc0[4][4], acc1[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc0[i][j] = acc1[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kBK) {
    for (int q = tid; q < kTileM * kBK; q += kThreads) {
      int r = q / kBK, k = q % kBK;
      int64_t tok = g.row_token ? (int64_t)g.row_token[m0 + r] : m0 + r;
      As[k][r] = (tok >= 0 && k0 + k < K) ? act[tok * K + k0 + k] : 0.0f;
    }
    for (int q = tid; q < (SWIGLU ? 2 : 1) * kBN * kBK; q += kThreads) {
      int r = q / kBK, k = q % kBK;
      const float* W = r < kBN ? W0 : W1;
      int n = n0 + (r % kBN);
      Bs[k][r] = (n < N && k0 + k < K) ? W[(size_t)n * K + k0 + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][4 * ty + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs[k][4 * tx + j];
        if (SWIGLU) b1[j] = Bs[k][kBN + 4 * tx + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
          if (SWIGLU) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
        }
    }
    __syncthreads();
  }
  float* out = static_cast<float*>(g.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= N) continue;
      float v = acc0[i][j];
      if (SWIGLU) v = v / (1.0f + expf(-v)) * acc1[i][j];
      out[row * N + n] = v;
    }
  }
}

template <bool SWIGLU>
hipError_t launch_f32(const GemmOperands& g, hipStream_t st) {
  dim3 grid((unsigned)g.max_tiles, (unsigned)ceil_div(g.N, kBN));
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<SWIGLU>, grid, dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32_swiglu(const GemmOperands& g, hipStream_t st) { return launch_f32<true>(g, st); }
hipError_t launch_gemm_f32_down(const GemmOperands& g, hipStream_t st) { return launch_f32<false>(g, st); }

}  // namespace moe
