// Grouped bf16 GEMMs of the layer backward whose operands are not K-contiguous.
//
// The backward of the expert FFNs of the h'_t equation (方法 §2, "DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437), with the weights stored [out, in] as in the forward:
//
//   DGRAD  out[r, n] = sum_k A[src(r), k] * B_e[k, n]      over the permuted rows r of segment e;
//          A is K-contiguous (optionally gathered through a row map), B_e = the expert's weight
//          matrix read as [K][N] (N-contiguous), optionally split along K over two matrices:
//          dH = dY W_down (B = W_down[e], [d][I]) and dX = [dA dB] [W_gate; W_up] (B rows
//          k < I from W_gate[e], the rest from W_up[e], both [I][d]);
//   WGRAD  out_e[m, n] = sum_{r in segment e} A[srcA(r), m] * scale(r) * B[srcB(r), n]
//          with both operands row-major [rows][features] (M- and N-contiguous): dW_down =
//          (g dY)^T H and [dW_gate; dW_up] = [dA dB]^T X.
//
// Tiles of 128 x 128 with BK = 64 and 4 wavefronts (64 x 64 each, v_mfma_f32_32x32x16_bf16
// with the N-side tile as the A operand, as in the forward).  Operands are staged through
// registers into two LDS buffers in K-contiguous rows with the 16-byte-chunk XOR swizzle of
// the forward kernels; an [K][X] operand is transposed on the way: each thread loads a 4 (k)
// x 8 (x) block as four 16-byte rows and writes eight 8-byte LDS rows of 4 k-values.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 128;   // tile rows and columns
constexpr int kBK = 64;
constexpr int kStageElems = 2 * kT * kBK;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
// element offset of 16-byte chunk c of LDS row r
__device__ __forceinline__ int loff(int r, int c) { return r * kBK + ((c ^ swz(r)) << 3); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t elem(const uint4& q, int x) {
  const uint32_t w = x < 4 ? (x < 2 ? q.x : q.y) : (x < 6 ? q.z : q.w);
  return (x & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
}

__device__ __forceinline__ uint4 scale8(const uint4& q, float s) {
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t lo = f32_to_bf16(__uint_as_float(w[i] << 16) * s);
    const uint16_t hi = f32_to_bf16(__uint_as_float(w[i] & 0xFFFF0000u) * s);
    w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// the thread's 4 (k) x 8 (x) block, transposed into eight LDS rows x0 + j at k-offset k4
__device__ __forceinline__ void store_transposed(uint16_t* tile, const uint4 (&v)[4], int x0, int k4) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = x0 + j;
    const uint32_t lo = (uint32_t)elem(v[0], j) | ((uint32_t)elem(v[1], j) << 16);
    const uint32_t hi = (uint32_t)elem(v[2], j) | ((uint32_t)elem(v[3], j) << 16);
    *reinterpret_cast<uint2*>(tile + row * kBK + (((k4 >> 3) ^ swz(row)) << 3) + (k4 & 7)) = make_uint2(lo, hi);
  }
}

// 64 x 64 per wavefront from one LDS stage: A-side rows [0, 128), N-side rows [128, 256)
__device__ __forceinline__ void mma_stage(const uint16_t* st, f32x16 (&acc)[2][2], int wm, int wn, int l32,
                                          int khalf) {
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int c = kk * 2 + khalf;
    bf16x8 xf[2], wf[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) xf[mb] = *reinterpret_cast<const bf16x8*>(st + loff(wm * 64 + mb * 32 + l32, c));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      wf[nb] = *reinterpret_cast<const bf16x8*>(st + loff(kT + wn * 64 + nb * 32 + l32, c));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[mb][nb], 0, 0, 0);
  }
}

// lane holds row m + 32 mb + l32 and columns n + 32 nb + 8 q + 4 khalf + (0..3)
__device__ __forceinline__ void store_acc(const f32x16 (&acc)[2][2], uint16_t* out, int64_t ldo, int64_t m, int n,
                                          int l32, int khalf) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    uint16_t* orow = out + (m + mb * 32 + l32) * ldo;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = n + nb * 32 + q * 8 + khalf * 4;
        *reinterpret_cast<uint2*>(orow + f) =
            make_uint2((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 0]) | ((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 1]) << 16),
                       (uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 2]) | ((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 3]) << 16));
      }
  }
}

__global__ void __launch_bounds__(kThreads) dgrad_kernel(BwdDgrad g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int mt = blockIdx.x;
  const int seg = g.tile_seg[mt];
  if (seg < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
  const int64_t m0 = (int64_t)mt * kT;
  const int n0 = blockIdx.y * kT;
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  const uint16_t* B0 = (shared ? g.b_shared[0] : g.b_routed[0]) + (int64_t)e * g.b_estride;
  const uint16_t* B1 = (shared ? g.b_shared[1] : g.b_routed[1]);
  if (B1) B1 += (int64_t)e * g.b_estride;
  // A: K-contiguous rows (t >> 3) + 32 i, chunk t & 7
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = m0 + (tid >> 3) + 32 * i;
    int64_t src = g.a_gather ? (int64_t)g.a_gather[r] : r;
    if (src < 0) src = 0;  // padding row: any valid row (its result is never used)
    asrc[i] = g.a + src * g.lda + (tid & 7) * 8;
  }
  // B: [K][N], the thread's 4 x 8 block at k4 = 4 (t >> 4), n8 = 8 (t & 15)
  const int k4 = 4 * (tid >> 4), n8 = 8 * (tid & 15);
  uint4 ra[4], rb[4];
  auto load = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(asrc[i] + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + k4 + j;
      const uint16_t* row = k < g.b_split ? B0 + (int64_t)k * g.ldb : B1 + (int64_t)(k - g.b_split) * g.ldb;
      rb[j] = *reinterpret_cast<const uint4*>(row + n0 + n8);
    }
  };
  auto store = [&](int buf) {
    uint16_t* st = lds + buf * kStageElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(st + loff((tid >> 3) + 32 * i, tid & 7)) = ra[i];
    store_transposed(st + kT * kBK, rb, n8, k4);
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  const int nk = g.K / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    mma_stage(lds + (kt & 1) * kStageElems, acc, wm, wn, l32, khalf);
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }
  store_acc(acc, g.out, g.ldo, m0 + wm * 64, n0 + wn * 64, l32, khalf);
}

__global__ void __launch_bounds__(kThreads) wgrad_kernel(BwdWgrad g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int e_seg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
  const int m0 = blockIdx.x * kT, n0 = blockIdx.y * kT;
  const int r_begin = g.seg_off[e_seg], r_end = g.seg_off[e_seg + 1];   // multiples of 128
  const int k4 = 4 * (tid >> 4), x8 = 8 * (tid & 15);
  uint4 ra[4], rb[4];
  auto load = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r_begin + kt * kBK + k4 + j;
      int64_t sa = g.a_gather ? (int64_t)g.a_gather[r] : r;
      int64_t sb = g.b_gather ? (int64_t)g.b_gather[r] : r;
      if (sa < 0) sa = 0;  // padding row: its scale (or its other operand row) is zero
      if (sb < 0) sb = 0;
      ra[j] = *reinterpret_cast<const uint4*>(g.a + sa * g.lda + m0 + x8);
      if (g.a_scale) ra[j] = scale8(ra[j], g.a_scale[r]);
      rb[j] = *reinterpret_cast<const uint4*>(g.b + sb * g.ldb + n0 + x8);
    }
  };
  auto store = [&](int buf) {
    uint16_t* st = lds + buf * kStageElems;
    store_transposed(st, ra, x8, k4);
    store_transposed(st + kT * kBK, rb, x8, k4);
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  const int nk = (r_end - r_begin) / kBK;
  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) load(kt + 1);
      mma_stage(lds + (kt & 1) * kStageElems, acc, wm, wn, l32, khalf);
      if (kt + 1 < nk) store((kt + 1) & 1);
      __syncthreads();
    }
  }
  // segment e_seg's gradient: routed experts first, then the shared ones; output rows
  // m < out_split go to matrix 0, the rest to matrix 1 (at m - out_split)
  const bool shared = e_seg >= g.n_routed;
  const int e = shared ? e_seg - g.n_routed : e_seg;
  const int which = m0 < g.out_split ? 0 : 1;
  uint16_t* out = (shared ? g.out_shared[which] : g.out_routed[which]) + (int64_t)e * g.out_estride;
  store_acc(acc, out, g.ldo, (which ? m0 - g.out_split : m0) + wm * 64, n0 + wn * 64, l32, khalf);
}

}  // namespace

hipError_t launch_bwd_dgrad(const BwdDgrad& g, hipStream_t st) {
  const size_t lds_bytes = 2 * kStageElems * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dgrad_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(dgrad_kernel, dim3((unsigned)g.max_tiles, (unsigned)(g.N / kT)), dim3(kThreads), lds_bytes, st,
                     g);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const BwdWgrad& g, int n_segments, hipStream_t st) {
  const size_t lds_bytes = 2 * kStageElems * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)(g.M / kT), (unsigned)(g.N / kT), (unsigned)n_segments),
                     dim3(kThreads), lds_bytes, st, g);
  return hipGetLastError();
}

}  // namespace moe
