// Combine: out_t = u_t + sum_s Y[shared row of t] + sum_k gate[t,k] * Y[perm_row[t,k]].
//
// The outer sums of the h'_t equation (方法 §2, "DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437): the residual, the always-on shared experts
// (gate 1) and the gate-weighted routed experts, gathered back from the permuted
// layout.  One workgroup of up to 128 threads per token, each thread owning 8
// consecutive features per pass; a thread issues all K_r + N_s + 1 row loads before
// summing them in fp32 in a fixed order (residual, shared experts in order, routed slots
// in order), so the result is bit-reproducible.  HBM-bound: (K_r + N_s + 2) * d * elem
// bytes per token.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxThreads = 128;
constexpr int kVec = 8;

// threads per token: one per 8 features up to two wavefronts (short workgroups keep many
// tokens in flight per CU, which measured faster than one thread per chunk)
inline int combine_threads(int d) {
  const int chunks = (d + kVec - 1) / kVec;
  return chunks > 64 ? 128 : 64;
}

struct Vec8 {
  float v[kVec];
};

__device__ __forceinline__ Vec8 load8(const uint16_t* p) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  Vec8 o;
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.v[2 * i] = __uint_as_float(w[i] << 16);
    o.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return o;
}
__device__ __forceinline__ Vec8 load8(const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  return Vec8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
  r.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T, int KMAX, int SMAX>
__global__ void __launch_bounds__(kMaxThreads) combine_kernel(const T* __restrict__ u, const T* __restrict__ y,
                                                           const float* __restrict__ gate,
                                                           const int32_t* __restrict__ perm_row,
                                                           const int32_t* __restrict__ seg_off, int d, int K, int N,
                                                           int Ns, T* __restrict__ out) {
  const int64_t t = blockIdx.x;
  int64_t rows[KMAX + SMAX];
  float gk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rows[k] = -1;
    gk[k] = 0.0f;
    if (k < K) {
      int r = perm_row[t * K + k];
      rows[k] = r;
      gk[k] = gate[t * K + k];
    }
  }
#pragma unroll
  for (int s = 0; s < SMAX; ++s) rows[KMAX + s] = s < Ns ? (int64_t)seg_off[N + s] + t : -1;

  for (int j = threadIdx.x * kVec; j < d; j += blockDim.x * kVec) {
    Vec8 acc = load8(u + t * d + j);
    Vec8 parts[KMAX + SMAX];
#pragma unroll
    for (int q = 0; q < KMAX + SMAX; ++q)
      if (rows[q] >= 0) parts[q] = load8(y + rows[q] * d + j);
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (rows[KMAX + s] >= 0)
#pragma unroll
        for (int i = 0; i < kVec; ++i) acc.v[i] += parts[KMAX + s].v[i];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (rows[k] >= 0)
#pragma unroll
        for (int i = 0; i < kVec; ++i) acc.v[i] = fmaf(gk[k], parts[k].v[i], acc.v[i]);
    store8(out + t * d + j, acc.v);
  }
}

template <typename T, int KMAX, int SMAX>
hipError_t launch_t(const moe_shape& s, const void* u, const float* gate, const WorkspacePlan& p, const char* ws,
                    void* out, hipStream_t st) {
  const T* y = reinterpret_cast<const T*>(ws + p.y);
  const int32_t* perm_row = reinterpret_cast<const int32_t*>(ws + p.perm_row);
  const int32_t* seg_off = reinterpret_cast<const int32_t*>(ws + p.seg_off);
  hipLaunchKernelGGL((combine_kernel<T, KMAX, SMAX>), dim3((unsigned)s.tokens), dim3(combine_threads(s.hidden)), 0, st,
                     static_cast<const T*>(u), y, gate, perm_row, seg_off, s.hidden, s.top_k, s.n_routed,
                     s.n_shared, static_cast<T*>(out));
  return hipGetLastError();
}

template <typename T>
hipError_t launch_k(const moe_shape& s, const void* u, const float* gate, const WorkspacePlan& p, const char* ws,
                    void* out, hipStream_t st) {
  const int K = s.top_k, S = s.n_shared;
  if (K <= 8 && S <= 2) return launch_t<T, 8, 2>(s, u, gate, p, ws, out, st);
  if (K <= 16 && S <= 4) return launch_t<T, 16, 4>(s, u, gate, p, ws, out, st);
  return hipErrorInvalidValue;  // host validation routes larger shapes to the looped kernel
}

// general shapes: loop over the slots instead of holding them in registers
template <typename T>
__global__ void __launch_bounds__(kMaxThreads) combine_loop_kernel(const T* __restrict__ u, const T* __restrict__ y,
                                                                const float* __restrict__ gate,
                                                                const int32_t* __restrict__ perm_row,
                                                                const int32_t* __restrict__ seg_off, int d, int K,
                                                                int N, int Ns, T* __restrict__ out) {
  const int64_t t = blockIdx.x;
  for (int j = threadIdx.x * kVec; j < d; j += blockDim.x * kVec) {
    Vec8 acc = load8(u + t * d + j);
    for (int s = 0; s < Ns; ++s) {
      Vec8 p = load8(y + ((int64_t)seg_off[N + s] + t) * d + j);
#pragma unroll
      for (int i = 0; i < kVec; ++i) acc.v[i] += p.v[i];
    }
    for (int k = 0; k < K; ++k) {
      int r = perm_row[t * K + k];
      if (r < 0) continue;
      float gk = gate[t * K + k];
      Vec8 p = load8(y + (int64_t)r * d + j);
#pragma unroll
      for (int i = 0; i < kVec; ++i) acc.v[i] = fmaf(gk, p.v[i], acc.v[i]);
    }
    store8(out + t * d + j, acc.v);
  }
}

template <typename T>
hipError_t launch_any(const moe_shape& s, const void* u, const float* gate, const WorkspacePlan& p, const char* ws,
                      void* out, hipStream_t st) {
  if (s.top_k <= 16 && s.n_shared <= 4) return launch_k<T>(s, u, gate, p, ws, out, st);
  hipLaunchKernelGGL(combine_loop_kernel<T>, dim3((unsigned)s.tokens), dim3(combine_threads(s.hidden)), 0, st,
                     static_cast<const T*>(u), reinterpret_cast<const T*>(ws + p.y), gate,
                     reinterpret_cast<const int32_t*>(ws + p.perm_row), reinterpret_cast<const int32_t*>(ws + p.seg_off),
                     s.hidden, s.top_k, s.n_routed, s.n_shared, static_cast<T*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* u, const float* gate, const WorkspacePlan& p,
                          const char* ws, void* out, hipStream_t st) {
  if (s.dtype == MOE_DTYPE_F32) return launch_any<float>(s, u, gate, p, ws, out, st);
  return launch_any<uint16_t>(s, u, gate, p, ws, out, st);
}

}  // namespace moe
