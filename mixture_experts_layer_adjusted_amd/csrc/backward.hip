// Layer backward: the non-GEMM kernels.
//
// Gradients of L = <dout, h'> for the h'_t equation of 方法 §2 ("DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437) with the selection held fixed (the Topk is piecewise
// constant; the bias never enters a gate, so it gets no gradient).  With g_k = s_k / S over the
// selected experts (S = their sum of s) and dg_k = <dout_t, FFN_k(u_t)>:
//   ds_k = dg_k / S - (sum_j dg_j s_j) / S^2,   dz_k = ds_k s_k (1 - s_k),
//   du_t = dout_t + sum over the token's rows of dX + sum_k dz_k e_{idx_k},
//   de_i = sum over the (token, slot) pairs that picked i of dz u_t.
//
//  row_gate:   the gate of every permuted row (its (token, slot) gate; 1 for shared-expert rows;
//              0 for padding rows), which scales dY = g dout in the backward GEMMs;
//  router_bwd: one workgroup per token: the K_r logits z = u_t . e_k are recomputed in fp32
//              (blocked partial sums in a fixed order), dg_k is the fixed-order sum of the
//              per-tile partials the gate/up backward GEMM wrote, then dz, and du_t summed in a
//              fixed order (residual, routed rows, shared rows, centroid terms);
//  dcentroid:  de_i in two fixed-order passes: per 128-row tile of segment i (rows in order), then
//              over the segment's tiles (in order).
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 128;

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// one thread per (token, slot) pair, then per (token, shared expert)
__global__ void row_gate_kernel(const int32_t* __restrict__ perm_row, const float* __restrict__ gate,
                                const int32_t* __restrict__ seg_off, int T, int K, int N, int Ns,
                                float* __restrict__ row_gate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t routed = (int64_t)T * K;
  if (i < routed) {
    const int r = perm_row[i];
    if (r >= 0) row_gate[r] = gate[i];
  } else if (i < routed + (int64_t)T * Ns) {
    const int64_t j = i - routed;
    const int s = (int)(j / T), t = (int)(j % T);
    row_gate[seg_off[N + s] + t] = 1.0f;
  }
}

__global__ void __launch_bounds__(kRouterThreads) router_bwd_kernel(
    const uint16_t* __restrict__ u, const float* __restrict__ E, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm_row, const float* __restrict__ dg_part, int NT,
    const int32_t* __restrict__ seg_off, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ dX, int d,
    int N, int K, int Ns, uint16_t* __restrict__ du, float* __restrict__ row_dz) {
  __shared__ float wsum[kRouterThreads / 64][kMaxTopK];
  __shared__ float s_k[kMaxTopK], dg_k[kMaxTopK], dz_k[kMaxTopK];
  __shared__ int32_t e_k[kMaxTopK], row_k[kMaxTopK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < K) {
    const int e = idx[t * K + tid];
    const int r = perm_row[t * K + tid];
    const bool ok = e >= 0 && e < N && r >= 0;
    e_k[tid] = ok ? e : -1;
    row_k[tid] = ok ? r : -1;
  }
  __syncthreads();
  // logits of the selected experts, eight at a time: per-thread partial dot products over the
  // thread's 8-column slices (the u slice loaded once for all eight), then a fixed-order butterfly
  // within each wavefront and the wavefronts' sums in order
  const uint16_t* urow = u + t * d;
  for (int k0 = 0; k0 < K; k0 += 8) {
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = tid * 8; j < d; j += kRouterThreads * 8) {
      float uv[8];
      load8(urow + j, uv);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int e = k0 + kk < K ? e_k[k0 + kk] : -1;
        if (e < 0) continue;
        const float* erow = E + (int64_t)e * d + j;
        const float4 e0 = *reinterpret_cast<const float4*>(erow);
        const float4 e1 = *reinterpret_cast<const float4*>(erow + 4);
        float part = 0.0f;
        part = fmaf(uv[0], e0.x, part);
        part = fmaf(uv[1], e0.y, part);
        part = fmaf(uv[2], e0.z, part);
        part = fmaf(uv[3], e0.w, part);
        part = fmaf(uv[4], e1.x, part);
        part = fmaf(uv[5], e1.y, part);
        part = fmaf(uv[6], e1.z, part);
        part = fmaf(uv[7], e1.w, part);
        acc[kk] += part;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      float v = acc[kk];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if ((tid & 63) == 0 && k0 + kk < K) wsum[tid >> 6][k0 + kk] = v;
    }
  }
  __syncthreads();
  if (tid < K) {
    float z = 0.0f;
    for (int w = 0; w < kRouterThreads / 64; ++w) z += wsum[w][tid];
    float dg = 0.0f;
    const int r = row_k[tid];
    if (r >= 0)
      for (int q = 0; q < NT; ++q) dg += dg_part[(int64_t)r * NT + q];
    s_k[tid] = r >= 0 ? 1.0f / (1.0f + expf(-z)) : 0.0f;
    dg_k[tid] = dg;
  }
  __syncthreads();
  if (tid < K) {
    float S = 0.0f, D = 0.0f;
    for (int k = 0; k < K; ++k) {
      S += s_k[k];
      D += dg_k[k] * s_k[k];
    }
    const float s = s_k[tid];
    const float ds = dg_k[tid] / S - D / (S * S);
    const float dz = row_k[tid] >= 0 ? ds * s * (1.0f - s) : 0.0f;
    dz_k[tid] = dz;
    if (row_k[tid] >= 0) row_dz[row_k[tid]] = dz;
  }
  __syncthreads();
  for (int j = tid * 8; j < d; j += kRouterThreads * 8) {
    float acc[8], v[8];
    load8(dout + t * d + j, acc);
    for (int k = 0; k < K; ++k) {
      if (row_k[k] < 0) continue;
      load8(dX + (int64_t)row_k[k] * d + j, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    for (int s = 0; s < Ns; ++s) {
      load8(dX + ((int64_t)seg_off[N + s] + t) * d + j, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    for (int k = 0; k < K; ++k) {
      if (e_k[k] < 0) continue;
      const float* erow = E + (int64_t)e_k[k] * d + j;
      const float4 e0 = *reinterpret_cast<const float4*>(erow);
      const float4 e1 = *reinterpret_cast<const float4*>(erow + 4);
      const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(dz_k[k], ev[i], acc[i]);
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(du + t * d + j) = o;
  }
}

// de in two fixed-order passes, so that a segment with many rows (the Zipf head) does not hold
// one workgroup while the rest of the chip idles.  Pass 1, one workgroup per (128-row M-tile of a
// routed segment, 1024 columns): part[t, j] = sum over the real rows r of tile t, in row order,
// of row_dz[r] * u[row_token[r], j], 8 columns per lane from 16-byte loads.  Pass 2:
// de[i, j] = sum over the M-tiles t of segment i, in tile order, of part[t, j]; a segment without
// rows writes zeros.  d is a multiple of 8.
constexpr int kDcThreads = 128;
constexpr int kDcCols = kDcThreads * 8;

__global__ void __launch_bounds__(kDcThreads) dcentroid_part_kernel(const uint16_t* __restrict__ u,
                                                                    const int32_t* __restrict__ row_token,
                                                                    const float* __restrict__ row_dz,
                                                                    const int32_t* __restrict__ tile_seg,
                                                                    int n_routed, int d, float* __restrict__ part) {
  const int t = blockIdx.x;
  const int e = tile_seg[t];
  if (e < 0 || e >= n_routed) return;   // a shared-expert tile or past the last one: never read
  __shared__ int32_t tok[kTileM];
  __shared__ float dz[kTileM];
  for (int i = threadIdx.x; i < kTileM; i += kDcThreads) {
    const int64_t r = (int64_t)t * kTileM + i;
    tok[i] = row_token[r];
    dz[i] = row_dz[r];
  }
  __syncthreads();
  const int j = blockIdx.y * kDcCols + threadIdx.x * 8;
  if (j >= d) return;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int i = 0; i < kTileM; ++i) {
    const int tk = tok[i];
    if (tk < 0) continue;   // padding row
    const uint4 q = *reinterpret_cast<const uint4*>(u + (int64_t)tk * d + j);
    const float w = dz[i];
    const uint32_t x[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = fmaf(w, __uint_as_float(x[k] << 16), acc[2 * k]);
      acc[2 * k + 1] = fmaf(w, __uint_as_float(x[k] & 0xFFFF0000u), acc[2 * k + 1]);
    }
  }
  float* o = part + (int64_t)t * d + j;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

__global__ void __launch_bounds__(kDcThreads) dcentroid_sum_kernel(const float* __restrict__ part,
                                                                   const int32_t* __restrict__ seg_off, int d,
                                                                   float* __restrict__ de) {
  const int e = blockIdx.x;
  const int j = blockIdx.y * kDcCols + threadIdx.x * 8;
  if (j >= d) return;
  const int t0 = seg_off[e] / kTileM, t1 = seg_off[e + 1] / kTileM;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f), b = a;
  for (int t = t0; t < t1; ++t) {
    const float* p = part + (int64_t)t * d + j;
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
  }
  float* o = de + (int64_t)e * d + j;
  *reinterpret_cast<float4*>(o) = a;
  *reinterpret_cast<float4*>(o + 4) = b;
}

// dst[b][c * ldd + off + r] = scale[r] * src[b][gather[r] * lds + c] for r < R, c < C (bf16):
// 64 x 64 tiles through LDS.  Each thread loads rows 2p and 2p + 1 at 8 consecutive columns
// (two 16-byte loads) and stores the 8 column pairs as 32-bit words tile[c][p] (the pitch of 33
// words keeps a wavefront's writes on distinct banks); the store phase reads 4 words = 8
// consecutive rows of one column and writes them with one 16-byte store.  A row whose gather
// entry is negative (padding) is written as zeros.
__device__ __forceinline__ uint4 load_row8(const TransposeArgs& a, const uint16_t* src, int r, int c) {
  if (r >= a.R || c >= a.C) return make_uint4(0u, 0u, 0u, 0u);
  const int64_t srow = a.gather ? (int64_t)a.gather[r] : r;
  if (srow < 0) return make_uint4(0u, 0u, 0u, 0u);
  uint4 q = *reinterpret_cast<const uint4*>(src + srow * a.lds + c);
  if (a.scale) {
    const float s = a.scale[r];
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)f32_to_bf16(__uint_as_float(w[j] << 16) * s) |
             ((uint32_t)f32_to_bf16(__uint_as_float(w[j] & 0xFFFF0000u) * s) << 16);
    q = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return q;
}

__global__ void __launch_bounds__(256) transpose_kernel(TransposeArgs a) {
  __shared__ uint32_t tile[64][33];
  const int64_t b = blockIdx.z;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* src = a.src + b * a.src_bstride;
  uint16_t* dst = a.dst + b * a.dst_bstride;
  const int tid = threadIdx.x;
  {
    const int p = tid >> 3, cl = (tid & 7) * 8;
    const uint4 q0 = load_row8(a, src, r0 + 2 * p, c0 + cl);
    const uint4 q1 = load_row8(a, src, r0 + 2 * p + 1, c0 + cl);
    const uint32_t w0[4] = {q0.x, q0.y, q0.z, q0.w}, w1[4] = {q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[cl + 2 * j][p] = (w0[j] & 0xFFFFu) | (w1[j] << 16);
      tile[cl + 2 * j + 1][p] = (w0[j] >> 16) | (w1[j] & 0xFFFF0000u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + 256 * i;          // 512 stores of 8 rows
    const int cl = v >> 3, rg = v & 7;
    const int r = r0 + 8 * rg, c = c0 + cl;
    if (c < a.C && r < a.R)
      *reinterpret_cast<uint4*>(dst + (int64_t)c * a.ldd + a.off + r) =
          make_uint4(tile[cl][4 * rg], tile[cl][4 * rg + 1], tile[cl][4 * rg + 2], tile[cl][4 * rg + 3]);
  }
}

// Activations transposed and quantised along the rows: for column c and each run of 128 rows
// j0..j0+127 (j0 a multiple of 128), v[j] = scale[j] * src[gather ? row_token[j] : j][c] in fp32
// (0 where row_token[j] < 0), one scale amax / 448 (1 when the run is all zero) and the E4M3 codes
// of v / scale: dst[c * ldd + j], dst_scale[c * (ldd / 128) + j / 128].  A 128-row x 64-column
// block goes through LDS as fp32 [64][129]: each thread loads 32 columns of one row (four 16-byte
// loads), then four consecutive threads take one column's 128 rows, 32 each.
__global__ void __launch_bounds__(256) transpose_quant_kernel(TransposeQuantArgs a) {
  __shared__ float tile[64][129];
  const int64_t j0 = (int64_t)blockIdx.x * 128;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int jl = tid >> 1, half = tid & 1;
    const int64_t j = j0 + jl;
    const int tok = a.row_token[j];
    float v[32];
    if (tok < 0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    } else {
      const int64_t srow = a.gather ? (int64_t)tok : j;
      const float sc = a.scale ? a.scale[j] : 1.0f;
      const uint16_t* p = a.src + srow * a.lds + c0 + 32 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float w[8];
        load8(p + 8 * q, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[8 * q + i] = w[i] * sc;
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) tile[32 * half + i][jl] = v[i];
  }
  __syncthreads();
  const int c = tid >> 2, q = tid & 3;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = tile[c][32 * q + i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const float scale = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w[k] = e4m3x4_from_f32(__fdiv_rn(v[4 * k], scale), __fdiv_rn(v[4 * k + 1], scale), __fdiv_rn(v[4 * k + 2], scale),
                           __fdiv_rn(v[4 * k + 3], scale));
  uint8_t* drow = a.dst + (int64_t)(c0 + c) * a.ldd + j0 + 32 * q;
  *reinterpret_cast<uint4*>(drow) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(drow + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  if (q == 0) a.dst_scale[(int64_t)(c0 + c) * (a.ldd / 128) + j0 / 128] = scale;
}

// SwiGLU backward from the saved inputs [a b] of the forward (ab [rows, 2I]: a then b, bf16):
// with dH before the gate (dhu [rows, I]) and dh = row_gate * dH, for every feature
//   dA = dh b sg (1 + a (1 - sg)),  dB = dh a sg,  H = a sg b   (sg = sigmoid(a)),
// written to dab ([rows, 2I]: dA then dB) and h ([rows, I]); dg_part[row, n] = sum over the
// features 128 n + [0, 128) of dH H (16 lanes of 8 features, added pairwise in a fixed order).
// Padding rows (row_token < 0) are written as zeros.  Only the rows [0, seg_off[n_seg]) the
// segments use are touched.  Each lane takes kSavedUnroll runs of 8 features per grid step, all
// loads issued before any arithmetic.
constexpr int kSavedThreads = 256, kSavedUnroll = 4;

__global__ void __launch_bounds__(kSavedThreads) swiglu_bwd_saved_kernel(
    const uint16_t* __restrict__ ab, const uint16_t* __restrict__ dhu, const float* __restrict__ row_gate,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ seg_end, int I, uint16_t* __restrict__ dab,
    uint16_t* __restrict__ h, float* __restrict__ dg_part) {
  const int runs = I / 8;                        // runs of 8 features per row, a multiple of 16
  const int total = seg_end[0] * runs;           // < 2^27: rows * 2I * 2 bytes < 2^32
  const int step = gridDim.x * kSavedThreads * kSavedUnroll;
  for (int base = blockIdx.x * kSavedThreads * kSavedUnroll + threadIdx.x; base < total; base += step) {
    uint4 qa[kSavedUnroll], qb[kSavedUnroll], qd[kSavedUnroll];
    float rg[kSavedUnroll];
    int tok[kSavedUnroll];
#pragma unroll
    for (int k = 0; k < kSavedUnroll; ++k) {
      const int i = base + k * kSavedThreads;
      if (i < total) {
        const int r = i / runs, f = (i - r * runs) * 8;
        qa[k] = *reinterpret_cast<const uint4*>(ab + (int64_t)r * 2 * I + f);
        qb[k] = *reinterpret_cast<const uint4*>(ab + (int64_t)r * 2 * I + I + f);
        qd[k] = *reinterpret_cast<const uint4*>(dhu + (int64_t)r * I + f);
        rg[k] = row_gate[r];
        tok[k] = row_token[r];
      }
    }
#pragma unroll
    for (int k = 0; k < kSavedUnroll; ++k) {
      const int i = base + k * kSavedThreads;
      // i < total holds for all 16 lanes of a run group or for none (total and the groups are
      // multiples of 16), so the shuffles below read only lanes of the same group
      if (i < total) {
        const int r = i / runs, f = (i - r * runs) * 8;
        const uint32_t wa[4] = {qa[k].x, qa[k].y, qa[k].z, qa[k].w};
        const uint32_t wb[4] = {qb[k].x, qb[k].y, qb[k].z, qb[k].w};
        const uint32_t wd[4] = {qd[k].x, qd[k].y, qd[k].z, qd[k].w};
        const bool pad = tok[k] < 0;
        uint32_t oa[4], ob[4], oh[4];
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float va[2], vb[2], vh[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float a = __uint_as_float(t ? wa[j] & 0xFFFF0000u : wa[j] << 16);
            const float b = __uint_as_float(t ? wb[j] & 0xFFFF0000u : wb[j] << 16);
            const float du = __uint_as_float(t ? wd[j] & 0xFFFF0000u : wd[j] << 16);
            const float sg = 1.0f / (1.0f + __expf(-a));
            const float dh = rg[k] * du;
            va[t] = pad ? 0.0f : dh * b * sg * (1.0f + a * (1.0f - sg));
            vb[t] = pad ? 0.0f : dh * a * sg;
            vh[t] = pad ? 0.0f : a * sg * b;
            part += du * vh[t];
          }
          oa[j] = (uint32_t)f32_to_bf16(va[0]) | ((uint32_t)f32_to_bf16(va[1]) << 16);
          ob[j] = (uint32_t)f32_to_bf16(vb[0]) | ((uint32_t)f32_to_bf16(vb[1]) << 16);
          oh[j] = (uint32_t)f32_to_bf16(vh[0]) | ((uint32_t)f32_to_bf16(vh[1]) << 16);
        }
        *reinterpret_cast<uint4*>(dab + (int64_t)r * 2 * I + f) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
        *reinterpret_cast<uint4*>(dab + (int64_t)r * 2 * I + I + f) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        *reinterpret_cast<uint4*>(h + (int64_t)r * I + f) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        part += __shfl_xor(part, 4, 64);
        part += __shfl_xor(part, 8, 64);
        if ((threadIdx.x & 15) == 0) dg_part[(int64_t)r * (I / 128) + f / 128] = part;
      }
    }
  }
}

}  // namespace

hipError_t launch_row_gate(const moe_shape& s, const int32_t* perm_row, const float* gate, const int32_t* seg_off,
                           int64_t max_rows, float* row_gate, float* row_dz, hipStream_t st) {
  const int64_t fill_blocks = std::min<int64_t>(ceil_div(max_rows, 256), 4096);
  if (fill_blocks > 0) {
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, st, row_gate, max_rows);
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, st, row_dz, max_rows);
  }
  const int64_t n = (int64_t)s.tokens * (s.top_k + s.n_shared);
  if (n > 0)
    hipLaunchKernelGGL(row_gate_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, perm_row, gate, seg_off,
                       s.tokens, s.top_k, s.n_routed, s.n_shared, row_gate);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_saved(const void* ab, const void* dhu, const float* row_gate, const int32_t* row_token,
                                  const int32_t* seg_end, int64_t max_rows, int I, void* dab, void* h, float* dg_part,
                                  hipStream_t st) {
  if (I % 128 != 0 || max_rows * 2 * I * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const int64_t per_block = (int64_t)kSavedThreads * kSavedUnroll;
  const int64_t blocks = std::min<int64_t>(ceil_div(max_rows * (I / 8), per_block), 2048);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_saved_kernel, dim3((unsigned)blocks), dim3(kSavedThreads), 0, st,
                     static_cast<const uint16_t*>(ab), static_cast<const uint16_t*>(dhu), row_gate, row_token, seg_end,
                     I, static_cast<uint16_t*>(dab), static_cast<uint16_t*>(h), dg_part);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const moe_shape& s, const void* u, const float* centroids, const int32_t* idx,
                             const int32_t* perm_row, const float* dg_part, const int32_t* seg_off, const void* dout,
                             const void* dX, void* du, float* row_dz, hipStream_t st) {
  if (s.tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)s.tokens), dim3(kRouterThreads), 0, st,
                     static_cast<const uint16_t*>(u), centroids, idx, perm_row, dg_part, s.inter / 128, seg_off,
                     static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(dX), s.hidden, s.n_routed,
                     s.top_k, s.n_shared, static_cast<uint16_t*>(du), row_dz);
  return hipGetLastError();
}

hipError_t launch_dcentroid(const moe_shape& s, const void* u, const int32_t* row_token, const float* row_dz,
                            const int32_t* seg_off, const int32_t* tile_seg, int64_t max_tiles, float* part, float* de,
                            hipStream_t st) {
  if (s.hidden % 8 != 0) return hipErrorInvalidValue;
  const unsigned cols = (unsigned)ceil_div(s.hidden, kDcCols);
  if (max_tiles > 0) {
    hipLaunchKernelGGL(dcentroid_part_kernel, dim3((unsigned)max_tiles, cols), dim3(kDcThreads), 0, st,
                       static_cast<const uint16_t*>(u), row_token, row_dz, tile_seg, s.n_routed, s.hidden, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(dcentroid_sum_kernel, dim3((unsigned)s.n_routed, cols), dim3(kDcThreads), 0, st, part, seg_off,
                     s.hidden, de);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

hipError_t launch_transpose_quant(const TransposeQuantArgs& a, hipStream_t st) {
  if (a.rows == 0 || a.C == 0) return hipSuccess;
  if (a.rows % 128 != 0 || a.C % 64 != 0 || a.ldd < a.rows || a.ldd % 128 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_quant_kernel, dim3((unsigned)(a.rows / 128), (unsigned)(a.C / 64)), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, int batch, hipStream_t st) {
  if (a.R == 0 || a.C == 0 || batch == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)ceil_div(a.R, 64), (unsigned)ceil_div(a.C, 64), (unsigned)batch),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
