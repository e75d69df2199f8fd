// Bias update and FP8 (E4M3FN) quantisers.
//
// Bias update: the end-of-step rule of 方法 §2 of "DeepSeek-V3 技術報告"
// (xyznot.com/zh-tw/paper/2412.19437): an expert above the step's mean load
// T*K_r/N_r (compared exactly as load*N_r vs T*K_r in 64-bit integers) loses
// gamma, one below it gains gamma, one exactly at it keeps its bias.
//
// Quantisers: the fine-grained FP8 scheme of the same page's 核心概念 list, one
// fp32 scale per 1x128 activation tile and per 128x128 weight block:
// scale = amax / 448 (the E4M3FN maximum; 1 for an all-zero tile), code = E4M3FN
// round-to-nearest-even of the correctly rounded fp32 quotient x / scale,
// saturating at +-448, by gfx950's packed conversion instruction (fp8_codec.h;
// OCP OFP8 layout: bias 7, 3 mantissa bits, S.1111.111 = NaN).
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ void update_bias_kernel(int32_t n, int64_t total, const int32_t* __restrict__ load,
                                   float* __restrict__ bias, float gamma) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t l = (int64_t)load[i] * n;
  float b = bias[i];
  if (l > total) b = __fsub_rn(b, gamma);
  else if (l < total) b = __fadd_rn(b, gamma);
  bias[i] = b;
}

// 16 lanes per 1x128 tile (8 consecutive elements each, one 16-byte load), 16 tiles per
// 256-thread workgroup, grid-stride over the tiles
__global__ void __launch_bounds__(256) quant_act_kernel(const uint16_t* __restrict__ x, int64_t rows, int32_t cols,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int sub = threadIdx.x & 15;
  const int64_t tiles_per_row = cols / 128;
  const int64_t tiles = rows * tiles_per_row;
  for (int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); tile - (threadIdx.x >> 4) < tiles;
       tile += (int64_t)gridDim.x * 16) {
    // every lane of a wave stays in the loop (the shuffles below need all 64): lanes past the
    // last tile work on a copy of tile 0 and store nothing
    const bool live = tile < tiles;
    const int64_t t = live ? tile : 0;
    const int64_t r = t / tiles_per_row, c0 = (t % tiles_per_row) * 128 + 8 * sub;
    const uint4 q = *reinterpret_cast<const uint4*>(x + r * cols + c0);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float scale = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      o[h] = e4m3x4_from_f32(__fdiv_rn(v[4 * h], scale), __fdiv_rn(v[4 * h + 1], scale), __fdiv_rn(v[4 * h + 2], scale),
                             __fdiv_rn(v[4 * h + 3], scale));
    if (live) {
      *reinterpret_cast<uint2*>(codes + r * cols + c0) = make_uint2(o[0], o[1]);
      if (sub == 0) scales[t] = scale;
    }
  }
}

// one workgroup (256 threads) per 128x128 block: each thread handles 64 elements
__global__ void __launch_bounds__(256) quant_weight_kernel(const uint16_t* __restrict__ w, int32_t rows,
                                                           int32_t cols, uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int bc = cols / 128, br = rows / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)br * bc);
  const int rb = (int)((blk / bc) % br), cb = (int)(blk % bc);
  const uint16_t* src = w + mat * (int64_t)rows * cols + (int64_t)rb * 128 * cols + cb * 128;
  uint8_t* dst = codes + mat * (int64_t)rows * cols + (int64_t)rb * 128 * cols + cb * 128;
  // thread: row (tid >> 1) , columns 64 * (tid & 1) .. + 64
  const int r = tid >> 1, c = (tid & 1) * 64;
  float v[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 q = *reinterpret_cast<const uint4*>(src + (int64_t)r * cols + c + 8 * i);
    uint32_t ww[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(ww[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 16 * i + 4 * j;
      o[j] = e4m3x4_from_f32(__fdiv_rn(v[b], scale), __fdiv_rn(v[b + 1], scale), __fdiv_rn(v[b + 2], scale),
                             __fdiv_rn(v[b + 3], scale));
    }
    *reinterpret_cast<uint4*>(dst + (int64_t)r * cols + c + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (tid == 0) scales[blk] = scale;
}

}  // namespace

hipError_t launch_update_bias(int32_t n, int64_t total, const int32_t* load, float* bias, float gamma,
                              hipStream_t st) {
  hipLaunchKernelGGL(update_bias_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, n, total, load, bias,
                     gamma);
  return hipGetLastError();
}

hipError_t launch_quantize_act(int64_t rows, int32_t cols, const void* x, uint8_t* codes, float* scales,
                               hipStream_t st) {
  const int64_t tiles = rows * (cols / 128);
  if (tiles == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(ceil_div(tiles, 16), 8192);
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, const void* w, uint8_t* codes,
                                   float* scales, hipStream_t st) {
  const int64_t blocks = (int64_t)n_mats * (rows / 128) * (cols / 128);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(w),
                     rows, cols, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
