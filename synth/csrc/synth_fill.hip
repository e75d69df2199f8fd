// Device (HIP, gfx950) filler for the seeded synthetic input streams.
//
// Same definition as the numpy reference in synth/__init__.py and the host
// filler in synth_host.c: SplitMix64 outputs (Steele, Lea and Flood, OOPSLA
// 2014) of a per-tensor key, eight 16-bit fields summed (Irwin-Hall of order 8),
// recentred to an exact integer, converted exactly to fp32 and scaled by one
// correctly rounded fp32 multiply; bf16 output is the round-to-nearest-even of
// that fp32 value.  Holds no arithmetic of the MoE method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kG = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ int32_t ih8(uint64_t key, uint64_t n) {
  uint64_t w0 = mix64(key + (2 * n + 1) * kG);
  uint64_t w1 = mix64(key + (2 * n + 2) * kG);
  int32_t s = 0;
#pragma unroll
  for (int sh = 0; sh < 64; sh += 16) s += (int32_t)((w0 >> sh) & 0xFFFF) + (int32_t)((w1 >> sh) & 0xFFFF);
  return s - 262140;
}

template <int kKind>
__global__ void __launch_bounds__(256) fill_kernel(void* __restrict__ out, int64_t n, int64_t start,
                                                   uint64_t key, float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float v = __fmul_rn((float)ih8(key, (uint64_t)(start + i)), scale);
    if (kKind == 0) {
      static_cast<float*>(out)[i] = v;
    } else {
      uint32_t b = __float_as_uint(v);
      static_cast<uint16_t*>(out)[i] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    }
  }
}

}  // namespace

// Fill out[0..n) (device memory) with elements [start, start+n) of stream `key`,
// asynchronously on `stream`. out_kind: 0 = fp32, 1 = bf16 bits.
// Returns 0, -1 on bad arguments, -4 if the launch failed.
extern "C" int synth_fill_normal_device(void* out, int64_t n, int64_t start, uint64_t key, float scale,
                                        int out_kind, hipStream_t stream) {
  if (n < 0 || start < 0 || (out_kind != 0 && out_kind != 1)) return -1;
  if (n == 0) return 0;
  if (!out) return -1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (out_kind == 0)
    hipLaunchKernelGGL(fill_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, out, n, start, key, scale);
  else
    hipLaunchKernelGGL(fill_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, out, n, start, key, scale);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
