// Grouped bf16 expert GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// The expert FFNs of the h'_t equation (方法 §2, "DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437), each a SwiGLU FFN, run as two grouped GEMMs
// over the padded per-expert layout built by the permutation:
//   gate/up:  H[r, n] = SiLU(x_r . Wg[e][n]) * (x_r . Wu[e][n]),  x_r = u[row_token[r]]
//   down:     Y[r, n] = H[r] . Wd[e][n]
// where e is the expert (routed or shared) owning row r's M-tile.  The gate/up
// GEMM reads token rows straight from u through row_token, so the permuted
// activation matrix is never materialised.
//
// Tiling: a workgroup of 256 threads (4 wavefronts) owns 128 rows x 256 weight
// rows (gate/up: 128 gate + the matching 128 up features; down: 256 output
// features) and walks K in 64-wide steps through a double-buffered LDS stage
// (16 KB activations + 32 KB weights per stage).  Each wavefront computes 64 rows x
// 4 blocks of 32 weight rows with 8 MFMA accumulators; the MFMA's A operand is the
// weight tile and its B operand the activation tile, so each lane ends up holding
// four runs of 4 consecutive output features of one row.  LDS rows are 128 bytes;
// the 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so the 8 lanes of a
// fragment read that share a chunk index hit 8 different bank groups.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kWRows = 256;
constexpr int kStageElems = (kTileM + kWRows) * kBK;  // bf16 elements per LDS stage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

template <bool SWIGLU>
__global__ void __launch_bounds__(kThreads) grouped_gemm_bf16_kernel(GemmOperands g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int mt = blockIdx.x;
  const int seg = g.tile_seg[mt];
  if (seg < 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = g.K, N = g.N;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int n0 = blockIdx.y * (SWIGLU ? kWRows / 2 : kWRows);
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  const size_t wstride = (size_t)N * K;
  const uint16_t* W0 = static_cast<const uint16_t*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride;
  const uint16_t* W1 = SWIGLU ? static_cast<const uint16_t*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride
                              : nullptr;
  const uint16_t* act = static_cast<const uint16_t*>(g.act);

  // ---- per-thread global source rows (fixed chunk column, rows tid/8 + 32 i)
  const int ch = tid & 7;
  const int rbase = tid >> 3;
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t r = m0 + rbase + 32 * i;
    int64_t tok = g.row_token ? (int64_t)g.row_token[r] : r;
    asrc[i] = tok >= 0 ? act + tok * K + ch * 8 : nullptr;
  }
  const uint16_t* wsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = rbase + 32 * i;  // 0..255 within the weight tile
    const uint16_t* base;
    int n;
    if (SWIGLU) {
      base = r < 128 ? W0 : W1;
      n = n0 + (r & 127);
    } else {
      base = W0;
      n = n0 + r;
    }
    wsrc[i] = n < N ? base + (size_t)n * K + ch * 8 : nullptr;
  }

  u32x4 ra[4], rw[8];
  auto load_stage = [&](int k0) {
    const bool kin = k0 + ch * 8 < K;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = (kin && asrc[i]) ? *reinterpret_cast<const u32x4*>(asrc[i] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rw[i] = (kin && wsrc[i]) ? *reinterpret_cast<const u32x4*>(wsrc[i] + k0) : u32x4{0, 0, 0, 0};
  };
  auto store_stage = [&](int buf) {
    uint16_t* st = lds + buf * kStageElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(st + lds_off(rbase + 32 * i, ch)) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(st + lds_off(kTileM + rbase + 32 * i, ch)) = rw[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // weight-tile rows of this wavefront's four 32-row blocks
  int wrow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    wrow[nb] = SWIGLU ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32) : (wn * 128 + nb * 32);
  const int l32 = lane & 31, khalf = lane >> 5;

  const int nk = (K + kBK - 1) / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_stage((kt + 1) * kBK);
    const uint16_t* st = lds + (kt & 1) * kStageElems;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + khalf;
      bf16x8 xf[2], wf[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        xf[mb] = *reinterpret_cast<const bf16x8*>(st + lds_off(wm * 64 + mb * 32 + l32, c));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        wf[nb] = *reinterpret_cast<const bf16x8*>(st + lds_off(kTileM + wrow[nb] + l32, c));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[mb][nb], 0, 0, 0);
    }
    if (more) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds row (l32) and features 8 q + 4 khalf + (0..3) of each 32-block
  uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t row = m0 + wm * 64 + mb * 32 + l32;
    uint16_t* orow = out + row * N;
    if (SWIGLU) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = n0 + wn * 64 + nb * 32 + q * 8 + khalf * 4;
          uint16_t h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = f32_to_bf16(silu(acc[mb][nb][q * 4 + v]) * acc[mb][nb + 2][q * 4 + v]);
          if (f + 3 < N) {
            *reinterpret_cast<uint2*>(orow + f) =
                make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (f + v < N) orow[f + v] = h[v];
          }
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = n0 + wn * 128 + nb * 32 + q * 8 + khalf * 4;
          uint16_t h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = f32_to_bf16(acc[mb][nb][q * 4 + v]);
          if (f + 3 < N) {
            *reinterpret_cast<uint2*>(orow + f) =
                make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (f + v < N) orow[f + v] = h[v];
          }
        }
      }
    }
  }
}

template <bool SWIGLU>
hipError_t launch_bf16(const GemmOperands& g, hipStream_t st) {
  const size_t lds_bytes = 2 * kStageElems * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_bf16_kernel<SWIGLU>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int ntile = SWIGLU ? kWRows / 2 : kWRows;
  dim3 grid((unsigned)g.max_tiles, (unsigned)ceil_div(g.N, ntile));
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<SWIGLU>, grid, dim3(kThreads), lds_bytes, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_swiglu(const GemmOperands& g, hipStream_t st) { return launch_bf16<true>(g, st); }
hipError_t launch_gemm_bf16_down(const GemmOperands& g, hipStream_t st) { return launch_bf16<false>(g, st); }

}  // namespace moe
