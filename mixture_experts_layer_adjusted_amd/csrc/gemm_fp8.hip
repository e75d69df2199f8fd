// Grouped FP8 (E4M3FN) expert GEMMs with 1x128 activation and 128x128 weight block scales.
//
// The expert FFNs of the h'_t equation (方法 §2, "DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437) in the FP8 scheme of the same page's 核心概念
// list: E4M3 operands, one fp32 scale per 1x128 activation tile and per 128x128 weight
// block, accumulation in fp32.  The page's design for its hardware moves the partial
// sums of every 128-element K block out of the tensor cores into fp32 registers and
// scales them there; gfx950's MFMA accumulates in full fp32 already, so the same
// arithmetic is laid out as: per 128-wide K-step (one scale block) a fresh MFMA
// accumulator collects the raw E4M3 products (v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit E8M0 scales), which is then added to the fp32 result with the factor
// act_scale[row][kb] * weight_scale[feature block][kb].
//
//   gate/up:  H[r, n] = SiLU(x_r . Wg[e][n]) * (x_r . Wu[e][n]), then H is quantised per
//             1x128 tile along I (scale = amax / 448, round to nearest even, saturate);
//             the 128 features of a tile are exactly the workgroup's N-tile, so the row
//             amax is a reduction across the four wavefronts that share the row
//   down:     Y[r, n] = H[r] . Wd[e][n] in bf16
//
// Tiling: 512 threads (8 wavefronts, two per SIMD), 128 rows x 256 weight rows (gate/up: 128
// gate + the matching 128 up features; down: 256 output features), wavefront (wm, wn) of the
// 2 x 4 grid owning 64 rows x 64 weight rows.  One K-step is 128 bytes of every row, the LDS
// row pitch of the bf16 kernels, with the same XOR swizzle (conflict-free 16-lane reads), three
// 48 KB stages filled by direct global->LDS loads two K-steps ahead, and the same XCD-aware
// tile order (blocks of 4 M-tiles x 8 N-tiles of one expert per XCD).
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kBK = 128;            // K elements (bytes) per step = one scale block
constexpr int kWRows = 256;
constexpr int kStages = 3;
constexpr int kDataBytes = (kTileM + kWRows) * kBK;   // 48 KB of operands per stage
constexpr int kScaleBytes = 1024;                      // 128 row scales + 2 weight-block scales, padded
constexpr int kStageBytes = kDataBytes + kScaleBytes;
constexpr int kXcds = 8;
constexpr int kXcdChunk = 32;
constexpr int kGroupM = 4;
constexpr int kDmaPerStage = 7;     // loads per wavefront per stage: 2 activation + 4 weight (1 KB) + 1 scale
constexpr int kE8M0One = 127;       // E8M0 encoding of 2^0

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int boff(int r, int c) { return r * kBK + ((c ^ swz(r)) << 4); }  // c: 16-byte chunk

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 32 bytes of row r starting at 16-byte chunk c (c even): two swizzled 16-byte reads
__device__ __forceinline__ i32x8 frag32(const uint8_t* st, int r, int c) {
  u32x4 a = *reinterpret_cast<const u32x4*>(st + boff(r, c));
  u32x4 b = *reinterpret_cast<const u32x4*>(st + boff(r, c + 1));
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

template <bool SWIGLU>
__global__ void __launch_bounds__(kThreads) grouped_gemm_fp8_kernel(GemmOperands g, int NT) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float row_amax[kTileM][4];
  // ---- logical tile (same XCD-aware order as the bf16 streaming kernel)
  const int b = blockIdx.x;
  const int64_t L = (int64_t)(b / (kXcds * kXcdChunk)) * (kXcds * kXcdChunk) + (b % kXcds) * kXcdChunk +
                    (b / kXcds) % kXcdChunk;
  const int64_t mt_glob = L / NT;
  if (mt_glob >= g.max_tiles) return;
  const int seg = g.tile_seg[mt_glob];
  if (seg < 0) return;
  const int seg_m0 = g.seg_off[seg] / kTileM;
  const int seg_mt = g.seg_off[seg + 1] / kTileM - seg_m0;
  const int64_t lam = L - (int64_t)seg_m0 * NT;
  const int grp = (int)(lam / (kGroupM * NT));
  const int gm = min(kGroupM, seg_mt - grp * kGroupM);
  const int rem = (int)(lam - (int64_t)grp * kGroupM * NT);
  const int mt = seg_m0 + grp * kGroupM + rem % gm;
  const int nt = rem / gm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int K = g.K, N = g.N, KB = K / kBK;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int n0 = nt * (SWIGLU ? kWRows / 2 : kWRows);
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  const size_t wstride = (size_t)N * K;
  const size_t sstride = (size_t)(N / kBK) * KB;  // scales per expert matrix
  const uint8_t* W0 = static_cast<const uint8_t*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride;
  const uint8_t* W1 =
      SWIGLU ? static_cast<const uint8_t*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride : nullptr;
  const float* S0 = (shared ? g.s_shared[0] : g.s_routed[0]) + e * sstride;
  const float* S1 = SWIGLU ? (shared ? g.s_shared[1] : g.s_routed[1]) + e * sstride : nullptr;
  const uint8_t* act = static_cast<const uint8_t*>(g.act);

  // ---- direct-load sources: wave w fills activation rows [16w, 16w+16) and weight-tile rows
  // [32w, 32w+32), 8 rows of 128 bytes per load; lane l covers row l >> 3, slot l & 7
  const int lrow = lane >> 3, lslot = lane & 7;
  const uint8_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wave * 16 + i * 8 + lrow;
    int64_t tok = g.row_token ? (int64_t)g.row_token[m0 + row] : m0 + row;
    if (tok < 0) tok = 0;  // padding row: any valid row (outputs never read)
    asrc[i] = act + tok * K + ((lslot ^ swz(row)) << 4);
  }
  const uint8_t* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + lrow;  // 0..255 within the weight tile
    const uint8_t* base;
    int n;
    if (SWIGLU) {
      base = r < kWRows / 2 ? W0 : W1;
      n = n0 + (r & (kWRows / 2 - 1));
    } else {
      base = W0;
      n = n0 + r;
    }
    if (n >= N) n = N - 1;  // beyond the last feature: any valid row (outputs masked)
    wsrc[i] = base + (size_t)n * K + ((lslot ^ swz(kTileM + r)) << 4);
  }
  // ---- scale sources: every wave loads the activation scales of rows [16w, 16w+16) (lanes 0..15,
  // 4 bytes each) into the stage's scale area; wave 7's lanes 16 and 17 load the scales of the
  // two 128-row weight blocks of the tile, landing right after the 128 row scales
  const int l32 = lane & 31, khalf = lane >> 5;
  const float* ssrc = nullptr;
  if (lane < 16) {
    const int row = wave * 16 + lane;
    int64_t tok = g.row_token ? (int64_t)g.row_token[m0 + row] : m0 + row;
    if (tok < 0) tok = 0;
    ssrc = g.act_scale + tok * KB;
  } else if (wave == 7 && lane < 18) {
    const int nb = lane - 16;
    if (SWIGLU) {
      ssrc = (nb == 0 ? S0 : S1) + (size_t)(n0 / kBK) * KB;  // gate block, then the matching up block
    } else {
      const int n = min(n0 + nb * kBK, N - 1);
      ssrc = S0 + (size_t)(n / kBK) * KB;
    }
  }
  auto issue_stage = [&](int kt) {
    uint8_t* st = lds + (kt % kStages) * kStageBytes;
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(asrc[i] + k0, (lds_void_t*)(st + (wave * 16 + i * 8) * kBK), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(wsrc[i] + k0, (lds_void_t*)(st + (kTileM + wave * 32 + i * 8) * kBK), 16, 0,
                                       0);
    // lanes without a scale to load stay inactive for this one load (it still counts once)
    if (ssrc) __builtin_amdgcn_global_load_lds(ssrc + kt, (lds_void_t*)(st + kDataBytes + wave * 64), 4, 0, 0);
  };

  // weight rows of the wave's two 32-row blocks, and the 128-row scale block each falls in
  int wrow[2], wblk[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if (SWIGLU) {
      wrow[nb] = nb * (kWRows / 2) + wn * 32;      // gate block, then the matching up block
      wblk[nb] = nb;
    } else {
      wrow[nb] = wn * 64 + nb * 32;
      wblk[nb] = wrow[nb] / kBK;
    }
  }

  float acc[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

  const int nk = KB;
  issue_stage(0);
  if (nk > 1) issue_stage(1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vmcnt<kDmaPerStage>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // stage kt landed for every wave; stage kt-1 is no longer read
    if (kt + 2 < nk) issue_stage(kt + 2);
    const uint8_t* st = lds + (kt % kStages) * kStageBytes;
    const float* sc = reinterpret_cast<const float*>(st + kDataBytes);
    f32x16 part[2][2];
#pragma unroll
    for (int kk = 0; kk < kBK / 64; ++kk) {
      const int c = kk * 4 + khalf * 2;  // this lane's 32 bytes of the 64-byte slice
      i32x8 xf[2], wf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) xf[mb] = frag32(st, wm * 64 + mb * 32 + l32, c);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) wf[nb] = frag32(st, kTileM + wrow[nb] + l32, c);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (kk == 0) {
            f32x16 z;
#pragma unroll
            for (int v = 0; v < 16; ++v) z[v] = 0.0f;
            part[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[nb], xf[mb], z, 0, 0, 0, kE8M0One, 0,
                                                                           kE8M0One);
          } else {
            part[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[nb], xf[mb], part[mb][nb], 0, 0, 0,
                                                                           kE8M0One, 0, kE8M0One);
          }
        }
    }
    // fold the block's products into the fp32 result with act_scale * weight_scale
    const float sw0 = sc[kTileM + wblk[0]], sw1 = sc[kTileM + wblk[1]];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float sa = sc[wm * 64 + mb * 32 + l32];
      const float f0 = sa * sw0, f1 = sa * sw1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[mb][0][v] = fmaf(part[mb][0][v], f0, acc[mb][0][v]);
        acc[mb][1][v] = fmaf(part[mb][1][v], f1, acc[mb][1][v]);
      }
    }
  }

  // ---- epilogue.  Lane holds row 64 wm + 32 mb + l32 and, per 32-row weight block, features
  // 8 q + 4 khalf + (0..3) of that block
  if (SWIGLU) {
    uint8_t* out = static_cast<uint8_t*>(g.out);
    const int IB = N / kBK;
    float h[2][16];
    float amax[2] = {0.0f, 0.0f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        h[mb][v] = silu(acc[mb][0][v]) * acc[mb][1][v];
        amax[mb] = fmaxf(amax[mb], fabsf(h[mb][v]));
      }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      amax[mb] = fmaxf(amax[mb], __shfl_xor(amax[mb], 32, 64));
      if (khalf == 0) row_amax[wm * 64 + mb * 32 + l32][wn] = amax[mb];
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = wm * 64 + mb * 32 + l32;
      const float a = fmaxf(fmaxf(row_amax[r][0], row_amax[r][1]), fmaxf(row_amax[r][2], row_amax[r][3]));
      const float scale = a > 0.0f ? __fdiv_rn(a, 448.0f) : 1.0f;
      uint8_t* orow = out + (m0 + r) * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = n0 + wn * 32 + q * 8 + khalf * 4;
        uint32_t w = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) w |= e4m3_from_f32(__fdiv_rn(h[mb][q * 4 + v], scale)) << (8 * v);
        *reinterpret_cast<uint32_t*>(orow + f) = w;
      }
      if (wn == 0 && khalf == 0) g.out_scale[(m0 + r) * IB + n0 / kBK] = scale;
    }
  } else {
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      uint16_t* orow = out + (m0 + wm * 64 + mb * 32 + l32) * N;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = n0 + wrow[nb] + q * 8 + khalf * 4;
          if (f + 3 < N) {
            *reinterpret_cast<uint2*>(orow + f) =
                make_uint2((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 0]) |
                               ((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 1]) << 16),
                           (uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 2]) |
                               ((uint32_t)f32_to_bf16(acc[mb][nb][q * 4 + 3]) << 16));
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (f + v < N) orow[f + v] = f32_to_bf16(acc[mb][nb][q * 4 + v]);
          }
        }
    }
  }
}

template <bool SWIGLU>
hipError_t launch_fp8(const GemmOperands& g, hipStream_t st) {
  if (g.K % kBK != 0 || g.N % kBK != 0) return hipErrorInvalidValue;
  const size_t lds_bytes = kStages * kStageBytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_fp8_kernel<SWIGLU>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int NT = (int)ceil_div(g.N, SWIGLU ? kWRows / 2 : kWRows);
  const int64_t tiles = g.max_tiles * NT;
  const int64_t grid = ceil_div(tiles, kXcds * kXcdChunk) * (kXcds * kXcdChunk);
  hipLaunchKernelGGL(grouped_gemm_fp8_kernel<SWIGLU>, dim3((unsigned)grid), dim3(kThreads), lds_bytes, st, g, NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_swiglu(const GemmOperands& g, hipStream_t st) { return launch_fp8<true>(g, st); }
hipError_t launch_gemm_fp8_down(const GemmOperands& g, hipStream_t st) { return launch_fp8<false>(g, st); }

}  // namespace moe
