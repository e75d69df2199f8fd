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
// Two kernels:
//  * the streaming kernel (contraction length a multiple of 64): a workgroup of 8 wavefronts
//    owns 256 rows (two M-tiles of one segment) x 256 weight rows (gate/up: 128 gate + the
//    matching 128 up features; down: 256 output features), or 128 rows x 512 weight rows when
//    segments hold few rows (decode-like batches).  Each wavefront computes 128 x 64 with
//    v_mfma_f32_32x32x16_bf16; the MFMA's A operand is the weight tile and its B operand the
//    activation tile, so a lane ends with runs of four consecutive output features of one row.
//    Two 64 KB LDS stages are filled by direct loads into LDS (buffer_load_dwordx4 ... lds) one
//    K-step ahead; LDS rows are XOR-swizzled in 16-byte chunks so that fragment reads are free
//    of bank conflicts.  Tiles come in an XCD-aware order: the 8 XCDs of MI355X each receive
//    workgroups round-robin, so workgroup b runs on XCD b % 8, and logical tiles are handed out
//    so that the 32 workgroups an XCD holds at once form one block of M-tiles x N-tiles of the
//    same expert (operands reused through that XCD's L2), experts in order.  The backward uses
//    it with other epilogues (SwiGLU backward, weight gradients) and, for the input-gradient
//    products, with the weights read K-major as stored through transposing LDS reads;
//  * the register-staged kernel (any contraction length that is a multiple of 8): 4 wavefronts
//    on 128 x 256, loads through registers with zero fill of the K tail, in plain grid order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kWRows = 256;
constexpr int kStageElems = (kTileM + kWRows) * kBK;  // bf16 elements per LDS stage

#ifndef MOE_STREAM_BK
#define MOE_STREAM_BK 64
#endif
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
#ifndef MOE_STREAM_WAVES
#define MOE_STREAM_WAVES 8
#endif
#ifndef MOE_STREAM_WROWS
#define MOE_STREAM_WROWS 256
#endif
#ifndef MOE_STREAM_WGS
#define MOE_STREAM_WGS 1
#endif
#ifndef MOE_STREAM_WM
#define MOE_STREAM_WM 2
#endif
#ifndef MOE_STREAM_TM
#define MOE_STREAM_TM 256
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// K-major weight tile in LDS: BK rows of 256 features (512 bytes); the 16-byte feature chunk c
// of row r sits at slot c ^ kn_swz(r), so that the eight rows a transposing read touches (rows
// kb..kb+3 and kb+8..kb+11 at one 32-feature block) fall on distinct bank groups
__device__ __forceinline__ int kn_swz(int r) { return 4 * (r & 3); }
__device__ __forceinline__ int kn_off(int r, int col) { return r * 256 + (((col >> 3) ^ kn_swz(r)) << 3) + (col & 7); }
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS rows are 128 bytes (64 bf16).  The 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7):
// a ds_read_b128 is served 16 lanes per pass by 64 four-byte banks (256 bytes), and the 16 lanes
// of a fragment read (rows r..r+15, one logical chunk) then cover all 64 banks exactly once
// (rows 2j and 2j+1 share a chunk slot but sit in opposite bank halves).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ swz(row)) << 3); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }


// Epilogue: the lane holds, for row r0 + 32 mb + l32, features 8 q + 4 khalf + (0..3) of each
// 32-feature block; SwiGLU pairs gate block nb with up block nb + NBW/2, the gate blocks covering
// features fbase + 32 nb.
template <bool SWIGLU, int MB = 2, int NBW = 4>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MB][NBW], uint16_t* out, int64_t r0, int fbase,
                                           int N, int l32, int khalf) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    uint16_t* orow = out + (r0 + mb * 32 + l32) * N;
#pragma unroll
    for (int nb = 0; nb < (SWIGLU ? NBW / 2 : NBW); ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = fbase + nb * 32 + q * 8 + khalf * 4;
        uint16_t h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          h[v] = SWIGLU ? f32_to_bf16(silu(acc[mb][nb][q * 4 + v]) * acc[mb][nb + NBW / 2][q * 4 + v])
                        : f32_to_bf16(acc[mb][nb][q * 4 + v]);
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

  store_tile<SWIGLU>(acc, static_cast<uint16_t*>(g.out), m0 + wm * 64, n0 + (SWIGLU ? wn * 64 : wn * 128), N, l32,
                     khalf);
}


// ---------------------------------------------------------------------------- streaming variant
//
// WAVES wavefronts own TM rows (128, one M-tile; or 256, two M-tiles of the same segment) x
// WROWS weight rows (gate/up: WROWS/2 gate + the matching WROWS/2 up features; down: WROWS
// output features); wavefront (wm, wn) of the WM x (WAVES/WM) grid computes TM/WM rows x
// WROWS/(WAVES/WM) weight rows.  WGS workgroups share a CU, each with 160 KB / WGS of LDS
// holding as many stages of (TM + WROWS) x BK bf16 as fit; direct global->LDS loads run
// (stages - 1) K-steps ahead of the MFMAs.  With TM = 256 a segment with an odd number of
// M-tiles ends in a half tile: its second 128 rows belong to the next segment, so they load
// a valid row and the wavefronts owning them skip their MFMAs and stores.

constexpr int kLdsBytes = 163840;
constexpr int kXcds = 8;          // MI355X: 8 XCDs of 32 CUs, workgroups dealt round-robin
constexpr int kCusPerXcd = 32;
constexpr int kGroupM = MOE_GROUP_M;  // M-tiles per block of the within-expert order

template <int BK, int WAVES, int WROWS, int WGS, int TM>
struct StreamCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kChunks = BK / 8;                       // 16-byte chunks per LDS row
  static constexpr int kRowsPer256 = 256 / kRowBytes;          // rows sharing one pass of the 64 banks
  static constexpr int kStageElems = (TM + WROWS) * BK;
  static constexpr int kStages = (kLdsBytes / WGS) / (kStageElems * 2);
  static constexpr int kRowsPerDma = 1024 / kRowBytes;          // rows one wave-wide 1 KB load fills
  static constexpr int kADma = TM / kRowsPerDma / WAVES;        // activation loads per wave per stage
  static constexpr int kWDma = WROWS / kRowsPerDma / WAVES;     // weight loads per wave per stage
  static constexpr int kDmaPerStage = kADma + kWDma;
  static constexpr int kXcdChunk = kCusPerXcd * WGS;            // workgroups an XCD holds at once
  static_assert(kStages >= 2, "at least two LDS stages");
  static_assert(kADma * kRowsPerDma * WAVES == TM && kWDma * kRowsPerDma * WAVES == WROWS, "load split");
  static_assert((WROWS / WAVES) % kRowsPerDma == 0 && (WROWS / 2) % (WROWS / WAVES) == 0,
                "gate/up split on a wave boundary");
  // chunk c of row r sits at slot c ^ swz(r): the 16 rows of a 16-lane read pass then cover all
  // 64 banks once (rows in one 256-byte bank span differ in their bank offset, rows in different
  // spans in their slot)
  __device__ static __forceinline__ int swz(int r) { return (r / kRowsPer256) % kChunks; }
  __device__ static __forceinline__ int off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_dma16(const void* src, uint16_t* lds_base) {
  // each lane's 16 bytes land at lds_base + 16 * lane (the destination is wave-uniform)
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds_base), 16, 0, 0);
}

// The same 16-byte-per-lane load into LDS in buffer form: address = base + voff + soff, with soff
// wave-uniform (the K-step's byte offset).  A raw buffer of 2^32 - 1 bytes covers every 32-bit
// offset the kernels form (the launchers check that their operands stay below 4 GiB).  Measured
// 2-4% faster than the global form on the same tiles.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ void lds_buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds_base), 16, voff, soff, 0, 0);
}

#ifndef MOE_BUFFER_LOADS
#define MOE_BUFFER_LOADS 1
#endif

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (split field on gfx9: bits 3:0 and 15:14), expcnt and lgkmcnt not waited
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS traffic of this wavefront done (lgkmcnt 0; vmcnt 63 and expcnt 7 are no wait), then a bare
// barrier: unlike __syncthreads() it leaves global loads, LDS DMA and stores in flight.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Staged epilogues of the 256 x 256 tile kernels (eight wavefronts; wavefront (wm, wn) holds rows
// wm * 128 + [0, 128) of the tile in MB = 4 blocks of 32 and 64 output columns (plain) or 32
// gate + the matching 32 up features (SwiGLU) in NBW = 2 blocks of 32).  The 32 x 32 MFMA result
// layout gives each lane runs of 4 columns of one row, so direct stores write 32 rows x 16 bytes
// per instruction; staged through an LDS stage no load is filling, each store instead writes
// whole 256- or 512-byte row spans (8 full 128-byte lines).  Staged 16-byte chunk c of row r sits
// at slot c ^ (r mod chunks per row), so neither side piles onto a few banks.  The LDS accesses
// are typed (64-bit and 4 x 32-bit integers), which keeps the compiler from making them wait for
// the global loads and stores in flight.  The caller has passed lds_barrier() since the stage was
// last read.  Every store instruction has an active lane (chunk 0 lies below N; N is a multiple
// of 8), so the return value, the stores this wavefront issued, is exact for vmcnt accounting.
constexpr int kStagedRounds = 8;   // row-span stores per wavefront per 64 KB of staged output

// four values rounded to bf16 (nearest even, as f32_to_bf16 for finite values) by the packed
// conversion instruction, lowest address first
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint64_t pack_bf16x4(float a, float b, float c, float d) {
  const bf16x2_t lo = {(__bf16)a, (__bf16)b};
  const bf16x2_t hi = {(__bf16)c, (__bf16)d};
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}

// plain 256 x 256 tile (rows m0 + [0, tile_rows), tile_rows 128 or 256, columns n0 + [0, 256)
// below N) in two passes of 512-byte rows: pass p stages accumulator blocks 2p and 2p + 1 of
// every wavefront (tile rows wm * 128 + p * 64 + [0, 64) as staged rows wm * 64 + [0, 64)), so
// half of each wavefront's accumulators are dead before any row is read back
__device__ __forceinline__ int store_tile_staged(const f32x16 (&acc)[4][2], uint16_t* stg, uint16_t* out,
                                                 int64_t m0, int n0, int N, int tile_rows, int wave, int wm,
                                                 int wn, int lane) {
  // the lane index made opaque: the per-lane LDS offsets below are then computed per tile rather
  // than hoisted out of the caller's tile loop, where they would hold registers across the MFMAs
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, khalf = lane >> 5;
  // staged rows 64 and up belong to wavefronts wm = 1, absent from a half tile
  const int rounds = tile_rows > 128 ? kStagedRounds : kStagedRounds / 2;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p > 0) lds_barrier();   // the first pass has been read back
    if (wm * 128 < tile_rows) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = wm * 64 + h * 32 + l32;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * 8 + nb * 4 + q;
            const f32x16& a = acc[2 * p + h][nb];
            *reinterpret_cast<uint64_t*>(stg + r * 256 + ((c ^ (r & 31)) << 3) + khalf * 4) =
                pack_bf16x4(a[q * 4], a[q * 4 + 1], a[q * 4 + 2], a[q * 4 + 3]);
          }
      }
    }
    lds_barrier();
    const int c = lane & 31;
    const int f = n0 + c * 8;
#pragma unroll
    for (int i = 0; i < kStagedRounds; ++i) {
      if (i < rounds) {
        const int r = (i * 8 + wave) * 2 + (lane >> 5);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * 256 + ((c ^ (r & 31)) << 3));
        const int64_t row = m0 + (r >> 6) * 128 + p * 64 + (r & 63);
        if (f < N) *reinterpret_cast<u32x4*>(out + row * N + f) = v;
      }
    }
  }
  return 2 * rounds;
}

// SwiGLU 256 x 128 tile H = silu(gate) * up in one pass of 256-byte rows (rows m0 + [0, tile_rows),
// features n0 + [0, 128) below N)
__device__ __forceinline__ int store_tile_staged_swiglu(const f32x16 (&acc)[4][2], uint16_t* stg, uint16_t* out,
                                                        int64_t m0, int n0, int N, int tile_rows, int wave, int wm,
                                                        int wn, int lane) {
  asm volatile("" : "+v"(lane));   // as in store_tile_staged
  const int l32 = lane & 31, khalf = lane >> 5;
  if (wm * 128 < tile_rows) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 128 + mb * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * 4 + q;
        const f32x16& ga = acc[mb][0];
        const f32x16& ua = acc[mb][1];
        *reinterpret_cast<uint64_t*>(stg + r * 128 + ((c ^ (r & 15)) << 3) + khalf * 4) =
            pack_bf16x4(silu(ga[q * 4]) * ua[q * 4], silu(ga[q * 4 + 1]) * ua[q * 4 + 1],
                        silu(ga[q * 4 + 2]) * ua[q * 4 + 2], silu(ga[q * 4 + 3]) * ua[q * 4 + 3]);
      }
    }
  }
  lds_barrier();
  const int c = lane & 15;
  const int f = n0 + c * 8;
  const int rounds = tile_rows > 128 ? kStagedRounds : kStagedRounds / 2;
#pragma unroll
  for (int i = 0; i < kStagedRounds; ++i) {
    if (i < rounds) {
      const int r = (i * 8 + wave) * 4 + (lane >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * 128 + ((c ^ (r & 15)) << 3));
      if (f < N) *reinterpret_cast<u32x4*>(out + (m0 + r) * N + f) = v;
    }
  }
  return rounds;
}

// The SwiGLU inputs of a 256 x 128 tile, a (gate accumulators) to columns n0 + [0, 128) and b (up)
// to columns N + n0 + [0, 128) of out (row stride 2N, rows m0 + [0, tile_rows)): two staged passes
// of 256-byte row spans as in store_tile_staged_swiglu.  The caller has passed lds_barrier() since
// the stage was last read (the SwiGLU pass before it ends with its row reads).
__device__ __forceinline__ int store_tile_staged_ab(const f32x16 (&acc)[4][2], uint16_t* stg, uint16_t* out,
                                                    int64_t m0, int n0, int N, int tile_rows, int wave, int wm,
                                                    int wn, int lane) {
  asm volatile("" : "+v"(lane));   // as in store_tile_staged
  const int l32 = lane & 31, khalf = lane >> 5;
  const int rounds = tile_rows > 128 ? kStagedRounds : kStagedRounds / 2;
  const int c = lane & 15;
  const int f = n0 + c * 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lds_barrier();   // the stage's previous rows have been read
    if (wm * 128 < tile_rows) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r = wm * 128 + mb * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cc = wn * 4 + q;
          const f32x16& a = acc[mb][h];
          *reinterpret_cast<uint64_t*>(stg + r * 128 + ((cc ^ (r & 15)) << 3) + khalf * 4) =
              pack_bf16x4(a[q * 4], a[q * 4 + 1], a[q * 4 + 2], a[q * 4 + 3]);
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kStagedRounds; ++i) {
      if (i < rounds) {
        const int r = (i * 8 + wave) * 4 + (lane >> 4);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * 128 + ((c ^ (r & 15)) << 3));
        if (f < N) *reinterpret_cast<u32x4*>(out + (m0 + r) * 2 * (int64_t)N + h * N + f) = v;
      }
    }
  }
  return 2 * rounds;
}

// SwiGLU backward epilogue of a 256 x 128 tile (a, b = the gate and up accumulators of features
// n0 + [0, 128), rows m0 + [0, tile_rows)), through an LDS stage no load is filling:
//   dH before the gate (g.dh, [rows, N]) comes in by direct loads into the stage (256-byte rows
//   whose 16-byte chunk c sits at slot c ^ (row mod 16)) and is read into registers in the
//   accumulator layout;
//   with dh = row_gate * dH:  dA = dh b sg (1 + a (1 - sg)),  dB = dh a sg,  H = a sg b
//   (sg = sigmoid(a)), written to g.out ([rows, 2N]: dA then dB) and g.out2 ([rows, N]);
//   g.dg_part[row, nt] = sum over the 128 features of dH H, the four wavefronts of a row added in
//   order through red.
// Four passes, pass p taking accumulator block p of every wavefront (tile rows wm * 128 + 32 p +
// [0, 32), staged rows 32 wm + [0, 32)): its dA, dB and H (3 x 16 KB) go through the stage and
// out as whole 256-byte row spans, after which that block's accumulators are dead.  Waits for
// every load in flight (the prefetched K-step included) before reading dH.  Returns the stores
// every wavefront issued (some issue one more: the dg_part rows).
__device__ __forceinline__ int store_tile_staged_swiglu_bwd(const f32x16 (&acc)[4][2], uint16_t* stg,
                                                            const GemmOperands& g, int64_t m0, int n0, int nt,
                                                            int tile_rows, int wave, int wm, int wn, int lane,
                                                            float (*red)[4]) {
  asm volatile("" : "+v"(lane));   // as in store_tile_staged
  const int N = g.N;
  const int l32 = lane & 31, khalf = lane >> 5;
  const bool full = tile_rows > 128;
  // dH rows m0 + r (r beyond the tile: its last row), four rows per 1 KB load
  {
    const uint16_t* dh = static_cast<const uint16_t*>(g.dh);
    const int slot = lane & 15;
#pragma unroll
    for (int i = 0; i < kStagedRounds; ++i) {
      const int r = (i * 8 + wave) * 4 + (lane >> 4);
      const int rr = r < tile_rows ? r : tile_rows - 1;
      int f = n0 + 8 * (slot ^ (r & 15));
      if (f + 8 > N) f = N - 8;   // beyond the last feature: any valid chunk (never stored)
      lds_dma16(dh + (m0 + rr) * N + f, stg + (i * 8 + wave) * 4 * 128);
    }
  }
  float rg[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int r = wm * 128 + mb * 32 + l32;
    rg[mb] = g.row_gate[m0 + (r < tile_rows ? r : tile_rows - 1)];
  }
  wait_vmcnt<0>();
  lds_barrier();
  const bool active = wm * 128 < tile_rows;
  uint64_t dq[4][4];
  if (active) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 128 + mb * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * 4 + q;
        dq[mb][q] = *reinterpret_cast<const uint64_t*>(stg + r * 128 + ((c ^ (r & 15)) << 3) + khalf * 4);
      }
    }
  }
  uint16_t* dab = static_cast<uint16_t*>(g.out);
  uint16_t* hout = static_cast<uint16_t*>(g.out2);
  const int c = lane & 15;
  const int f = n0 + c * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    lds_barrier();   // the stage's previous contents (dH, or the last pass) have been read
    if (active) {
      const int sr = wm * 32 + l32;   // staged row
      float part = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float oa[4], ob[4], oh[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float dhu = __uint_as_float(((uint32_t)(dq[p][q] >> (16 * v)) & 0xFFFFu) << 16);
          const float a = acc[p][0][q * 4 + v], b = acc[p][1][q * 4 + v];
          const float sg = 1.0f / (1.0f + __expf(-a));
          const float dhv = rg[p] * dhu;
          oa[v] = dhv * b * sg * (1.0f + a * (1.0f - sg));
          ob[v] = dhv * a * sg;
          oh[v] = a * sg * b;
          part += dhu * oh[v];
        }
        const int off = sr * 128 + (((wn * 4 + q) ^ (sr & 15)) << 3) + khalf * 4;
        *reinterpret_cast<uint64_t*>(stg + off) = pack_bf16x4(oa[0], oa[1], oa[2], oa[3]);
        *reinterpret_cast<uint64_t*>(stg + 8192 + off) = pack_bf16x4(ob[0], ob[1], ob[2], ob[3]);
        *reinterpret_cast<uint64_t*>(stg + 16384 + off) = pack_bf16x4(oh[0], oh[1], oh[2], oh[3]);
      }
      part += __shfl_xor(part, 32, 64);
      if (khalf == 0) red[wm * 128 + p * 32 + l32][wn] = part;
    }
    lds_barrier();
    // 3 outputs x 64 staged rows x 16 chunks: each load/store covers four rows of one output;
    // staged rows 32 and up (wavefronts wm = 1) are absent from a half tile
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int blk = i * 8 + wave;          // 0..47
      const int o = blk >> 4;                // dA, dB, H
      const int sr = (blk & 15) * 4 + (lane >> 4);
      if (full || (blk & 15) < 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + o * 8192 + sr * 128 + ((c ^ (sr & 15)) << 3));
        const int64_t row = m0 + (sr >> 5) * 128 + p * 32 + (sr & 31);
        uint16_t* dst = o == 2 ? hout + row * N + f : dab + row * 2 * (int64_t)N + (o == 1 ? N : 0) + f;
        if (f < N) *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
  // red was complete at the last pass's second barrier
  const int t = wave * 64 + lane;
  if (t < tile_rows) g.dg_part[(m0 + t) * (N / 128) + nt] = red[t][0] + red[t][1] + red[t][2] + red[t][3];
  return full ? 24 : 12;
}

// wait until at most n (0, 4, 8, 12, 16 or 24: the stores a staged epilogue issued after the
// loads being waited for) vector memory operations are outstanding
__device__ __forceinline__ void wait_loads_behind_stores(int n) {
  if (n == 24)
    wait_vmcnt<24>();
  else if (n == 16)
    wait_vmcnt<16>();
  else if (n == 12)
    wait_vmcnt<12>();
  else if (n == 8)
    wait_vmcnt<8>();
  else if (n == 4)
    wait_vmcnt<4>();
  else
    wait_vmcnt<0>();
}

// wait until at most `ahead` stages of this wave's loads are still in flight
template <int PER, int MAXAHEAD>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXAHEAD >= 3) {
    if (ahead >= 3) { wait_vmcnt<3 * PER>(); return; }
  }
  if constexpr (MAXAHEAD >= 2) {
    if (ahead == 2) { wait_vmcnt<2 * PER>(); return; }
  }
  if constexpr (MAXAHEAD >= 1) {
    if (ahead == 1) { wait_vmcnt<PER>(); return; }
  }
  wait_vmcnt<0>();
}

// SwiGLU backward epilogue: acc[mb][0] holds the gate pre-activations a and acc[mb][1] the up
// values b of rows r0 + 32 mb + l32, features fbase + 8 q + 4 khalf + (0..3).  With
// sg = sigmoid(a), h = a sg b and dh = row_gate * dh_in (the gate of the row's (token, slot)):
// dA = dh b sg (1 + a (1 - sg)) and dB = dh a sg go to out = [dA dB], h to out2, and the
// row's sum of dh_in * h over the workgroup's 128 features (its share of <dY, FFN(x)>, the
// gate gradient) to dg_part[row, nt], reduced across the wavefronts sharing the row.
template <int MB>
__device__ __forceinline__ void store_swiglu_bwd(const f32x16 (&acc)[MB][2], const GemmOperands& g, int64_t m0,
                                                 int mrow0, int fbase, int nt, int wn, int tile_rows, bool active,
                                                 int l32, int khalf, float (*red)[4]) {
  const int N = g.N;
  const uint16_t* dhp = static_cast<const uint16_t*>(g.dh);
  uint16_t* dab = static_cast<uint16_t*>(g.out);
  uint16_t* hout = static_cast<uint16_t*>(g.out2);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rl = mrow0 + mb * 32 + l32;
    const int64_t r = m0 + rl;
    float part = 0.0f;
    if (active) {
      const float rg = g.row_gate[r];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = fbase + q * 8 + khalf * 4;
        const uint2 dq = *reinterpret_cast<const uint2*>(dhp + r * N + f);
        const float dhu[4] = {__uint_as_float(dq.x << 16), __uint_as_float(dq.x & 0xFFFF0000u),
                              __uint_as_float(dq.y << 16), __uint_as_float(dq.y & 0xFFFF0000u)};
        uint16_t da[4], db[4], hh[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc[mb][0][q * 4 + v], b = acc[mb][1][q * 4 + v];
          const float sg = 1.0f / (1.0f + __expf(-a));
          const float h = a * sg * b;
          const float dh = rg * dhu[v];
          da[v] = f32_to_bf16(dh * b * sg * (1.0f + a * (1.0f - sg)));
          db[v] = f32_to_bf16(dh * a * sg);
          hh[v] = f32_to_bf16(h);
          part += dhu[v] * h;
        }
        *reinterpret_cast<uint2*>(dab + r * 2 * N + f) =
            make_uint2((uint32_t)da[0] | ((uint32_t)da[1] << 16), (uint32_t)da[2] | ((uint32_t)da[3] << 16));
        *reinterpret_cast<uint2*>(dab + r * 2 * N + N + f) =
            make_uint2((uint32_t)db[0] | ((uint32_t)db[1] << 16), (uint32_t)db[2] | ((uint32_t)db[3] << 16));
        *reinterpret_cast<uint2*>(hout + r * N + f) =
            make_uint2((uint32_t)hh[0] | ((uint32_t)hh[1] << 16), (uint32_t)hh[2] | ((uint32_t)hh[3] << 16));
      }
    }
    part += __shfl_xor(part, 32, 64);
    if (khalf == 0) red[rl][wn] = part;
  }
  __syncthreads();
  for (int row = threadIdx.x; row < tile_rows; row += blockDim.x)
    g.dg_part[(m0 + row) * (N / 128) + nt] = red[row][0] + red[row][1] + red[row][2] + red[row][3];
}

// EPI: 0 plain store (down GEMM), 1 SwiGLU (gate/up GEMM), 2 SwiGLU backward (gate/up recomputed)
// WKN: the weight operand is stored with K as its row index ([K][N], N contiguous), as a
// weight matrix is for an input-gradient product; see kn_off below
template <int EPI, int BK, int WAVES, int WROWS, int WGS, int WM, int TM, bool WKN = false>
__global__ void __launch_bounds__(WAVES * 64, WGS) grouped_gemm_bf16_stream_kernel(GemmOperands g, int NT) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2;
  static_assert(!WKN || (EPI == 0 && BK == 64 && WROWS == 256 && WAVES == 8 && TM == 256),
                "K-major weights: the 256 x 256 plain-store tile");
  using C = StreamCfg<BK, WAVES, WROWS, WGS, TM>;
  constexpr int WN = WAVES / WM;           // wavefront grid WM x WN
  constexpr int RW = TM / WM;              // rows per wavefront
  constexpr int MB = RW / 32;              // 32-row blocks per wavefront
  constexpr int WRW = WROWS / WN;          // weight rows per wavefront
  constexpr int NBW = WRW / 32;            // 32-row weight blocks per wavefront
  static_assert(TM == kTileM || TM == 2 * kTileM, "tile of one or two M-tiles");
  static_assert(!SWIGLU || NBW % 2 == 0, "SwiGLU pairs gate and up blocks");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  // ---- logical tile of this workgroup (see the file comment)
  const int64_t L = xcd_logical(blockIdx.x, C::kXcdChunk);
  int seg, nt, tile_rows, nk;
  int64_t m0;
  {
    const int64_t slot = L / NT;             // M-tile (TM = 128) or pair of M-tiles (TM = 256)
    if (slot >= g.max_tiles) return;
    seg = TM == kTileM ? g.tile_seg[slot] : g.pair_seg[slot];
    if (seg < 0) return;
    const int seg_first = TM == kTileM ? g.seg_off[seg] / kTileM : g.pair_off[seg];
    const int seg_count = TM == kTileM ? g.seg_off[seg + 1] / kTileM - seg_first : g.pair_off[seg + 1] - seg_first;
    // rows of this tile that belong to the segment (a half tile has 128)
    const WalkTile t = walk_tile(L, NT, kGroupM, TM, seg_first, seg_count, g.seg_off[seg], g.seg_off[seg + 1]);
    nt = t.nt;
    m0 = t.m0;
    tile_rows = t.tile_rows;
    nk = g.K / BK;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS offsets stay scalar
  const int wm = wave / WN, wn = wave % WN;
  const int K = g.K, N = g.N;
  const int n0 = nt * (SWIGLU ? WROWS / 2 : WROWS);
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  // K-major weights may be two matrices stacked along K: rows [0, kn_split) of the first,
  // the rest of the second (the gate and up weights of one expert)
  const int kn_split = WKN ? g.kn_split : K;
  const size_t wstride = (size_t)N * (WKN ? kn_split : K);
  // row strides (elements): rows of length K; K-major weights have rows of length N
  const int64_t lda = K, ldw = WKN ? N : K;
  const char* W0 = static_cast<const char*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride * 2;
  const char* W1 = SWIGLU || (WKN && kn_split < K)
                       ? static_cast<const char*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride * 2
                       : nullptr;
  const char* act = static_cast<const char*>(g.act);

  // ---- per-lane sources, as 32-bit byte offsets from a wave-uniform base (the launcher checks that
  // the activation matrix and one expert's weight matrix stay below 4 GiB): wave w fills activation
  // rows [w * TM/WAVES, +TM/WAVES) and weight-tile rows [w * WROWS/WAVES, +WROWS/WAVES),
  // kRowsPerDma rows per load; lane l covers row l / kChunks of its load and slot l % kChunks,
  // which holds logical chunk slot ^ swz(row)
  const int lrow = lane / C::kChunks;
  const int lslot = lane % C::kChunks;
  uint32_t aoff[C::kADma];
#pragma unroll
  for (int i = 0; i < C::kADma; ++i) {
    const int row = wave * (TM / WAVES) + i * C::kRowsPerDma + lrow;
    const int64_t r = m0 + (row < tile_rows ? row : 0);  // rows past a half tile: a valid row
    int64_t tok = g.row_token ? (int64_t)g.row_token[r] : r;
    if (tok < 0) tok = 0;  // padding row: any valid row (its outputs are never read)
    aoff[i] = (uint32_t)(tok * lda * 2) + ((lslot ^ C::swz(row)) << 4);
  }
  uint32_t woff[C::kWDma];
#pragma unroll
  for (int i = 0; i < C::kWDma; ++i) {
    if constexpr (WKN) {
      // K-major weight tile: BK rows of WROWS features (512 bytes), two rows per 1 KB load; lane
      // l fills row 2 (4 w + i) + l / 32 at slot l % 32, which holds feature chunk slot ^ kn_swz(row)
      const int kr = 2 * (wave * C::kWDma + i) + (lane >> 5);
      int n = n0 + 8 * ((lane & 31) ^ kn_swz(kr));
      if (n + 8 > N) n = N - 8;  // beyond the last feature: any valid chunk (outputs masked)
      woff[i] = (uint32_t)((kr * ldw + n) * 2);
    } else {
      const int r = wave * (WROWS / WAVES) + i * C::kRowsPerDma + lrow;  // row within the weight tile
      int n = n0 + (SWIGLU ? r % (WROWS / 2) : r);
      if (n >= N) n = N - 1;  // beyond the last feature: any valid row (outputs masked)
      woff[i] = (uint32_t)(n * ldw * 2) + ((lslot ^ C::swz(TM + r)) << 4);
    }
  }
  // gate rows come from W0, up rows from W1; the split falls on a wave boundary
  const char* wbase = (SWIGLU && wave * (WROWS / WAVES) >= WROWS / 2) ? W1 : W0;
  const __amdgpu_buffer_rsrc_t act_buf = raw_buffer(act);
  auto issue_stage = [&](int kt) {
    uint16_t* st = lds + (kt % C::kStages) * C::kStageElems;
    const int k0 = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < C::kADma; ++i)
      lds_buf16(act_buf, aoff[i], (uint32_t)k0, st + (wave * (TM / WAVES) + i * C::kRowsPerDma) * BK);
    // K-major weights advance by BK rows per step, switching matrix at kn_split
    const int kr0 = kt * BK;
    const char* wm_base = !WKN ? wbase : (kr0 < kn_split ? W0 : W1);
    const uint32_t wk = !WKN ? (uint32_t)k0 : (uint32_t)((int64_t)(kr0 < kn_split ? kr0 : kr0 - kn_split) * ldw * 2);
    const __amdgpu_buffer_rsrc_t w_buf = raw_buffer(wm_base);
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i)
      lds_buf16(w_buf, woff[i], wk, st + (TM + wave * (WROWS / WAVES) + i * C::kRowsPerDma) * BK);
  };

  f32x16 acc[MB][NBW];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int c = 0; c < NBW; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
  int wrow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (SWIGLU)
      wrow[nb] = nb < NBW / 2 ? wn * (WRW / 2) + nb * 32 : WROWS / 2 + wn * (WRW / 2) + (nb - NBW / 2) * 32;
    else
      wrow[nb] = wn * WRW + nb * 32;
  }
  const int l32 = lane & 31, khalf = lane >> 5;
  const int mrow0 = wm * RW;
  // rows of the tile holding the segment's rows (all of them when no real row counts are given);
  // a wavefront with none idles (the upper half of a half tile, or segment padding)
  const int real_rows = g.seg_rows ? min(tile_rows, max(0, g.seg_rows[seg] - (int)(m0 - g.seg_off[seg]))) : tile_rows;
  const bool active = mrow0 < real_rows;
  constexpr bool kAccInAgprs = MB * NBW * 16 > 128;

  constexpr int kAhead = C::kStages - 1;
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < nk) issue_stage(s);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt have landed once only the later issued stages are in flight
    wait_stages<C::kDmaPerStage, kAhead - 1>(min(kAhead - 1, nk - 1 - kt));
    // a bare barrier: after it all of stage kt is in LDS and every wave is done reading stage
    // kt-1, whose buffer the next loads overwrite (__syncthreads() would add a memory fence
    // that also drains the loads still in flight)
    __builtin_amdgcn_s_barrier();
    const uint16_t* st = lds + (kt % C::kStages) * C::kStageElems;
    // fragments of sub-step kk+1 are read while the MFMAs of sub-step kk run
    auto mma_stage = [&]() {
      bf16x8 xf[2][MB], wf[2][NBW];
      auto load_frags = [&](int buf, int kk) {
        const int c = kk * 2 + khalf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xf[buf][mb] = *reinterpret_cast<const bf16x8*>(st + C::off(mrow0 + mb * 32 + l32, c));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          if constexpr (WKN) {
            // two transposing reads (ds_read_b64_tr_b16) give the lane K rows kb..kb+3 and
            // kb+4..kb+7 of feature wrow + l32: within each 16-lane group, lane s names row
            // kb + s / 4 at features +4 (s % 4)..+3 of the group's 16, and receives its own
            // feature's four rows
            const int kb = kk * 16 + khalf * 8;
            const int col = wrow[nb] + (l32 & 16) + 4 * (lane & 3);
            const int r0 = kb + ((lane & 15) >> 2);
            const uint16_t* wt = st + TM * BK;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + kn_off(r0, col)));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + kn_off(r0 + 4, col)));
            wf[buf][nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            wf[buf][nb] = *reinterpret_cast<const bf16x8*>(st + C::off(TM + wrow[nb] + l32, c));
          }
        }
      };
      load_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < BK / 16) load_frags(cur ^ 1, kk + 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][nb], xf[cur][mb], acc[mb][nb], 0, 0, 0);
        // the next stage's loads go out once this sub-step's MFMAs are queued
        if (kk == 0 && kt + kAhead < nk) issue_stage(kt + kAhead);
      }
    };
    if constexpr (kAccInAgprs) {
      // accumulators beyond 256 VGPRs live in AGPRs; a branch around the MFMAs would make the
      // compiler copy them to VGPRs and back every K-step, so the upper half of a half tile
      // computes on its copied valid row and only skips its stores
      mma_stage();
    } else if (active) {
      mma_stage();
    } else if (kt + kAhead < nk) {
      issue_stage(kt + kAhead);
    }
  }
  if constexpr (EPI == 2) {
    static_assert(NBW == 2 && WN == 4, "one gate and one up block per wavefront, four wavefronts per row");
    __shared__ float red[TM][4];
    store_swiglu_bwd<MB>(acc, g, m0, mrow0, n0 + wn * (WRW / 2), nt, wn, tile_rows, active, l32, khalf, red);
  } else if (active) {
    store_tile<SWIGLU, MB, NBW>(acc, static_cast<uint16_t*>(g.out), m0 + mrow0,
                                n0 + wn * (SWIGLU ? WRW / 2 : WRW), N, l32, khalf);
  }
}

// The streaming kernel's 256 x 256 plain-store and SwiGLU forms (and the K-major input-gradient
// form), persistent: one workgroup per CU walks logical tiles i * G + 32 x + j (slot j of XCD x,
// G workgroups: the same tile-to-XCD assignment as the one-tile grid when G = 256) and issues the
// first K-step of its next tile during the last K-step of the current one, so a tile's pipeline
// fill overlaps its neighbour's MFMAs.  The output goes out through LDS as whole row spans
// (store_tile_staged*), after those loads, and the next tile's first wait counts the stores
// (vmcnt retires in issue order): the stores stay in flight through that tile's first K-step.
// The tile after next is described before the stores, whose table reads would otherwise wait for
// them.  Tiles past the last 256-row tile end the walk (their slots only grow).
template <int EPI, bool WKN>
__global__ void __launch_bounds__(512) grouped_gemm_bf16_persistent_kernel(GemmOperands g, int NT) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2 || EPI == 3;
  static_assert(EPI >= 0 && EPI <= 3, "plain store, SwiGLU, SwiGLU backward or SwiGLU saving its inputs");
  static_assert(!WKN || EPI == 0, "K-major weights: plain store");
  constexpr int BK = 64, TM = 256, WROWS = 256, WAVES = 8, WN = 4, RW = 128, MB = 4, WRW = 64, NBW = 2;
  using C = StreamCfg<BK, WAVES, WROWS, 1, TM>;
  static_assert(C::kStages == 2, "two LDS stages");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int K = g.K, N = g.N, nk = K / BK;
  const int kn_split = WKN ? g.kn_split : K;
  const size_t wstride = (size_t)N * kn_split;
  const int64_t lda = K, ldw = WKN ? N : K;
  const int G = gridDim.x;
  const int max_slots = (int)g.max_tiles;
  int L = persistent_first((int)blockIdx.x, G);

  struct Tile {
    int seg, nt, tile_rows;
    int64_t m0;
  };
  // the 256-row tile of logical index l, in the XCD-aware within-expert order of the streaming
  // kernel; seg < 0 past the last one
  // The per-segment tables, copied to LDS behind the operand stages: describing a tile then
  // takes one global read, the segment of its 256-row slot (seg_of), which the walk issues a
  // tile ahead of use.
  int32_t* s_pair_off = reinterpret_cast<int32_t*>(lds + C::kStages * C::kStageElems);
  int32_t* s_seg_off = s_pair_off + g.n_seg + 1;
  // SwiGLU backward: per-row partials of the gate gradient, one per wavefront of the row
  float(*red)[4] = reinterpret_cast<float(*)[4]>(s_seg_off + g.n_seg + 1);
  for (int i = tid; i <= g.n_seg; i += C::kThreads) {
    s_pair_off[i] = g.pair_off[i];
    s_seg_off[i] = g.seg_off[i];
  }
  __syncthreads();
  // (tile indices, walk included, stay below 2^31: the launcher checks)
  auto seg_of = [&](int l) {
    const int slot = l / NT;
    return slot < max_slots ? g.pair_seg[slot] : -1;
  };
  auto describe = [&](int l, int seg_read) {
    Tile t{-1, 0, 0, 0};
    // wave-uniform table entries, kept in scalar registers
    const int seg = __builtin_amdgcn_readfirstlane(seg_read);
    if (seg < 0) return t;
    const int seg_first = __builtin_amdgcn_readfirstlane(s_pair_off[seg]);
    const int seg_count = __builtin_amdgcn_readfirstlane(s_pair_off[seg + 1]) - seg_first;
    const WalkTile w = walk_tile(l, NT, kGroupM, TM, seg_first, seg_count,
                                 __builtin_amdgcn_readfirstlane(s_seg_off[seg]),
                                 __builtin_amdgcn_readfirstlane(s_seg_off[seg + 1]));
    t.seg = seg;
    t.nt = w.nt;
    t.m0 = w.m0;
    t.tile_rows = w.tile_rows;
    return t;
  };
  // per-lane load sources of the tile being loaded (as in the streaming kernel)
  const int lrow = lane / C::kChunks, lslot = lane % C::kChunks;
  const char* act = static_cast<const char*>(g.act);
  uint32_t aoff[C::kADma], woff[C::kWDma];
  const char* W0 = nullptr;
  const char* W1 = nullptr;
  auto prepare = [&](const Tile& t) {
    const int n0 = t.nt * (SWIGLU ? WROWS / 2 : WROWS);
    const bool shared = t.seg >= g.n_routed;
    const int e = shared ? t.seg - g.n_routed : t.seg;
    W0 = static_cast<const char*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride * 2;
    W1 = SWIGLU || (WKN && kn_split < K)
             ? static_cast<const char*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride * 2
             : W0;
    // rows past a half tile: a valid row; the token gathers are issued together (one branch,
    // one round trip)
    int tok[C::kADma];
#pragma unroll
    for (int i = 0; i < C::kADma; ++i) {
      const int row = wave * (TM / WAVES) + i * C::kRowsPerDma + lrow;
      tok[i] = (int)t.m0 + (row < t.tile_rows ? row : 0);
    }
    if (g.row_token) {
#pragma unroll
      for (int i = 0; i < C::kADma; ++i) tok[i] = g.row_token[tok[i]];
    }
#pragma unroll
    for (int i = 0; i < C::kADma; ++i) {
      const int row = wave * (TM / WAVES) + i * C::kRowsPerDma + lrow;
      const int64_t r = tok[i] < 0 ? 0 : tok[i];  // padding row: any valid row (its outputs are never read)
      aoff[i] = (uint32_t)(r * lda * 2) + ((lslot ^ C::swz(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      if constexpr (WKN) {
        const int kr = 2 * (wave * C::kWDma + i) + (lane >> 5);
        int n = n0 + 8 * ((lane & 31) ^ kn_swz(kr));
        if (n + 8 > N) n = N - 8;
        woff[i] = (uint32_t)((kr * ldw + n) * 2);
      } else {
        const int r = wave * (WROWS / WAVES) + i * C::kRowsPerDma + lrow;
        int n = n0 + (SWIGLU ? r % (WROWS / 2) : r);
        if (n >= N) n = N - 1;
        woff[i] = (uint32_t)(n * ldw * 2) + ((lslot ^ C::swz(TM + r)) << 4);
      }
    }
  };
  int issued = 0, consumed = 0;
  const __amdgpu_buffer_rsrc_t act_buf = raw_buffer(act);
  auto issue = [&](int kt) {
    uint16_t* st = lds + (issued % C::kStages) * C::kStageElems;
    const int k0 = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < C::kADma; ++i) {
      uint16_t* dst = st + (wave * (TM / WAVES) + i * C::kRowsPerDma) * BK;
      if (MOE_BUFFER_LOADS)
        lds_buf16(act_buf, aoff[i], (uint32_t)k0, dst);
      else
        lds_dma16(act + k0 + aoff[i], dst);
    }
    const int kr0 = kt * BK;
    // gate rows come from W0, up rows from W1 (the split falls on a wave boundary); K-major
    // weights advance by BK rows per step, switching matrix at kn_split
    const char* wm_base = WKN ? (kr0 < kn_split ? W0 : W1)
                              : ((SWIGLU && wave * (WROWS / WAVES) >= WROWS / 2) ? W1 : W0);
    const uint32_t wk = WKN ? (uint32_t)((int64_t)(kr0 < kn_split ? kr0 : kr0 - kn_split) * ldw * 2) : (uint32_t)k0;
    const __amdgpu_buffer_rsrc_t w_buf = raw_buffer(wm_base);
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      uint16_t* dst = st + (TM + wave * (WROWS / WAVES) + i * C::kRowsPerDma) * BK;
      if (MOE_BUFFER_LOADS)
        lds_buf16(w_buf, woff[i], wk, dst);
      else
        lds_dma16(wm_base + wk + woff[i], dst);
    }
    ++issued;
  };

  int wrow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (SWIGLU)
      wrow[nb] = nb < NBW / 2 ? wn * (WRW / 2) + nb * 32 : WROWS / 2 + wn * (WRW / 2) + (nb - NBW / 2) * 32;
    else
      wrow[nb] = wn * WRW + nb * 32;
  }
  const int l32 = lane & 31, khalf = lane >> 5;
  const int mrow0 = wm * RW;

  Tile cur = describe(L, seg_of(L));
  if (cur.seg < 0) return;
  prepare(cur);
  issue(0);
  Tile nxt = describe(L + G, seg_of(L + G));
  // stores the previous tile issued after this tile's first K-step loads: vmcnt retires in
  // issue order, so a count of that many means the K-step has landed while the stores may still
  // be in flight
  int stores_behind = 0;
  while (true) {
    // the segment of the tile after next, read here so that its latency passes under this tile's
    // first K-step (it is issued after the previous tile's stores, which only makes the counted
    // wait below stricter)
    const int seg2 = nxt.seg >= 0 ? seg_of(L + 2 * G) : -1;
    const bool active = mrow0 < cur.tile_rows;   // false only for the upper half of a half tile
    // the loads of the step after kt: this tile's next one, or the next tile's first
    auto issue_next = [&](int kt) {
      if (kt + 1 < nk) {
        issue(kt + 1);
      } else if (nxt.seg >= 0) {
        prepare(nxt);
        issue(0);
      }
    };
    f32x16 acc[MB][NBW];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int c = 0; c < NBW; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
    // the first K-step's loads
    wait_loads_behind_stores(stores_behind);
    for (int kt = 0; kt < nk; ++kt) {
      // a bare barrier: stage `consumed` has landed and the other buffer is no longer read
      __builtin_amdgcn_s_barrier();
      if (active) {
        const uint16_t* st = lds + (consumed % C::kStages) * C::kStageElems;
        bf16x8 xf[2][MB], wf[2][NBW];
        auto load_frags = [&](int buf, int kk) {
          const int c = kk * 2 + khalf;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            xf[buf][mb] = *reinterpret_cast<const bf16x8*>(st + C::off(mrow0 + mb * 32 + l32, c));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            if constexpr (WKN) {
              const int kb = kk * 16 + khalf * 8;
              const int col = wrow[nb] + (l32 & 16) + 4 * (lane & 3);
              const int r0 = kb + ((lane & 15) >> 2);
              const uint16_t* wt = st + TM * BK;
              const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + kn_off(r0, col)));
              const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + kn_off(r0 + 4, col)));
              wf[buf][nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
              wf[buf][nb] = *reinterpret_cast<const bf16x8*>(st + C::off(TM + wrow[nb] + l32, c));
            }
          }
        };
        load_frags(0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          __builtin_amdgcn_iglp_opt(1);   // the compiler interleaves LDS reads with the MFMAs
          const int cb = kk & 1;
          if (kk + 1 < BK / 16) load_frags(cb ^ 1, kk + 1);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][nb], xf[cb][mb], acc[mb][nb], 0, 0, 0);
          // the next step's loads go out once this sub-step's MFMAs are queued
          if (kk == 0) issue_next(kt);
        }
      } else {
        issue_next(kt);
      }
      ++consumed;
      // the next K-step's loads
      if (kt + 1 < nk) wait_vmcnt<0>();
    }
    // the tile after next, described from LDS before this tile's stores go out
    const Tile nxt2 = describe(L + 2 * G, seg2);
    // the tile's output through the stage no load is filling (stage `issued` mod 2, the one the
    // last K-step read)
    lds_barrier();   // every wavefront is done reading the stage
    uint16_t* stg = lds + (issued % C::kStages) * C::kStageElems;
    if constexpr (EPI == 2)
      stores_behind = store_tile_staged_swiglu_bwd(acc, stg, g, cur.m0, cur.nt * (WROWS / 2), cur.nt, cur.tile_rows,
                                                   wave, wm, wn, lane, red);
    else if constexpr (SWIGLU) {
      stores_behind = store_tile_staged_swiglu(acc, stg, static_cast<uint16_t*>(g.out), cur.m0, cur.nt * (WROWS / 2),
                                               N, cur.tile_rows, wave, wm, wn, lane);
      if constexpr (EPI == 3)   // and the SwiGLU inputs a, b to out2 ([rows, 2N])
        stores_behind += store_tile_staged_ab(acc, stg, static_cast<uint16_t*>(g.out2), cur.m0, cur.nt * (WROWS / 2),
                                              N, cur.tile_rows, wave, wm, wn, lane);
    }
    else
      stores_behind = store_tile_staged(acc, stg, static_cast<uint16_t*>(g.out), cur.m0, cur.nt * WROWS, N,
                                        cur.tile_rows, wave, wm, wn, lane);
    if (nxt.seg < 0) break;
    cur = nxt;
    nxt = nxt2;
    L += G;
  }
}

#ifndef MOE_PERSISTENT_GEMM
#define MOE_PERSISTENT_GEMM 1
#endif

template <int EPI, bool WKN>
hipError_t launch_persistent(const GemmOperands& g, hipStream_t st) {
  using SC = StreamCfg<64, 8, 256, 1, 256>;
  // operand stages, then the pair_off and seg_off tables (n_seg + 1 entries each), then (SwiGLU
  // backward) the per-row gate-gradient partials
  constexpr size_t red_bytes = EPI == 2 ? 256 * 4 * sizeof(float) : 0;
  const size_t stage_bytes = SC::kStages * SC::kStageElems * sizeof(uint16_t);
  const size_t max_lds = stage_bytes + 2 * (size_t)(kMaxRouted + kMaxShared + 1) * sizeof(int32_t) + red_bytes;
  static_assert(SC::kStages * SC::kStageElems * 2 + 2 * (kMaxRouted + kMaxShared + 1) * 4 + 4096 <= kLdsBytes, "LDS");
  if (g.n_seg < 1 || g.n_seg > kMaxRouted + kMaxShared) return hipErrorInvalidValue;
  const size_t lds_bytes = stage_bytes + 2 * (size_t)(g.n_seg + 1) * sizeof(int32_t) + red_bytes;
  auto kern = &grouped_gemm_bf16_persistent_kernel<EPI, WKN>;
  int n_cu = 0;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)max_lds);
  if (err != hipSuccess || (err = device_cu_count(&n_cu)) != hipSuccess) return err;
  const int NT = (int)ceil_div(g.N, EPI == 0 ? 256 : 128);
  if (g.max_pairs * NT == 0) return hipSuccess;
  if (EPI == 2 && g.N % 128 != 0) return hipErrorInvalidValue;   // dg_part holds N / 128 tiles per row
  // one workgroup per CU (the LDS stages allow no more), a multiple of the 8 x 32 tile block
  const int64_t span = kXcds * SC::kXcdChunk;
  const int64_t grid = std::max<int64_t>(span, (int64_t)n_cu / span * span);
  // the walk's tile indices (up to two grid strides past the last tile) and the table slots are int
  if (g.max_tiles * NT + 2 * grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds_bytes, st, g, NT);
  return hipGetLastError();
}

// Weight gradient, persistent: out_e[m, n] = sum over the columns k of segment e of A[m, k] B[n, k]
// (transposed activations, row strides lda and ldw).  With a few hundred rows per expert a
// 256 x 256 output tile has only a handful of K-steps, so a one-tile workgroup spends much of its
// time filling its pipeline and draining its stores.  Each workgroup instead walks a fixed
// sequence of tiles (logical tile i * G + 32 x + j for the workgroup in slot j of XCD x, G
// workgroups, so an XCD keeps a run of one expert's tiles: blocks of 4 M-tiles x all N-tiles)
// and issues the first K-step of its next tile during the last K-step of the current one; the
// output goes out through LDS as whole row spans after those loads and stays in flight through
// the next tile's first K-step, as in the persistent kernel above.  The segment table is copied
// to LDS, so describing a tile takes no global load.  The stage ring runs on across tiles (the
// issued and consumed stage counts pick the LDS buffer).
__global__ void __launch_bounds__(512) grouped_wgrad_bf16_kernel(GemmOperands g, int NT, int64_t n_tiles) {
  constexpr int BK = 64, TM = 256, WROWS = 256, WAVES = 8, WN = 4, RW = 128, MB = 4, WRW = 64, NBW = 2;
  using C = StreamCfg<BK, WAVES, WROWS, 1, TM>;
  static_assert(C::kStages == 2, "two LDS stages");
  static_assert(C::kStageElems == (TM / 2) * WROWS, "a stage holds half an output tile");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int N = g.N;
  const int64_t lda = g.lda, ldw = g.ldw;
  const int MT = (g.wg_m + TM - 1) / TM;
  const int64_t per = (int64_t)MT * NT;
  const int64_t G = gridDim.x;
  int64_t L = persistent_first((int)blockIdx.x, (int)G);
  if (L >= n_tiles) return;

  // The segment table, copied to LDS behind the operand stages: a tile's description then
  // needs no global load, whose wait would also drain the previous tile's stores.
  int32_t* seg_off = reinterpret_cast<int32_t*>(lds + C::kStages * C::kStageElems);
  for (int i = tid; i <= g.n_seg; i += C::kThreads) seg_off[i] = g.seg_off[i];
  __syncthreads();

  struct Tile {
    int seg, nt, tile_rows, nk;
    int64_t m0, k_base;
  };
  // an expert's tiles in blocks of kGM M-tiles x all N-tiles, M fastest: the 32 workgroups of an
  // XCD then hold about kGM M-tiles x 32 / kGM N-tiles and share both operands' slices in L2
  constexpr int kGM = 4;
  auto describe = [&](int64_t l) {
    Tile t;
    t.seg = (int)(l / per);
    const int rem = (int)(l - (int64_t)t.seg * per);
    const int blk = rem / (kGM * NT);
    const int gm = min(kGM, MT - blk * kGM);
    const int r2 = rem - blk * kGM * NT;
    t.nt = r2 / gm;
    t.m0 = (int64_t)(blk * kGM + r2 % gm) * TM;
    t.tile_rows = min(TM, g.wg_m - (int)t.m0);
    const int k0 = __builtin_amdgcn_readfirstlane(seg_off[t.seg]);
    const int k1 = __builtin_amdgcn_readfirstlane(seg_off[t.seg + 1]);
    t.k_base = k0;
    t.nk = (k1 - k0) / BK;
    return t;
  };
  // per-lane load sources of the tile being loaded, as in the streaming kernel
  const int lrow = lane / C::kChunks, lslot = lane % C::kChunks;
  uint32_t aoff[C::kADma], woff[C::kWDma];
  uint32_t k_bytes = 0;   // the tile's first K column (segment start) in bytes: the loads' scalar offset
  auto prepare = [&](const Tile& t) {
    const int n0 = t.nt * WROWS;
#pragma unroll
    for (int i = 0; i < C::kADma; ++i) {
      const int row = wave * (TM / WAVES) + i * C::kRowsPerDma + lrow;
      aoff[i] = (uint32_t)((t.m0 + (row < t.tile_rows ? row : 0)) * lda * 2) + ((lslot ^ C::swz(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i) {
      const int r = wave * (WROWS / WAVES) + i * C::kRowsPerDma + lrow;
      woff[i] = (uint32_t)((int64_t)min(n0 + r, N - 1) * ldw * 2) + ((lslot ^ C::swz(TM + r)) << 4);
    }
    k_bytes = (uint32_t)(t.k_base * 2);
  };
  // buffer-form loads: wave-uniform bases, the lane's 32-bit offset, the K offset in a scalar (the
  // launcher keeps both operand matrices below 4 GiB)
  const __amdgpu_buffer_rsrc_t act_buf = raw_buffer(g.act);
  const __amdgpu_buffer_rsrc_t w_buf = raw_buffer(g.w_routed[0]);
  int issued = 0, consumed = 0;
  auto issue = [&](int kt) {
    uint16_t* st = lds + (issued % C::kStages) * C::kStageElems;
    const uint32_t k0 = k_bytes + (uint32_t)(kt * BK * 2);
#pragma unroll
    for (int i = 0; i < C::kADma; ++i)
      lds_buf16(act_buf, aoff[i], k0, st + (wave * (TM / WAVES) + i * C::kRowsPerDma) * BK);
#pragma unroll
    for (int i = 0; i < C::kWDma; ++i)
      lds_buf16(w_buf, woff[i], k0, st + (TM + wave * (WROWS / WAVES) + i * C::kRowsPerDma) * BK);
    ++issued;
  };

  int wrow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wrow[nb] = wn * WRW + nb * 32;
  const int l32 = lane & 31, khalf = lane >> 5;
  const int mrow0 = wm * RW;

  Tile cur = describe(L);
  prepare(cur);
  if (cur.nk > 0) issue(0);
  // stores the previous tile issued after this tile's first K-step loads: vmcnt retires in
  // issue order, so a count of that many means the K-step has landed while the stores may still
  // be in flight
  int stores_behind = 0;
  while (true) {
    const int64_t Ln = L + G;
    const bool has_next = Ln < n_tiles;
    const Tile nxt = has_next ? describe(Ln) : cur;
    // the next tile's first K-step, issued once this tile's last one is being computed
    auto prefetch_next = [&]() {
      if (has_next && nxt.nk > 0) {
        prepare(nxt);
        issue(0);
      }
    };
    const bool active = mrow0 < cur.tile_rows;   // false only for the upper half of a half tile
    f32x16 acc[MB][NBW];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int c = 0; c < NBW; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
    // the first K-step's loads
    wait_loads_behind_stores(stores_behind);
    for (int kt = 0; kt < cur.nk; ++kt) {
      // a bare barrier: stage `consumed` has landed and the other buffer is no longer read
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < cur.nk)
        issue(kt + 1);
      else
        prefetch_next();
      if (active) {
        const uint16_t* st = lds + (consumed % C::kStages) * C::kStageElems;
        bf16x8 xf[2][MB], wf[2][NBW];
        auto load_frags = [&](int buf, int kk) {
          const int c = kk * 2 + khalf;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            xf[buf][mb] = *reinterpret_cast<const bf16x8*>(st + C::off(mrow0 + mb * 32 + l32, c));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
            wf[buf][nb] = *reinterpret_cast<const bf16x8*>(st + C::off(TM + wrow[nb] + l32, c));
        };
        load_frags(0, 0);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          __builtin_amdgcn_iglp_opt(1);   // the compiler interleaves LDS reads with the MFMAs
          const int cb = kk & 1;
          if (kk + 1 < BK / 16) load_frags(cb ^ 1, kk + 1);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][nb], xf[cb][mb], acc[mb][nb], 0, 0, 0);
        }
      }
      ++consumed;
      // the next K-step's loads (issued before this step's MFMAs)
      if (kt + 1 < cur.nk) wait_vmcnt<0>();
    }
    // a tile without K-steps (an empty segment) prefetched nothing for the next one; its loads
    // go to the stage the previous tile's rows were read back from, once every wavefront is
    // done with them
    if (cur.nk == 0) {
      lds_barrier();
      prefetch_next();
    }
    // segment cur.seg's matrix of the routed or shared output (an empty segment writes zeros),
    // staged through the stage no load is filling: stage `issued` mod 2, the one this tile's last
    // K-step read
    {
      const bool shared = cur.seg >= g.n_routed;
      const int e = shared ? cur.seg - g.n_routed : cur.seg;
      uint16_t* out = static_cast<uint16_t*>(shared ? g.out2 : g.out) + (int64_t)e * g.wg_m * N;
      lds_barrier();   // every wavefront is done reading the stage
      stores_behind = store_tile_staged(acc, lds + (issued % C::kStages) * C::kStageElems, out, cur.m0,
                                        cur.nt * WROWS, N, cur.tile_rows, wave, wm, wn, lane);
    }
    if (!has_next) break;
    cur = nxt;
    L = Ln;
  }
}

hipError_t launch_wgrad_bf16(const GemmOperands& g, hipStream_t st) {
  using C = StreamCfg<64, 8, 256, 1, 256>;
  if (g.wg_m % 128 != 0 || g.N % 8 != 0) return hipErrorInvalidValue;
  // 32-bit byte offsets address the transposed activation matrices
  if ((int64_t)g.wg_m * g.lda * 2 >= (int64_t(1) << 32) || (int64_t)g.N * g.ldw * 2 >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  // operand stages, then the segment table (n_seg + 1 offsets)
  const size_t stage_bytes = C::kStages * C::kStageElems * sizeof(uint16_t);
  const size_t max_lds = stage_bytes + (size_t)(kMaxRouted + kMaxShared + 1) * sizeof(int32_t);
  if (max_lds > (size_t)kLdsBytes) return hipErrorInvalidValue;
  const size_t lds_bytes = stage_bytes + (size_t)(g.n_seg + 1) * sizeof(int32_t);
  int n_cu = 0;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&grouped_wgrad_bf16_kernel), (int)max_lds);
  if (err != hipSuccess || (err = device_cu_count(&n_cu)) != hipSuccess) return err;
  const int NT = (int)ceil_div(g.N, 256);
  const int64_t tiles = (int64_t)g.n_seg * ceil_div(g.wg_m, 256) * NT;
  if (tiles == 0) return hipSuccess;
  // one workgroup per CU (the LDS stages allow no more), a multiple of the XCD count
  const int64_t grid = std::max<int64_t>(kXcds, (int64_t)n_cu / kXcds * kXcds);
  hipLaunchKernelGGL(grouped_wgrad_bf16_kernel, dim3((unsigned)grid), dim3(512), lds_bytes, st, g, NT, tiles);
  return hipGetLastError();
}

template <int EPI, int SBK, int SW, int SR, int SG, int SM, int STM, bool WKN = false>
hipError_t launch_stream(const GemmOperands& g, hipStream_t st) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2;
  using SC = StreamCfg<SBK, SW, SR, SG, STM>;
  const int NT = (int)ceil_div(g.N, SWIGLU ? SR / 2 : SR);
  const size_t lds_bytes = SC::kStages * SC::kStageElems * sizeof(uint16_t);
  auto kern = &grouped_gemm_bf16_stream_kernel<EPI, SBK, SW, SR, SG, SM, STM, WKN>;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds_bytes);
  if (err != hipSuccess) return err;
  const int64_t tiles = (STM == kTileM ? g.max_tiles : g.max_pairs) * NT;
  const int64_t span = kXcds * SC::kXcdChunk;
  const int64_t grid = ceil_div(tiles, span) * span;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(SC::kThreads), lds_bytes, st, g, NT);
  return hipGetLastError();
}

#ifndef MOE_SMALL_SEGMENT_TILE
#define MOE_SMALL_SEGMENT_TILE 1
#endif

template <int EPI>
hipError_t launch_bf16(const GemmOperands& g, hipStream_t st) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2;
  constexpr int SBK = MOE_STREAM_BK;
  // the streaming kernel addresses its sources with 32-bit byte offsets
  const bool offsets_fit = g.act_rows * g.K * 2 < (int64_t(1) << 32) && (int64_t)g.N * g.K * 2 < (int64_t(1) << 32);
  if (g.K % SBK == 0 && offsets_fit) {
    if constexpr (EPI == 2) {
      // 256 x 256 tiles (the SwiGLU-backward epilogue assumes four wavefronts of one gate and
      // one up block per row)
      if (MOE_PERSISTENT_GEMM) return launch_persistent<EPI, false>(g, st);
      return launch_stream<EPI, 64, 8, 256, 1, 2, 256>(g, st);
    } else {
      // segments of a few rows (decode-like batches, expected routed rows per expert below one
      // M-tile): 128-row tiles x 512 weight rows put 80% of every stage's loads on weights
      if (MOE_SMALL_SEGMENT_TILE && g.small_segments) return launch_stream<EPI, 64, 8, 512, 1, 2, 128>(g, st);
      if (MOE_PERSISTENT_GEMM && SBK == 64 && MOE_STREAM_WAVES == 8 && MOE_STREAM_WROWS == 256 &&
          MOE_STREAM_WGS == 1 && MOE_STREAM_WM == 2 && MOE_STREAM_TM == 256)
        return launch_persistent<EPI, false>(g, st);
      return launch_stream<EPI, SBK, MOE_STREAM_WAVES, MOE_STREAM_WROWS, MOE_STREAM_WGS, MOE_STREAM_WM,
                           MOE_STREAM_TM>(g, st);
    }
  }
  if (EPI == 2) return hipErrorInvalidValue;   // the backward mode exists in the streaming kernel only
  const size_t lds_bytes = 2 * kStageElems * sizeof(uint16_t);
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&grouped_gemm_bf16_kernel<SWIGLU>), (int)lds_bytes);
  if (err != hipSuccess) return err;
  dim3 grid((unsigned)g.max_tiles, (unsigned)ceil_div(g.N, SWIGLU ? kWRows / 2 : kWRows));
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<SWIGLU>, grid, dim3(kThreads), lds_bytes, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_swiglu(const GemmOperands& g, hipStream_t st) { return launch_bf16<1>(g, st); }
// SwiGLU that also writes its inputs [a b] of every row to g.out2 ([rows, 2N]); always the
// persistent 256 x 256 form
hipError_t launch_gemm_bf16_swiglu_save(const GemmOperands& g, hipStream_t st) {
  if (g.K % 64 != 0 || g.N % 8 != 0 || !g.out2) return hipErrorInvalidValue;
  if (g.act_rows * g.K * 2 >= (int64_t(1) << 32) || (int64_t)g.N * g.K * 2 >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  return launch_persistent<3, false>(g, st);
}
hipError_t launch_gemm_bf16_down(const GemmOperands& g, hipStream_t st) { return launch_bf16<0>(g, st); }
hipError_t launch_gemm_bf16_swiglu_bwd(const GemmOperands& g, hipStream_t st) { return launch_bf16<2>(g, st); }
hipError_t launch_gemm_bf16_wgrad(const GemmOperands& g, hipStream_t st) { return launch_wgrad_bf16(g, st); }

// Input-gradient product on K-major weights (as stored), no transposed copy: out[r, n] =
// sum_k act[r, k] W[k, n] with W = rows [0, kn_split) of w_*[0] then the rest of w_*[1]
hipError_t launch_gemm_bf16_dgrad(const GemmOperands& g, hipStream_t st) {
  if (g.K % 64 != 0 || g.N % 128 != 0 || g.kn_split % 64 != 0 || g.kn_split <= 0 || g.kn_split > g.K)
    return hipErrorInvalidValue;
  // 32-bit byte offsets: the activation matrix and one stacked weight matrix (K rows of N)
  if (g.act_rows * g.K * 2 >= (int64_t(1) << 32) || (int64_t)g.N * g.K * 2 >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  if (MOE_PERSISTENT_GEMM) return launch_persistent<0, true>(g, st);
  return launch_stream<0, 64, 8, 256, 1, 2, 256, true>(g, st);
}

}  // namespace moe
