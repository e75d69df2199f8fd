// Grouped FP8 (E4M3FN) expert GEMMs with 1x128 activation and 128x128 weight block scales.
//
// The expert FFNs of the h'_t equation (方法 §2, "DeepSeek-V3 技術報告",
// xyznot.com/zh-tw/paper/2412.19437) in the FP8 scheme of the same page's 核心概念
// list: E4M3 operands, one fp32 scale per 1x128 activation tile and per 128x128 weight
// block, accumulation in fp32.  The page's design for its hardware moves the partial
// sums of every 128-element K block out of the tensor cores into fp32 registers and
// scales them there.  On gfx950 one v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales)
// contracts a whole 128-element scale block of a 16x16 output block, so every MFMA result
// is that block's raw partial sum: it is folded into the fp32 result at once with the
// factor act_scale[row][kb] * weight_scale[feature block][kb], and no partial accumulator
// outlives its MFMA.
//
//   gate/up:  H[r, n] = SiLU(x_r . Wg[e][n]) * (x_r . Wu[e][n]), then H is quantised per
//             1x128 tile along I (scale = amax / 448, round to nearest even, saturate);
//             the 128 features of a tile are exactly the workgroup's N-tile, so the row
//             amax is a reduction across the four wavefronts that share the row
//   down:     Y[r, n] = H[r] . Wd[e][n] in bf16
//
// The layer backward runs its three GEMM kinds on the same operand path (the page lists the
// input-gradient and weight-gradient products as FP8 GEMMs too):
//   plain:    the down form above with other operands: dH = dout W_down (weights transposed
//             to [I, d] blocks) and dX = [dA dB] [W_gate; W_up] (transposed to [d, 2I])
//   SwiGLU backward: the gate/up products recomputed, then from dH (before the gate, bf16)
//             and the row gate: H, dA = g dH b SiLU'(a), dB = g dH SiLU(a) (bf16) and per row
//             and 128-feature tile the partial sum of dH * H
//   weight gradient (grouped_wgrad_fp8_kernel, persistent): out_e[m, n] = sum over the rows k
//             of segment e of A[m, k] B[n, k] with both operands transposed activations
//             quantised per 1x128 run of rows, so the second operand also has one scale per
//             row and K block, and K runs over the segment's rows only
//
// Tiling: 512 threads (8 wavefronts, two per SIMD), 256 rows (two M-tiles of one segment;
// a segment with an odd M-tile count ends in a half tile whose upper wavefronts idle) x
// 256 weight rows (gate/up: 128 gate + the matching 128 up features; down: 256 output
// features).  Wavefront (wm, wn) of the 2 x 4 grid owns 128 rows x 64 weight rows as 8 x 4
// blocks of 16 x 16.  One K-step is one 128-byte scale block of every row, staged in LDS
// with its 16-byte chunks reordered and XOR-swizzled (conflict-free reads) by direct global->LDS loads
// one K-step ahead, in the XCD-aware tile order of the bf16 kernels.  The weight-gradient form
// tiles each segment's M x N output in 256 x 256 blocks.
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kTM = 2 * kTileM;     // activation rows per workgroup
constexpr int kBK = 128;            // K elements (bytes) per step = one scale block
constexpr int kWRows = 256;
constexpr int kStages = 2;
constexpr int kDataBytes = (kTM + kWRows) * kBK;      // 64 KB of operands per stage
constexpr int kScaleBytes = 2048;                      // 256 row scales + 2 weight-block scales, padded
constexpr int kStageBytes = kDataBytes + kScaleBytes;   // per stage of the ring, operands and scales
constexpr int kRowsPerDma = 8;                         // 128-byte rows one wave-wide 1 KB load fills
constexpr int kADma = kTM / kRowsPerDma / kWaves;      // 4
constexpr int kWDma = kWRows / kRowsPerDma / kWaves;   // 4
constexpr int kXcds = 8;
constexpr int kXcdChunk = 32;
constexpr int kGroupM = 4;          // 256-row tiles per block of the within-expert order
constexpr int kE8M0One = 127;       // E8M0 encoding of 2^0
constexpr int kMB = 8;              // 16-row token blocks per wavefront
constexpr int kNB = 4;              // 16-row weight blocks per wavefront

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// A staged operand row holds one 128-byte K block as eight 16-byte chunks.  A fragment read
// gives lane (l16, kq) chunks 2 kq and 2 kq + 1 of row l16, and one 16x16x128 read instruction
// therefore touches chunks {0, 2, 4, 6} (or {1, 3, 5, 7}) of 16 rows.  Stored in K order that
// pattern costs the LDS two passes per instruction (measured: 8 LDS cycles per 1 KB read against 4
// for contiguous or 32-row patterns, under any XOR swizzle of the rows), so chunk 2 kq + h is kept
// at slot 4 h + kq instead, and each read takes 64 contiguous bytes of every row; the slots of a
// row are then XOR-swizzled by row / 2 (conflict-free 16-lane reads).  The lanes' registers hold
// the same bytes as with the plain order.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int kslot(int q) { return ((q & 1) << 2) | (q >> 1); }     // slot of K chunk q
__device__ __forceinline__ int kchunk(int s) { return ((s & 3) << 1) | (s >> 2); }    // K chunk of slot s

// K-major weight tile (input-gradient products): 128 K rows of 256 feature bytes; the 16-byte
// feature chunk c of row r sits at slot c ^ kn8_swz(r), so that the 32 rows one transposing read
// touches (8 j + 0..7 in each K quarter) fall on each bank group twice
__device__ __forceinline__ int kn8_swz(int r) { return (r & 7) | (((r >> 5) & 1) << 3); }
__device__ __forceinline__ int kn8_off(int r, int col) { return r * 256 + (((col >> 4) ^ kn8_swz(r)) << 4) + (col & 15); }
// global byte offset, within its row, of the chunk that LDS slot s of row r holds
__device__ __forceinline__ int src_chunk(int r, int s) { return kchunk(s ^ swz(r)) << 4; }

// LDS ring of the forward and input-gradient kernels: kStages operand stages of kDataBytes,
// then kStages scale areas of kScaleBytes.  An operand stage then spans exactly 64 KB, so each
// fragment read below is a per-lane base plus a constant within the LDS instructions' 16-bit
// offset, and a K-step adds its stage's start to four bases (measured: the SwiGLU GEMM's integer
// VALU per K-step 34 -> 6 instructions, 2-4% faster at T=8192).
__device__ __forceinline__ int stage_off(int s) { return (s % kStages) * kDataBytes; }
__device__ __forceinline__ int scale_off(int s) { return kStages * kDataBytes + (s % kStages) * kScaleBytes; }

// Byte offsets, within a stage, of the two 16-byte halves (K chunks 2 kq and 2 kq + 1) of the
// lane's fragment of token block 0 (rows mrow0 + l16) and weight block 0 (weight-tile rows
// wrow0 + l16).  mrow0, wrow0 and kTM are multiples of 16, so every row 16 b + l16 has the
// swizzle of l16 and block b lies 16 b rows further on.
struct FragBase {
  uint32_t x0, x1, w0, w1;
};
__device__ __forceinline__ FragBase frag_base(int mrow0, int wrow0, int l16, int kq) {
  const int s = swz(l16);
  const uint32_t c0 = (uint32_t)((kslot(2 * kq) ^ s) << 4), c1 = (uint32_t)((kslot(2 * kq + 1) ^ s) << 4);
  const uint32_t xr = (uint32_t)(mrow0 + l16) * kBK, wr = (uint32_t)(kTM + wrow0 + l16) * kBK;
  return {xr + c0, xr + c1, wr + c0, wr + c1};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS traffic of this wavefront done (lgkmcnt 0; vmcnt 63 and expcnt 7 are no wait), then a bare
// barrier that leaves global loads, LDS DMA and stores in flight; the empty asm statements keep
// the compiler from moving memory accesses across it
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// 32 bytes of a staged row, K chunks 2 kq and 2 kq + 1: the halves at st + o0 + off and
// st + o1 + off (o0, o1 from frag_base)
__device__ __forceinline__ i32x8 frag_at(const uint8_t* st, uint32_t o0, uint32_t o1, int off) {
  u32x4 a = *reinterpret_cast<const u32x4*>(st + o0 + off);
  u32x4 b = *reinterpret_cast<const u32x4*>(st + o1 + off);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// A 256 x 256 bf16 output tile held in the 16 x 16 MFMA layout (wavefront (wm, wn): rows
// wm * 128 + 16 mb + (lane mod 16), columns wn * 64 + 16 nb + 4 (lane / 16) + 0..3) written to
// out (row stride N, rows m0 + [0, tile_rows), columns n0 + [0, 256) below N) through an LDS stage
// of at least 64 KB that no load is filling, as whole 512-byte row spans: pass p stages
// accumulator blocks 4p..4p+3 of every wavefront (tile rows wm * 128 + 64 p + [0, 64) as staged
// rows wm * 64 + [0, 64)), 16-byte chunk c of a staged row at slot c ^ (row mod 32).  The LDS
// accesses are typed so that the compiler does not make them wait for memory traffic in flight.
// Every store has an active lane (N is a multiple of 128), so the returned count of this
// wavefront's stores is exact.
__device__ __forceinline__ int store_tile_staged16(const f32x4 (&acc)[kMB][kNB], uint8_t* stage, uint16_t* out,
                                                   int64_t m0, int n0, int N, int tile_rows, int wave, int wm,
                                                   int wn, int lane) {
  constexpr int kRounds = 8;   // row-span stores per wavefront per staged half
  asm volatile("" : "+v"(lane));   // per-lane offsets computed here, not hoisted across the MFMAs
  uint16_t* stg = reinterpret_cast<uint16_t*>(stage);
  const bool active = wm * (kTM / 2) < tile_rows;
  const int rounds = tile_rows > kTM / 2 ? kRounds : kRounds / 2;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p > 0) lds_barrier();   // the first pass has been read back
    if (active) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int r = wm * 64 + h * 16 + (lane & 15);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = wn * 8 + nb * 2 + ((lane >> 4) >> 1);
          const f32x4& a = acc[4 * p + h][nb];
          const uint64_t lo = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
          const uint64_t hi = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
          *reinterpret_cast<uint64_t*>(stg + r * 256 + ((c ^ (r & 31)) << 3) + ((lane >> 4) & 1) * 4) = lo | (hi << 32);
        }
      }
    }
    lds_barrier();
    const int c = lane & 31;
    const int f = n0 + c * 8;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      if (i < rounds) {
        const int r = (i * kWaves + wave) * 2 + (lane >> 5);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * 256 + ((c ^ (r & 31)) << 3));
        const int64_t row = m0 + (r >> 6) * 128 + p * 64 + (r & 63);
        if (f < N) *reinterpret_cast<u32x4*>(out + row * N + f) = v;
      }
    }
  }
  return 2 * rounds;
}

// EPI: 0 plain bf16 store, 1 SwiGLU with H quantised, 2 SwiGLU backward.
// WKN (with EPI 0): the weight codes are read K-major as stored ([K rows][N features] per
// expert, rows [0, kn_split) of w_*[0] and the rest of w_*[1]; block scales [K/128][N/128]),
// through transposing LDS reads, for the input-gradient products of the backward
template <int EPI, bool WKN = false>
__global__ void __launch_bounds__(kThreads) grouped_gemm_fp8_kernel(GemmOperands g, int NT) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2 || EPI == 3;
  static_assert(!WKN || EPI == 0, "K-major weights: plain store");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float row_red[kTM][4];   // per-row reductions across the four wavefronts of a row
  // ---- logical tile (same XCD-aware order as the bf16 streaming kernels, over 256-row tiles)
  const int64_t L = xcd_logical(blockIdx.x, kXcdChunk);
  const int64_t slot = L / NT;
  if (slot >= g.max_tiles) return;
  const int seg = g.pair_seg[slot];
  if (seg < 0) return;
  const int seg_first = g.pair_off[seg];
  const WalkTile wt = walk_tile(L, NT, kGroupM, kTM, seg_first, g.pair_off[seg + 1] - seg_first, g.seg_off[seg],
                                g.seg_off[seg + 1]);
  const int nt = wt.nt;
  const int64_t m0 = wt.m0;
  const int tile_rows = wt.tile_rows;  // 256, or 128 for a half tile
  const int nk = g.K / kBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int K = g.K, N = g.N, KB = K / kBK;
  const int n0 = nt * (SWIGLU ? kWRows / 2 : kWRows);
  const bool shared = seg >= g.n_routed;
  const int e = shared ? seg - g.n_routed : seg;
  const int kn_split = WKN ? g.kn_split : K;   // K rows of the first stacked matrix
  const size_t wstride = (size_t)N * kn_split;
  const size_t sstride = (size_t)(N / kBK) * (kn_split / kBK);  // scales per expert matrix
  const bool two = SWIGLU || (WKN && kn_split < K);
  const uint8_t* W0 = static_cast<const uint8_t*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * wstride;
  const uint8_t* W1 =
      two ? static_cast<const uint8_t*>(shared ? g.w_shared[1] : g.w_routed[1]) + e * wstride : nullptr;
  const float* S0 = (shared ? g.s_shared[0] : g.s_routed[0]) + e * sstride;
  const float* S1 = two ? (shared ? g.s_shared[1] : g.s_routed[1]) + e * sstride : nullptr;
  const uint8_t* act = static_cast<const uint8_t*>(g.act);

  // ---- direct-load sources as 32-bit byte offsets (the launcher checks the sizes): wave w fills
  // activation rows [32w, 32w+32) and weight-tile rows [32w, 32w+32), 8 rows of 128 bytes per
  // load; lane l covers row l >> 3 of its load and slot l & 7, which holds K chunk src_chunk(row, slot)
  const int lrow = lane >> 3, lslot = lane & 7;
  uint32_t aoff[kADma];
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int row = wave * (kTM / kWaves) + i * kRowsPerDma + lrow;
    const int64_t r = m0 + (row < tile_rows ? row : 0);  // rows past a half tile: a valid row
    int64_t tok = g.row_token ? (int64_t)g.row_token[r] : r;
    if (tok < 0) tok = 0;  // padding row: any valid row (outputs never read)
    aoff[i] = (uint32_t)(tok * K) + src_chunk(row, lslot);
  }
  uint32_t woff[kWDma];
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    if constexpr (WKN) {
      // K-major weight tile: 128 K rows of 256 feature bytes, four rows per 1 KB load; lane l
      // fills row 4 (4 w + i) + l / 16 at slot l % 16, which holds feature chunk slot ^ kn8_swz(row)
      const int kr = 4 * (wave * kWDma + i) + (lane >> 4);
      int n = n0 + 16 * ((lane & 15) ^ kn8_swz(kr));
      if (n + 16 > N) n = N - 16;  // beyond the last feature: any valid chunk (outputs masked)
      woff[i] = (uint32_t)(kr * N + n);
    } else {
      const int r = wave * (kWRows / kWaves) + i * kRowsPerDma + lrow;  // 0..255 within the weight tile
      int n = n0 + (SWIGLU ? (r & (kWRows / 2 - 1)) : r);
      if (n >= N) n = N - 1;  // beyond the last feature: any valid row (outputs masked)
      woff[i] = (uint32_t)n * (uint32_t)K + src_chunk(kTM + r, lslot);
    }
  }
  // gate rows (waves 0-3) come from W0, up rows (waves 4-7) from W1
  const uint8_t* wbase = (SWIGLU && wave >= kWaves / 2) ? W1 : W0;
  // ---- scale sources: lanes 0..31 of wave w load the activation scales of rows [32w, 32w+32)
  // into the stage's scale area; wave 7's lanes 32 and 33 load the scales of the tile's two
  // 128-row weight blocks, landing right after the 256 row scales.  The loads are buffer loads
  // (counted by vmcnt only, so that the waits for the fragment reads can stay partial) at a
  // per-lane byte offset from the scale array each lane reads: act_scale, S0, or S1 (the up
  // projection's scales, lane 33 of the SwiGLU forms; K-major weights past kn_split)
  uint32_t s_off = 0;
  if (lane < 32) {
    const int row = wave * 32 + lane;
    const int64_t r = m0 + (row < tile_rows ? row : 0);
    int64_t tok = g.row_token ? (int64_t)g.row_token[r] : r;
    if (tok < 0) tok = 0;
    s_off = (uint32_t)(tok * KB) * 4;
  } else if (wave == kWaves - 1 && lane < 34) {
    const int nb = lane - 32;
    if (SWIGLU) {
      s_off = (uint32_t)((n0 / kBK) * KB) * 4;  // gate block (S0), then the matching up block (S1)
    } else if (WKN) {
      s_off = (uint32_t)(min(n0 + nb * kBK, N - 1) / kBK) * 4;  // row 0 of the [K/128][N/128] scales
    } else {
      s_off = (uint32_t)((min(n0 + nb * kBK, N - 1) / kBK) * KB) * 4;
    }
  }
  const __amdgpu_buffer_rsrc_t as_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g.act_scale), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t s0_buf = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(S0), (short)0, -1,
                                                                         0x00020000);
  const __amdgpu_buffer_rsrc_t s1_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(S1 ? S1 : S0), (short)0, -1, 0x00020000);
  // operand loads in buffer form (address = base + 32-bit lane offset + the K-step's offset in a
  // scalar; the launcher keeps both matrices below 4 GiB): measured faster than the global form
  const __amdgpu_buffer_rsrc_t act_buf = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(act), (short)0, -1,
                                                                          0x00020000);
  auto issue_stage = [&](int kt) {
    uint8_t* st = lds + stage_off(kt);
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < kADma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_buf,
                                               (lds_void_t*)(st + (wave * (kTM / kWaves) + i * kRowsPerDma) * kBK),
                                               16, aoff[i], (uint32_t)k0, 0, 0);
    // K-major weights advance by 128 rows per step, switching matrix at kn_split
    const uint8_t* wm_base = !WKN ? wbase : (k0 < kn_split ? W0 : W1);
    const uint32_t wk = !WKN ? (uint32_t)k0 : (uint32_t)((int64_t)(k0 < kn_split ? k0 : k0 - kn_split) * N);
    const __amdgpu_buffer_rsrc_t w_buf =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wm_base), (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_buf, (lds_void_t*)(st + (kTM + wave * (kWRows / kWaves) + i * kRowsPerDma) * kBK), 16, woff[i], wk, 0,
          0);
    // scales: one dword per lane at the lane's offset plus the K block's (K-major weight scales
    // step by a row of N/128 blocks per K block)
    lds_void_t* sdst = (lds_void_t*)(lds + scale_off(kt) + wave * 128);
    if (lane < 32) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(as_buf, sdst, 4, s_off, (uint32_t)kt * 4, 0, 0);
    } else if (wave == kWaves - 1 && lane < 34) {
      if constexpr (WKN) {
        const int split = kn_split / kBK;
        if (kt < split)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(s0_buf, sdst, 4, s_off, (uint32_t)(kt * (N / kBK)) * 4, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(s1_buf, sdst, 4, s_off, (uint32_t)((kt - split) * (N / kBK)) * 4,
                                                   0, 0);
      } else if (SWIGLU && lane == 33) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s1_buf, sdst, 4, s_off, (uint32_t)kt * 4, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s0_buf, sdst, 4, s_off, (uint32_t)kt * 4, 0, 0);
      }
    }
  };

  // weight rows of the wave's four 16-row blocks, and the 128-row scale block each falls in
  int wrow[kNB], wblk[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (SWIGLU) {
      wrow[nb] = (nb < 2 ? 0 : kWRows / 2) + wn * 32 + (nb & 1) * 16;  // gate blocks, then the matching up blocks
      wblk[nb] = nb < 2 ? 0 : 1;
    } else {
      wrow[nb] = wn * 64 + nb * 16;
      wblk[nb] = wrow[nb] / kBK;
    }
  }
  const int l16 = lane & 15, kq = lane >> 4;  // token of the 16x16 block; K quarter and feature group
  const int mrow0 = wm * (kTM / 2);
  const bool active = mrow0 < tile_rows;      // false only for the upper half of a half tile
  const int wrow0 = wrow[0];                  // wrow[nb] - wrow0 is a constant
  const FragBase fb = frag_base(mrow0, wrow0, l16, kq);

  f32x4 acc[kMB][kNB];
#pragma unroll
  for (int a = 0; a < kMB; ++a)
#pragma unroll
    for (int c = 0; c < kNB; ++c) acc[a][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

  issue_stage(0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<0>();
    // a bare barrier: every wave's loads of stage kt have landed and stage kt-1 is no longer read
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < nk) issue_stage(kt + 1);
    if (active) {
      const uint8_t* st = lds + stage_off(kt);
      const float* sc = reinterpret_cast<const float*>(lds + scale_off(kt));
      i32x8 wf[kNB];
      float sw[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        if constexpr (WKN) {
          // four transposing reads (ds_read_b64_tr_b8) give the lane K rows 32 kq + 8 j + (0..7)
          // of feature wrow + l16: within each 16-lane group, lane s names row 8 j + s / 2 at
          // features +8 (s % 2)..+7 of the group's 16, and receives its own feature's eight rows
          const uint8_t* wt = st + kTM * kBK;
          const int col = wrow[nb] + 8 * (lane & 1);
          i32x8 f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 32 * kq + 8 * j + ((lane & 15) >> 1);
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(wt + kn8_off(r, col)));
            f[2 * j] = v[0];
            f[2 * j + 1] = v[1];
          }
          wf[nb] = f;
        } else {
          wf[nb] = frag_at(st, fb.w0, fb.w1, (wrow[nb] - wrow0) * kBK);
        }
        sw[nb] = sc[kTM + wblk[nb]];
      }
      // token fragments one block ahead, so that each block's LDS reads are in flight while the
      // previous block's MFMAs run
      const float* sa_row = sc + mrow0 + l16;
      i32x8 xf_next = frag_at(st, fb.x0, fb.x1, 0);
      float sa_next = sa_row[0];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const i32x8 xf = xf_next;
        const float sa = sa_next;
        if (mb + 1 < kMB) {
          xf_next = frag_at(st, fb.x0, fb.x1, (mb + 1) * 16 * kBK);
          sa_next = sa_row[(mb + 1) * 16];
        }
        // plain-store form: keeps the compiler from sinking those reads below the MFMAs (which it
        // otherwise does, exposing each block's LDS latency again; down GEMM 2.12 -> 2.02 ms at
        // T=8192).  The SwiGLU forms measured slower with it (gate/up 3.64 -> 3.81 ms).
        if constexpr (EPI == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[nb], xf, zero, 0, 0, 0, kE8M0One, 0,
                                                                              kE8M0One);
          const float f = sa * sw[nb];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(part[v], f, acc[mb][nb][v]);
        }
      }
    }
  }

  // ---- epilogue.  Lane holds, for token row mrow0 + 16 mb + l16, features 4 kq + (0..3) of
  // each 16-row weight block
  if constexpr (EPI == 2) {
    // gate block nb and up block nb + 2 hold the same features
    const uint16_t* dhp = static_cast<const uint16_t*>(g.dh);
    uint16_t* dab = static_cast<uint16_t*>(g.out);
    uint16_t* hout = static_cast<uint16_t*>(g.out2);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int rl = mrow0 + mb * 16 + l16;
      const int64_t r = m0 + rl;
      float part = 0.0f;
      if (active) {
        const float rg = g.row_gate[r];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int f = n0 + wn * 32 + nb * 16 + kq * 4;
          const uint2 dq = *reinterpret_cast<const uint2*>(dhp + r * N + f);
          const float dhu[4] = {__uint_as_float(dq.x << 16), __uint_as_float(dq.x & 0xFFFF0000u),
                                __uint_as_float(dq.y << 16), __uint_as_float(dq.y & 0xFFFF0000u)};
          uint16_t da[4], db[4], hh[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float a = acc[mb][nb][v], bu = acc[mb][nb + 2][v];
            const float sg = 1.0f / (1.0f + __expf(-a));
            const float h = a * sg * bu;
            const float dh = rg * dhu[v];
            da[v] = f32_to_bf16(dh * bu * sg * (1.0f + a * (1.0f - sg)));
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
      // lanes of one row: l16 + 16 kq
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (kq == 0) row_red[rl][wn] = part;
    }
    __syncthreads();
    for (int row = tid; row < tile_rows; row += kThreads)
      g.dg_part[(m0 + row) * (N / kBK) + nt] = row_red[row][0] + row_red[row][1] + row_red[row][2] + row_red[row][3];
  } else if constexpr (EPI == 1 || EPI == 3) {
    uint8_t* out = static_cast<uint8_t*>(g.out);
    const int IB = N / kBK;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      if constexpr (EPI == 3) {
        // the SwiGLU inputs a (gate) and b (up) of the row, bf16, to out2 ([rows, 2N]: a then b)
        if (active) {
          uint16_t* ab = static_cast<uint16_t*>(g.out2) + (m0 + mrow0 + mb * 16 + l16) * 2 * N;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int f = n0 + wn * 32 + nb * 16 + kq * 4;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4& v = acc[mb][nb + 2 * h];
              *reinterpret_cast<uint2*>(ab + h * N + f) =
                  make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
            }
          }
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[mb][nb][v] = silu(acc[mb][nb][v]) * acc[mb][nb + 2][v];  // h, in place of the gate value
          amax = fmaxf(amax, fabsf(acc[mb][nb][v]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      if (kq == 0) row_red[mrow0 + mb * 16 + l16][wn] = amax;
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const int r = mrow0 + mb * 16 + l16;
        const float a = fmaxf(fmaxf(row_red[r][0], row_red[r][1]), fmaxf(row_red[r][2], row_red[r][3]));
        const float scale = a > 0.0f ? __fdiv_rn(a, 448.0f) : 1.0f;
        uint8_t* orow = out + (m0 + r) * N;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int f = n0 + wn * 32 + nb * 16 + kq * 4;
          const uint32_t w = e4m3x4_from_f32(__fdiv_rn(acc[mb][nb][0], scale), __fdiv_rn(acc[mb][nb][1], scale),
                                             __fdiv_rn(acc[mb][nb][2], scale), __fdiv_rn(acc[mb][nb][3], scale));
          *reinterpret_cast<uint32_t*>(orow + f) = w;
        }
        if (wn == 0 && kq == 0) g.out_scale[(m0 + r) * IB + n0 / kBK] = scale;
      }
    }
  } else {
    // whole row spans through stage nk mod 2: the last K-step read the other stage, and every
    // wavefront passed that step's barrier after its reads of this one (nk = 1: never used)
    store_tile_staged16(acc, lds + stage_off(nk), static_cast<uint16_t*>(g.out), m0, n0, N, tile_rows, wave, wm, wn,
                        lane);
  }
}

// The forward down GEMM (plain bf16 store), persistent: one workgroup
// per CU walks the 256-row tiles the one-tile grid gives workgroups b, b + G, b + 2G, ... (G
// workgroups, a multiple of 256: the same tile-to-XCD assignment), so that the CU's MFMAs do not
// idle while a tile's first K-step loads or its output drains.  The next tile's first K-step's
// loads go out during the current tile's last K-step; the current tile's output then leaves,
// through LDS, while they are in flight.  The stores stay in flight through the next tile's first
// K-step: that wait counts them (vmcnt retires in issue order).  The rows are the activation
// matrix's own (H in the permuted layout: no gather).  The per-segment tables are copied to LDS
// behind the operand stages, so describing a tile takes one global read, the segment of its
// 256-row slot, issued a tile ahead.  The K-step body is the one-tile kernel's (kept as a copy:
// moved into a shared inline function it compiled to a different register allocation that
// spilled in the plain-store form).  The SwiGLU form stays one tile per workgroup: persistent,
// its K-loop scheduled with less overlap of the fold and the MFMAs (measured at T=8192: gate/up
// 3.36 -> 3.71 ms, down 1.82 -> 1.72 ms).
__global__ void __launch_bounds__(kThreads) grouped_gemm_fp8_persistent_kernel(GemmOperands g, int NT) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int K = g.K, N = g.N, KB = K / kBK, nk = K / kBK;
  const int G = gridDim.x;
  const int max_slots = (int)g.max_tiles;
  int32_t* s_pair_off = reinterpret_cast<int32_t*>(lds + kStages * kStageBytes);
  int32_t* s_seg_off = s_pair_off + g.n_seg + 1;
  for (int i = tid; i <= g.n_seg; i += kThreads) {
    s_pair_off[i] = g.pair_off[i];
    s_seg_off[i] = g.seg_off[i];
  }
  __syncthreads();

  struct Tile {
    int seg, nt, tile_rows;
    int64_t m0;
  };
  // (tile indices, walk included, stay below 2^31: the launcher checks)
  auto seg_of = [&](int l) {
    const int slot = l / NT;
    return slot < max_slots ? g.pair_seg[slot] : -1;
  };
  auto describe = [&](int l, int seg_read) {
    Tile t{-1, 0, 0, 0};
    const int seg = __builtin_amdgcn_readfirstlane(seg_read);
    if (seg < 0) return t;
    const int seg_first = __builtin_amdgcn_readfirstlane(s_pair_off[seg]);
    const int seg_count = __builtin_amdgcn_readfirstlane(s_pair_off[seg + 1]) - seg_first;
    const int row_start = __builtin_amdgcn_readfirstlane(s_seg_off[seg]);
    const WalkTile w = walk_tile(l, NT, kGroupM, kTM, seg_first, seg_count, row_start,
                                 __builtin_amdgcn_readfirstlane(s_seg_off[seg + 1]));
    t.seg = seg;
    t.nt = w.nt;
    t.m0 = w.m0;
    t.tile_rows = w.tile_rows;
    return t;
  };

  // ---- per-lane load sources of the tile being loaded (as in grouped_gemm_fp8_kernel): 32-bit
  // byte offsets of the lane's four operand rows and its scale row
  const int lrow = lane >> 3, lslot = lane & 7;
  // the row of each of the lane's operand rows, then of its scale row (lanes 0..31; the other
  // lanes' copy is unused)
  auto tile_row = [&](const Tile& t, int i) {
    const int row = i < kADma ? wave * (kTM / kWaves) + i * kRowsPerDma + lrow : wave * 32 + (lane & 31);
    return (int)t.m0 + (row < t.tile_rows ? row : 0);  // rows past a half tile: a valid row
  };
  uint32_t aoff[kADma], woff[kWDma], s_off = 0;
  const uint8_t* wbase = nullptr;
  const float* S0 = nullptr;
  auto prepare = [&](const Tile& t) {
    const int n0 = t.nt * kWRows;
    const bool shared = t.seg >= g.n_routed;
    const int e = shared ? t.seg - g.n_routed : t.seg;
    wbase = static_cast<const uint8_t*>(shared ? g.w_shared[0] : g.w_routed[0]) + e * ((size_t)N * K);
    S0 = (shared ? g.s_shared[0] : g.s_routed[0]) + e * ((size_t)(N / kBK) * KB);
#pragma unroll
    for (int i = 0; i < kADma; ++i) {
      const int row = wave * (kTM / kWaves) + i * kRowsPerDma + lrow;
      aoff[i] = (uint32_t)((int64_t)tile_row(t, i) * K) + src_chunk(row, lslot);
    }
#pragma unroll
    for (int i = 0; i < kWDma; ++i) {
      const int r = wave * (kWRows / kWaves) + i * kRowsPerDma + lrow;  // 0..255 within the weight tile
      const int n = min(n0 + r, N - 1);  // beyond the last feature: any valid row (outputs masked)
      woff[i] = (uint32_t)n * (uint32_t)K + src_chunk(kTM + r, lslot);
    }
    // scale sources: lanes 0..31 the activation scales of rows [32w, 32w+32), wave 7's lanes 32
    // and 33 the scales of the tile's two 128-row weight blocks (byte offsets into act_scale, S0)
    if (lane < 32) {
      s_off = (uint32_t)((int64_t)tile_row(t, kADma) * KB) * 4;
    } else if (wave == kWaves - 1 && lane < 34) {
      s_off = (uint32_t)((min(n0 + (lane - 32) * kBK, N - 1) / kBK) * KB) * 4;
    }
  };
  const __amdgpu_buffer_rsrc_t act_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.act), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t as_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g.act_scale), (short)0, -1, 0x00020000);
  // K-step kt of the prepared tile into LDS stage `stage`
  auto issue = [&](int kt, int stage) {
    uint8_t* st = lds + stage_off(stage);
    const uint32_t k0 = (uint32_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < kADma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_buf,
                                               (lds_void_t*)(st + (wave * (kTM / kWaves) + i * kRowsPerDma) * kBK),
                                               16, aoff[i], k0, 0, 0);
    const __amdgpu_buffer_rsrc_t w_buf =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wbase), (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_buf, (lds_void_t*)(st + (kTM + wave * (kWRows / kWaves) + i * kRowsPerDma) * kBK), 16, woff[i], k0, 0,
          0);
    lds_void_t* sdst = (lds_void_t*)(lds + scale_off(stage) + wave * 128);
    if (lane < 32) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(as_buf, sdst, 4, s_off, (uint32_t)kt * 4, 0, 0);
    } else if (wave == kWaves - 1 && lane < 34) {
      const __amdgpu_buffer_rsrc_t s0_buf =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(S0), (short)0, -1, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s0_buf, sdst, 4, s_off, (uint32_t)kt * 4, 0, 0);
    }
  };

  // weight rows of the wave's four 16-row blocks, and the 128-row scale block each falls in
  int wrow[kNB], wblk[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    wrow[nb] = wn * 64 + nb * 16;
    wblk[nb] = wrow[nb] / kBK;
  }
  const int l16 = lane & 15, kq = lane >> 4;
  const int mrow0 = wm * (kTM / 2);
  const FragBase fb = frag_base(mrow0, wrow[0], l16, kq);
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

  int L = persistent_first((int)blockIdx.x, G);
  Tile cur = describe(L, seg_of(L));
  if (cur.seg < 0) return;
  prepare(cur);
  issue(0, 0);
  int step = 0;           // K-steps consumed so far (the stage ring runs on across tiles)
  int stores_behind = 0;  // this wavefront's output stores issued after the current tile's first loads
  while (true) {
    const int Ln = L + G;
    const int seg_next = seg_of(Ln);
    const bool active = mrow0 < cur.tile_rows;   // false only for the upper half of a half tile
    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int a = 0; a < kMB; ++a)
#pragma unroll
      for (int c = 0; c < kNB; ++c) acc[a][c] = zero;
    // this tile's first K-step has landed: all but the previous tile's output stores, which were
    // issued after its loads
    if (stores_behind == 16)
      wait_vmcnt<16>();
    else if (stores_behind == 8)
      wait_vmcnt<8>();
    else
      wait_vmcnt<0>();
    auto compute = [&]() {
      if (active) {
        const uint8_t* st = lds + stage_off(step);
        const float* sc = reinterpret_cast<const float*>(lds + scale_off(step));
        i32x8 wf[kNB];
        float sw[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          wf[nb] = frag_at(st, fb.w0, fb.w1, nb * 16 * kBK);
          sw[nb] = sc[kTM + wblk[nb]];
        }
        // token fragments one block ahead, so that each block's LDS reads are in flight while the
        // previous block's MFMAs run
        const float* sa_row = sc + mrow0 + l16;
        i32x8 xf_next = frag_at(st, fb.x0, fb.x1, 0);
        float sa_next = sa_row[0];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const i32x8 xf = xf_next;
          const float sa = sa_next;
          if (mb + 1 < kMB) {
            xf_next = frag_at(st, fb.x0, fb.x1, (mb + 1) * 16 * kBK);
            sa_next = sa_row[(mb + 1) * 16];
          }
          __builtin_amdgcn_sched_barrier(0);   // as in the one-tile plain-store form
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[nb], xf, zero, 0, 0, 0, kE8M0One,
                                                                                0, kE8M0One);
            const float f = sa * sw[nb];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(part[v], f, acc[mb][nb][v]);
          }
        }
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) {
      if (kt > 0) wait_vmcnt<0>();
      // a bare barrier: every wave's loads of this stage have landed and the other stage is no
      // longer read
      __builtin_amdgcn_s_barrier();
      issue(kt + 1, step + 1);
      compute();
      ++step;
    }
    // the last K-step: the next tile's first K-step goes out before it is computed
    if (nk > 1) wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    {
      const Tile nxt = describe(Ln, seg_next);
      if (nxt.seg >= 0) {
        prepare(nxt);
        issue(0, step + 1);
      }
    }
    compute();
    ++step;

    // ---- epilogue of the current tile, while the next tile's first K-step loads are in flight.
    // Lane holds, for token row mrow0 + 16 mb + l16, features 4 kq + (0..3) of each 16-row
    // weight block
    // whole row spans through the stage the last K-step read (the next tile's first K-step fills
    // the other one), once every wavefront is done reading it
    lds_barrier();
    stores_behind = store_tile_staged16(acc, lds + stage_off(step - 1), static_cast<uint16_t*>(g.out), cur.m0,
                                        cur.nt * kWRows, N, cur.tile_rows, wave, wm, wn, lane);
    const Tile nxt = describe(Ln, seg_next);
    if (nxt.seg < 0) break;
    cur = nxt;
    L = Ln;
  }
}

// Weight gradient, persistent: out_e[m, n] = sum over the rows k of segment e of A[m, k] B[n, k]
// (both operands transposed activations, one scale per row and 128-row K block).  An expert's
// segment holds a few hundred rows, so a 256 x 256 output tile has only a few K-steps and a
// one-tile workgroup spends most of its time filling its pipeline and draining its stores.
// Here each workgroup walks a fixed sequence of tiles (logical tile i * G + 32 x + j for the
// workgroup in slot j of XCD x, G workgroups, so an XCD keeps a run of one expert's tiles: blocks
// of 4 M-tiles x all N-tiles) and the loads of a tile's first K-step go out during the last K-step
// of the tile before it.  The bf16 output goes out through LDS as whole 512-byte row spans (the
// 16 x 16 MFMA layout gives 16 rows x 32 bytes per store instruction), after those loads, and
// stays in flight through the next tile's first K-step: that wait counts the stores (vmcnt
// retires in issue order).  The segment table is copied to LDS, so describing a tile takes no
// global load, whose wait would drain the stores.  The stage ring runs on across tiles: the
// consumed and issued stage counts pick the LDS buffer.
__global__ void __launch_bounds__(kThreads) grouped_wgrad_fp8_kernel(GemmOperands g, int NT, int64_t n_tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  static_assert(kDataBytes == 128 * 512, "a stage's operand bytes hold 128 rows of bf16 output");
  constexpr int kRounds = 8;   // row-span stores per wavefront per staged half
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int N = g.N;
  const int64_t lda = g.lda, ldw = g.ldw;
  const int MT = (g.wg_m + kTM - 1) / kTM;
  const int per = MT * NT;
  const int G = gridDim.x;
  int L = persistent_first((int)blockIdx.x, G);
  if (L >= n_tiles) return;

  int32_t* seg_off = reinterpret_cast<int32_t*>(lds + kStages * kStageBytes);
  for (int i = tid; i <= g.n_seg; i += kThreads) seg_off[i] = g.seg_off[i];
  __syncthreads();

  struct Tile {
    int seg, nt, tile_rows, nk, m0, k_base;
  };
  // an expert's tiles in blocks of kGM M-tiles x all N-tiles, M fastest (the launcher keeps the
  // tile indices, walk included, below 2^31; row and column indices fit 32 bits)
  constexpr int kGM = 4;
  auto describe = [&](int l) {
    Tile t;
    t.seg = l / per;
    const int rem = l - t.seg * per;
    const int blk = rem / (kGM * NT);
    const int gm = min(kGM, MT - blk * kGM);
    const int r2 = rem - blk * kGM * NT;
    t.nt = r2 / gm;
    t.m0 = (blk * kGM + r2 % gm) * kTM;
    t.tile_rows = min(kTM, g.wg_m - t.m0);
    const int k0 = __builtin_amdgcn_readfirstlane(seg_off[t.seg]);
    const int k1 = __builtin_amdgcn_readfirstlane(seg_off[t.seg + 1]);
    t.k_base = k0;
    t.nk = (k1 - k0) / kBK;
    return t;
  };
  // per-lane load sources of the tile being loaded (as in grouped_gemm_fp8_kernel): 32-bit byte
  // offsets; waves 0-3 load the scales of activation rows [64w, 64w + 64) into scale slots
  // [64w, 64w + 64), waves 4-7 those of weight rows [64(w - 4), 64(w - 4) + 64) into slots
  // 256 + the row (one scale array per wave, so that the array is wave-uniform)
  uint32_t aoff[kADma], woff[kWDma], s_off = 0;
  int k_base = 0;   // the tile's first K column (segment start), the loads' scalar offset base
  // (32-bit offset arithmetic: the launcher checks wg_m * lda and N * ldw against 2^32)
  const uint32_t lda32 = (uint32_t)lda, ldw32 = (uint32_t)ldw;
  auto prepare = [&](const Tile& t) {
    // the per-lane parts are derived here from an opaque lane index rather than kept live
    // across the MFMAs, where registers are short
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lrow = ln >> 3, lslot = ln & 7;
    const int n0 = t.nt * kWRows;
#pragma unroll
    for (int i = 0; i < kADma; ++i) {
      const int row = wave * (kTM / kWaves) + i * kRowsPerDma + lrow;
      aoff[i] = (uint32_t)(t.m0 + (row < t.tile_rows ? row : 0)) * lda32 + src_chunk(row, lslot);
    }
#pragma unroll
    for (int i = 0; i < kWDma; ++i) {
      const int r = wave * (kWRows / kWaves) + i * kRowsPerDma + lrow;
      woff[i] = (uint32_t)min(n0 + r, N - 1) * ldw32 + src_chunk(kTM + r, lslot);
    }
    k_base = t.k_base;
    // scale byte offsets (before the K block): activation rows from act_scale, weight rows from
    // s_routed[0]
    const int srow = (wave & 3) * 64 + ln;
    if (wave < 4)
      s_off = (uint32_t)(t.m0 + (srow < t.tile_rows ? srow : 0)) * (lda32 / kBK) * 4;
    else
      s_off = (uint32_t)min(n0 + srow, N - 1) * (ldw32 / kBK) * 4;
  };
  // operand and scale loads in buffer form: a wave-uniform base, the lane's 32-bit offset and the
  // K-step's offset in a scalar
  const __amdgpu_buffer_rsrc_t act_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.act), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t w_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.w_routed[0]), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t as_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g.act_scale), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t ws_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g.s_routed[0]), (short)0, -1, 0x00020000);
  int issued = 0, consumed = 0;
  auto issue = [&](int kt) {
    uint8_t* st = lds + stage_off(issued);
    const uint32_t k0 = (uint32_t)(k_base + kt * kBK);
#pragma unroll
    for (int i = 0; i < kADma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(act_buf,
                                               (lds_void_t*)(st + (wave * (kTM / kWaves) + i * kRowsPerDma) * kBK),
                                               16, aoff[i], k0, 0, 0);
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_buf, (lds_void_t*)(st + (kTM + wave * (kWRows / kWaves) + i * kRowsPerDma) * kBK), 16, woff[i], k0, 0,
          0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wave < 4 ? as_buf : ws_buf,
                                             (lds_void_t*)(lds + scale_off(issued) + wave * 256), 4, s_off,
                                             (uint32_t)(k_base / kBK + kt) * 4, 0, 0);
    ++issued;
  };

  const int l16 = lane & 15, kq = lane >> 4;
  const int mrow0 = wm * (kTM / 2);
  const FragBase fb = frag_base(mrow0, wn * 64, l16, kq);
  // scale slots of activation row mrow0 + 16 mb + l16 and of the lane's four weight rows
  // wn * 64 + 16 nb + 4 kq + (0..3)
  const int sa_base = mrow0 + l16;
  const int sw_base = kTM + wn * 64 + 4 * kq;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

  Tile cur = describe(L);
  prepare(cur);
  if (cur.nk > 0) issue(0);
  // stores the previous tile issued after this tile's first K-step loads
  int stores_behind = 0;
  while (true) {
    const int Ln = L + G;
    const bool has_next = Ln < n_tiles;
    // the next tile's first K-step, issued once this tile's last one is being computed (a
    // description is two LDS reads, so it is not carried across the K-loop, where scalar
    // registers are short)
    auto prefetch_next = [&]() {
      if (!has_next) return;
      const Tile t = describe(Ln);
      if (t.nk > 0) {
        prepare(t);
        issue(0);
      }
    };
    const bool active = mrow0 < cur.tile_rows;   // false only for the upper half of a half tile
    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int a = 0; a < kMB; ++a)
#pragma unroll
      for (int c = 0; c < kNB; ++c) acc[a][c] = zero;
    // the first K-step's loads
    if (stores_behind == 2 * kRounds)
      wait_vmcnt<2 * kRounds>();
    else if (stores_behind == kRounds)
      wait_vmcnt<kRounds>();
    else
      wait_vmcnt<0>();
    for (int kt = 0; kt < cur.nk; ++kt) {
      // a bare barrier: stage `consumed` has landed and the other buffer is no longer read
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < cur.nk)
        issue(kt + 1);
      else
        prefetch_next();
      if (active) {
        const uint8_t* st = lds + stage_off(consumed);
        const float* sc = reinterpret_cast<const float*>(lds + scale_off(consumed));
        i32x8 wf[kNB];
        f32x4 swr[kNB];   // scales of the lane's four weight rows (one group of 32)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          wf[nb] = frag_at(st, fb.w0, fb.w1, nb * 16 * kBK);
          swr[nb] = *reinterpret_cast<const f32x4*>(sc + sw_base + 16 * nb);
        }
        // token fragments one block ahead (as in grouped_gemm_fp8_kernel)
        i32x8 xf_next = frag_at(st, fb.x0, fb.x1, 0);
        float sa_next = sc[sa_base];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const i32x8 xf = xf_next;
          const float sa = sa_next;
          if (mb + 1 < kMB) {
            xf_next = frag_at(st, fb.x0, fb.x1, (mb + 1) * 16 * kBK);
            sa_next = sc[sa_base + (mb + 1) * 16];
          }
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[nb], xf, zero, 0, 0, 0, kE8M0One,
                                                                                0, kE8M0One);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(part[v], sa * swr[nb][v], acc[mb][nb][v]);
          }
        }
      }
      ++consumed;
      // the next K-step's loads
      if (kt + 1 < cur.nk) wait_vmcnt<0>();
    }
    // a tile without K-steps (an empty segment) prefetched nothing for the next one; its loads
    // go to the stage the previous tile's rows were read back from, once every wavefront is
    // done with them
    if (cur.nk == 0) {
      lds_barrier();
      prefetch_next();
    }
    // ---- epilogue: segment cur.seg's matrix of the routed or shared output (an empty segment
    // writes zeros) as staged row spans, through the stage no load is filling (stage `issued`
    // mod 2, the one the last K-step read)
    {
      const bool shared = cur.seg >= g.n_routed;
      const int e = shared ? cur.seg - g.n_routed : cur.seg;
      uint16_t* out = static_cast<uint16_t*>(shared ? g.out2 : g.out) + (int64_t)e * g.wg_m * N;
      lds_barrier();   // every wavefront is done reading the stage
      stores_behind = store_tile_staged16(acc, lds + stage_off(issued), out, cur.m0, cur.nt * kWRows, N,
                                          cur.tile_rows, wave, wm, wn, lane);
    }
    if (!has_next) break;
    cur = describe(Ln);
    L = Ln;
  }
}

hipError_t launch_wgrad_fp8(const GemmOperands& g, hipStream_t st) {
  if (g.K % kBK != 0 || g.N % kBK != 0 || g.wg_m % kBK != 0 || g.lda % kBK != 0 || g.ldw % kBK != 0)
    return hipErrorInvalidValue;
  if ((int64_t)g.wg_m * g.lda >= (int64_t(1) << 32) || (int64_t)g.N * g.ldw >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  // operand stages, then the segment table (n_seg + 1 offsets)
  const size_t stage_bytes = (size_t)kStages * kStageBytes;
  const size_t max_lds = stage_bytes + (size_t)(kMaxRouted + kMaxShared + 1) * sizeof(int32_t);
  if (max_lds > 163840) return hipErrorInvalidValue;
  const size_t lds_bytes = stage_bytes + (size_t)(g.n_seg + 1) * sizeof(int32_t);
  int n_cu = 0;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&grouped_wgrad_fp8_kernel), (int)max_lds);
  if (err != hipSuccess || (err = device_cu_count(&n_cu)) != hipSuccess) return err;
  const int NT = (int)ceil_div(g.N, kWRows);
  const int64_t tiles = (int64_t)g.n_seg * ceil_div(g.wg_m, kTM) * NT;
  if (tiles == 0) return hipSuccess;
  // one workgroup per CU (the LDS stages allow no more), a multiple of the XCD count
  const int64_t grid = std::max<int64_t>(kXcds, (int64_t)n_cu / kXcds * kXcds);
  // tile indices, walk included, are int
  if (tiles + grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_wgrad_fp8_kernel, dim3((unsigned)grid), dim3(kThreads), lds_bytes, st, g, NT, tiles);
  return hipGetLastError();
}

template <int EPI, bool WKN = false>
hipError_t launch_fp8(const GemmOperands& g, hipStream_t st) {
  constexpr bool SWIGLU = EPI == 1 || EPI == 2 || EPI == 3;
  if (EPI == 3 && !g.out2) return hipErrorInvalidValue;
  if (WKN && (g.kn_split % kBK != 0 || g.kn_split <= 0 || g.kn_split > g.K)) return hipErrorInvalidValue;
  if (g.K % kBK != 0 || g.N % kBK != 0) return hipErrorInvalidValue;
  // 32-bit byte offsets address the activation matrix and one expert's weight matrix
  if (g.act_rows * g.K >= (int64_t(1) << 32) || (int64_t)g.N * g.K >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const size_t lds_bytes = kStages * kStageBytes;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&grouped_gemm_fp8_kernel<EPI, WKN>), (int)lds_bytes);
  if (err != hipSuccess) return err;
  const int NT = (int)ceil_div(g.N, SWIGLU ? kWRows / 2 : kWRows);
  const int64_t tiles = g.max_pairs * NT;
  const int64_t grid = ceil_div(tiles, kXcds * kXcdChunk) * (kXcds * kXcdChunk);
  if (grid == 0) return hipSuccess;
  auto kern = &grouped_gemm_fp8_kernel<EPI, WKN>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds_bytes, st, g, NT);
  return hipGetLastError();
}

#ifndef MOE_FP8_PERSISTENT
#define MOE_FP8_PERSISTENT 1
#endif

// the forward down GEMM, persistent (one workgroup per CU, a multiple of the 8 x 32 tile block)
hipError_t launch_fp8_down_persistent(const GemmOperands& g, hipStream_t st) {
  if (g.K % kBK != 0 || g.N % kBK != 0) return hipErrorInvalidValue;
  if (g.act_rows * g.K >= (int64_t(1) << 32) || (int64_t)g.N * g.K >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  if (g.n_seg < 1 || g.n_seg > kMaxRouted + kMaxShared) return hipErrorInvalidValue;
  if (g.row_token) return launch_fp8<0>(g, st);   // gathered rows: the one-tile kernel
  // operand stages, then the pair_off and seg_off tables (n_seg + 1 entries each)
  const size_t stage_bytes = (size_t)kStages * kStageBytes;
  const size_t max_lds = stage_bytes + 2 * (size_t)(kMaxRouted + kMaxShared + 1) * sizeof(int32_t);
  static_assert(kStages * kStageBytes + 2 * (kMaxRouted + kMaxShared + 1) * 4 <= 163840, "LDS");
  const size_t lds_bytes = stage_bytes + 2 * (size_t)(g.n_seg + 1) * sizeof(int32_t);
  auto kern = &grouped_gemm_fp8_persistent_kernel;
  int n_cu = 0;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)max_lds);
  if (err != hipSuccess || (err = device_cu_count(&n_cu)) != hipSuccess) return err;
  const int NT = (int)ceil_div(g.N, kWRows);
  if (g.max_pairs * NT == 0) return hipSuccess;
  const int64_t span = kXcds * kXcdChunk;
  const int64_t grid = std::max<int64_t>(span, (int64_t)n_cu / span * span);
  // the walk's tile indices (up to a grid stride past the last tile) and the table slots are int
  if (g.max_tiles * NT + 2 * grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds_bytes, st, g, NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_swiglu(const GemmOperands& g, hipStream_t st) { return launch_fp8<1>(g, st); }
// SwiGLU with H quantised, also writing the inputs [a b] of every row to g.out2 ([rows, 2N] bf16)
hipError_t launch_gemm_fp8_swiglu_save(const GemmOperands& g, hipStream_t st) { return launch_fp8<3>(g, st); }
hipError_t launch_gemm_fp8_down(const GemmOperands& g, hipStream_t st) {
  return MOE_FP8_PERSISTENT ? launch_fp8_down_persistent(g, st) : launch_fp8<0>(g, st);
}
hipError_t launch_gemm_fp8_swiglu_bwd(const GemmOperands& g, hipStream_t st) { return launch_fp8<2>(g, st); }
hipError_t launch_gemm_fp8_wgrad(const GemmOperands& g, hipStream_t st) { return launch_wgrad_fp8(g, st); }
hipError_t launch_gemm_fp8_dgrad(const GemmOperands& g, hipStream_t st) { return launch_fp8<0, true>(g, st); }

}  // namespace moe
