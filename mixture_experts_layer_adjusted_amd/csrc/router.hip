// Router: sigmoid affinities, biased top-K_r, normalised gates and per-expert loads.
//
// Implements the s_{i,t} and g'_{i,t} equations of 方法 §2 of the page
// "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437), with the bias
// entering the ranking only and the gate normalised over the selected unbiased
// affinities.
//
// Two implementations:
//
// MFMA path (bf16 tokens, d a multiple of 64, N_r <= 512):
//  1. split: every fp32 centroid element is written exactly as hi + mid + lo, three bf16 values
//     holding consecutive 8-bit slices of its 24-bit significand, so u . e = u . hi + u . mid +
//     u . lo with every bf16 x bf16 product exact in fp32;
//  2. logits: one bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16) over tokens x experts with the three
//     parts as three B operands, 128 x 128 tiles on 8 wavefronts (two per SIMD, each 64 tokens x
//     32 experts of every part), LDS stages filled by direct global->LDS loads;
//     every two 64-wide K-steps start a fresh accumulator that is then added to an fp32 running
//     sum (blocked summation keeps the logit error near 1e-7 of the sum of |terms|); s = sigmoid(z)
//     is written to the workspace; with fewer than 128 output tiles (decode-sized batches) the
//     contraction splits into up to 16 K-slices whose partial logits a second kernel adds in
//     slice order;
//  3. top-K: one wavefront per token on s + b, as in step 3 below, plus per-workgroup counts;
//     with a group limit (moe_route_grouped) the lanes first find the best c of every expert
//     group and mask the experts of the groups outside the topk_groups best;
//  4. counts: a fixed-order reduction of the per-workgroup counts into expert_load.
//
// Fused VALU path (fp32 tokens, or any other shape).  One workgroup (256 threads) owns
// kRouteTokens tokens:
//  1. logits z = u . e_i for its tokens and all experts, fp32 FMAs over LDS-staged
//     32-wide slices of d; each slice is summed in a fresh register and then added
//     to the running total (blocked summation keeps the rounding error of the
//     7168-long contraction near 1e-7 relative);
//  2. s = 1 / (1 + exp(-z)) written to LDS;
//  3. one wavefront per token: each lane holds ceil(N_r/64) candidate keys
//     (orderable bits of s+b in the high word, bit-inverted expert index in the
//     low word, so the 64-bit maximum is the highest score and, among equal
//     scores, the lowest index; NaN maps to the lowest key), K_r rounds of a
//     wave-wide 64-bit max pick the experts in order;
//  4. the workgroup's picks are counted per expert by a plain scan of its LDS
//     copy (no atomics) and written as one row of partial counts; a second
//     kernel sums the partial rows in a fixed order into expert_load.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;        // contraction slice staged in LDS
constexpr int kExpertTile = 256;  // experts per logit pass
constexpr int kEsPitch = kExpertTile + 1;

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

__device__ __forceinline__ uint64_t score_key(float c, int e) {
  uint32_t b = __float_as_uint(c);
  uint32_t ord;
  if (c != c) {
    ord = 0u;                              // NaN ranks below every number
  } else {
    if (c == 0.0f) b = 0u;                 // -0 and +0 are the same score
    ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

// one step of a wave-wide 64-bit maximum: v = max(v, v moved by the DPP control `ctrl` over the
// rows in row_mask); lanes without a source keep their own value, which leaves the maximum as is
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t mlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t mhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)mhi << 32) | mlo;
  return o > v ? o : v;
}

// maximum of v over the 64 lanes, returned to every lane: running maxima within each row of 16
// lanes by row shifts of 1, 2, 4 and 8 (lane 15 of a row then holds the row's maximum), row 1
// and 3 take in the row before through row_bcast:15, rows 2 and 3 take in lane 31 through
// row_bcast:31, so lane 63 ends with the maximum, read out as a scalar.  DPP moves stay in the
// VALU; the xor-shuffle form went through the LDS crossbar (ds_bpermute) twice per step.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xF>(v);   // row_shr:1
  v = dpp_max_step<0x112, 0xF>(v);   // row_shr:2
  v = dpp_max_step<0x114, 0xF>(v);   // row_shr:4
  v = dpp_max_step<0x118, 0xF>(v);   // row_shr:8
  v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Group limit (the per-token node limit of the page's cross-node all-to-all section, with the
// group score it leaves open read as the group's best biased score): the N_r experts form
// n_groups equal contiguous groups, only the topk_groups groups with the highest best s+b
// (ties to the lower group index) stay eligible, and the K_r picks are made among their
// experts.  Returns the lanes' "taken" bits of the ineligible candidates; gm is this
// wavefront's 64-entry LDS scratch.  topk_groups >= n_groups disables the limit.
template <int CPL>
__device__ __forceinline__ uint32_t group_limit_taken(const uint64_t (&key)[CPL], int N, int n_groups,
                                                      int topk_groups, int lane, uint32_t* gm) {
  if (topk_groups >= n_groups) return 0u;
  const int gs = N / n_groups;
  if (lane < n_groups) gm[lane] = 0u;
  // LDS operations of one wavefront take effect in program order
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int e = lane + 64 * j;
    if (e < N) atomicMax(&gm[e / gs], (uint32_t)(key[j] >> 32));
  }
  const uint64_t gk = lane < n_groups ? (((uint64_t)gm[lane] << 32) | (uint32_t)(~(uint32_t)lane)) : 0ull;
  uint64_t sel = 0ull;
  for (int r = 0; r < topk_groups; ++r) {
    const uint64_t w = wave_max_u64(((sel >> lane) & 1ull) ? 0ull : gk);
    sel |= 1ull << (int)(~(uint32_t)w);
  }
  uint32_t taken = 0u;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int e = lane + 64 * j;
    if (e < N && !((sel >> (e / gs)) & 1ull)) taken |= 1u << j;
  }
  return taken;
}

template <int CPL, typename TIn>
__global__ void __launch_bounds__(kThreads) route_kernel(const TIn* __restrict__ u, const float* __restrict__ E,
                                                         const float* __restrict__ bias, int T, int d, int N, int K,
                                                         GroupLimit gl, int32_t* __restrict__ idx_out,
                                                         float* __restrict__ gate_out, int32_t* __restrict__ partial,
                                                         float* __restrict__ s_out) {
  __shared__ float Us[kSlice][kRouteTokens + 1];
  __shared__ uint32_t gmax[kThreads / 64][64];
  __shared__ float Es[kSlice][kEsPitch];
  __shared__ float S[kRouteTokens][CPL * 64];
  __shared__ int32_t picks[kRouteTokens * kMaxTopK];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  const int tx = tid & 31;   // experts tx + 32 j
  const int ty = tid >> 5;   // tokens 4 ty .. 4 ty + 3

  for (int e0 = 0; e0 < N; e0 += kExpertTile) {
    float total[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) total[i][j] = 0.0f;

    for (int k0 = 0; k0 < d; k0 += kSlice) {
      // stage u[t0 .. t0+32, k0 .. k0+32] transposed into Us[k][t]
      for (int q = tid; q < kRouteTokens * kSlice; q += kThreads) {
        int t = q / kSlice, k = q % kSlice;
        float v = 0.0f;
        if (t0 + t < T && k0 + k < d) v = load_elem(u, (int64_t)(t0 + t) * d + k0 + k);
        Us[k][t] = v;
      }
      // stage E[e0 .. e0+256, k0 .. k0+32] transposed into Es[k][e]
      for (int q = tid; q < kExpertTile * kSlice; q += kThreads) {
        int e = q / kSlice, k = q % kSlice;
        float v = 0.0f;
        if (e0 + e < N && k0 + k < d) v = E[(int64_t)(e0 + e) * d + k0 + k];
        Es[k][e] = v;
      }
      __syncthreads();
      float acc[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
#pragma unroll 8
      for (int k = 0; k < kSlice; ++k) {
        float a[4], b[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = Us[k][4 * ty + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Es[k][tx + 32 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) total[i][j] += acc[i][j];
      __syncthreads();
    }
    // sigmoid into S
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int e = e0 + tx + 32 * j;
        if (e < CPL * 64) S[4 * ty + i][e] = 1.0f / (1.0f + expf(-total[i][j]));
      }
  }
  for (int q = tid; q < kRouteTokens * kMaxTopK; q += kThreads) picks[q] = -1;
  __syncthreads();
  if (s_out) {   // the affinities of the workgroup's tokens, for the balance statistic
    for (int q = tid; q < kRouteTokens * N; q += kThreads) {
      const int tt = q / N, e = q % N;
      if (t0 + tt < T) s_out[(int64_t)(t0 + tt) * N + e] = S[tt][e];
    }
  }

  // top-K: one wavefront per token
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float bl[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int e = lane + 64 * j;
    bl[j] = e < N ? bias[e] : 0.0f;
  }
  for (int tt = wave; tt < kRouteTokens; tt += kThreads / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    uint64_t key[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int e = lane + 64 * j;
      key[j] = e < N ? score_key(S[tt][e] + bl[j], e) : 0ull;
    }
    uint32_t taken = group_limit_taken<CPL>(key, N, gl.n_groups, gl.topk_groups, lane, gmax[wave]);
    float mys = 0.0f, sum = 0.0f;
    int myidx = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
      int bj = -1;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int e = lane + 64 * j;
        if (e < N && !((taken >> j) & 1u) && (bj < 0 || key[j] > best)) {
          best = key[j];
          bj = j;
        }
      }
      uint64_t win = wave_max_u64(bj < 0 ? 0ull : best);
      int we = (int)(~(uint32_t)win);
      if (bj >= 0 && best == win) taken |= 1u << bj;
      float sw = S[tt][we];
      sum += sw;
      if (lane == k) {
        mys = sw;
        myidx = we;
      }
    }
    if (lane < K) {
      idx_out[(int64_t)t * K + lane] = myidx;
      gate_out[(int64_t)t * K + lane] = mys / sum;
      picks[tt * K + lane] = myidx;
    }
  }
  __syncthreads();
  // partial per-expert counts of this workgroup's picks (plain scan, no atomics)
  for (int e = tid; e < N; e += kThreads) {
    int c = 0;
    for (int q = 0; q < kRouteTokens * K; ++q) c += (picks[q] == e);
    partial[(int64_t)blockIdx.x * N + e] = c;
  }
}

// one 64-lane workgroup per expert: lane j sums partial rows j, j+64, ...; then a fixed
// butterfly over the lanes (integer sums, so the order does not change the result anyway)
__global__ void __launch_bounds__(64) load_reduce_kernel(const int32_t* __restrict__ partial, int64_t blocks, int N,
                                                         int32_t* __restrict__ load) {
  const int e = blockIdx.x;
  int32_t s = 0;
  for (int64_t b = threadIdx.x; b < blocks; b += 64) s += partial[b * N + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (threadIdx.x == 0) load[e] = s;
}

__global__ void zero_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}


// ---------------------------------------------------------------------------- MFMA path

constexpr int kLT = 128;           // tokens per logits tile
constexpr int kLE = 128;           // experts per logits tile
constexpr int kLBK = 64;           // contraction per K-step
constexpr int kLStageElems = (kLT + 3 * kLE) * kLBK;  // 64 KB
constexpr int kLWaves = 8;         // two wavefronts per SIMD
constexpr int kTopkTokens = 64;    // tokens per top-K workgroup
constexpr int kTopkThreads = 1024; // 16 wavefronts, four tokens each: latency of the K rounds of
                                   // wave-wide maxima hidden across the wavefronts
static_assert(kTopkTokens * kMaxTopK % 4 == 0 && kTopkTokens % 4 == 0, "picks counted four at a time");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int roff(int r, int c) { return r * kLBK + ((c ^ rswz(r)) << 3); }

// e = hi + mid + lo exactly: hi keeps the sign, exponent and top 7 stored significand bits;
// the two remainders are exact fp32 differences with at most 16 and 8 significant bits
__global__ void split_centroids_kernel(const float* __restrict__ E, int64_t n_elems, int64_t n_pad_elems,
                                       uint16_t* __restrict__ hi, uint16_t* __restrict__ mid,
                                       uint16_t* __restrict__ lo) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pad_elems;
       i += (int64_t)gridDim.x * blockDim.x) {
    float x = i < n_elems ? E[i] : 0.0f;
    uint32_t h = __float_as_uint(x) & 0xFFFF0000u;
    float r1 = __fsub_rn(x, __uint_as_float(h));
    uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    float r2 = __fsub_rn(r1, __uint_as_float(m));
    hi[i] = (uint16_t)(h >> 16);
    mid[i] = (uint16_t)(m >> 16);
    lo[i] = (uint16_t)(__float_as_uint(r2) >> 16);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// logits tile: 256 threads, waves (wm, wn) in 2 x 2 own 64 tokens x 64 experts; two LDS stages
// kBuf: operand loads in buffer form (a base per matrix, 32-bit byte offsets; u below 4 GiB),
// else in global form
template <bool kBuf>
__global__ void __launch_bounds__(kLWaves * 64) router_logits_kernel(const uint16_t* __restrict__ u,
                                                                     const uint16_t* __restrict__ ehi,
                                                                     const uint16_t* __restrict__ emid,
                                                                     const uint16_t* __restrict__ elo, int T, int d,
                                                                     int N, float* __restrict__ s_out, int nk_per,
                                                                     float* __restrict__ z_part) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;   // 2 x 4 grid: 64 tokens x 32 experts (of each part) per wave
  const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
  const int lrow = lane >> 3, lslot = lane & 7;
  // DMA sources (element offsets from each matrix's base): wave w fills token rows [16w, 16w+16)
  // and, for each part, expert rows [16w, 16w+16)
  int64_t off[8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wave * 16 + i * 8 + lrow;
    const int t = min(t0 + row, T - 1);  // rows past T: any valid row (outputs discarded)
    off[i] = (int64_t)t * d + ((lslot ^ rswz(row)) << 3);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 16 + i * 8 + lrow;         // expert row within the part
      const int lrow_lds = kLT + p * kLE + row;          // LDS row
      off[2 + p * 2 + i] = (int64_t)(e0 + row) * d + ((lslot ^ rswz(lrow_lds)) << 3);
    }
  }
  const uint16_t* base[4] = {u, ehi, emid, elo};
  __amdgpu_buffer_rsrc_t buf[4];
  uint32_t voff[8];
  if constexpr (kBuf) {
#pragma unroll
    for (int m = 0; m < 4; ++m) buf[m] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base[m]), (short)0, -1,
                                                                            0x00020000);
#pragma unroll
    for (int j = 0; j < 8; ++j) voff[j] = (uint32_t)(off[j] * 2);
  }
  auto issue = [&](int kt) {
    uint16_t* st = lds + (kt & 1) * kLStageElems;
    const int k0 = kt * kLBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = j < 2 ? 0 : 1 + (j - 2) / 2;   // matrix: u, then the three parts
      const int lds_row = j < 2 ? wave * 16 + j * 8 : kLT + (m - 1) * kLE + wave * 16 + (j & 1) * 8;
      lds_void_t* dst = (lds_void_t*)(st + lds_row * kLBK);
      if constexpr (kBuf)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf[m], dst, 16, voff[j], (uint32_t)k0 * 2, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(base[m] + off[j] + k0, dst, 16, 0, 0);
    }
  };
  float zsum[2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) zsum[a][v] = 0.0f;
  const int l32 = lane & 31, khalf = lane >> 5;
  // K-steps [kt0, kt1) of the contraction: all of it, or slice blockIdx.z when it is split
  const int kt0 = blockIdx.z * nk_per, kt1 = min(d / kLBK, kt0 + nk_per);
  if (kt0 < kt1) issue(kt0);   // a slice past the end contributes zeros
  // one K-step's MFMAs on stage kt into acc (which the first of them starts from zero when
  // `fresh`); the partial logits of every two K-steps are then added to the fp32 running sum
  f32x16 acc[2];
  auto kstep = [&](int kt, auto fresh) {
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // stage kt landed for every wave; stage kt-1 no longer read
    if (kt + 1 < kt1) issue(kt + 1);
    const uint16_t* st = lds + (kt & 1) * kLStageElems;
    if constexpr (decltype(fresh)::value) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][v] = 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < kLBK / 16; ++kk) {
      const int c = kk * 2 + khalf;
      bf16x8 tf[2], ef[3];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) tf[mb] = *reinterpret_cast<const bf16x8*>(st + roff(wm * 64 + mb * 32 + l32, c));
#pragma unroll
      for (int p = 0; p < 3; ++p)
        ef[p] = *reinterpret_cast<const bf16x8*>(st + roff(kLT + p * kLE + wn * 32 + l32, c));
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[p], tf[mb], acc[mb], 0, 0, 0);
    }
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    kstep(kt, std::true_type{});
    if (kt + 1 < kt1) kstep(kt + 1, std::false_type{});
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) zsum[a][v] += acc[a][v];
  }
  // lane holds token t0 + 64 wm + 32 mb + l32 and experts e0 + 32 wn + 8 q + 4 khalf + (0..3)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int t = t0 + wm * 64 + mb * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + wn * 32 + q * 8 + khalf * 4;
      if (z_part) {   // a slice's partial logits, summed in slice order by logit_reduce_kernel
        float* zrow = z_part + ((int64_t)blockIdx.z * T + t) * N;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (e + v < N) zrow[e + v] = zsum[mb][q * 4 + v];
        continue;
      }
      float4 o;
      o.x = 1.0f / (1.0f + expf(-zsum[mb][q * 4 + 0]));
      o.y = 1.0f / (1.0f + expf(-zsum[mb][q * 4 + 1]));
      o.z = 1.0f / (1.0f + expf(-zsum[mb][q * 4 + 2]));
      o.w = 1.0f / (1.0f + expf(-zsum[mb][q * 4 + 3]));
      if (e + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(s_out + (int64_t)t * N + e) = o;
      } else {
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (e + v < N) s_out[(int64_t)t * N + e + v] = ov[v];
      }
    }
  }
}

// s = sigmoid(sum of the slices' partial logits, in slice order)
__global__ void logit_reduce_kernel(const float* __restrict__ z_part, int splits, int64_t n, float* __restrict__ s_out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float z = 0.0f;
    for (int q = 0; q < splits; ++q) z += z_part[q * n + i];
    s_out[i] = 1.0f / (1.0f + expf(-z));
  }
}

// top-K over precomputed affinities: one wavefront per token, kTopkTokens tokens per workgroup
template <int CPL>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ s_in,
                                                            const float* __restrict__ bias, int T, int N, int K,
                                                            GroupLimit gl, int32_t* __restrict__ idx_out,
                                                            float* __restrict__ gate_out,
                                                            int32_t* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) int32_t picks[kTopkTokens * kMaxTopK];
  __shared__ uint32_t gmax[kTopkThreads / 64][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTopkTokens;
  for (int q = tid; q < kTopkTokens * kMaxTopK; q += kTopkThreads) picks[q] = -1;
  float bl[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int e = lane + 64 * j;
    bl[j] = e < N ? bias[e] : 0.0f;
  }
  __syncthreads();
  for (int tt = wave; tt < kTopkTokens; tt += kTopkThreads / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* srow = s_in + (int64_t)t * N;
    float sv[CPL];
    uint64_t key[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int e = lane + 64 * j;
      sv[j] = e < N ? srow[e] : 0.0f;
      key[j] = e < N ? score_key(sv[j] + bl[j], e) : 0ull;
    }
    uint32_t taken = group_limit_taken<CPL>(key, N, gl.n_groups, gl.topk_groups, lane, gmax[wave]);
    float mys = 0.0f, sum = 0.0f;
    int myidx = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
      int bj = -1;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int e = lane + 64 * j;
        if (e < N && !((taken >> j) & 1u) && (bj < 0 || key[j] > best)) {
          best = key[j];
          bj = j;
        }
      }
      uint64_t win = wave_max_u64(bj < 0 ? 0ull : best);
      int we = (int)(~(uint32_t)win);
      float sw = 0.0f;
      if (bj >= 0 && best == win) {
        taken |= 1u << bj;
      }
      // the winner's affinity, broadcast from the lane that holds it
      const int owner = we & 63, oj = we >> 6;
      float cand = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        if (j == oj) cand = sv[j];
      sw = __shfl(cand, owner, 64);
      sum += sw;
      if (lane == k) {
        mys = sw;
        myidx = we;
      }
    }
    if (lane < K) {
      idx_out[(int64_t)t * K + lane] = myidx;
      gate_out[(int64_t)t * K + lane] = mys / sum;
      picks[tt * K + lane] = myidx;
    }
  }
  __syncthreads();
  // the workgroup's picks of each expert, four LDS entries per read (64 K entries, unused ones -1)
  for (int e = tid; e < N; e += kTopkThreads) {
    int c = 0;
    for (int q = 0; q < kTopkTokens * K; q += 4) {
      const int4 p = *reinterpret_cast<const int4*>(&picks[q]);
      c += (p.x == e) + (p.y == e) + (p.z == e) + (p.w == e);
    }
    partial[(int64_t)blockIdx.x * N + e] = c;
  }
}

template <typename TIn>
hipError_t launch_route_t(const moe_shape& s, const TIn* u, const float* centroids, const float* bias,
                          GroupLimit gl, int32_t* idx, float* gate, int32_t* load, int32_t* partial, int64_t blocks,
                          float* s_out, hipStream_t st) {
  const int N = s.n_routed;
  dim3 grid((unsigned)blocks), block(kThreads);
#define MOE_ROUTE_CASE(C)                                                                                  \
  hipLaunchKernelGGL((route_kernel<C, TIn>), grid, block, 0, st, u, centroids, bias, s.tokens, s.hidden, N, \
                     s.top_k, gl, idx, gate, partial, s_out)
  if (N <= 64) MOE_ROUTE_CASE(1);
  else if (N <= 128) MOE_ROUTE_CASE(2);
  else if (N <= 256) MOE_ROUTE_CASE(4);
  else MOE_ROUTE_CASE(8);
#undef MOE_ROUTE_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(load_reduce_kernel, dim3((unsigned)N), dim3(64), 0, st, partial, blocks, N, load);
  return hipGetLastError();
}

hipError_t launch_route_mfma(const moe_shape& s, const uint16_t* u, const float* centroids, const float* bias,
                             GroupLimit gl, int32_t* idx, float* gate, int32_t* load, const RouteWorkspace& w,
                             hipStream_t st) {
  const int T = s.tokens, d = s.hidden, N = s.n_routed;
  const int64_t npad = ceil_div(N, kLE) * kLE;
  hipLaunchKernelGGL(split_centroids_kernel, dim3(1024), dim3(256), 0, st, centroids, (int64_t)N * d, npad * d,
                     w.e_hi, w.e_mid, w.e_lo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds_bytes = 2 * kLStageElems * sizeof(uint16_t);
  // buffer-form loads address u and the split centroids with 32-bit byte offsets
  const bool buf = (int64_t)T * d * 2 < (int64_t(1) << 32) && npad * d * 2 < (int64_t(1) << 32);
  auto kern = buf ? &router_logits_kernel<true> : &router_logits_kernel<false>;
  if ((err = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds_bytes)) != hipSuccess) return err;
  const int splits = route_logit_splits(s);
  const int nk = d / kLBK, nk_per = (int)ceil_div(nk, splits);
  hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(T, kLT), (unsigned)(npad / kLE), (unsigned)splits),
                     dim3(kLWaves * 64), lds_bytes, st, u, w.e_hi, w.e_mid, w.e_lo, T, d, N, w.scores, nk_per,
                     splits > 1 ? w.zpart : nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (splits > 1) {
    const int64_t n = (int64_t)T * N;
    hipLaunchKernelGGL(logit_reduce_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(n, 256), 2048)), dim3(256), 0, st,
                       w.zpart, splits, n, w.scores);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t blocks = ceil_div(T, kTopkTokens);
  dim3 grid((unsigned)blocks), block(kTopkThreads);
#define MOE_TOPK_CASE(C) \
  hipLaunchKernelGGL((topk_kernel<C>), grid, block, 0, st, w.scores, bias, T, N, s.top_k, gl, idx, gate, w.partial)
  if (N <= 64) MOE_TOPK_CASE(1);
  else if (N <= 128) MOE_TOPK_CASE(2);
  else if (N <= 256) MOE_TOPK_CASE(4);
  else MOE_TOPK_CASE(8);
#undef MOE_TOPK_CASE
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(load_reduce_kernel, dim3((unsigned)N), dim3(64), 0, st, w.partial, blocks, N, load);
  return hipGetLastError();
}

}  // namespace

bool route_uses_mfma(const moe_shape& s) {
  return s.dtype != MOE_DTYPE_F32 && s.hidden % kLBK == 0 && s.n_routed <= kMaxRouted;
}

// K slices of the MFMA logits: with few 128 x 128 tiles (small T) the contraction is split so
// that about 256 workgroups run; the slices' partial sums are added in a fixed order
int route_logit_splits(const moe_shape& s) {
  if (!route_uses_mfma(s) || s.tokens == 0) return 1;
  const int64_t tiles = ceil_div(s.tokens, kLT) * ceil_div(s.n_routed, kLE);
  if (tiles >= 128) return 1;
  const int64_t nk = s.hidden / kLBK;
  return (int)std::max<int64_t>(1, std::min<int64_t>({16, 256 / tiles, nk}));
}

int64_t route_mfma_blocks(const moe_shape& s) { return ceil_div(s.tokens, kTopkTokens); }

hipError_t launch_route(const moe_shape& s, const void* u, const float* centroids, const float* bias,
                        GroupLimit gl, int32_t* idx, float* gate, int32_t* load, const RouteWorkspace& w,
                        hipStream_t st) {
  if (s.tokens > 0 && route_uses_mfma(s))
    return launch_route_mfma(s, static_cast<const uint16_t*>(u), centroids, bias, gl, idx, gate, load, w, st);
  int32_t* partial = w.partial;
  const int64_t blocks = ceil_div(s.tokens, kRouteTokens);
  if (s.tokens == 0) {
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)ceil_div(s.n_routed, 256)), dim3(256), 0, st, load, s.n_routed);
    return hipGetLastError();
  }
  if (s.dtype == MOE_DTYPE_F32)
    return launch_route_t(s, static_cast<const float*>(u), centroids, bias, gl, idx, gate, load, partial, blocks,
                          w.scores, st);
  return launch_route_t(s, static_cast<const uint16_t*>(u), centroids, bias, gl, idx, gate, load, partial, blocks,
                        w.scores, st);
}

namespace {

// Sequence-wise balance statistic, one workgroup per sequence of L tokens (the reading of the
// page's "tiny sequence-level balance loss"): loss = alpha * sum_i f_i P_i with
// f_i = N_r / (K_r L) * (the sequence's picks of expert i) and P_i = (1/L) sum_t s_{i,t} / S_t,
// S_t = sum_j s_{j,t}.  Picks are counted with LDS increments (exact); every float sum runs in a
// fixed order (per-lane strided sums, a fixed tree, then token order), so the result is the
// same on every run.
__global__ void __launch_bounds__(256) seq_balance_kernel(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                          int N, int K, int L, float alpha,
                                                          float* __restrict__ loss) {
  extern __shared__ float dyn[];
  float* St = dyn;                                          // [L]
  int32_t* cnt = reinterpret_cast<int32_t*>(dyn + L);       // [N]
  __shared__ float red[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * L;
  for (int e = tid; e < N; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int q = tid; q < L * K; q += 256) {
    const int e = idx[t0 * K + q];
    if (e >= 0 && e < N) atomicAdd(&cnt[e], 1);
  }
  for (int t = wave; t < L; t += 4) {
    const float* row = s + (t0 + t) * N;
    float v = 0.0f;
    for (int e = lane; e < N; e += 64) v += row[e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) St[t] = v;
  }
  __syncthreads();
  float term = 0.0f;
  for (int e = tid; e < N; e += 256) {
    float p = 0.0f;
    for (int t = 0; t < L; ++t) p += s[(t0 + t) * N + e] / St[t];
    const float f = (float)cnt[e] * (float)N / ((float)K * (float)L);
    term += f * (p / (float)L);
  }
  red[tid] = term;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) loss[blockIdx.x] = alpha * red[0];
}

// Long sequences (L >= 64) in two passes so that the whole chip takes part: the first pass gives
// every chunk of up to 64 tokens of a sequence its own workgroup, which writes the chunk's
// partial sum over its tokens of s_{i,t} / S_t for every expert (S_t summed as above); the
// second adds the chunk partials of each sequence in chunk order and forms the loss.
__global__ void __launch_bounds__(256) seq_balance_part_kernel(const float* __restrict__ s, int N, int L, int cps,
                                                               float* __restrict__ part) {
  __shared__ float St[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int64_t seq = c / cps;
  const int ci = (int)(c % cps);
  const int64_t t0 = seq * L + (int64_t)ci * 64;
  const int nt = min(64, L - ci * 64);
  for (int t = wave; t < nt; t += 4) {
    const float* row = s + (t0 + t) * N;
    float v = 0.0f;
    for (int e = lane; e < N; e += 64) v += row[e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) St[t] = v;
  }
  __syncthreads();
  for (int e = tid; e < N; e += 256) {
    float p = 0.0f;
    for (int t = 0; t < nt; ++t) p += s[(t0 + t) * N + e] / St[t];
    part[c * N + e] = p;
  }
}

__global__ void __launch_bounds__(256) seq_balance_final_kernel(const float* __restrict__ part,
                                                                const int32_t* __restrict__ idx, int N, int K, int L,
                                                                int cps, float alpha, float* __restrict__ loss) {
  extern __shared__ int32_t cnt[];   // [N]
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * L;
  for (int e = tid; e < N; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int q = tid; q < L * K; q += 256) {
    const int e = idx[t0 * K + q];
    if (e >= 0 && e < N) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  float term = 0.0f;
  const float* pc = part + (int64_t)blockIdx.x * cps * N;
  for (int e = tid; e < N; e += 256) {
    float p = 0.0f;
    for (int c = 0; c < cps; ++c) p += pc[(int64_t)c * N + e];
    const float f = (float)cnt[e] * (float)N / ((float)K * (float)L);
    term += f * (p / (float)L);
  }
  red[tid] = term;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) loss[blockIdx.x] = alpha * red[0];
}

}  // namespace

hipError_t launch_seq_balance(const moe_shape& s, int seq_len, float alpha, const float* scores, const int32_t* idx,
                              float* part, float* loss, hipStream_t st) {
  const int64_t n_seq = s.tokens / seq_len;
  if (n_seq == 0) return hipSuccess;
  if (seq_len >= 64) {
    const int cps = (int)ceil_div(seq_len, 64);
    hipLaunchKernelGGL(seq_balance_part_kernel, dim3((unsigned)(n_seq * cps)), dim3(256), 0, st, scores, s.n_routed,
                       seq_len, cps, part);
    hipLaunchKernelGGL(seq_balance_final_kernel, dim3((unsigned)n_seq), dim3(256), (size_t)s.n_routed * 4, st, part,
                       idx, s.n_routed, s.top_k, seq_len, cps, alpha, loss);
    return hipGetLastError();
  }
  const size_t lds = (size_t)seq_len * 4 + (size_t)s.n_routed * 4;
  hipError_t err = ensure_dynamic_lds(reinterpret_cast<const void*>(&seq_balance_kernel), 65536 + 4 * kMaxRouted);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(seq_balance_kernel, dim3((unsigned)n_seq), dim3(256), lds, st, scores, idx, s.n_routed, s.top_k,
                     seq_len, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
