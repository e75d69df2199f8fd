/* Host (C/OpenMP) filler for the seeded synthetic input streams.
 *
 * Same definition as the numpy reference in synth/__init__.py and the device
 * filler in synth_fill.hip: SplitMix64 outputs (Steele, Lea and Flood, OOPSLA
 * 2014) of a per-tensor key, eight 16-bit fields summed (Irwin-Hall of order 8),
 * recentred to an exact integer, converted exactly to fp32 and scaled by one
 * correctly rounded fp32 multiply; bf16 output is the round-to-nearest-even of
 * that fp32 value.  Built with -ffp-contract=off.  Holds no arithmetic of the
 * MoE method.
 */
#include <stdint.h>
#include <string.h>

#define SYNTH_G 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline int32_t ih8(uint64_t key, uint64_t n) {
  uint64_t w0 = mix64(key + (2 * n + 1) * SYNTH_G);
  uint64_t w1 = mix64(key + (2 * n + 2) * SYNTH_G);
  int32_t s = 0;
  for (int sh = 0; sh < 64; sh += 16) s += (int32_t)((w0 >> sh) & 0xFFFF) + (int32_t)((w1 >> sh) & 0xFFFF);
  return s - 262140;
}

static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

/* Fill out[0..n) with elements [start, start+n) of the stream `key`.
 * out_kind: 0 = fp32, 1 = bf16 (uint16 bit patterns). Returns 0, or -1 on bad arguments. */
int synth_fill_normal_host(void* out, int64_t n, int64_t start, uint64_t key, float scale, int out_kind) {
  if (!out || n < 0 || start < 0 || (out_kind != 0 && out_kind != 1)) return -1;
  if (out_kind == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      float x = (float)ih8(key, (uint64_t)(start + i));
      o[i] = x * scale;
    }
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      float x = (float)ih8(key, (uint64_t)(start + i));
      o[i] = f32_to_bf16_rne(x * scale);
    }
  }
  return 0;
}
