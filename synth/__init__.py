"""Seeded synthetic inputs for the MoE layer, shared by the oracle and the GPU path.

This module holds no arithmetic of the method itself: it only draws numbers.
Every tensor is a pure function of (seed, config id, tensor tag, expert index,
element index), so any subset can be regenerated independently on the host
(numpy reference or the C/OpenMP filler in ``csrc/synth_host.c``) or on the
device (the HIP filler in ``csrc/synth_fill.hip``); the three agree bit for bit.

Definition (the same in all three implementations):

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014), and ``G`` its
  golden-ratio increment 0x9E3779B97F4A7C15.  All arithmetic is mod 2**64.
* stream key: ``k0 = mix64(seed + G)``, ``k1 = mix64(k0 ^ (cfg + G))``,
  ``k2 = mix64(k1 ^ (tag + G))``, ``key = mix64(k2 ^ (expert + G))``.
* element ``n`` of a stream uses the two words ``w_j = mix64(key + (2n+j+1)*G)``,
  j = 0, 1 (outputs 2n+1 and 2n+2 of a SplitMix64 generator started at ``key``).
* "normal" values: the eight 16-bit fields of w0, w1 are summed (Irwin-Hall of
  order 8, an integer in [0, 8*65535]); ``x = sum - 262140`` is an integer of
  magnitude below 2**24, so ``float32(x)`` is exact; the value is
  ``float32(x) * scale32`` (one correctly rounded fp32 multiply), where
  ``scale32 = float32(sigma / IH8_STD)`` and ``IH8_STD = 65536*sqrt(2/3)``
  (more precisely sqrt(8*(65536**2-1)/12)), the standard deviation of the sum.
  The result has mean 0, standard deviation sigma, and tails bounded at
  about 4.9 sigma.
* bf16 tensors are the fp32 values rounded to nearest-even bf16.
* "uniform" values (only used for the small bias vector): ``(w0 >> 11) * 2**-53``
  in float64, then an affine map, then rounded to fp32.
"""
from __future__ import annotations

import math

import numpy as np

G = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
IH8_STD = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)
IH8_MEAN = 262140

# tensor tags
TAG_U, TAG_CENTROID, TAG_BIAS = 1, 2, 3
TAG_W_GATE, TAG_W_UP, TAG_W_DOWN = 4, 5, 6
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN = 7, 8, 9
TAG_PERM = 10
TAG_DOUT = 11          # upstream gradient dL/dh' of the backward

_MASK64 = (1 << 64) - 1


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, cfg: int, tag: int, expert: int) -> int:
    """64-bit key of one tensor stream (see the module docstring)."""
    g = int(G)
    k = _mix64_int(seed + g)
    k = _mix64_int(k ^ ((cfg + g) & _MASK64))
    k = _mix64_int(k ^ ((tag + g) & _MASK64))
    return _mix64_int(k ^ ((expert + g) & _MASK64))


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _words(key: int, start: int, n: int):
    idx = np.arange(start, start + n, dtype=np.uint64)
    base = np.uint64(key)
    with np.errstate(over="ignore"):
        c0 = base + (np.uint64(2) * idx + np.uint64(1)) * G
        c1 = base + (np.uint64(2) * idx + np.uint64(2)) * G
    return _mix64(c0), _mix64(c1)


def normal_scale32(sigma: float) -> np.float32:
    return np.float32(sigma / IH8_STD)


def normal_f32(key: int, n: int, sigma: float, start: int = 0) -> np.ndarray:
    """Elements [start, start+n) of the approximately N(0, sigma^2) stream, fp32."""
    w0, w1 = _words(key, start, n)
    m = np.uint64(0xFFFF)
    s = np.zeros(n, dtype=np.int64)
    for w in (w0, w1):
        for sh in (0, 16, 32, 48):
            s += ((w >> np.uint64(sh)) & m).astype(np.int64)
    x = (s - IH8_MEAN).astype(np.float32)
    return x * normal_scale32(sigma)


def uniform_f64(key: int, n: int, start: int = 0) -> np.ndarray:
    w0, _ = _words(key, start, n)
    return (w0 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to nearest-even bf16; returns the uint16 bit patterns (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


from .configs import CONFIGS, LayerConfig, get_config  # noqa: E402
from .host import make_host_inputs, zipf_centroid_scales, bias_vector  # noqa: E402

__all__ = [
    "G", "IH8_STD", "stream_key", "normal_f32", "uniform_f64", "normal_scale32",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "CONFIGS", "LayerConfig", "get_config",
    "make_host_inputs", "zipf_centroid_scales", "bias_vector",
    "TAG_U", "TAG_CENTROID", "TAG_BIAS", "TAG_W_GATE", "TAG_W_UP", "TAG_W_DOWN",
    "TAG_SH_GATE", "TAG_SH_UP", "TAG_SH_DOWN", "TAG_PERM",
]
