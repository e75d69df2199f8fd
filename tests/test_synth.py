"""The seeded input streams: numpy reference vs the C filler, bf16 rounding, moments, Zipf recipe."""
import math

import numpy as np
import pytest
import torch

import synth
from synth import host
from synth.configs import CONFIGS
from synth.native import host_lib


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_stream_moments_and_independence():
    k1 = synth.stream_key(0, 3, synth.TAG_U, 0)
    k2 = synth.stream_key(0, 3, synth.TAG_U, 1)
    a = synth.normal_f32(k1, 200000, 2.0).astype(np.float64)
    b = synth.normal_f32(k2, 200000, 2.0).astype(np.float64)
    assert abs(a.mean()) < 0.02 and abs(a.std() - 2.0) < 0.02
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.01
    assert abs(np.corrcoef(a[:-1], a[1:])[0, 1]) < 0.01
    # offsets address the same stream
    assert np.array_equal(synth.normal_f32(k1, 100, 2.0, 5000), synth.normal_f32(k1, 5100, 2.0)[5000:])


def test_key_matches_python_int_reference():
    # the key chain evaluated with Python integers mod 2^64 (independent of numpy overflow rules)
    m = (1 << 64) - 1
    g = 0x9E3779B97F4A7C15

    def mix(z):
        z &= m
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
        return z ^ (z >> 31)
    key = synth.stream_key(7, 2, 5, 11)
    want = mix(mix(mix(mix(7 + g) ^ (2 + g)) ^ (5 + g)) ^ (11 + g))
    assert key == want
    # element 3 of the stream from Python ints
    w0, w1 = mix(key + 7 * g), mix(key + 8 * g)
    s = sum((w >> sh) & 0xFFFF for w in (w0, w1) for sh in (0, 16, 32, 48)) - 262140
    assert synth.normal_f32(key, 1, 1.0, 3)[0] == np.float32(s) * synth.normal_scale32(1.0)


@pytest.mark.skipif(host_lib() is None, reason="C filler not built")
@pytest.mark.parametrize("bf16", [False, True])
def test_c_filler_matches_numpy(bf16):
    key = synth.stream_key(0, 4, synth.TAG_W_DOWN, 17)
    sig = 1.0 / math.sqrt(2048)
    a = host.host_normal(key, 300001, sig, 123456789, bf16)
    v = synth.normal_f32(key, 300001, sig, 123456789)
    b = synth.f32_to_bf16_bits(v) if bf16 else v
    assert np.array_equal(a, b)


def test_zipf_scales():
    lam = host.zipf_centroid_scales(CONFIGS[3])
    assert lam.shape == (256,)
    assert abs(lam.max() - 32 ** 0.3) < 1e-5       # capped top share 1/K_r -> (0.125*256)^0.3
    assert lam.min() > 0.5
    assert len(np.unique(lam)) > 200


def test_bias_distributions():
    assert np.all(host.bias_vector(CONFIGS[0]) == 0)
    b1 = host.bias_vector(CONFIGS[1])
    assert b1.min() >= -0.01 and b1.max() <= 0.01 and b1.std() > 0.004
    b2 = host.bias_vector(CONFIGS[2])
    assert 0.07 < b2.std() < 0.13
