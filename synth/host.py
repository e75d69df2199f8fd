"""Host-side assembly of the seeded synthetic inputs (numpy arrays).

bf16 tensors are returned as uint16 bit patterns (numpy has no bf16); fp32
tensors as float32.  Expert weights are stored [out_features, in_features]
per expert: gate/up projections [N, I, d], down projection [N, d, I].
"""
from __future__ import annotations

import ctypes
import math

import numpy as np

from . import (TAG_BIAS, TAG_CENTROID, TAG_PERM, TAG_SH_DOWN, TAG_SH_GATE, TAG_SH_UP, TAG_U,
               TAG_W_DOWN, TAG_W_GATE, TAG_W_UP, f32_to_bf16_bits, normal_f32, normal_scale32,
               stream_key, uniform_f64, _mix64)
from .configs import LayerConfig
from .native import host_lib


def host_normal(key: int, n: int, sigma: float, start: int = 0, bf16: bool = False) -> np.ndarray:
    """Elements [start, start+n) of a normal stream: C/OpenMP filler if built, else numpy."""
    lib = host_lib()
    if lib is None or n < 4096:
        v = normal_f32(key, n, sigma, start)
        return f32_to_bf16_bits(v) if bf16 else v
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    rc = lib.synth_fill_normal_host(out.ctypes.data_as(ctypes.c_void_p), n, start, key,
                                    float(normal_scale32(sigma)), 1 if bf16 else 0)
    if rc != 0:
        raise RuntimeError("synth_fill_normal_host failed")
    return out


def storage_is_bf16(cfg: LayerConfig) -> bool:
    return cfg.dtype in ("bf16", "fp8")


def zipf_centroid_scales(cfg: LayerConfig, s: float = 1.1, power: float = 0.3) -> np.ndarray:
    """Per-expert centroid norm multipliers lambda_i (fp32) for Zipf-like popularity.

    Target shares q_r ~ r**-s over ranks 1..N_r, water-filled to the per-token
    cap 1/K_r (an expert can be picked at most once per token); ranks are mapped
    to experts by a seeded permutation; lambda_i = (q_i * N_r) ** power.
    """
    n, k = cfg.n_routed, cfg.top_k
    q = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    q /= q.sum()
    cap = 1.0 / k
    capped = np.zeros(n, dtype=bool)
    for _ in range(n):
        over = (q > cap) & ~capped
        if not over.any():
            break
        capped |= over
        free = ~capped
        q[capped] = cap
        rest = 1.0 - cap * capped.sum()
        q[free] *= rest / q[free].sum()
    key = stream_key(cfg.seed, cfg.cid, TAG_PERM, 0)
    draws = _mix64(np.uint64(key) + (np.arange(n, dtype=np.uint64) + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15))
    rank_to_expert = np.argsort(draws, kind="stable")
    lam = np.empty(n, dtype=np.float64)
    lam[rank_to_expert] = (q * n) ** power
    return lam.astype(np.float32)


def bias_vector(cfg: LayerConfig) -> np.ndarray:
    key = stream_key(cfg.seed, cfg.cid, TAG_BIAS, 0)
    n = cfg.n_routed
    if cfg.bias == "zero":
        return np.zeros(n, dtype=np.float32)
    if cfg.bias == "uniform0.01":
        return (-0.01 + 0.02 * uniform_f64(key, n)).astype(np.float32)
    if cfg.bias == "normal_var0.01":  # variance 0.01, standard deviation 0.1
        return normal_f32(key, n, 0.1)
    raise ValueError(cfg.bias)


def centroids(cfg: LayerConfig) -> np.ndarray:
    d = cfg.hidden
    e = np.stack([normal_f32(stream_key(cfg.seed, cfg.cid, TAG_CENTROID, i), d, 1.0 / math.sqrt(d))
                  for i in range(cfg.n_routed)])
    if cfg.zipf:
        e = (e * zipf_centroid_scales(cfg)[:, None]).astype(np.float32)
    return e


def token_rows(cfg: LayerConfig, rows=None) -> np.ndarray:
    """Rows of u [T, d] (all rows if rows is None), in storage format."""
    d = cfg.hidden
    key = stream_key(cfg.seed, cfg.cid, TAG_U, 0)
    bf = storage_is_bf16(cfg)
    if rows is None:
        return host_normal(key, cfg.tokens * d, 1.0, 0, bf).reshape(cfg.tokens, d)
    return np.stack([host_normal(key, d, 1.0, int(t) * d, bf) for t in rows])


def expert_weights(cfg: LayerConfig, e: int, shared: bool = False):
    """(w_gate [I,d], w_up [I,d], w_down [d,I]) of routed expert e (or shared expert e)."""
    d, I = cfg.hidden, cfg.inter
    tg, tu, td = (TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN) if shared else (TAG_W_GATE, TAG_W_UP, TAG_W_DOWN)
    bf = storage_is_bf16(cfg)
    wg = host_normal(stream_key(cfg.seed, cfg.cid, tg, e), I * d, 1.0 / math.sqrt(d), 0, bf).reshape(I, d)
    wu = host_normal(stream_key(cfg.seed, cfg.cid, tu, e), I * d, 1.0 / math.sqrt(d), 0, bf).reshape(I, d)
    wd = host_normal(stream_key(cfg.seed, cfg.cid, td, e), d * I, 1.0 / math.sqrt(I), 0, bf).reshape(d, I)
    return wg, wu, wd


def make_host_inputs(cfg: LayerConfig, with_weights: bool = True) -> dict:
    """All inputs of a configuration as host arrays (use for the small configurations)."""
    out = {
        "u": token_rows(cfg),
        "centroids": centroids(cfg),
        "bias": bias_vector(cfg),
    }
    if with_weights:
        ws = [expert_weights(cfg, e) for e in range(cfg.n_routed)]
        out["w_gate"] = np.stack([w[0] for w in ws])
        out["w_up"] = np.stack([w[1] for w in ws])
        out["w_down"] = np.stack([w[2] for w in ws])
        if cfg.n_shared:
            ss = [expert_weights(cfg, s, shared=True) for s in range(cfg.n_shared)]
            out["sh_gate"] = np.stack([w[0] for w in ss])
            out["sh_up"] = np.stack([w[1] for w in ss])
            out["sh_down"] = np.stack([w[2] for w in ss])
        else:
            z = np.uint16 if storage_is_bf16(cfg) else np.float32
            out["sh_gate"] = np.zeros((0, cfg.inter, cfg.hidden), dtype=z)
            out["sh_up"] = np.zeros((0, cfg.inter, cfg.hidden), dtype=z)
            out["sh_down"] = np.zeros((0, cfg.hidden, cfg.inter), dtype=z)
    return out
