"""Shared pieces of the GPU parity tests: run the library, run the oracle, compare.

Matching rules (the layer of 方法 §2, "DeepSeek-V3 技術報告"):
* indices: the GPU's picks equal the oracle's as a set for every token whose
  oracle margin c_(K) - c_(K+1) is >= 1e-6; for the other ("exempt") tokens
  every GPU pick must still be legal, c >= c_(K) - 1e-6; the order must be
  non-increasing in the oracle's c up to 1e-6;
* loads: exactly bincount of the GPU's picks, and equal to the oracle's loads
  for every expert once the exempt tokens' swaps are applied;
* gates: within 1e-5 of the oracle's gates evaluated at the GPU's picks;
* bias: bit-exact;
* outputs: max over tokens of ||y_gpu - y||_inf / ||y||_inf within the dtype's
  tolerance (fp32 1e-5, bf16 2e-2, fp8 6e-2 against the unquantised oracle,
  2e-2 against the quantisation-faithful one), on the whole output and on the
  expert part y - u alone; the oracle forward is driven by the GPU's routing
  so that an exempt token's legal swap is not counted as an output error.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import threading

import numpy as np
import torch

import mixture_experts_layer_adjusted_amd as moe
from oracle import moe_oracle as O
from synth import bf16_bits_to_f32, host
from synth.device import bf16_to_numpy_bits

GAP_EXEMPT = 1e-6
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "fp8_faithful": 2e-2}
DTYPE = {"f32": moe.MOE_DTYPE_F32, "bf16": moe.MOE_DTYPE_BF16, "fp8": moe.MOE_DTYPE_FP8_B128}


def shape_of(cfg, tokens=None):
    return moe.make_shape(cfg.tokens if tokens is None else tokens, cfg.hidden, cfg.n_routed, cfg.top_k,
                          cfg.n_shared, cfg.inter, DTYPE[cfg.dtype])


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(bf16_to_numpy_bits(t))
    return t.detach().float().cpu().numpy()


class Runner:
    """Holds device inputs and the workspace of one configuration."""

    def __init__(self, cfg, dev: dict, tokens=None):
        self.cfg = cfg
        self.dev = dev
        self.T = cfg.tokens if tokens is None else tokens
        self.shape = shape_of(cfg, self.T)
        nbytes = moe.moe_workspace_size(self.shape)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        K = cfg.top_k
        self.idx = torch.empty((self.T, K), dtype=torch.int32, device="cuda")
        self.gate = torch.empty((self.T, K), dtype=torch.float32, device="cuda")
        self.load = torch.empty((cfg.n_routed,), dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(dev["u"][: self.T] if dev["u"].dtype != torch.uint8 else dev["u"])
        self.weights = self.make_weights()

    def make_weights(self):
        d = self.dev
        sc = None
        if self.cfg.dtype == "fp8":
            sc = {k: d.get(k) for k in ("w_gate_scale", "w_up_scale", "w_down_scale", "sh_gate_scale",
                                        "sh_up_scale", "sh_down_scale")}
            return moe.make_weights(d["w_gate_q"], d["w_up_q"], d["w_down_q"], d.get("sh_gate_q"),
                                    d.get("sh_up_q"), d.get("sh_down_q"), scales=sc)
        ns = self.cfg.n_shared > 0
        return moe.make_weights(d["w_gate"], d["w_up"], d["w_down"], d["sh_gate"] if ns else None,
                                d["sh_up"] if ns else None, d["sh_down"] if ns else None)

    def route(self, bias=None):
        moe.moe_route(self.shape, self.dev["u"], self.dev["centroids"], self.dev["bias"] if bias is None else bias,
                      self.idx, self.gate, self.load, self.ws)

    def forward(self, idx=None, gate=None):
        moe.moe_forward(self.shape, self.dev["u"], self.weights, self.idx if idx is None else idx,
                        self.gate if gate is None else gate, self.out, self.ws)

    def update_bias(self, bias):
        moe.moe_update_bias(self.cfg.n_routed, self.T * self.cfg.top_k, self.load, bias, self.cfg.gamma)


def quantize_fp8_weights(dev: dict, cfg):
    """The library's own FP8 weight preparation (moe_quantize_weights) on the bf16 device weights."""
    for name in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        w = dev[name]
        n, r, c = w.shape
        codes = torch.empty((n, r, c), dtype=torch.uint8, device="cuda")
        scales = torch.empty((n, r // 128, c // 128), dtype=torch.float32, device="cuda")
        if n:
            moe.moe_quantize_weights(n, r, c, w, codes, scales)
        dev[name + "_q"] = codes
        dev[name + "_scale"] = scales
    return dev


def check_routing(idx_gpu, gate_gpu, load_gpu, s_or, c_or, idx_or, gap_or, n_routed):
    """Returns the boolean mask of exempt tokens; asserts every matching rule."""
    T, K = idx_gpu.shape
    assert np.array_equal(load_gpu, np.bincount(idx_gpu.ravel(), minlength=n_routed))
    assert np.all((idx_gpu >= 0) & (idx_gpu < n_routed))
    assert all(len(set(r)) == K for r in idx_gpu.tolist())
    exempt = gap_or < GAP_EXEMPT
    same = np.sort(idx_gpu, 1) == np.sort(idx_or, 1)
    bad = ~same.all(1) & ~exempt
    assert not bad.any(), f"{bad.sum()} non-exempt tokens differ, e.g. {np.nonzero(bad)[0][:5]}"
    c64 = c_or.astype(np.float64)
    ck = np.take_along_axis(c64, idx_or[:, K - 1:K], 1)
    cg = np.take_along_axis(c64, idx_gpu, 1)
    assert np.all(cg >= ck - GAP_EXEMPT), "an exempt token picked an illegal expert"
    assert np.all(cg[:, :-1] >= cg[:, 1:] - GAP_EXEMPT), "picks not ordered by score"
    g_or = O.gates(s_or, idx_gpu.astype(np.int64))
    np.testing.assert_allclose(gate_gpu, g_or, rtol=0, atol=1e-5)
    load_or = O.expert_load(idx_or, n_routed)
    # apply the exempt tokens' swaps to the oracle's load and compare exactly
    adj = load_or.copy()
    for t in np.nonzero(exempt)[0]:
        for e in idx_or[t]:
            adj[e] -= 1
        for e in idx_gpu[t]:
            adj[e] += 1
    assert np.array_equal(adj, load_gpu)
    return exempt


def check_grouped_routing(idx_gpu, gate_gpu, load_gpu, s_or, c_or, n_groups, topk_groups, n_routed):
    """Group-limited routing (R13) against the oracle; returns the mask of exempt tokens.

    Tokens whose oracle expert margin or group margin is below GAP_EXEMPT are exempt from the
    exact-set check; their picks must still come from at most topk_groups groups whose scores
    are within GAP_EXEMPT of the last eligible group's, be legal among those groups' experts,
    and be ordered by score.
    """
    T, K = idx_gpu.shape
    idx_or, gap, ggap = O.select_topk_grouped(c_or, K, n_groups, topk_groups)
    assert np.array_equal(load_gpu, np.bincount(idx_gpu.ravel(), minlength=n_routed))
    assert np.all((idx_gpu >= 0) & (idx_gpu < n_routed))
    assert all(len(set(r)) == K for r in idx_gpu.tolist())
    gs = n_routed // n_groups
    assert all(len(set((r // gs).tolist())) <= topk_groups for r in idx_gpu)
    exempt = (gap < GAP_EXEMPT) | (ggap < GAP_EXEMPT)
    same = np.sort(idx_gpu, 1) == np.sort(idx_or, 1)
    bad = ~same.all(1) & ~exempt
    assert not bad.any(), f"{bad.sum()} non-exempt tokens differ, e.g. {np.nonzero(bad)[0][:5]}"
    c64 = c_or.astype(np.float64)
    gsc = O.group_scores(c_or, n_groups)
    g_last = np.sort(gsc, 1)[:, ::-1][:, topk_groups - 1]
    for t in np.nonzero(exempt)[0]:
        groups = sorted(set((idx_gpu[t] // gs).tolist()))
        assert all(gsc[t, q] >= g_last[t] - GAP_EXEMPT for q in groups)
        allowed = [q for q in range(n_groups) if gsc[t, q] >= g_last[t] - GAP_EXEMPT]
        elig = np.concatenate([c64[t, q * gs:(q + 1) * gs] for q in allowed])
        ck = np.sort(elig)[::-1][K - 1]
        assert np.all(c64[t, idx_gpu[t]] >= ck - GAP_EXEMPT), "an exempt token picked an illegal expert"
    cg = np.take_along_axis(c64, idx_gpu, 1)
    assert np.all(cg[:, :-1] >= cg[:, 1:] - GAP_EXEMPT), "picks not ordered by score"
    np.testing.assert_allclose(gate_gpu, O.gates(s_or, idx_gpu.astype(np.int64)), rtol=0, atol=1e-5)
    return exempt


def rel_err(y_gpu, y_ref, u=None):
    """max_t ||y_gpu - y_ref||_inf / ||y_ref||_inf (and the same on y - u when u is given)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    e = np.max(np.abs(y_gpu - y_ref), 1) / np.maximum(np.max(np.abs(y_ref), 1), 1e-30)
    if u is None:
        return float(e.max())
    ue = np.asarray(u, np.float64)
    d_ref = y_ref - ue
    e2 = np.max(np.abs((y_gpu - ue) - d_ref), 1) / np.maximum(np.max(np.abs(d_ref), 1), 1e-30)
    return float(e.max()), float(e2.max())


# ----------------------------------------------------------------------------- sampling at the V3 shapes

def tile_covering_tokens(idx, n_routed, n_shared=1, seed=0, tile=128):
    """Tokens whose rows reach every 128-row M-tile of the padded permuted layout.

    Routed expert e's segment holds the tokens that picked e in increasing token order, and
    each shared segment holds every token in order; both start on a 128-row boundary, and
    the grouped GEMMs walk them in 256-row tiles (a segment's odd last M-tile is a half tile).
    Every M-tile of every segment gets at least one sampled row at a random position in the
    tile, so every 256-row tile, every half tile and every tile of the most loaded expert is
    compared.  Greedy: a tile that already holds a sampled token is skipped."""
    idx = np.asarray(idx)
    T = idx.shape[0]
    rng = np.random.default_rng(seed)
    mark = np.zeros(T, dtype=bool)
    segments = [np.nonzero((idx == e).any(axis=1))[0] for e in rng.permutation(n_routed)]
    if n_shared:
        segments.append(np.arange(T))
    for toks in segments:
        for m in range(0, len(toks), tile):
            rows = toks[m:m + tile]
            if not mark[rows].any():
                mark[rng.choice(rows)] = True
    return np.nonzero(mark)[0]


def oracle_pool():
    """Threads for the oracle's per-expert terms (numpy releases the GIL in its kernels)."""
    return cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1)))


def _f32(a):
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


class HostExperts:
    """Oracle-side expert weights regenerated from the seeded streams on the host; with fp8=True
    each matrix is quantised by the oracle's 128x128 block quantiser.  Nothing is copied from
    the device."""

    def __init__(self, cfg, fp8=False, report_every=32):
        self.cfg = cfg
        self.fp8 = fp8
        self._lock = threading.Lock()
        self._done = 0
        self._every = report_every

    @staticmethod
    def _quantize(w):
        # one 128-row strip of blocks at a time: blocks are independent, and the strips keep the
        # oracle's temporaries small enough for several threads to quantise at once
        parts = [O.quantize_weight_128x128(w[r:r + 128]) for r in range(0, w.shape[0], 128)]
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])

    def _prep(self, ws):
        ws = tuple(_f32(w) for w in ws)
        return tuple(self._quantize(w) for w in ws) if self.fp8 else ws

    def routed(self, e):
        w = self._prep(host.expert_weights(self.cfg, int(e)))
        with self._lock:
            self._done += 1
            if self._done % self._every == 0:
                print(f"  oracle: {self._done} routed experts prepared ({'fp8' if self.fp8 else 'bf16'})", flush=True)
        return w

    def shared(self):
        return [self._prep(host.expert_weights(self.cfg, s, shared=True)) for s in range(self.cfg.n_shared)]
