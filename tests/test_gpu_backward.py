"""GPU parity of the layer backward (moe_backward) against the oracle's float64 backward.

Gradients of <dout, h'> for the h'_t equation of 方法 §2 ("DeepSeek-V3 技術報告",
xyznot.com/zh-tw/paper/2412.19437), routing held fixed (reading R14 of oracle/moe_oracle.py,
pinned by tests/test_oracle_backward.py).  Metric as for the forward: per token (or per expert
row / matrix) max-abs error over max-abs value, against the bf16 tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
import synth
from oracle import moe_oracle as O
from synth import bf16_bits_to_f32, host
from synth.configs import CONFIGS, LayerConfig
from synth.device import fill_normal_, host_to_device, make_device_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from helpers import TOL, Runner, to_host_f32

BWD_TOL = 2e-2


def _f(a):
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def _rel(x, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x)))


def _row_rel(x, ref):
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(np.max(np.abs(x - ref), axis=1) / np.where(den > 0, den, 1.0)))


def _dout(cfg, T):
    key = synth.stream_key(cfg.seed, cfg.cid, synth.TAG_DOUT, 0)
    dev = fill_normal_(torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda"), key, 1.0)
    return dev, _f(host.host_normal(key, T * cfg.hidden, 1.0, bf16=True).reshape(T, cfg.hidden))


def _grads_like(dev, ns):
    g = {k: torch.empty_like(dev[k]) for k in ("w_gate", "w_up", "w_down")}
    for k in ("sh_gate", "sh_up", "sh_down"):
        g[k] = torch.empty_like(dev[k]) if ns else None
    return g


def _run_backward(cfg, r, dev, dout_d):
    T = r.T
    du = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    de = torch.empty((cfg.n_routed, cfg.hidden), dtype=torch.float32, device="cuda")
    g = _grads_like(dev, cfg.n_shared)
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    moe.moe_backward(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout_d, du, de, wg, ws)
    torch.cuda.synchronize()
    return du, de, g


def _small(name, T, d, N, K, Ns, I, bias="uniform0.01", cid=60):
    return LayerConfig(cid, name, T, d, N, K, Ns, I, "bf16", bias)


@pytest.mark.parametrize("cfg", [
    _small("bwd-small", 200, 256, 16, 4, 1, 128),
    _small("bwd-two-shared", 512, 512, 16, 4, 2, 256, cid=61),
    _small("bwd-no-shared-ragged", 77, 384, 8, 3, 0, 384, cid=62),
    # the most segments the library takes (512 routed + 64 shared): the segment tables the
    # persistent kernels copy to LDS at their largest; at T=512 most routed segments hold a few
    # rows or none (weight-gradient tiles without K-steps), at T=8192 the input-gradient
    # products run on full 256-row tiles
    _small("bwd-max-segments-sparse", 512, 128, 512, 8, 64, 128, cid=66),
    _small("bwd-max-segments", 8192, 128, 512, 8, 64, 128, cid=67),
], ids=lambda c: c.name)
def test_backward_parity_small(cfg):
    print(f"backward: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} K={cfg.top_k} "
          f"Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    hf = {k: _f(v) for k, v in h.items()}
    dev = host_to_device(h)
    r = Runner(cfg, dev)
    r.route()
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _run_backward(cfg, r, dev, dout_d)
    idx = r.idx.cpu().numpy().astype(np.int64)
    shared = list(zip(hf["sh_gate"], hf["sh_up"], hf["sh_down"]))
    du_o, de_o, dr_o, dsh_o = O.layer_backward(hf["u"], hf["centroids"], idx,
                                               O.stacked(hf["w_gate"], hf["w_up"], hf["w_down"]), shared, dout_h)
    errs = {"du": _row_rel(to_host_f32(du), du_o)}
    de_g = de.cpu().numpy()
    used = sorted(dr_o)
    # the centroid gradient of an expert with one or two tokens is ill-conditioned (ds cancels):
    # it is held to the oracle's bf16 storage model (reading R17), the exact value is printed
    _, de_m, _, _ = O.layer_backward_steps(hf["u"], hf["centroids"], idx,
                                           O.stacked(hf["w_gate"], hf["w_up"], hf["w_down"]), shared, dout_h,
                                           O.Bf16Policy)
    errs["de"] = _row_rel(de_g[used], de_m[used])
    print(f"de against the exact backward (not asserted): {_row_rel(de_g[used], de_o[used]):.5f}", flush=True)
    unused = [e for e in range(cfg.n_routed) if e not in dr_o]
    assert np.all(de_g[unused] == 0)
    wmax = 0.0
    for name, j in (("w_gate", 0), ("w_up", 1), ("w_down", 2)):
        got = to_host_f32(g[name])
        for e in range(cfg.n_routed):
            if e in dr_o:
                wmax = max(wmax, _rel(got[e], dr_o[e][j]))
            else:
                assert np.all(got[e] == 0), (name, e)
    errs["dW_routed"] = wmax
    smax = 0.0
    for s_i, grads in enumerate(dsh_o):
        for name, j in (("sh_gate", 0), ("sh_up", 1), ("sh_down", 2)):
            smax = max(smax, _rel(to_host_f32(g[name])[s_i], grads[j]))
    errs["dW_shared"] = smax
    print("relative errors:", {k: round(v, 5) for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL, (k, v)


def test_backward_is_deterministic():
    cfg = _small("bwd-det", 300, 256, 16, 4, 1, 256, cid=63)
    h = host.make_host_inputs(cfg)
    dev = host_to_device(h)
    r = Runner(cfg, dev)
    r.route()
    dout_d, _ = _dout(cfg, cfg.tokens)
    a = _run_backward(cfg, r, dev, dout_d)
    b = _run_backward(cfg, r, dev, dout_d)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    for k in a[2]:
        if a[2][k] is not None:
            assert torch.equal(a[2][k].view(torch.int16), b[2][k].view(torch.int16)), k


def test_backward_v3_decode_shape_sampled():
    cfg = CONFIGS[2]   # T=256, d=7168, N_r=256, K_r=8, N_s=1, I=2048
    print("backward: V3 decode shape, sampled tokens and experts", flush=True)
    dev = make_device_inputs(cfg)
    r = Runner(cfg, dev)
    r.route()
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _run_backward(cfg, r, dev, dout_d)
    idx = r.idx.cpu().numpy().astype(np.int64)
    u_h = _f(host.token_rows(cfg))
    c_h = host.centroids(cfg)
    experts = [int(e) for e in np.unique(idx)[:: max(1, len(np.unique(idx)) // 3)][:3]]
    toks = sorted(set(np.arange(0, cfg.tokens, 61).tolist()) | set(np.nonzero(np.isin(idx, experts).any(1))[0].tolist()))
    toks = np.array(toks)
    cache = {}

    def routed(e):
        if e not in cache:
            cache[e] = tuple(_f(w) for w in host.expert_weights(cfg, e))
        return cache[e]

    shared = [tuple(_f(w) for w in host.expert_weights(cfg, s, shared=True)) for s in range(cfg.n_shared)]
    du_o, de_o, dr_o, _ = O.layer_backward(u_h[toks], c_h, idx[toks], routed, shared, dout_h[toks])
    e_du = _row_rel(to_host_f32(du)[toks], du_o)
    de_g = de.cpu().numpy()
    e_de = _row_rel(de_g[experts], de_o[experts])
    e_w = 0.0
    for e in experts:
        for name, j in (("w_gate", 0), ("w_up", 1), ("w_down", 2)):
            e_w = max(e_w, _rel(to_host_f32(g[name][e]), dr_o[e][j]))
    print(f"relative errors: du {e_du:.5f} de {e_de:.5f} dW {e_w:.5f} over {len(toks)} tokens, experts {experts}")
    assert e_du <= BWD_TOL and e_de <= BWD_TOL and e_w <= BWD_TOL


def test_backward_ignores_stale_workspace():
    """Every row of the permuted layout that the backward's passes touch is defined by the call
    itself: a workspace holding arbitrary bytes from earlier use gives the same gradients."""
    cfg = _small("bwd-stale", 77, 384, 8, 3, 0, 384, cid=65)
    h = host.make_host_inputs(cfg)
    dev = host_to_device(h)
    r = Runner(cfg, dev)
    r.route()
    dout_d, _ = _dout(cfg, cfg.tokens)
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    outs = []
    for fill in (0x00, 0x55):
        ws.fill_(fill)
        du = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        de = torch.empty((cfg.n_routed, cfg.hidden), dtype=torch.float32, device="cuda")
        g = _grads_like(dev, 0)
        wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"])
        moe.moe_backward(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout_d, du, de, wg, ws)
        torch.cuda.synchronize()
        outs.append((du, de, g))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    for k in ("w_gate", "w_up", "w_down"):
        assert torch.equal(outs[0][2][k].view(torch.int16), outs[1][2][k].view(torch.int16)), k


def test_backward_zero_tokens_writes_zero_gradients():
    cfg = _small("bwd-empty", 64, 256, 8, 2, 1, 128, cid=64)
    h = host.make_host_inputs(cfg)
    dev = host_to_device(h)
    r = Runner(cfg, dev, tokens=0)
    shape = r.shape
    g = _grads_like(dev, 1)
    for t in g.values():
        t.fill_(1.0)
    de = torch.full((cfg.n_routed, cfg.hidden), 1.0, dtype=torch.float32, device="cuda")
    du = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dout = torch.zeros((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_backward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    moe.moe_backward(shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout, du, de, wg, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(de) == 0
    for k, t in g.items():
        assert torch.count_nonzero(t) == 0, k
