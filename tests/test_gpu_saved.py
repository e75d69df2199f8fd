"""GPU parity of the saved-input training pair (moe_forward_train, moe_backward_saved).

The forward keeps the SwiGLU inputs a = W_gate x and b = W_up x of every (token, expert) row
(方法 §2, "DeepSeek-V3 技術報告", xyznot.com/zh-tw/paper/2412.19437: the expert FFN is SwiGLU) and
the backward reads them in place of a second gate/up product.  Checked here:
* the forward's output is bit-identical to moe_forward's (same kernels, same epilogue);
* every saved row holds a, b of its (token, expert) pair, against the float64 products, with
  the rows placed by the permuted layout the forward documents (segment i: the tokens that
  picked routed expert i in token order, then one full-token segment per shared expert, each
  segment starting on a multiple of 128 rows);
* the gradients against the oracle's float64 backward, to the bf16 backward tolerance, and close
  to moe_backward's (the two differ only in rounding a and b to bf16);
* padding and unused rows of the saved buffer and the workspace never reach a gradient;
* FP8_B128: the same pair on E4M3 weights, against the oracle's FP8 backward with a and b held
  in bf16 (reading R17 on R16), to the FP8 backward's Frobenius / max-abs bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
from oracle import moe_oracle as O
from synth import host
from synth.configs import CONFIGS, LayerConfig
from synth.device import host_to_device, make_device_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from helpers import HostExperts, Runner, oracle_pool, to_host_f32
    from test_gpu_backward import BWD_TOL, _dout, _f, _grads_like, _rel, _row_rel
    from test_gpu_backward_fp8 import _check, _fro, _setup, _weights_q


def _small(name, T, d, N, K, Ns, I, cid, dtype="bf16"):
    return LayerConfig(cid, name, T, d, N, K, Ns, I, dtype, "uniform0.01")


def _saved_buffer(shape, fill=None):
    t = torch.empty(moe.moe_saved_inputs_size(shape) // 2, dtype=torch.bfloat16, device="cuda")
    if fill is not None:
        t.view(torch.uint8).fill_(fill)
    return t


def _backward_saved(cfg, r, dev, dout_d, saved, ws=None):
    T = r.T
    du = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    de = torch.empty((cfg.n_routed, cfg.hidden), dtype=torch.float32, device="cuda")
    g = _grads_like(dev, cfg.n_shared)
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    if ws is None:
        ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    moe.moe_backward_saved(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, saved, dout_d, du, de, wg,
                           ws)
    torch.cuda.synchronize()
    return du, de, g


def _backward(cfg, r, dev, dout_d):
    du = torch.empty((r.T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    de = torch.empty((cfg.n_routed, cfg.hidden), dtype=torch.float32, device="cuda")
    g = _grads_like(dev, cfg.n_shared)
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    moe.moe_backward(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout_d, du, de, wg, ws)
    torch.cuda.synchronize()
    return du, de, g


def _rows_of_layout(idx, T, n_routed, n_shared):
    """(row, token, expert) of every non-padding row of the permuted layout."""
    rows = []
    off = 0
    for e in range(n_routed):
        toks = np.nonzero((idx == e).any(1))[0]
        rows += [(off + j, int(t), e) for j, t in enumerate(toks)]
        off += -(-len(toks) // 128) * 128
    for s in range(n_shared):
        rows += [(off + t, t, n_routed + s) for t in range(T)]
        off += -(-T // 128) * 128
    return rows


CASES = [
    _small("saved-small", 200, 256, 16, 4, 1, 128, cid=80),
    _small("saved-two-shared", 512, 512, 16, 4, 2, 256, cid=81),
    _small("saved-no-shared-ragged", 77, 384, 8, 3, 0, 384, cid=82),
    # 512 routed + 64 shared segments, most routed ones a few rows or empty
    _small("saved-max-segments-sparse", 512, 128, 512, 8, 64, 128, cid=83),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_train_output_and_saved_rows(cfg):
    print(f"forward_train: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} K={cfg.top_k} "
          f"Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    hf = {k: _f(v) for k, v in h.items()}
    dev = host_to_device(h)
    r = Runner(cfg, dev)
    r.route()
    r.forward()
    ref_out = r.out.clone()
    saved = _saved_buffer(r.shape, fill=0xFF)
    out = torch.empty_like(ref_out)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, out, saved, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    idx = r.idx.cpu().numpy().astype(np.int64)
    I = cfg.inter
    sv = to_host_f32(saved.view(-1, 2 * I))
    u = hf["u"].astype(np.float64)
    worst = 0.0
    for row, t, e in _rows_of_layout(idx, cfg.tokens, cfg.n_routed, cfg.n_shared):
        if e < cfg.n_routed:
            wg_, wu_ = hf["w_gate"][e], hf["w_up"][e]
        else:
            wg_, wu_ = hf["sh_gate"][e - cfg.n_routed], hf["sh_up"][e - cfg.n_routed]
        ab = np.concatenate([wg_.astype(np.float64) @ u[t], wu_.astype(np.float64) @ u[t]])
        worst = max(worst, float(np.max(np.abs(sv[row] - ab)) / np.max(np.abs(ab))))
    print(f"saved [a b] rows: worst row-relative error {worst:.5f}", flush=True)
    assert worst <= 1e-2


# the largest segment count with full 256-row tiles in the input-gradient products (backward
# only: the saved-row walk above would take minutes at 590 K rows)
BWD_CASES = CASES + [_small("saved-max-segments", 8192, 128, 512, 8, 64, 128, cid=89)]


@pytest.mark.parametrize("cfg", BWD_CASES, ids=lambda c: c.name)
def test_backward_saved_parity(cfg):
    print(f"backward_saved: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} K={cfg.top_k} "
          f"Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    hf = {k: _f(v) for k, v in h.items()}
    dev = host_to_device(h)
    r = Runner(cfg, dev)
    r.route()
    saved = _saved_buffer(r.shape, fill=0xFF)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _backward_saved(cfg, r, dev, dout_d, saved)
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
                                           O.Bf16SavedPolicy)
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
    # against the recomputing backward: the same gradients up to the bf16 rounding of a and b
    du_r, de_r, g_r = _backward(cfg, r, dev, dout_d)
    errs["du_vs_recompute"] = _row_rel(to_host_f32(du), to_host_f32(du_r))
    print("relative errors:", {k: round(v, 5) for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= BWD_TOL, (k, v)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_backward_saved_ignores_poisoned_padding(dtype):
    """Saved buffer and workspace filled with NaN / arbitrary bytes before the calls give the
    same, finite gradients as zero-filled ones: padding rows and rows past the last segment are
    never read into a gradient."""
    cfg = _small("saved-poison", 77, 384, 8, 3, 1, 384, cid=84, dtype=dtype)
    h = host.make_host_inputs(cfg)
    dev = host_to_device(h)
    if dtype == "fp8":
        dev, r = _setup(cfg, dev)
    else:
        r = Runner(cfg, dev)
        r.route()
    dout_d, _ = _dout(cfg, cfg.tokens)
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    outs = []
    for fill in (0x00, 0xFF):
        saved = _saved_buffer(r.shape, fill=fill)
        r.ws.fill_(fill)
        ws.fill_(0x55 if fill else 0x00)
        moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
        outs.append(_backward_saved(cfg, r, dev, dout_d, saved, ws))
    for t in (outs[1][0], outs[1][1]):
        assert torch.isfinite(t.float()).all()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    for k, t in outs[0][2].items():
        if t is not None:
            assert torch.isfinite(outs[1][2][k].float()).all(), k
            assert torch.equal(t.view(torch.int16), outs[1][2][k].view(torch.int16)), k


def test_backward_saved_v3_decode_shape_sampled():
    cfg = CONFIGS[2]   # T=256, d=7168, N_r=256, K_r=8, N_s=1, I=2048
    print("backward_saved: V3 decode shape, sampled tokens and experts", flush=True)
    dev = make_device_inputs(cfg)
    r = Runner(cfg, dev)
    r.route()
    saved = _saved_buffer(r.shape)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _backward_saved(cfg, r, dev, dout_d, saved)
    idx = r.idx.cpu().numpy().astype(np.int64)
    u_h = _f(host.token_rows(cfg))
    c_h = host.centroids(cfg)
    uniq = np.unique(idx)
    experts = [int(e) for e in uniq[:: max(1, len(uniq) // 3)][:3]]
    toks = sorted(set(np.arange(0, cfg.tokens, 61).tolist()) | set(np.nonzero(np.isin(idx, experts).any(1))[0].tolist()))
    toks = np.array(toks)
    cache = {}

    def routed(e):
        if e not in cache:
            cache[e] = tuple(_f(w) for w in host.expert_weights(cfg, e))
        return cache[e]

    shared = [tuple(_f(w) for w in host.expert_weights(cfg, s, shared=True)) for s in range(cfg.n_shared)]
    du_o, de_o, dr_o, _ = O.layer_backward(u_h[toks], c_h, idx[toks], routed, shared, dout_h[toks])
    _, de_m, _, _ = O.layer_backward_steps(u_h[toks], c_h, idx[toks], routed, shared, dout_h[toks],
                                           O.Bf16SavedPolicy)
    e_du = _row_rel(to_host_f32(du)[toks], du_o)
    e_de = _row_rel(de.cpu().numpy()[experts], de_m[experts])   # against the storage model (R17)
    print(f"de against the exact backward (not asserted): {_row_rel(de.cpu().numpy()[experts], de_o[experts]):.5f}")
    e_w = 0.0
    for e in experts:
        for name, j in (("w_gate", 0), ("w_up", 1), ("w_down", 2)):
            e_w = max(e_w, _rel(to_host_f32(g[name][e]), dr_o[e][j]))
    print(f"relative errors: du {e_du:.5f} de {e_de:.5f} dW {e_w:.5f} over {len(toks)} tokens, experts {experts}")
    assert e_du <= BWD_TOL and e_de <= BWD_TOL and e_w <= BWD_TOL


def _pick_experts(load):
    """The most loaded expert, and one whose segment has at least one full 256-row tile and
    ends in a half tile (an odd count of 128-row M-tiles)."""
    top = int(np.argmax(load))
    mt = -(-load // 128)
    half = np.nonzero((mt % 2 == 1) & (load > 256))[0]
    return top, int(half[np.argsort(load[half])[len(half) // 2]])


def test_backward_prefill_shape_against_oracle():
    """T = 16384 at the V3 shape (Zipf routing): moe_backward and moe_backward_saved against the
    float64 oracle (R14).  du on sampled tokens, each from the oracle over that token's own rows,
    and every weight gradient of two experts from the oracle's steps over exactly that expert's
    rows: the most loaded one (its segment spans some 18 256-row tiles) and one whose segment ends
    in a half tile."""
    cfg = CONFIGS[3]   # T=16384, d=7168, N_r=256, K_r=8, N_s=1, I=2048
    print("backward and backward_saved vs the oracle: V3 prefill shape", flush=True)
    dev = make_device_inputs(cfg)
    r = Runner(cfg, dev)
    r.route()
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    idx = r.idx.cpu().numpy().astype(np.int64)
    load = np.bincount(idx.ravel(), minlength=cfg.n_routed)
    experts = _pick_experts(load)
    toks = np.random.default_rng(16).choice(cfg.tokens, 16, replace=False)
    got = {}
    for kind in ("recompute", "saved"):
        if kind == "saved":
            saved = _saved_buffer(r.shape)
            moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
            du, de, g = _backward_saved(cfg, r, dev, dout_d, saved)
            del saved
        else:
            du, de, g = _backward(cfg, r, dev, dout_d)
        got[kind] = (to_host_f32(du)[toks],
                     {e: tuple(to_host_f32(g[n][e]) for n in ("w_gate", "w_up", "w_down")) for e in experts})
        del du, de, g
        torch.cuda.empty_cache()
    u_h = _f(host.token_rows(cfg))
    c_h = host.centroids(cfg)
    ex = HostExperts(cfg)
    with oracle_pool() as pool:
        du_o, _, _, _ = O.layer_backward(u_h[toks], c_h, idx[toks], ex.routed, ex.shared(), dout_h[toks],
                                         map=pool.map)
    s_all = O.affinity64(u_h, c_h)
    dw_o = {}
    for e in experts:
        rows, slots = np.nonzero(idx == e)
        ssel = np.take_along_axis(s_all[rows], idx[rows], axis=1)
        gate = ssel[np.arange(len(rows)), slots] / ssel.sum(axis=1)
        P = O.ExactPolicy
        _, _, dw_o[e] = O.expert_backward(u_h[rows], dout_h[rows], u_h[rows], dout_h[rows], gate, *ex.routed(e), P)
    print(f"tokens {sorted(toks.tolist())}; experts {experts} with {[int(load[e]) for e in experts]} rows", flush=True)
    for kind, (du_g, dw_g) in got.items():
        errs = {"du": _row_rel(du_g, du_o)}
        for e in experts:
            for j, name in enumerate(("dWg", "dWu", "dWd")):
                errs[f"{name}[{e}]"] = _rel(dw_g[e][j], dw_o[e][j])
        print(kind, "relative errors:", {k: round(v, 5) for k, v in errs.items()}, flush=True)
        for k, v in errs.items():
            assert v <= BWD_TOL, (kind, k, v)


FP8_CASES = [
    _small("saved-fp8-small", 200, 256, 16, 4, 1, 128, cid=85, dtype="fp8"),
    _small("saved-fp8-two-shared", 512, 512, 16, 4, 2, 256, cid=86, dtype="fp8"),
    _small("saved-fp8-max-segments-sparse", 512, 128, 512, 8, 64, 128, cid=87, dtype="fp8"),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=lambda c: c.name)
def test_fp8_saved_pair_parity(cfg):
    print(f"fp8 saved pair: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} K={cfg.top_k} "
          f"Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    hf = {k: _f(v) for k, v in h.items()}
    dev, r = _setup(cfg, host_to_device(h))
    r.forward()
    ref_out = r.out.clone()
    saved = _saved_buffer(r.shape, fill=0xFF)
    out = torch.empty_like(ref_out)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, out, saved, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _backward_saved(cfg, r, dev, dout_d, saved)
    idx = r.idx.cpu().numpy().astype(np.int64)
    shq = _weights_q(hf, "sh_")
    du_o, de_o, dr_o, dsh_o = O.layer_backward_fp8(hf["u"], hf["centroids"], idx, _weights_q(hf, "w_"),
                                                   [shq(s) for s in range(cfg.n_shared)], dout_h, saved=True)
    du_g = to_host_f32(du)
    errs = {"du": (_fro(du_g - dout_h, du_o - dout_h), _row_rel(du_g, du_o))}
    de_g = de.cpu().numpy()
    used = sorted(dr_o)
    errs["de"] = (_fro(de_g[used], de_o[used]), _row_rel(de_g[used], de_o[used]))
    assert np.all(de_g[[e for e in range(cfg.n_routed) if e not in dr_o]] == 0)
    w = (0.0, 0.0)
    for name, j in (("w_gate", 0), ("w_up", 1), ("w_down", 2)):
        got = to_host_f32(g[name])
        for e in range(cfg.n_routed):
            if e in dr_o:
                w = (max(w[0], _fro(got[e], dr_o[e][j])), max(w[1], _rel(got[e], dr_o[e][j])))
            else:
                assert np.all(got[e] == 0), (name, e)
    errs["dW_routed"] = w
    w = (0.0, 0.0)
    for s_i, grads in enumerate(dsh_o):
        for name, j in (("sh_gate", 0), ("sh_up", 1), ("sh_down", 2)):
            got = to_host_f32(g[name])[s_i]
            w = (max(w[0], _fro(got, grads[j])), max(w[1], _rel(got, grads[j])))
    errs["dW_shared"] = w
    _check(errs)


# Two FP8 models apart: a, b rounded to bf16 move some E4M3 codes of dA and dB by one step.  The
# oracle bounds that distance between its own two FP8 variants by 2e-2 (Frobenius,
# tests/test_oracle_backward_bf16.py); one E4M3 step moves an element by at most 1/8 of itself.
FP8_SAVED_VS_RECOMPUTE_FRO = 2e-2
FP8_SAVED_VS_RECOMPUTE_MAX = 0.125


def test_fp8_saved_prefill_shape_matches_recompute():
    """T = 8192 at the V3 shape: the FP8 saved path against the FP8 recomputing backward, per
    expert matrix and on du - dout, within the distance the two FP8 models allow each other (the
    oracle's parity of each is checked on the small cases)."""
    cfg = CONFIGS[4]
    print("fp8 backward_saved vs moe_backward: V3 prefill shape, T=8192", flush=True)
    dev, r = _setup(cfg, make_device_inputs(cfg))
    saved = _saved_buffer(r.shape)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
    dout_d, _ = _dout(cfg, cfg.tokens)
    a = _backward_saved(cfg, r, dev, dout_d, saved)
    del saved
    b = _backward(cfg, r, dev, dout_d)
    x, y = a[0].float() - dout_d.float(), b[0].float() - dout_d.float()
    worst = {"du": ((x - y).norm() / y.norm()).item()}
    for k in ("w_gate", "w_up", "w_down"):
        x, y = a[2][k].float(), b[2][k].float()
        used = y.flatten(1).abs().amax(1) > 0
        fro = ((x - y)[used].flatten(1).norm(dim=1) / y[used].flatten(1).norm(dim=1)).max().item()
        mx = ((x - y)[used].flatten(1).abs().amax(1) / y[used].flatten(1).abs().amax(1)).max().item()
        worst[k] = (fro, mx)
        del x, y
    print("relative differences (frobenius[, max-abs]):", worst, flush=True)
    assert worst["du"] <= FP8_SAVED_VS_RECOMPUTE_FRO
    for k in ("w_gate", "w_up", "w_down"):
        assert worst[k][0] <= FP8_SAVED_VS_RECOMPUTE_FRO and worst[k][1] <= FP8_SAVED_VS_RECOMPUTE_MAX, (k, worst[k])


def test_saved_pair_zero_tokens():
    """T = 0: moe_forward_train is a no-op (a null saved buffer is allowed) and moe_backward_saved
    writes zero weight and centroid gradients, as moe_backward does."""
    cfg = _small("saved-empty", 64, 256, 8, 2, 1, 128, cid=64)
    dev = host_to_device(host.make_host_inputs(cfg))
    r = Runner(cfg, dev, tokens=0)
    moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, None, r.ws)
    g = _grads_like(dev, 1)
    for t in g.values():
        t.fill_(1.0)
    de = torch.full((cfg.n_routed, cfg.hidden), 1.0, dtype=torch.float32, device="cuda")
    du = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dout = torch.zeros((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    saved = _saved_buffer(r.shape, fill=0xFF)
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    moe.moe_backward_saved(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, saved, dout, du, de, wg, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(de) == 0
    for k, t in g.items():
        assert torch.count_nonzero(t) == 0, k
