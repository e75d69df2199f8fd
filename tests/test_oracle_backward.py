"""Pins of the oracle's layer backward (reading R14 of oracle/moe_oracle.py).

The gradients of L = <dout, h'> (h' of 方法 §2, "DeepSeek-V3 技術報告",
xyznot.com/zh-tw/paper/2412.19437) for a fixed selection are checked against
central finite differences of the oracle's own float64 forward, against reverse-mode
differentiation of an independent torch float64 statement of the same forward on the CPU,
and against the closed form when every expert's down projection is zero.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _layer(seed=0, T=5, d=8, N=6, K=2, I=4, Ns=2):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, d))
    e = rng.standard_normal((N, d)) / np.sqrt(d)
    b = rng.standard_normal(N) * 0.1
    wg = rng.standard_normal((N, I, d)) / np.sqrt(d)
    wu = rng.standard_normal((N, I, d)) / np.sqrt(d)
    wd = rng.standard_normal((N, d, I)) / np.sqrt(I)
    sh = [tuple(rng.standard_normal(sz) / np.sqrt(sz[1]) for sz in ((I, d), (I, d), (d, I))) for _ in range(Ns)]
    dout = rng.standard_normal((T, d))
    c = O.affinity64(u, e) + b
    idx, _ = O.select_topk(c, K)
    return dict(u=u, e=e, wg=wg, wu=wu, wd=wd, sh=sh, dout=dout, idx=idx)


def _loss(L):
    s = O.affinity64(L["u"], L["e"])
    ssel = np.take_along_axis(s, L["idx"], 1)
    gate = ssel / ssel.sum(1, keepdims=True)
    y = O.layer_forward(L["u"], L["idx"], gate, O.stacked(L["wg"], L["wu"], L["wd"]), L["sh"])
    return float(np.sum(L["dout"] * y))


def _grads(L):
    return O.layer_backward(L["u"], L["e"], L["idx"], O.stacked(L["wg"], L["wu"], L["wd"]), L["sh"], L["dout"])


def test_backward_matches_finite_differences():
    L = _layer()
    du, de, dr, dsh = _grads(L)
    rng = np.random.default_rng(1)
    eps = 1e-6

    def check(arr, pos, analytic):
        old = arr[pos]
        arr[pos] = old + eps
        lp = _loss(L)
        arr[pos] = old - eps
        lm = _loss(L)
        arr[pos] = old
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - analytic) <= 1e-7 + 1e-6 * abs(fd), (pos, fd, analytic)

    for _ in range(12):
        p = tuple(rng.integers(0, n) for n in L["u"].shape)
        check(L["u"], p, du[p])
        p = tuple(rng.integers(0, n) for n in L["e"].shape)
        check(L["e"], p, de[p])
    for ex, (dwg, dwu, dwd) in dr.items():
        for arr, g in ((L["wg"][ex], dwg), (L["wu"][ex], dwu), (L["wd"][ex], dwd)):
            p = tuple(rng.integers(0, n) for n in arr.shape)
            check(arr, p, g[p])
    for (wg, wu, wd), (dwg, dwu, dwd) in zip(L["sh"], dsh):
        for arr, g in ((wg, dwg), (wu, dwu), (wd, dwd)):
            p = tuple(rng.integers(0, n) for n in arr.shape)
            check(arr, p, g[p])
    # an expert never picked gets no weight gradient entry and a zero centroid gradient
    unused = sorted(set(range(L["e"].shape[0])) - set(L["idx"].ravel().tolist()))
    for ex in unused:
        assert ex not in dr and np.all(de[ex] == 0)


def test_backward_matches_torch_autograd():
    L = _layer(seed=3, T=7, d=12, N=8, K=3, I=6, Ns=1)
    du, de, dr, dsh = _grads(L)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in L.items() if k in ("u", "e", "wg", "wu", "wd")}
    sh = [tuple(torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in ws) for ws in L["sh"]]
    idx = torch.tensor(L["idx"])
    s = torch.sigmoid(t["u"] @ t["e"].T)
    ssel = torch.gather(s, 1, idx)
    gate = ssel / ssel.sum(1, keepdim=True)

    def ffn(x, wg, wu, wd):
        return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T

    out = t["u"].clone()
    for wg, wu, wd in sh:
        out = out + ffn(t["u"], wg, wu, wd)
    for tok in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            ex = int(idx[tok, k])
            out[tok] = out[tok] + gate[tok, k] * ffn(t["u"][tok:tok + 1], t["wg"][ex], t["wu"][ex], t["wd"][ex])[0]
    (out * torch.tensor(L["dout"])).sum().backward()
    np.testing.assert_allclose(du, t["u"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(de, t["e"].grad.numpy(), rtol=1e-10, atol=1e-12)
    for ex, (dwg, dwu, dwd) in dr.items():
        np.testing.assert_allclose(dwg, t["wg"].grad[ex].numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dwu, t["wu"].grad[ex].numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dwd, t["wd"].grad[ex].numpy(), rtol=1e-10, atol=1e-12)
    for ws, gs in zip(sh, dsh):
        for w, g in zip(ws, gs):
            np.testing.assert_allclose(g, w.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_with_zero_down_projections():
    L = _layer(seed=5)
    L["wd"][:] = 0.0
    L["sh"] = [(wg, wu, np.zeros_like(wd)) for wg, wu, wd in L["sh"]]
    du, de, dr, dsh = _grads(L)
    # every expert output is 0: du is the residual path alone, no gate or centroid gradient,
    # and only the down projections receive gradients
    assert np.array_equal(du, L["dout"])
    assert np.all(de == 0)
    for dwg, dwu, dwd in list(dr.values()) + dsh:
        assert np.all(dwg == 0) and np.all(dwu == 0) and np.any(dwd != 0)
