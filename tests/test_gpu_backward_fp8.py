"""GPU parity of the FP8 layer backward (moe_backward with FP8_B128 weights) against the oracle's
quantisation-faithful backward (reading R16 of oracle/moe_oracle.py, pinned by
tests/test_oracle_backward_fp8.py).

The page "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437) makes the forward GEMM and
both backward GEMMs FP8 (section 方法, FP8 Mixed Precision Training; 核心概念, FP8 item).  Both
sides quantise the same held values, so the comparison is to the quantisation-faithful
tolerance of the forward, with one difference.  In the backward a tensor's E4M3 codes are taken
from values that an earlier FP8 product and a bf16 store produced, so the GPU's fp32 accumulation
and the oracle's float64 can round a held value differently, which moves a code (or a run's
scale) by one step: the oracle itself moves by up to ~1% in max-abs terms under a 1e-6 relative
perturbation of its held values, while its Frobenius-norm change stays ~0.1%.  A misplaced
scale or operand moves either by >10%.  So each gradient matrix (and du - dout) is held to a
relative Frobenius-norm error of 1e-2, and to a max-abs error over max-abs value of 5e-2.
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
    from helpers import HostExperts, Runner, oracle_pool, quantize_fp8_weights, to_host_f32

FP8_BWD_FRO = 1e-2
FP8_BWD_MAX = 5e-2


def _f(a):
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def _rel(x, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x)))


def _fro(x, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def _check(errs):
    """errs: name -> (frobenius, max-abs)."""
    print("relative errors (frobenius, max-abs) vs the quantisation-faithful oracle:",
          {k: (round(a, 5), round(b, 5)) for k, (a, b) in errs.items()}, flush=True)
    for k, (a, b) in errs.items():
        assert a <= FP8_BWD_FRO and b <= FP8_BWD_MAX, (k, a, b)


def _row_rel(x, ref):
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(np.max(np.abs(x - ref), axis=1) / np.where(den > 0, den, 1.0)))


def _dout(cfg, T):
    key = synth.stream_key(cfg.seed, cfg.cid, synth.TAG_DOUT, 0)
    dev = fill_normal_(torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda"), key, 1.0)
    return dev, _f(host.host_normal(key, T * cfg.hidden, 1.0, bf16=True).reshape(T, cfg.hidden))


def _small(name, T, d, N, K, Ns, I, cid):
    return LayerConfig(cid, name, T, d, N, K, Ns, I, "fp8", "uniform0.01")


def _weights_q(hf, prefix):
    """Accessor e -> ((codes, scale) x 3): the oracle's 128x128 block quantiser applied to the host
    copies of the bf16 weights (nothing is read back from the device)."""
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = tuple(O.quantize_weight_128x128(hf[f"{prefix}{n}"][e]) for n in ("gate", "up", "down"))
        return cache[e]
    return get


def _run_backward(cfg, r, dev, dout_d):
    T = r.T
    du = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    de = torch.empty((cfg.n_routed, cfg.hidden), dtype=torch.float32, device="cuda")
    g = {k: torch.empty(dev[k].shape, dtype=torch.bfloat16, device="cuda") for k in ("w_gate", "w_up", "w_down")}
    for k in ("sh_gate", "sh_up", "sh_down"):
        g[k] = torch.empty(dev[k].shape, dtype=torch.bfloat16, device="cuda") if cfg.n_shared else None
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    moe.moe_backward(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout_d, du, de, wg, ws)
    torch.cuda.synchronize()
    return du, de, g


def _setup(cfg, dev=None):
    if dev is None:
        dev = host_to_device(host.make_host_inputs(cfg))
    dev = quantize_fp8_weights(dev, cfg)
    r = Runner(cfg, dev)
    r.route()
    return dev, r


@pytest.mark.parametrize("cfg", [
    _small("fp8-bwd-small", 200, 256, 16, 4, 1, 128, cid=70),
    _small("fp8-bwd-two-shared", 512, 512, 16, 4, 2, 256, cid=71),
    _small("fp8-bwd-no-shared-ragged", 77, 384, 8, 3, 0, 384, cid=72),
    # 512 routed + 64 shared segments (the largest segment table, copied to LDS by the
    # weight-gradient kernel), most routed segments with a few rows or none
    _small("fp8-bwd-max-segments-sparse", 512, 128, 512, 8, 64, 128, cid=77),
], ids=lambda c: c.name)
def test_fp8_backward_parity_small(cfg):
    print(f"fp8 backward: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} K={cfg.top_k} "
          f"Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    hf = {k: _f(v) for k, v in h.items()}
    dev, r = _setup(cfg, host_to_device(h))
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _run_backward(cfg, r, dev, dout_d)
    idx = r.idx.cpu().numpy().astype(np.int64)
    shq = _weights_q(hf, "sh_")
    du_o, de_o, dr_o, dsh_o = O.layer_backward_fp8(hf["u"], hf["centroids"], idx, _weights_q(hf, "w_"),
                                                   [shq(s) for s in range(cfg.n_shared)], dout_h)
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


def test_fp8_backward_is_deterministic():
    cfg = _small("fp8-bwd-det", 300, 256, 16, 4, 1, 256, cid=73)
    dev, r = _setup(cfg)
    dout_d, _ = _dout(cfg, cfg.tokens)
    a = _run_backward(cfg, r, dev, dout_d)
    b = _run_backward(cfg, r, dev, dout_d)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    for k in a[2]:
        if a[2][k] is not None:
            assert torch.equal(a[2][k].view(torch.int16), b[2][k].view(torch.int16)), k


def test_fp8_backward_v3_prefill_sampled():
    """T = 8192 at the V3 shape (d=7168, N_r=256, K_r=8, N_s=1, I=2048): du of sampled tokens and
    the weight gradients of one routed expert with more than one 128-row run, each from the
    oracle's steps over exactly the rows they depend on."""
    cfg = CONFIGS[4]
    print("fp8 backward: V3 prefill shape, sampled tokens and one expert", flush=True)
    dev, r = _setup(cfg, make_device_inputs(cfg))
    dout_d, dout_h = _dout(cfg, cfg.tokens)
    du, de, g = _run_backward(cfg, r, dev, dout_d)
    idx = r.idx.cpu().numpy().astype(np.int64)
    u_h = _f(host.token_rows(cfg))
    c_h = host.centroids(cfg)
    ex_q = HostExperts(cfg, fp8=True)
    deq = lambda ws: tuple(O.dequant_weight(*w) for w in ws)  # noqa: E731
    # du of a few tokens depends on those tokens' rows only
    toks = np.array([0, 4097, cfg.tokens - 1])
    with oracle_pool() as pool:
        du_o, _, _, _ = O.layer_backward_steps(u_h[toks], c_h, idx[toks], lambda e: deq(ex_q.routed(e)),
                                               [deq(w) for w in ex_q.shared()], dout_h[toks], O.Fp8Policy,
                                               map=pool.map)
    du_g = to_host_f32(du)[toks]
    errs = {"du": (_fro(du_g - dout_h[toks], du_o - dout_h[toks]), _row_rel(du_g, du_o))}
    # one routed expert's weight gradients depend on its rows (in token order) only
    load = np.bincount(idx.ravel(), minlength=cfg.n_routed)
    cand = np.nonzero(load > 128)[0]
    ex = int(cand[np.argsort(load[cand])[len(cand) // 2]])
    rows, slots = np.nonzero(idx == ex)
    s = O.affinity64(u_h[rows], c_h)
    ssel = np.take_along_axis(s, idx[rows], axis=1)
    gate = ssel[np.arange(len(rows)), slots] / ssel.sum(axis=1)
    P = O.Fp8Policy
    _, _, dw_o = O.expert_backward(P.tiles(u_h[rows]), P.tiles(dout_h[rows]), u_h[rows], dout_h[rows], gate,
                                   *deq(ex_q.routed(ex)), P)
    for name, j in (("w_gate", 0), ("w_up", 1), ("w_down", 2)):
        got = to_host_f32(g[name][ex])
        errs[f"d{name}"] = (_fro(got, dw_o[j]), _rel(got, dw_o[j]))
    print(f"tokens {toks.tolist()}, expert {ex} ({len(rows)} rows)", flush=True)
    _check(errs)


def test_fp8_backward_zero_tokens_writes_zero_gradients():
    cfg = _small("fp8-bwd-empty", 64, 256, 8, 2, 1, 128, cid=74)
    dev = quantize_fp8_weights(host_to_device(host.make_host_inputs(cfg)), cfg)
    r = Runner(cfg, dev, tokens=0)
    g = {k: torch.full(dev[k].shape, 1.0, dtype=torch.bfloat16, device="cuda")
         for k in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")}
    de = torch.full((cfg.n_routed, cfg.hidden), 1.0, dtype=torch.float32, device="cuda")
    du = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dout = torch.zeros((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    wg = moe.make_weight_grads(g["w_gate"], g["w_up"], g["w_down"], g["sh_gate"], g["sh_up"], g["sh_down"])
    moe.moe_backward(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, dout, du, de, wg, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(de) == 0
    for k, t in g.items():
        assert torch.count_nonzero(t) == 0, k
