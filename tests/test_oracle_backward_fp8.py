"""Pins of the oracle's FP8 layer backward (reading R16 of oracle/moe_oracle.py).

The page "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437) lists the forward GEMM and
both backward GEMMs as FP8 (section 方法, FP8 Mixed Precision Training; 核心概念, FP8 item: E4M3,
1x128 activation tiles, 128x128 weight blocks).  The oracle states the R14 backward step by step
with every GEMM operand passed through a quantisation policy; these tests pin
* the reduction to the R14 backward (itself pinned by finite differences and torch autograd)
  when every quantiser and storage rounding is the identity,
* exact equivariance of the whole FP8 chain under scaling dout by a power of two,
* the distance to the unquantised backward that the E4M3 grid allows,
* the row-run quantiser against a hand-written loop, and the bf16 rounding against torch.
"""
import numpy as np
import torch

from oracle import moe_oracle as O


def _layer(seed=0, T=160, d=256, N=4, K=2, I=128, Ns=1):
    rng = np.random.default_rng(seed)
    bf = lambda a: O.bf16_round(a)  # noqa: E731  (held inputs are bf16 values)
    u = bf(rng.standard_normal((T, d)))
    e = rng.standard_normal((N, d)) / np.sqrt(d)
    wg = bf(rng.standard_normal((N, I, d)) / np.sqrt(d))
    wu = bf(rng.standard_normal((N, I, d)) / np.sqrt(d))
    wd = bf(rng.standard_normal((N, d, I)) / np.sqrt(I))
    sh = [tuple(bf(rng.standard_normal(sz) / np.sqrt(sz[1])) for sz in ((I, d), (I, d), (d, I))) for _ in range(Ns)]
    dout = bf(rng.standard_normal((T, d)))
    idx, _ = O.select_topk(O.affinity64(u, e), K)
    L = dict(u=u, e=e, wg=wg, wu=wu, wd=wd, sh=sh, dout=dout, idx=idx)
    if d % 128 == 0 and I % 128 == 0:
        q = lambda w: tuple(O.quantize_weight_128x128(x) for x in w)  # noqa: E731
        L.update(rq=lambda ex: q((wg[ex], wu[ex], wd[ex])), shq=[q(w) for w in sh])
    return L


def _flat(res):
    du, de, dr, dsh = res
    out = {"du": du, "de": de}
    for ex, gr in dr.items():
        for name, g in zip(("wg", "wu", "wd"), gr):
            out[f"{name}{ex}"] = g
    for i, gr in enumerate(dsh):
        for name, g in zip(("wg", "wu", "wd"), gr):
            out[f"sh_{name}{i}"] = g
    return out


def _rel(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


def test_identity_policy_is_the_exact_backward():
    L = _layer(T=37, d=24, N=6, K=3, I=16, Ns=2)
    routed = O.stacked(L["wg"], L["wu"], L["wd"])
    got = _flat(O.layer_backward_steps(L["u"], L["e"], L["idx"], routed, L["sh"], L["dout"], O.ExactPolicy))
    ref = _flat(O.layer_backward(L["u"], L["e"], L["idx"], routed, L["sh"], L["dout"]))
    assert got.keys() == ref.keys()
    for k in ref:
        assert _rel(got[k], ref[k]) < 1e-12, k


def test_fp8_backward_scales_exactly_with_powers_of_two():
    L = _layer(seed=1)
    a = _flat(O.layer_backward_fp8(L["u"], L["e"], L["idx"], L["rq"], L["shq"], L["dout"]))
    b = _flat(O.layer_backward_fp8(L["u"], L["e"], L["idx"], L["rq"], L["shq"], 8.0 * L["dout"]))
    for k in a:
        assert np.array_equal(b[k], 8.0 * a[k]), k


def test_fp8_backward_within_the_e4m3_grid_of_the_exact_one():
    L = _layer(seed=2)
    deq = lambda ws: tuple(O.dequant_weight(*w) for w in ws)  # noqa: E731
    fp8 = _flat(O.layer_backward_fp8(L["u"], L["e"], L["idx"], L["rq"], L["shq"], L["dout"]))
    # the same weights (dequantised) without any activation quantisation or bf16 storage
    exact = _flat(O.layer_backward(L["u"], L["e"], L["idx"], lambda ex: deq(L["rq"](ex)),
                                   [deq(w) for w in L["shq"]], L["dout"]))
    errs = {k: _rel(fp8[k] - (L["dout"] if k == "du" else 0), exact[k] - (L["dout"] if k == "du" else 0))
            for k in exact}
    # E4M3 keeps 3 mantissa bits: an element moves by at most 1/16 of its magnitude and
    # independent rounding errors average down in every sum; a dropped or misplaced term
    # moves a gradient by a large fraction of its size
    assert max(errs.values()) < 0.12, errs
    assert min(errs.values()) > 1e-4, errs      # the quantisers are really applied


def test_row_runs_quantiser_by_hand():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((130, 3)).astype(np.float32)
    x[128:] *= 1e-3                     # the second run is small: its own scale keeps its precision
    x[5, 1] = 0.0
    x[:, 2] = 0.0                       # an all-zero column: scale 1, codes 0
    got = O.quantize_runs_of_rows(x)
    want = np.zeros_like(got)
    for c in range(3):
        for r0 in (0, 128):
            run = x[r0:r0 + 128, c]
            amax = np.float32(np.max(np.abs(run)))
            scale = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            for i, v in enumerate(run):
                want[r0 + i, c] = float(O.e4m3_round(np.float32(v / scale))) * float(scale)
    assert np.array_equal(got, want)
    assert np.all(got[:, 2] == 0)
    assert np.max(np.abs(got[128:, 0] - x[128:, 0])) <= np.max(np.abs(x[128:, 0])) / 16


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-8, 8, 4096),
                        # exact ties between two bf16 values: both parities of the kept bit
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0])])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x), want)


def test_fp8_input_gradient_quantises_each_token_on_its_own():
    # R16 quantises [dA dB] per 1x128 tile along 2I, i.e. within one token's row, and every
    # other step before du is per row as well.  So scaling one token's dout by a power of two
    # leaves every other token's du bit-identical and scales that token's du exactly; a
    # quantiser whose tiles ran down the rows (several tokens sharing a scale) would move
    # the neighbours' du through the shared scale.
    L = _layer(seed=5)
    t0 = 37
    d2 = L["dout"].copy()
    d2[t0] *= 8.0
    du1 = O.layer_backward_fp8(L["u"], L["e"], L["idx"], L["rq"], L["shq"], L["dout"])[0]
    du2 = O.layer_backward_fp8(L["u"], L["e"], L["idx"], L["rq"], L["shq"], d2)[0]
    others = np.arange(du1.shape[0]) != t0
    assert np.array_equal(du2[others], du1[others])
    assert np.array_equal(du2[t0] - d2[t0], 8.0 * (du1[t0] - L["dout"][t0]))
    assert np.any(du1[t0] != L["dout"][t0])
