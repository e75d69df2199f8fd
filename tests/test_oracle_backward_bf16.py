"""Pins of the oracle's bf16 backward storage model (reading R17 of oracle/moe_oracle.py).

The layer backward of 方法 §2 ("DeepSeek-V3 技術報告", xyznot.com/zh-tw/paper/2412.19437) taken
step by step (R16's steps) with bf16 storage between the steps, and, for the saved-input
variant, a and b held in bf16 from the forward.  Pinned by
* its rounding functions: bf16 storage and the once-rounded gate * dout against torch;
* the saved-input variant equalling the plain one bit for bit where a and b are bf16 values
  (small integers), and differing from it where they are not;
* the distance to the exact R14 backward that bf16 allows, on the well-conditioned outputs;
* the FP8 saved-input variant: R16's quantisers with a and b rounded to bf16, differing from the
  plain FP8 backward by no more than that rounding moves the E4M3 codes.
"""
import numpy as np
import torch

from oracle import moe_oracle as O


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


def _run(L, policy):
    return _flat(O.layer_backward_steps(L["u"], L["e"], L["idx"], O.stacked(L["wg"], L["wu"], L["wd"]), L["sh"],
                                        L["dout"], policy))


def _layer(rng, T, d, N, K, I, Ns, integer):
    if integer:
        # a = x Wg^T and b = x Wu^T are integers of magnitude <= 2 * d: bf16 values for d <= 64
        draw = lambda *sz: rng.integers(-1, 2, size=sz).astype(np.float64)  # noqa: E731
        u = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
        wg, wu = draw(N, I, d), draw(N, I, d)
        sh = [(draw(I, d), draw(I, d), O.bf16_round(rng.standard_normal((d, I)) / 4)) for _ in range(Ns)]
    else:
        bf = O.bf16_round
        u = bf(rng.standard_normal((T, d)))
        wg = bf(rng.standard_normal((N, I, d)) / np.sqrt(d))
        wu = bf(rng.standard_normal((N, I, d)) / np.sqrt(d))
        sh = [tuple(bf(rng.standard_normal(sz) / np.sqrt(sz[1])) for sz in ((I, d), (I, d), (d, I)))
              for _ in range(Ns)]
    wd = O.bf16_round(rng.standard_normal((N, d, I)) / np.sqrt(I))
    e = rng.standard_normal((N, d)) / np.sqrt(d)
    dout = O.bf16_round(rng.standard_normal((T, d)))
    idx, _ = O.select_topk(O.affinity64(u, e), K)
    return dict(u=u, e=e, wg=wg, wu=wu, wd=wd, sh=sh, dout=dout, idx=idx)


def test_bf16_storage_roundings_match_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 33)) * 10.0 ** rng.integers(-6, 6, size=(9, 33))
    g = rng.random(9)
    ref = (torch.tensor(g, dtype=torch.float32)[:, None] * torch.tensor(x, dtype=torch.float32)).to(torch.bfloat16)
    assert np.array_equal(O.Bf16Policy.scaled(g, x), ref.double().numpy())
    held = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.Bf16Policy.held(x), held)
    assert np.array_equal(O.Bf16SavedPolicy.saved(x), held)
    assert np.array_equal(O.Bf16Policy.saved(x), x)
    assert np.array_equal(O.Bf16Policy.tiles(x), x) and np.array_equal(O.Bf16Policy.runs(x), x)


def test_saved_variant_equals_plain_where_a_and_b_are_bf16_values():
    L = _layer(np.random.default_rng(1), T=40, d=32, N=5, K=2, I=24, Ns=1, integer=True)
    plain, saved = _run(L, O.Bf16Policy), _run(L, O.Bf16SavedPolicy)
    assert plain.keys() == saved.keys()
    for k in plain:
        assert np.array_equal(plain[k], saved[k]), k


def test_saved_variant_rounds_a_and_b():
    L = _layer(np.random.default_rng(2), T=40, d=32, N=5, K=2, I=24, Ns=1, integer=False)
    plain, saved = _run(L, O.Bf16Policy), _run(L, O.Bf16SavedPolicy)
    assert not np.array_equal(plain["de"], saved["de"])
    assert not np.array_equal(plain["wg0"], saved["wg0"])


def test_bf16_storage_within_bf16_of_the_exact_backward():
    L = _layer(np.random.default_rng(3), T=160, d=256, N=4, K=2, I=128, Ns=1, integer=False)
    exact = _run(L, O.ExactPolicy)
    for policy in (O.Bf16Policy, O.Bf16SavedPolicy):
        got = _run(L, policy)
        for k in exact:
            if k == "de":
                continue   # ill-conditioned where ds cancels: the reason the storage model exists
            ref = exact[k] - (L["dout"] if k == "du" else 0)
            err = _rel(got[k] - (L["dout"] if k == "du" else 0), ref)
            # a few bf16 roundings (relative 2^-9 each) on the path to every output
            assert err < 1.5e-2, (policy.__name__, k, err)
            assert err > 0, (policy.__name__, k)


def test_fp8_saved_variant_is_r16_with_bf16_a_and_b():
    assert O.Fp8SavedPolicy.tiles is O.Fp8Policy.tiles and O.Fp8SavedPolicy.runs is O.Fp8Policy.runs
    assert O.Fp8SavedPolicy.held is O.Fp8Policy.held and O.Fp8SavedPolicy.scaled is O.Fp8Policy.scaled
    x = np.random.default_rng(4).standard_normal((7, 19)) * 30.0
    assert np.array_equal(O.Fp8SavedPolicy.saved(x), O.bf16_round(x))
    assert np.array_equal(O.Fp8Policy.saved(x), x)
    L = _layer(np.random.default_rng(5), T=160, d=256, N=4, K=2, I=128, Ns=1, integer=False)
    q = lambda w: tuple(O.quantize_weight_128x128(m) for m in w)  # noqa: E731
    rq = lambda ex: q((L["wg"][ex], L["wu"][ex], L["wd"][ex]))  # noqa: E731
    shq = [q(w) for w in L["sh"]]
    plain = _flat(O.layer_backward_fp8(L["u"], L["e"], L["idx"], rq, shq, L["dout"]))
    saved = _flat(O.layer_backward_fp8(L["u"], L["e"], L["idx"], rq, shq, L["dout"], saved=True))
    assert not np.array_equal(plain["wg0"], saved["wg0"])
    for k in plain:
        if k == "de":
            continue
        ref = plain[k] - (L["dout"] if k == "du" else 0)
        got = saved[k] - (L["dout"] if k == "du" else 0)
        # bf16 a, b move some E4M3 codes of dA, dB by one step (1/16 at most): Frobenius small
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 2e-2, k
