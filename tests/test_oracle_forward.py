"""Pins of the oracle's expert/forward half and of its FP8 quantiser.

Sources: the h' equation of 方法 §2 of the page "DeepSeek-V3 技術報告"
(xyznot.com/zh-tw/paper/2412.19437), a hand-worked SwiGLU value, torch's
F.linear/F.silu as an independent library for the dense special case,
invariances the equation implies, and the OCP OFP8 E4M3 encoding (table values
and torch's float8_e4m3fn cast) for the quantiser.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O


def _rand_layer(rng, T=12, d=16, N=6, K=2, Ns=1, I=8):
    return dict(
        u=rng.standard_normal((T, d)),
        e=rng.standard_normal((N, d)) / math.sqrt(d),
        b=rng.uniform(-0.01, 0.01, N).astype(np.float32),
        wg=rng.standard_normal((N, I, d)) / math.sqrt(d),
        wu=rng.standard_normal((N, I, d)) / math.sqrt(d),
        wd=rng.standard_normal((N, d, I)) / math.sqrt(I),
        sg=rng.standard_normal((Ns, I, d)) / math.sqrt(d),
        su=rng.standard_normal((Ns, I, d)) / math.sqrt(d),
        sd=rng.standard_normal((Ns, d, I)) / math.sqrt(I),
        K=K,
    )


def _forward(L):
    idx, g, *_ = O.route(L["u"], L["e"], L["b"], L["K"])
    shared = list(zip(L["sg"], L["su"], L["sd"]))
    return O.layer_forward(L["u"], idx, g, O.stacked(L["wg"], L["wu"], L["wd"]), shared), idx, g


def test_swiglu_hand_value():
    # d = 2, I = 1: gate row [ln 3, 0], up row [0, 1], down column [1, -1]; x = [1, 2]
    # a = ln 3, b = 2, h = SiLU(ln 3) * 2 = (3/4 ln 3) * 2, y = [h, -h]
    x = np.array([[1.0, 2.0]])
    wg = np.array([[math.log(3.0), 0.0]])
    wu = np.array([[0.0, 1.0]])
    wd = np.array([[1.0], [-1.0]])
    h = 1.5 * math.log(3.0)
    np.testing.assert_allclose(O.swiglu_ffn(x, wg, wu, wd), [[h, -h]], rtol=1e-15)


def test_dense_special_case_matches_torch():
    # N_r = K_r = 1, N_s = 0: the layer is u + SwiGLU(u), gate 1
    rng = np.random.default_rng(11)
    L = _rand_layer(rng, N=1, K=1, Ns=0)
    out, idx, g = _forward(L)
    assert np.all(g == 1.0)
    x = torch.from_numpy(L["u"])
    ref = x + F.linear(F.silu(F.linear(x, torch.from_numpy(L["wg"][0]))) * F.linear(x, torch.from_numpy(L["wu"][0])),
                       torch.from_numpy(L["wd"][0]))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_identical_routed_experts_sum_to_one_ffn():
    rng = np.random.default_rng(12)
    L = _rand_layer(rng, N=5, K=3, Ns=1)
    for k in ("wg", "wu", "wd"):
        L[k] = np.repeat(L[k][:1], 5, axis=0)
    out, idx, g = _forward(L)
    x = L["u"]
    want = x + O.swiglu_ffn(x, L["sg"][0], L["su"][0], L["sd"][0]) + O.swiglu_ffn(x, L["wg"][0], L["wu"][0], L["wd"][0])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_gives_residual():
    rng = np.random.default_rng(13)
    L = _rand_layer(rng)
    L["wd"][:] = 0
    L["sd"][:] = 0
    out, *_ = _forward(L)
    assert np.array_equal(out, L["u"])


def test_token_permutation_equivariance():
    rng = np.random.default_rng(14)
    L = _rand_layer(rng, T=20)
    out, *_ = _forward(L)
    p = rng.permutation(20)
    L2 = dict(L, u=L["u"][p])
    out2, *_ = _forward(L2)
    np.testing.assert_allclose(out2, out[p], rtol=1e-13, atol=1e-13)


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(15)
    L = _rand_layer(rng, N=7, K=3)
    out, *_ = _forward(L)
    p = rng.permutation(7)
    L2 = dict(L, e=L["e"][p], b=L["b"][p], wg=L["wg"][p], wu=L["wu"][p], wd=L["wd"][p])
    out2, *_ = _forward(L2)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-13)


def test_two_shared_experts_equal_one_wide_ffn():
    rng = np.random.default_rng(16)
    L = _rand_layer(rng, Ns=2)
    idx, g, *_ = O.route(L["u"], L["e"], L["b"], L["K"])
    routed = O.stacked(L["wg"], L["wu"], L["wd"])
    two = O.layer_forward(L["u"], idx, g, routed, list(zip(L["sg"], L["su"], L["sd"])))
    wide = (np.concatenate(L["sg"], 0), np.concatenate(L["su"], 0), np.concatenate(L["sd"], 1))
    one = O.layer_forward(L["u"], idx, g, routed, [wide])
    np.testing.assert_allclose(two, one, rtol=1e-13, atol=1e-13)


def test_gate_weighting_is_linear_in_each_expert():
    # doubling expert j's down projection adds exactly g_j * FFN_j(u) again for tokens that picked j
    rng = np.random.default_rng(17)
    L = _rand_layer(rng, N=4, K=2, Ns=0)
    out, idx, g = _forward(L)
    j = int(idx[0, 0])
    L2 = dict(L, wd=L["wd"].copy())
    L2["wd"][j] *= 2
    out2, idx2, g2 = _forward(L2)
    assert np.array_equal(idx, idx2)
    rows, slots = np.nonzero(idx == j)
    extra = g[rows, slots][:, None] * O.swiglu_ffn(L["u"][rows], L["wg"][j], L["wu"][j], L["wd"][j])
    np.testing.assert_allclose(out2[rows] - out[rows], extra, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------- FP8 quantiser

def test_e4m3_table(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "e4m3_table.json")))
    for code_s, val_s in d["pairs"]:
        code = int(code_s, 16)
        neg = val_s.startswith("-")
        v = val_s.lstrip("-")
        if "^" in v:
            m, _, ex = v.partition("2^")
            m = float(m.rstrip("*")) if m else 1.0
            val = m * 2.0 ** int(ex)
        else:
            val = float(v)
        val = -val if neg else val
        assert O.e4m3_decode(np.array([code], np.uint8))[0] == val
        assert O.e4m3_encode(np.array([val]))[0] == code
        assert O.e4m3_round(np.array([val]))[0] == val


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(18)
    # wide magnitude range, exact midpoints of the grid, and subnormals
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
        (np.arange(-1000, 1000) + 0.5) * 2.0 ** -9,
        (np.arange(8, 16) + 0.5) * 2.0 ** 5,
        [0.0, -0.0, 448.0, -448.0, 464.0, -464.0],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    mine = O.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)
    codes = O.e4m3_encode(mine)
    assert np.array_equal(codes, torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3_saturates():
    assert O.e4m3_round(np.array([470.0, 1e6, -1e6]))[0] == 448.0
    assert O.e4m3_round(np.array([-1e6]))[0] == -448.0


def test_act_quantiser_against_torch():
    rng = np.random.default_rng(19)
    x = (rng.standard_normal((7, 384)) * rng.uniform(0.01, 30, (7, 1))).astype(np.float32)
    x[3, 128:256] = 0.0
    codes, scale = O.quantize_act_1x128(x)
    assert scale.shape == (7, 3) and scale.dtype == np.float32
    assert scale[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    for r in range(7):
        for j in range(3):
            blk = x[r, 128 * j:128 * (j + 1)]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert scale[r, j] == np.float32(amax) / np.float32(448.0)
            y = torch.from_numpy(blk) / torch.tensor(scale[r, j])   # fp32 division in torch
            ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, 128 * j:128 * (j + 1)], ref)
            # the amax element maps to +-448 (code 0x7e / 0xfe)
            k = int(np.argmax(np.abs(blk)))
            assert codes[r, 128 * j + k] & 0x7F == 0x7E


def test_weight_quantiser_blocks():
    rng = np.random.default_rng(20)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:, 256:] *= 1000.0
    codes, scale = O.quantize_weight_128x128(w)
    assert scale.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)]
            assert scale[bi, bj] == np.float32(np.abs(blk).max()) / np.float32(448.0)
            ref = (torch.from_numpy(blk) / torch.tensor(scale[bi, bj])).to(torch.float8_e4m3fn).view(torch.uint8)
            assert np.array_equal(codes[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)], ref.numpy())


def test_grid_values_round_trip_exactly():
    # values on the E4M3 grid times a power of two, with block amax exactly 448 * 2^k,
    # quantise losslessly: scale = 2^k exactly and every code decodes to the input
    rng = np.random.default_rng(21)
    grid = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    grid = grid[np.isfinite(grid)]
    x = rng.choice(grid, size=(4, 256)) * rng.choice([-1.0, 1.0], size=(4, 256))
    x[:, 0] = 448.0
    x[:, 128] = -448.0
    x = (x * 2.0 ** -5).astype(np.float32)
    codes, scale = O.quantize_act_1x128(x)
    assert np.all(scale == np.float32(2.0 ** -5))
    np.testing.assert_array_equal(O.dequant_act(codes, scale), x.astype(np.float64))


def test_fp8_forward_is_exact_for_grid_inputs_up_to_h():
    # when u and all weights are on the quantisation grid the only fp8 effect is the
    # quantisation of H; replacing H's quantiser by torch's cast gives the same output
    rng = np.random.default_rng(22)
    grid = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    grid = grid[np.isfinite(grid) & (grid <= 8)]

    def g(shape, s):
        a = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        a.reshape(-1, 128)[:, 0] = 448.0
        return (a * s).astype(np.float32)
    T, d, I = 4, 128, 128
    u = g((T, d), 2.0 ** -8)
    wg, wu = g((I, d), 2.0 ** -12), g((I, d), 2.0 ** -12)
    wd = g((d, I), 2.0 ** -12)
    q = [O.quantize_weight_128x128(w) for w in (wg, wu, wd)]
    idx = np.zeros((T, 1), np.int64)
    gate = np.ones((T, 1))
    out = O.layer_forward_fp8(u, idx, gate, lambda e: q, [])
    x = u.astype(np.float64)
    a = x @ wg.astype(np.float64).T
    b = x @ wu.astype(np.float64).T
    h = torch.from_numpy((O.silu(a) * b).astype(np.float32))
    amax = h.abs().reshape(T, 1, 128).amax(-1)
    sc = amax / 448.0
    hq = (h.reshape(T, 1, 128) / sc[..., None]).to(torch.float8_e4m3fn).to(torch.float64) * sc[..., None].double()
    want = x + hq.reshape(T, I).numpy() @ wd.astype(np.float64).T
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- FP8 forward, step by step

def _torch_tiles(x):
    """1x128 tiles along the last axis, each cast with torch's float8_e4m3fn (R8 scale rule)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    r, k = t.shape
    t = t.reshape(r, k // 128, 128)
    amax = t.abs().amax(-1, keepdim=True)
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    return ((t / sc).to(torch.float8_e4m3fn).to(torch.float64) * sc.double()).reshape(r, k)


def _torch_blocks(w):
    """128x128 blocks of a stored [out, in] matrix, each cast with torch's float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    n, k = t.shape
    t = t.reshape(n // 128, 128, k // 128, 128)
    amax = t.abs().amax(dim=(1, 3), keepdim=True)
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    return ((t / sc).to(torch.float8_e4m3fn).to(torch.float64) * sc.double()).reshape(n, k)


def _unequal_blocks(rng, n, k, spread):
    """Off-grid values whose 128x128 blocks differ in magnitude by the given factors."""
    w = rng.standard_normal((n, k)).astype(np.float32)
    f = rng.choice(spread, size=(n // 128, k // 128)).astype(np.float32)
    return (w.reshape(n // 128, 128, k // 128, 128) * f[:, None, :, None]).reshape(n, k)


def test_weight_dequant_per_block_against_torch():
    # every 128x128 block keeps its own scale: blocks that differ by factors up to 1e5
    # dequantise to torch's per-block cast exactly (a shared scale would move the small
    # blocks to zero and saturate the large ones)
    rng = np.random.default_rng(23)
    w = _unequal_blocks(rng, 384, 256, [1e-3, 0.37, 1.0, 7.5, 90.0])
    codes, scale = O.quantize_weight_128x128(w)
    assert len(np.unique(scale)) == scale.size
    got = O.dequant_weight(codes, scale)
    np.testing.assert_array_equal(got, _torch_blocks(w).numpy())
    # and each block alone quantises to the same values (no block sees another's amax)
    for bi in range(3):
        for bj in range(2):
            blk = w[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)]
            c1, s1 = O.quantize_weight_128x128(blk)
            np.testing.assert_array_equal(O.dequant_weight(c1, s1),
                                          got[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)])


def test_fp8_forward_against_torch_casts():
    # the whole quantisation-faithful layer on off-grid data: u tiles with unequal amax,
    # weights with unequal block scales, two routed experts per token and a shared expert.
    # The reference re-derives every quantisation with torch's float8_e4m3fn cast and the
    # float64 products with torch, so a tile or block scale applied to the wrong elements,
    # or a skipped quantisation of u or H, separates the two.
    rng = np.random.default_rng(24)
    T, d, I, N, K = 6, 256, 256, 3, 2
    u = rng.standard_normal((T, d)).astype(np.float32)
    u *= rng.choice([0.01, 0.3, 1.0, 40.0], size=(T, d // 128)).repeat(128, axis=1).astype(np.float32)
    ws = {n: [_unequal_blocks(rng, *shape, [0.002, 0.05, 0.4]) for shape in ((I, d), (I, d), (d, I))]
          for n in range(N + 1)}
    idx = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [2, 1], [1, 0]])
    gate = rng.uniform(0.2, 0.8, (T, K))
    gate /= gate.sum(axis=1, keepdims=True)
    q = {n: tuple(O.quantize_weight_128x128(w) for w in ws[n]) for n in ws}
    got = O.layer_forward_fp8(u, idx, gate, lambda e: q[e], [q[N]])

    x = _torch_tiles(u)

    def ffn(xr, n):
        wg, wu, wd = (_torch_blocks(w) for w in ws[n])
        a = xr @ wg.T
        b = xr @ wu.T
        h = (torch.nn.functional.silu(a) * b).to(torch.float32)
        return _torch_tiles(h.numpy()) @ wd.T

    want = torch.from_numpy(u.astype(np.float64)) + ffn(x, N)
    for t in range(T):
        for k in range(K):
            want[t] += gate[t, k] * ffn(x[t:t + 1], int(idx[t, k]))[0]
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12 * float(want.abs().max()))
    # the test separates an unquantised u from the quantised one by far more than its bar
    x_plain = torch.from_numpy(u.astype(np.float64))
    alt = x_plain + ffn(x_plain, N)
    shared_only = torch.from_numpy(u.astype(np.float64)) + ffn(x, N)
    assert float((alt - shared_only).abs().max()) > 1e-3 * float(shared_only.abs().max())


def test_concurrent_expert_terms_change_nothing():
    # the map option only changes how the per-expert terms are evaluated: the output is
    # bit-identical to the plain loop, forward and backward
    import concurrent.futures as cf
    rng = np.random.default_rng(25)
    L = _rand_layer(rng, T=40, N=9, K=3, Ns=2)
    idx, g, *_ = O.route(L["u"], L["e"], L["b"], L["K"])
    routed = O.stacked(L["wg"], L["wu"], L["wd"])
    shared = list(zip(L["sg"], L["su"], L["sd"]))
    dout = rng.standard_normal(L["u"].shape)
    with cf.ThreadPoolExecutor(4) as pool:
        a = O.layer_forward(L["u"], idx, g, routed, shared, map=pool.map)
        b1 = O.layer_backward(L["u"], L["e"], idx, routed, shared, dout, map=pool.map)
        b2 = O.layer_backward_steps(L["u"], L["e"], idx, routed, shared, dout, O.Bf16Policy, map=pool.map)
    assert np.array_equal(a, O.layer_forward(L["u"], idx, g, routed, shared))
    for x, y in ((b1, O.layer_backward(L["u"], L["e"], idx, routed, shared, dout)),
                 (b2, O.layer_backward_steps(L["u"], L["e"], idx, routed, shared, dout, O.Bf16Policy))):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        assert x[2].keys() == y[2].keys()
        for e in x[2]:
            assert all(np.array_equal(p, q) for p, q in zip(x[2][e], y[2][e]))
