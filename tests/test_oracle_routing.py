"""Pins of the oracle's routing half against facts fixed outside the oracle.

Sources: the page "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437),
方法 §2 (affinity, g' selection, normalisation, bias update), a hand-worked
fixture derived from those equations, closed forms, a brute-force search over
all K-subsets, and torch's own sigmoid/topk as independent library routines.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _frac(s):
    return float(Fraction(s))


def test_hand_worked_fixture(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "hand_route.json")))
    bias = np.array([_frac(x) for x in d["bias"]], dtype=np.float32)
    s = np.array([[_frac(x) for x in t["s"]] for t in d["tokens"]])
    c = O.selection_scores(s, bias)
    idx, gap = O.select_topk(c, d["top_k"])
    for t, tok in enumerate(d["tokens"]):
        assert idx[t].tolist() == tok["idx"]
        assert gap[t] == _frac(tok["gap"])
    g = O.gates(s, idx)
    want = np.array([[_frac(x) for x in t["gate"]] for t in d["tokens"]])
    np.testing.assert_allclose(g, want, rtol=0, atol=1e-15)
    load = O.expert_load(idx, d["n_routed"])
    assert load.tolist() == d["load"]
    b2 = O.update_bias(bias, load, len(d["tokens"]) * d["top_k"], d["gamma"])
    gm = np.float32(d["gamma"])
    for i, expr in enumerate(d["bias_after"]):
        base = np.float32(_frac(expr.split()[0]))
        want_i = base - gm if "- g" in expr else base + gm
        assert b2[i].view(np.uint32) == np.float32(want_i).view(np.uint32)


def test_affinity_closed_forms():
    d = 8
    u = np.zeros((3, d))
    e = np.random.default_rng(0).standard_normal((5, d))
    assert np.all(O.affinity(u, e) == 0.5)                      # z = 0
    u = np.random.default_rng(1).standard_normal((4, d))
    assert np.all(O.affinity(u, np.zeros((5, d))) == 0.5)       # e_i = 0
    # z = ln 3 -> 3/4 and z = -ln 3 -> 1/4
    u = np.zeros((1, d)); u[0, 0] = 1.0
    e = np.zeros((2, d)); e[0, 0] = math.log(3.0); e[1, 0] = -math.log(3.0)
    np.testing.assert_allclose(O.affinity(u, e)[0], [0.75, 0.25], rtol=0, atol=1e-15)


def test_affinity_matches_torch_sigmoid():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((17, 33))
    e = rng.standard_normal((9, 33)) / math.sqrt(33)
    want = torch.sigmoid(torch.from_numpy(u) @ torch.from_numpy(e).T).numpy()
    np.testing.assert_allclose(O.affinity(u, e), want, rtol=1e-14, atol=1e-15)
    # orientation: s[t, i] uses token t and centroid i
    s = O.affinity(u, e)
    assert s.shape == (17, 9)
    assert abs(s[3, 5] - 1 / (1 + math.exp(-float(u[3] @ e[5])))) < 1e-15


def _dominance_ok(c_row, subset):
    """Every picked expert beats every unpicked one under (c desc, index asc)."""
    out = [j for j in range(len(c_row)) if j not in subset]
    for i in subset:
        for j in out:
            ci, cj = c_row[i], c_row[j]
            if not (ci > cj or (ci == cj and i < j)):
                return False
    return True


@pytest.mark.parametrize("n,k", [(4, 1), (5, 2), (6, 3), (8, 4), (9, 8), (7, 7)])
def test_topk_brute_force_with_ties(n, k):
    rng = np.random.default_rng(n * 10 + k)
    # values from a small set so that ties are frequent
    c = (rng.integers(0, 4, size=(40, n)) * 0.25).astype(np.float32)
    idx, gap = O.select_topk(c, k)
    for t in range(c.shape[0]):
        winners = [set(sub) for sub in itertools.combinations(range(n), k) if _dominance_ok(c[t], set(sub))]
        assert len(winners) == 1
        assert set(idx[t].tolist()) == winners[0]
        # the winning set also maximises the sum of c
        best = max(sum(c[t][list(sub)]) for sub in itertools.combinations(range(n), k))
        assert sum(c[t][idx[t]]) == best
        # ordered by (c desc, index asc)
        keys = [(-c[t][i], i) for i in idx[t]]
        assert keys == sorted(keys)
        if k < n:
            rest = sorted((-c[t][j], j) for j in range(n) if j not in idx[t])
            assert gap[t] == c[t][idx[t][-1]] - (-rest[0][0])


def test_zero_bias_equals_torch_topk():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((50, 64))
    e = rng.standard_normal((32, 64)) / 8
    s = O.affinity(u, e)
    idx, _ = O.select_topk(O.selection_scores(s, np.zeros(32)), 6)
    tk = torch.topk(torch.from_numpy(s.astype(np.float32)), 6, dim=1, largest=True, sorted=True).indices.numpy()
    assert np.array_equal(idx, tk)


def test_large_bias_forces_or_excludes():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((64, 16))
    e = rng.standard_normal((12, 16)) / 4
    b = np.zeros(12, dtype=np.float32)
    b[7] = 10.0
    b[2] = -10.0
    idx, g, load, s, c, gap = O.route(u, e, b, 3)
    assert all(7 in row for row in idx.tolist())
    assert load[2] == 0 and load[7] == 64
    # the gate of expert 7 still comes from the unbiased s
    t = 5
    k = idx[t].tolist().index(7)
    assert abs(g[t, k] - s[t, 7] / s[t, idx[t]].sum()) < 1e-15


def test_identical_centroids_lower_index_wins():
    e = np.tile(np.random.default_rng(5).standard_normal((1, 10)), (8, 1))
    u = np.random.default_rng(6).standard_normal((5, 10))
    idx, g, load, *_ = O.route(u, e, np.zeros(8, np.float32), 3)
    assert np.all(idx == np.array([0, 1, 2]))
    np.testing.assert_allclose(g, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_k_equals_n_selects_all():
    rng = np.random.default_rng(7)
    u = rng.standard_normal((6, 8))
    e = rng.standard_normal((5, 8))
    idx, g, load, s, c, gap = O.route(u, e, np.zeros(5, np.float32), 5)
    assert all(sorted(r) == [0, 1, 2, 3, 4] for r in idx.tolist())
    assert np.all(np.isinf(gap))
    assert np.all(load == 6)
    np.testing.assert_allclose(np.take_along_axis(s, idx, 1) / s.sum(1, keepdims=True), g, rtol=1e-15)


def test_gates_properties():
    rng = np.random.default_rng(8)
    u = rng.standard_normal((100, 32))
    e = rng.standard_normal((16, 32)) / 5
    b = rng.uniform(-0.05, 0.05, 16).astype(np.float32)
    idx, g, load, s, c, gap = O.route(u, e, b, 4)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=4e-16)
    assert np.all(g > 0)
    # ratios of gates equal ratios of the unbiased affinities
    r = g[:, 0] / g[:, 1]
    rs = s[np.arange(100), idx[:, 0]] / s[np.arange(100), idx[:, 1]]
    np.testing.assert_allclose(r, rs, rtol=1e-14)
    idx1, g1, *_ = O.route(u, e, b, 1)
    assert np.all(g1 == 1.0)


def test_bias_moves_selection_not_gates():
    # s on a 2^-10 grid so that adding 0.5 to every bias is exact in fp32
    rng = np.random.default_rng(9)
    s = rng.integers(1, 1000, size=(30, 10)) / 1024.0
    b = (rng.integers(-50, 50, size=10) / 1024.0).astype(np.float32)
    i1, _ = O.select_topk(O.selection_scores(s, b), 3)
    i2, _ = O.select_topk(O.selection_scores(s, b + np.float32(0.5)), 3)
    assert np.array_equal(i1, i2)
    np.testing.assert_array_equal(O.gates(s, i1), O.gates(s, i2))


def test_load_counts():
    rng = np.random.default_rng(10)
    u = rng.standard_normal((200, 16))
    e = rng.standard_normal((20, 16)) / 4
    idx, g, load, *_ = O.route(u, e, np.zeros(20, np.float32), 5)
    assert load.sum() == 200 * 5
    assert all(len(set(r)) == 5 for r in idx.tolist())
    manual = np.zeros(20, np.int64)
    for r in idx.tolist():
        for i in r:
            manual[i] += 1
    assert np.array_equal(manual, load)


def test_nan_scores_rank_last():
    c = np.array([[0.1, np.nan, 0.3, 0.2]], dtype=np.float32)
    idx, _ = O.select_topk(c, 3)
    assert idx[0].tolist() == [2, 3, 0]


def test_update_bias_closed_forms():
    n = 8
    b0 = np.linspace(-0.02, 0.02, n).astype(np.float32)
    # balanced: every load equals the mean -> unchanged
    assert np.array_equal(O.update_bias(b0, np.full(n, 3), 3 * n), b0)
    # expert 0 overloaded for 25 steps: b = fp32 iterate of (b - fp32(0.001))
    load = np.array([10, 2, 3, 3, 3, 3, 3, 3])  # total 30 vs mean 30/8 = 3.75
    b = b0.copy()
    want0 = np.float32(b0[0])
    want3 = np.float32(b0[3])
    for _ in range(25):
        b = O.update_bias(b, load, int(load.sum()))
        want0 = np.float32(want0 - np.float32(0.001))
        want3 = np.float32(want3 + np.float32(0.001))
    assert b[0].view(np.uint32) == want0.view(np.uint32)
    assert b[3].view(np.uint32) == want3.view(np.uint32)
    assert b[0] < b0[0] and b[1] > b0[1]   # overloaded goes down, underloaded goes up


def test_update_bias_integer_mean_tie():
    # mean T*K/N = 4*2/4 = 2 exactly: load 2 is neither over nor under
    b = np.zeros(4, np.float32)
    out = O.update_bias(b, np.array([3, 2, 2, 1]), 8)
    assert out[1] == 0 and out[2] == 0 and out[0] < 0 and out[3] > 0
