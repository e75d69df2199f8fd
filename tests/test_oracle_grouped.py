"""Pins of the oracle's group-limited selection (reading R13 of oracle/moe_oracle.py).

The page ("DeepSeek-V3 技術報告", xyznot.com/zh-tw/paper/2412.19437, cross-node all-to-all
section) caps every token at experts on 4 nodes and prints no selection rule, so this rule is
pinned only by a hand-worked fixture, by invariants checked with plain loops, and by its
reduction to the ungrouped Topk of 方法 §2 (itself pinned in test_oracle_routing.py).
"""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O


def _c(strings):
    return np.array([float(v) for v in strings], dtype=np.float32)


def test_grouped_hand_worked_fixture(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "grouped_route.json")))
    c = np.stack([_c(t["c"]) for t in d["tokens"]])
    idx, gap, ggap = O.select_topk_grouped(c, d["top_k"], d["n_groups"], d["topk_groups"])
    assert idx.tolist() == [t["idx"] for t in d["tokens"]]
    ung, _ = O.select_topk(c, d["top_k"])
    assert ung.tolist() == [t["idx_ungrouped"] for t in d["tokens"]]
    # token 1 has a three-way group tie at the boundary and a four-way expert tie
    assert ggap[1] == 0 and gap[1] == 0


@pytest.mark.parametrize("n,k", [(64, 6), (16, 4), (256, 8)])
def test_grouped_reduces_to_ungrouped(n, k):
    rng = np.random.default_rng(n)
    c = rng.random((300, n)).astype(np.float32)
    ref, _ = O.select_topk(c, k)
    for g in (1, 2, 8):
        idx, _, _ = O.select_topk_grouped(c, k, g, g)       # every group eligible
        assert np.array_equal(idx, ref)
    idx, _, _ = O.select_topk_grouped(c, k, 1, 1)
    assert np.array_equal(idx, ref)


def _group_max_loop(row, n_groups):
    gs = len(row) // n_groups
    out = []
    for g in range(n_groups):
        vals = [float(v) for v in row[g * gs:(g + 1) * gs] if v == v]
        out.append(max(vals) if vals else float("-inf"))
    return out


@pytest.mark.parametrize("n,g,mg,k", [(32, 8, 3, 5), (64, 8, 4, 8), (12, 4, 2, 3), (256, 8, 4, 8)])
def test_grouped_invariants(n, g, mg, k):
    rng = np.random.default_rng(n * 100 + k)
    # coarse values so that ties between scores and between groups occur
    c = (rng.integers(0, 12, size=(400, n)) / 8.0).astype(np.float32)
    idx, _, _ = O.select_topk_grouped(c, k, g, mg)
    gs = n // g
    for t in range(c.shape[0]):
        row = c[t]
        picks = [int(e) for e in idx[t]]
        gmax = _group_max_loop(row, g)
        used = sorted({e // gs for e in picks})
        assert len(picks) == len(set(picks)) == k
        assert len(used) <= mg
        # the eligible groups: the mg best by (score desc, index asc), from a plain sort
        ranked = sorted(range(g), key=lambda q: (-gmax[q], q))
        kept = set(ranked[:mg])
        assert set(used) <= kept
        for q in ranked[mg:]:
            assert min(gmax[p] for p in kept) >= gmax[q]
        # picks are the best eligible experts, ordered by (c desc, index asc)
        elig = [e for e in range(n) if e // gs in kept]
        best = sorted(elig, key=lambda e: (-float(row[e]), e))[:k]
        assert picks == best


def test_route_grouped_gates_from_unbiased_s():
    rng = np.random.default_rng(7)
    u = rng.standard_normal((50, 32)).astype(np.float32)
    e = (rng.standard_normal((16, 32)) / np.sqrt(32)).astype(np.float32)
    b = (rng.standard_normal(16) * 0.1).astype(np.float32)
    idx, gate, load, s, c, gap, ggap = O.route_grouped(u, e, b, 4, 4, 2)
    np.testing.assert_allclose(gate.sum(1), 1.0, rtol=0, atol=1e-12)
    sel = np.take_along_axis(s.astype(np.float64), idx, 1)
    np.testing.assert_allclose(gate, sel / sel.sum(1, keepdims=True), rtol=0, atol=1e-15)
    assert np.array_equal(load, np.bincount(idx.ravel(), minlength=16))
    assert all(len(set((r // 4).tolist())) <= 2 for r in idx)


# ----------------------------------------------------------------------------- balance loss (R15)

def test_seq_balance_hand_worked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "seq_balance.json")))
    s = np.array([[float(v) for v in r] for r in d["s"]])
    loss = O.seq_balance_loss(s, np.array(d["idx"]), d["seq_len"], d["alpha"])
    np.testing.assert_allclose(loss, [float(v) for v in d["loss"]], rtol=1e-14)


def test_seq_balance_uniform_picks_give_alpha():
    # every expert picked equally often in each sequence: f_i = 1, and sum_i P_i = 1 always
    rng = np.random.default_rng(2)
    n, k, L = 8, 2, 12
    s = rng.random((3 * L, n)) + 0.01
    idx = np.array([[(2 * t) % n, (2 * t + 1) % n] for t in range(3 * L)])
    np.testing.assert_allclose(O.seq_balance_loss(s, idx, L, 0.5), 0.5, rtol=1e-13)


def test_seq_balance_collapsed_routing():
    # all tokens pick experts {0, 1}: f = N/K on them, so loss = alpha N/K (P_0 + P_1)
    rng = np.random.default_rng(3)
    n, k, L = 16, 2, 10
    s = rng.random((L, n)) + 0.01
    idx = np.tile([0, 1], (L, 1))
    sn = s / s.sum(1, keepdims=True)
    want = 1e-4 * n / k * (sn[:, 0].mean() + sn[:, 1].mean())
    np.testing.assert_allclose(O.seq_balance_loss(s, idx, L), [want], rtol=1e-13)
