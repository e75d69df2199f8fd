"""GPU routing on exact ties and NaN scores, asserted exactly (no 1e-6 exemption).

The g' equation of 方法 §2 of the page "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437)
selects a set by Topk and leaves ties open; the library's reading (its header) orders the picks by
s + b descending, ties to the lower expert index, with NaN scores below every number.  The inputs
are built so that every score the order depends on is either exactly equal to another one or far
from it: every centroid is alpha_i times one fixed direction v and every token has u . v > 0, so
s_i = sigmoid(alpha_i u . v) is ordered like alpha_i, experts sharing an alpha share every
product and therefore every s bit for bit, and distinct alphas are more than 0.02 apart in s.
The expected picks are then fixed by hand and equal to the oracle's, token by token.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

N = 16
# experts 3, 7 and 12 share the top level, 0 and 5 the second; the rest are distinct and lower
ALPHA = np.array([1.0, -0.5, -1.5, 2.0, -0.25, 1.0, -2.0, 2.0, -0.75, -1.0, 0.25, -1.25, 2.0, 0.5, -1.75, 0.0])


def _inputs(T, d, dtype, seed):
    rng = np.random.default_rng(seed)
    u = (1.0 + 0.5 * np.abs(rng.standard_normal((T, d)))).astype(np.float32)
    if dtype == "bf16":
        u = torch.from_numpy(u).to(torch.bfloat16).float().numpy()
    v = np.full(d, 1.0 / d, dtype=np.float32)          # one direction shared by every centroid
    e = (ALPHA[:, None].astype(np.float32) * v[None, :]).astype(np.float32)
    return u, e


def _route(u, e, bias, K, dtype, grouped=None):
    T, d = u.shape
    dt = moe.MOE_DTYPE_BF16 if dtype == "bf16" else moe.MOE_DTYPE_F32
    shape = moe.make_shape(T, d, N, K, 0, 128, dt)
    ud = torch.from_numpy(u).to("cuda")
    if dtype == "bf16":
        ud = ud.to(torch.bfloat16)
    ws = torch.empty(moe.moe_workspace_size(shape), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    load = torch.empty((N,), dtype=torch.int32, device="cuda")
    ed = torch.from_numpy(e).to("cuda")
    bd = torch.from_numpy(bias.astype(np.float32)).to("cuda")
    if grouped is None:
        moe.moe_route(shape, ud, ed, bd, idx, gate, load, ws)
    else:
        moe.moe_route_grouped(shape, grouped[0], grouped[1], ud, ed, bd, idx, gate, load, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gate.cpu().numpy(), load.cpu().numpy()


def _oracle(u, e, bias, K):
    s = O.affinity(u, e)
    c = O.selection_scores(s, bias)
    idx, _ = O.select_topk(c, K)
    return s, idx


# (T, d, dtype): the MFMA router with and without split contractions, and the fused VALU router
SHAPES = [(256, 1024, "bf16"), (8192, 1024, "bf16"), (300, 200, "bf16"), (513, 1024, "f32")]


@pytest.mark.parametrize("T,d,dtype", SHAPES)
def test_ties_go_to_the_lower_index(T, d, dtype):
    u, e = _inputs(T, d, dtype, seed=T)
    bias = np.zeros(N, np.float32)
    bias[[3, 7, 12]] = 0.01                   # equal biases keep the tie
    idx, gate, load = _route(u, e, bias, 4, dtype)
    want = np.array([3, 7, 12, 0])             # 0 and 5 tie for the last place: 0 wins
    assert np.array_equal(idx, np.broadcast_to(want, idx.shape))
    s, idx_o = _oracle(u, e, bias, 4)
    assert np.array_equal(idx_o, idx)
    assert np.array_equal(load, np.bincount(idx.ravel(), minlength=N))
    # tied experts have the same s bit for bit, hence the same gate
    assert np.array_equal(gate[:, 0], gate[:, 1]) and np.array_equal(gate[:, 0], gate[:, 2])
    np.testing.assert_allclose(gate, O.gates(s, idx.astype(np.int64)), rtol=0, atol=1e-5)


@pytest.mark.parametrize("T,d,dtype", SHAPES)
def test_nan_scores_rank_last(T, d, dtype):
    u, e = _inputs(T, d, dtype, seed=T + 1)
    bias = np.zeros(N, np.float32)
    bias[3] = np.nan
    idx, _, load = _route(u, e, bias, 4, dtype)
    assert np.array_equal(idx, np.broadcast_to(np.array([7, 12, 0, 5]), idx.shape))
    assert load[3] == 0
    # every expert picked: the finite scores in order (ties to the lower index), then the NaN
    # ones in index order
    bias[12] = np.nan
    idx, gate, load = _route(u, e, bias, N, dtype)
    order = [7, 0, 5, 13, 10, 15, 4, 1, 8, 9, 11, 2, 14, 6, 3, 12]
    assert np.array_equal(idx, np.broadcast_to(np.array(order), idx.shape))
    assert np.all(load == T)
    s, idx_o = _oracle(u, e, bias, N)
    assert np.array_equal(idx_o, idx)
    np.testing.assert_allclose(gate, O.gates(s, idx.astype(np.int64)), rtol=0, atol=1e-5)


@pytest.mark.parametrize("T,d,dtype", SHAPES[:2])
def test_group_ties_go_to_the_lower_group(T, d, dtype):
    # 4 groups of 4 experts; groups 0, 1 and 3 share the best score (experts 3, 7, 12), so the
    # two eligible groups are 0 and 1 and the picks come from experts 0..7 only
    u, e = _inputs(T, d, dtype, seed=T + 2)
    bias = np.zeros(N, np.float32)
    idx, _, load = _route(u, e, bias, 4, dtype, grouped=(4, 2))
    assert np.array_equal(idx, np.broadcast_to(np.array([3, 7, 0, 5]), idx.shape))
    s = O.affinity(u, e)
    idx_o, _, _ = O.select_topk_grouped(O.selection_scores(s, bias), 4, 4, 2)
    assert np.array_equal(idx_o, idx)
    assert load[12] == 0
