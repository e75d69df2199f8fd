"""CPU oracle of the DeepSeekMoE layer forward — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP library and must never be used as
a fallback for it.

It is a plain, slow, float64 statement of what the layer computes, following
the page "DeepSeek-V3 技術報告" (xyznot.com/zh-tw/paper/2412.19437),
section 方法 §2 ("具備無輔助損失平衡機制的 DeepSeekMoE"):

* output:    h'_t = u_t + sum_{i<=N_s} FFN^(s)_i(u_t) + sum_{i<=N_r} g_{i,t} FFN^(r)_i(u_t)
* affinity:  s_{i,t} = Sigmoid(u_t^T e_i)
* selection: g'_{i,t} = s_{i,t} if s_{i,t} + b_i is among the K_r largest of
             {s_{j,t} + b_j}, else 0;  g_{i,t} = g'_{i,t} normalised
* balance:   at the end of a step b_i <- b_i - gamma if expert i is overloaded,
             b_i + gamma if underloaded, gamma = 0.001
and, for the FP8 variant, the tile/block quantisation of the same page's
核心概念 list (E4M3, 1x128 activation tiles, 128x128 weight blocks).

Readings where the page leaves a step open (each is also listed with the
other design notes of the repository):

R1  "normalised" g = g' / sum_j g'_{j,t} (sum over the selected experts).
R2  Topk ties: higher s+b first, then the lower expert index; NaN ranks last.
R3  s is rounded to fp32 and s+b is an fp32 add before selection (the page fixes
    no precision; fp32 is the precision of the GPU kernel, so both sides take
    the integer decision in the same precision).
R4  over/underloaded is against the step mean T*K_r/N_r, compared exactly in
    integers as load_i*N_r vs T*K_r; equal loads leave b_i unchanged; the
    update is one fp32 add of fp32(gamma).
R5  a step is one routing call over a batch of T tokens.
R6  FFN_i(x) = (SiLU(x W_gate^T) * (x W_up^T)) W_down^T with SiLU(v) = v*sigmoid(v),
    no biases; weights stored [out_features, in_features]; all experts,
    shared ones included, have intermediate width I.
R7  no normalisation of u_t inside the layer; the residual is u_t as given.
R8  FP8: scale = fp32(amax / 448) (E4M3FN maximum), amax = 0 -> scale 1,
    code = E4M3FN round-to-nearest-even of fp32(x / scale), saturating at 448;
    activations per 1x128 tile along the contraction dimension, weights per
    128x128 block of the stored [out, in] matrix; both GEMM inputs quantised
    (u before the gate/up projections, H before the down projection); the
    residual and gates stay unquantised.
R13 group limit (the page's cross-node all-to-all section caps every token at 4 nodes
    and prints no rule): the N_r experts form n_groups equal contiguous groups; a
    group's score is the highest c = s+b among its experts (NaN below every number);
    the topk_groups best groups (ties to the lower group index) stay eligible and
    the K_r picks follow R2 among their experts.  Parity of this rule is pinned by
    a hand-worked example and by invariants only.
R15 sequence-wise balance loss (the page adds "a tiny sequence-level balance loss,
    alpha = 0.0001" to the bias rule and prints no formula; the reading here, parity
    unpinned beyond alpha): for each sequence of L consecutive tokens,
    f_i = N_r / (K_r L) * (number of the sequence's picks of expert i),
    P_i = (1/L) sum_t s_{i,t} / sum_j s_{j,t},  loss = alpha * sum_i f_i P_i.
R14 backward: gradients of L = <dout, h'> with the selection (idx) held fixed, as the Topk
    is piecewise constant; the bias gets no gradient (it never enters a gate); the
    gate path is differentiated through the unbiased s of the gate equation with s
    evaluated in float64 (no fp32 rounding, so that finite differences can pin it).
R16 FP8 backward (the page's FP8 paragraph names the forward GEMM and both backward
    GEMMs, input gradient and weight gradient, as FP8 and fixes only the tile and block
    shapes): a weight operand is quantised per 128x128 block of its stored matrix, so a
    transposed weight carries the transposed codes and scales; every other operand per
    1x128 tile along that GEMM's contraction axis: u and dout along d, [dA dB] along 2I
    for the input-gradient products, and, for the weight-gradient products, whose
    contraction runs over an expert's rows, along those rows taken in token order in runs
    of 128 (the last run zero-padded).  A tensor is quantised from the precision it is held
    in between two steps, the same on both sides so that equal inputs give equal codes:
    u, dout and the stored H, dA, dB and dH (= dout W_down before the gate) in bf16,
    gate * dout in fp32.  Gates, the router and the residual are not quantised (R14).
    Parity of this reading is pinned by its reduction to R14 with every quantiser and
    rounding replaced by the identity, by exact scaling under powers of two, and by the
    distance to R14 that the E4M3 grid allows.
R17 bf16 backward storage (the page fixes no precision for the bf16 path): R16's steps with
    no quantiser, the tensors held between steps (dH, H, dA, dB) rounded to bf16 and
    gate * dout rounded once to bf16 from its fp32 product; the saved-input variant also
    holds the SwiGLU inputs a and b in bf16 from the forward (for the FP8 backward of R16
    too: a and b then come from the FP8 forward product and are rounded to bf16).  Outputs whose condition
    number magnifies these roundings past the bf16 tolerance (the centroid gradient of an
    expert picked by one or two tokens, where the two terms of ds nearly cancel) are checked
    against this model; every other output against R14 itself.  Pinned by its reduction to
    R14 when the roundings are the identity, by the saved-input variant equalling the plain
    one where a and b are bf16 values, and by the distance to R14 that bf16 allows.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- routing

def affinity(u: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """s[t, i] = Sigmoid(u_t . e_i) in float64 (方法 §2, affinity equation)."""
    z = np.asarray(u, dtype=np.float64) @ np.asarray(centroids, dtype=np.float64).T
    return 1.0 / (1.0 + np.exp(-z))


def selection_scores(s: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """c[t, i] = fp32(fp32(s) + b_i), the key Topk ranks (方法 §2, g' equation; R3)."""
    return np.asarray(s, dtype=np.float32) + np.asarray(bias, dtype=np.float32)[None, :]


def select_topk(c: np.ndarray, k: int):
    """Indices of the K_r largest c per token, ordered by (c desc, index asc) (R2).

    Returns (idx [T, K] int64, gap [T] float64) where gap is c_(K) - c_(K+1),
    the margin by which the K-th pick beats the first unpicked expert
    (+inf when K = N_r).
    """
    c = np.asarray(c)
    order = np.argsort(-c, axis=1, kind="stable")
    idx = order[:, :k]
    if k < c.shape[1]:
        ck = np.take_along_axis(c, order[:, k - 1:k], axis=1)[:, 0].astype(np.float64)
        ck1 = np.take_along_axis(c, order[:, k:k + 1], axis=1)[:, 0].astype(np.float64)
        gap = ck - ck1
    else:
        gap = np.full(c.shape[0], np.inf)
    return idx, gap


def gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g[t, k] = s[t, idx[t,k]] / sum_k' s[t, idx[t,k']] (unbiased s; R1)."""
    sel = np.take_along_axis(np.asarray(s, dtype=np.float64), idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def expert_load(idx: np.ndarray, n_routed: int) -> np.ndarray:
    """load[i] = number of (token, slot) assignments to expert i in the step."""
    return np.bincount(np.asarray(idx).ravel(), minlength=n_routed).astype(np.int64)


def route(u, centroids, bias, k: int):
    """The routing half of the layer: (idx, gate, load, s, c, gap)."""
    s = affinity(u, centroids)
    c = selection_scores(s, bias)
    idx, gap = select_topk(c, k)
    return idx, gates(s, idx), expert_load(idx, np.asarray(centroids).shape[0]), s, c, gap


_NAN_RANK = -1e300   # below every score a sigmoid plus a bias can produce, above "not eligible"


def group_scores(c: np.ndarray, n_groups: int) -> np.ndarray:
    """Score of each of the n_groups contiguous expert groups: its highest c (R13)."""
    c = np.asarray(c, dtype=np.float64)
    v = np.where(np.isnan(c), _NAN_RANK, c)
    t, n = v.shape
    return v.reshape(t, n_groups, n // n_groups).max(axis=2)


def select_topk_grouped(c: np.ndarray, k: int, n_groups: int, topk_groups: int):
    """R13: the K_r picks among the experts of the topk_groups best groups.

    Returns (idx [T, K] int64, gap [T], group_gap [T]): gap is c_(K) - c_(K+1) among the
    eligible experts (+inf when all of them are picked), group_gap is the margin of the last
    eligible group's score over the best ineligible one (+inf when every group is eligible).
    """
    c = np.asarray(c)
    t, n = c.shape
    gs = n // n_groups
    gsc = group_scores(c, n_groups)
    gorder = np.argsort(-gsc, axis=1, kind="stable")
    keep = gorder[:, :topk_groups]
    eligible = ((np.arange(n) // gs)[None, :, None] == keep[:, None, :]).any(axis=2)
    v = np.where(np.isnan(c), _NAN_RANK, c.astype(np.float64))
    v = np.where(eligible, v, -np.inf)
    order = np.argsort(-v, axis=1, kind="stable")
    idx = order[:, :k]
    if k < eligible.sum(axis=1).min():
        vk = np.take_along_axis(v, order[:, k - 1:k], axis=1)[:, 0]
        vk1 = np.take_along_axis(v, order[:, k:k + 1], axis=1)[:, 0]
        gap = np.where(np.isfinite(vk1), vk - vk1, np.inf)
    else:
        gap = np.full(t, np.inf)
    if topk_groups < n_groups:
        g1 = np.take_along_axis(gsc, gorder[:, topk_groups - 1:topk_groups], axis=1)[:, 0]
        g2 = np.take_along_axis(gsc, gorder[:, topk_groups:topk_groups + 1], axis=1)[:, 0]
        group_gap = g1 - g2
    else:
        group_gap = np.full(t, np.inf)
    return idx, gap, group_gap


def route_grouped(u, centroids, bias, k: int, n_groups: int, topk_groups: int):
    """Group-limited routing (R13): (idx, gate, load, s, c, gap, group_gap)."""
    s = affinity(u, centroids)
    c = selection_scores(s, bias)
    idx, gap, group_gap = select_topk_grouped(c, k, n_groups, topk_groups)
    return idx, gates(s, idx), expert_load(idx, np.asarray(centroids).shape[0]), s, c, gap, group_gap


def update_bias(bias: np.ndarray, load: np.ndarray, total_assignments: int, gamma: float = 0.001) -> np.ndarray:
    """Auxiliary-loss-free bias update (方法 §2, last paragraph; R4)."""
    b = np.asarray(bias, dtype=np.float32).copy()
    n = b.shape[0]
    ld = np.asarray(load, dtype=np.int64) * n
    g = np.float32(gamma)
    over = ld > total_assignments
    under = ld < total_assignments
    b[over] = b[over] - g
    b[under] = b[under] + g
    return b


# ----------------------------------------------------------------------------- experts

def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def swiglu_ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert FFN (R6): (SiLU(x Wg^T) * (x Wu^T)) Wd^T in float64."""
    x = np.asarray(x, dtype=np.float64)
    a = x @ np.asarray(w_gate, dtype=np.float64).T
    b = x @ np.asarray(w_up, dtype=np.float64).T
    return (silu(a) * b) @ np.asarray(w_down, dtype=np.float64).T


def layer_forward(u, idx, gate, routed, shared, ffn=swiglu_ffn, x=None, map=map) -> np.ndarray:
    """h'_t = u_t + sum_s FFN^(s)_s(u_t) + sum_k gate[t,k] FFN^(r)_{idx[t,k]}(u_t) (方法 §2, h' equation).

    routed: callable e -> (w_gate, w_up, w_down) of routed expert e;
    shared: sequence of (w_gate, w_up, w_down), one per shared expert.
    x: what the expert FFNs read (defaults to u; the FP8 variant passes the
    fake-quantised u here while the residual stays u).
    map: how the routed experts' FFN terms are evaluated (an executor's map runs them
    concurrently; the terms are added in increasing expert order either way).
    Rows of u, idx and gate correspond; pass a subset of rows to evaluate
    only those tokens (every term is per token).
    """
    u = np.asarray(u, dtype=np.float64)
    x = u if x is None else np.asarray(x, dtype=np.float64)
    out = u.copy()
    for wg, wu, wd in shared:
        out += ffn(x, wg, wu, wd)
    idx = np.asarray(idx)
    gate = np.asarray(gate, dtype=np.float64)

    def term(e):
        rows, slots = np.nonzero(idx == e)
        wg, wu, wd = routed(int(e))
        return rows, gate[rows, slots][:, None] * ffn(x[rows], wg, wu, wd)

    for rows, y in map(term, np.unique(idx)):
        out[rows] += y
    return out


def seq_balance_loss(s, idx, seq_len: int, alpha: float = 1e-4) -> np.ndarray:
    """R15: one loss per sequence of seq_len consecutive tokens, float64."""
    s = np.asarray(s, dtype=np.float64)
    idx = np.asarray(idx)
    t_n, n = s.shape
    k = idx.shape[1]
    out = []
    for q in range(t_n // seq_len):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        counts = np.bincount(idx[rows].ravel(), minlength=n).astype(np.float64)
        f = counts * n / (k * seq_len)
        p = (s[rows] / s[rows].sum(axis=1, keepdims=True)).mean(axis=0)
        out.append(alpha * float(np.sum(f * p)))
    return np.array(out)


def affinity64(u, centroids) -> np.ndarray:
    """s = Sigmoid(u^T e) in float64 throughout (the smooth form the backward differentiates)."""
    z = np.asarray(u, dtype=np.float64) @ np.asarray(centroids, dtype=np.float64).T
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_ffn_backward(x, w_gate, w_up, w_down, dy):
    """Gradients of y = (SiLU(x Wg^T) * (x Wu^T)) Wd^T given dL/dy: (dx, dWg, dWu, dWd), float64.

    With a = x Wg^T, b = x Wu^T, h = SiLU(a) * b and SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))):
    dh = dy Wd, dWd = dy^T h, da = dh * b * SiLU'(a), db = dh * SiLU(a),
    dx = da Wg + db Wu, dWg = da^T x, dWu = db^T x.
    """
    x = np.asarray(x, dtype=np.float64)
    wg, wu, wd = (np.asarray(w, dtype=np.float64) for w in (w_gate, w_up, w_down))
    dy = np.asarray(dy, dtype=np.float64)
    a = x @ wg.T
    b = x @ wu.T
    sg = 1.0 / (1.0 + np.exp(-a))
    h = a * sg * b
    dh = dy @ wd
    da = dh * b * sg * (1.0 + a * (1.0 - sg))
    db = dh * a * sg
    return da @ wg + db @ wu, da.T @ x, db.T @ x, dy.T @ h


def layer_backward(u, centroids, idx, routed, shared, dout, map=map):
    """Backward of the layer (R14): gradients of <dout, h'> for a fixed selection idx.

    routed: e -> (w_gate, w_up, w_down); shared: sequence of (w_gate, w_up, w_down).
    Returns (du [T, d], d_centroids [N_r, d], d_routed {e: (dWg, dWu, dWd)} for the experts
    that appear in idx, d_shared [(dWg, dWu, dWd)] per shared expert), all float64.
    map: how the routed experts' terms are evaluated (as in layer_forward; they are added in
    increasing expert order either way).

    With g_k = s_k / S (S = sum of the selected s) and dg_k = <dout_t, FFN_k(u_t)>:
    ds_j = dg_j / S - (sum_k dg_k s_k) / S^2 for selected j (0 elsewhere),
    dz = ds * s (1 - s), du_t += sum_k dz_k e_k, de_k += dz_k u_t.
    """
    u = np.asarray(u, dtype=np.float64)
    e = np.asarray(centroids, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    idx = np.asarray(idx)
    t_n, k_n = idx.shape
    s = affinity64(u, e)
    ssel = np.take_along_axis(s, idx, axis=1)
    ssum = ssel.sum(axis=1, keepdims=True)
    gate = ssel / ssum
    du = dout.copy()
    d_shared = []
    for wg, wu, wd in shared:
        dx, dwg, dwu, dwd = swiglu_ffn_backward(u, wg, wu, wd, dout)
        du += dx
        d_shared.append((dwg, dwu, dwd))
    dg = np.zeros((t_n, k_n))
    d_routed = {}

    def term(ex):
        rows, slots = np.nonzero(idx == ex)
        wg, wu, wd = routed(int(ex))
        y = swiglu_ffn(u[rows], wg, wu, wd)
        dg_e = np.sum(dout[rows] * y, axis=1)
        return (int(ex), rows, slots, dg_e,
                *swiglu_ffn_backward(u[rows], wg, wu, wd, gate[rows, slots][:, None] * dout[rows]))

    for ex, rows, slots, dg_e, dx, dwg, dwu, dwd in map(term, np.unique(idx)):
        dg[rows, slots] = dg_e
        du[rows] += dx
        d_routed[ex] = (dwg, dwu, dwd)
    ds = dg / ssum - np.sum(dg * ssel, axis=1, keepdims=True) / ssum ** 2
    dz = ds * ssel * (1.0 - ssel)
    de = np.zeros_like(e)
    for k in range(k_n):
        du += dz[:, k:k + 1] * e[idx[:, k]]
        np.add.at(de, idx[:, k], dz[:, k:k + 1] * u)
    return du, de, d_routed, d_shared


def stacked(w_gate, w_up, w_down):
    """Accessor e -> (w_gate[e], w_up[e], w_down[e]) over stacked [N, ...] arrays."""
    return lambda e: (w_gate[e], w_up[e], w_down[e])


# ----------------------------------------------------------------------------- FP8 (E4M3FN)

def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to even, saturating at +-448 (R8).

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normal values
    2^(e-7) * (1 + m/8), e = 1..15 (e = 15, m = 7 is NaN, so 448 is the
    largest finite value); subnormals m/8 * 2^-6, spacing 2^-9.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # unbiased exponent of a, floored at the subnormal range
    quantum = np.ldexp(1.0, e - 3)           # spacing of the 3-bit mantissa grid at that exponent
    q = np.round(a / quantum) * quantum      # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, y)


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """Bit patterns (uint8) of E4M3FN values that are already on the grid."""
    q = np.asarray(q, dtype=np.float64)
    sign = (np.signbit(q)).astype(np.uint8) << 7
    a = np.abs(q)
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    code[sub] = np.round(a[sub] / 2.0 ** -9).astype(np.uint8)
    nz = ~sub
    _, ex = np.frexp(a[nz])
    e = ex - 1
    m = np.round((a[nz] / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    code[nz] = ((e + 7) << 3 | m).astype(np.uint8)
    return code | sign


def _e4m3_values(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


_E4M3_TABLE = _e4m3_values(np.arange(256))


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Values of E4M3FN bit patterns (through the 256-entry table of the formula above)."""
    return _E4M3_TABLE[np.asarray(code, dtype=np.uint8)]


def _quant_block(x32: np.ndarray, axis_len_elems):
    amax = np.max(np.abs(x32), axis=axis_len_elems)
    scale = np.where(amax > 0, amax.astype(np.float32) / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return scale


def quantize_act_1x128(x: np.ndarray):
    """Per-row, per-128-column tile quantisation of an activation matrix [rows, K] (R8).

    Returns (codes uint8 [rows, K], scales fp32 [rows, K/128]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    r, k = x32.shape
    assert k % 128 == 0
    t = x32.reshape(r, k // 128, 128)
    scale = _quant_block(t, 2)
    y = (t / scale[:, :, None]).astype(np.float32)      # one fp32 division per element
    q = e4m3_round(y)
    return e4m3_encode(q).reshape(r, k), scale


def quantize_weight_128x128(w: np.ndarray):
    """Per-128x128-block quantisation of a stored [out, in] weight matrix (R8).

    Returns (codes uint8 [out, in], scales fp32 [out/128, in/128]).
    """
    w32 = np.asarray(w, dtype=np.float32)
    n, k = w32.shape
    assert n % 128 == 0 and k % 128 == 0
    t = w32.reshape(n // 128, 128, k // 128, 128)
    scale = _quant_block(t, (1, 3))
    y = (t / scale[:, None, :, None]).astype(np.float32)
    q = e4m3_round(y)
    return e4m3_encode(q).reshape(n, k), scale


def dequant_act(codes, scale) -> np.ndarray:
    r, k = codes.shape
    return (e4m3_decode(codes).reshape(r, k // 128, 128) * np.asarray(scale, np.float64)[:, :, None]).reshape(r, k)


def dequant_weight(codes, scale) -> np.ndarray:
    n, k = codes.shape
    v = e4m3_decode(codes).reshape(n // 128, 128, k // 128, 128) * np.asarray(scale, np.float64)[:, None, :, None]
    return v.reshape(n, k)


def swiglu_ffn_fp8(x_deq: np.ndarray, wq_gate, wq_up, wq_down) -> np.ndarray:
    """Quantisation-faithful expert FFN: inputs already fake-quantised; H is quantised
    per 1x128 tile along I after SiLU(a)*b, in fp32, before the down projection (R8)."""
    a = x_deq @ dequant_weight(*wq_gate).T
    b = x_deq @ dequant_weight(*wq_up).T
    h = (silu(a) * b).astype(np.float32)
    hq = dequant_act(*quantize_act_1x128(h))
    return hq @ dequant_weight(*wq_down).T


def layer_forward_fp8(u, idx, gate, routed_q, shared_q, map=map) -> np.ndarray:
    """Quantisation-faithful FP8 layer: u quantised per 1x128 tile, weights per 128x128 block
    (routed_q(e) / shared_q entries are ((codes, scale) x 3) from quantize_weight_128x128),
    H quantised per 1x128 tile; float64 arithmetic on the dequantised values (R8)."""
    u32 = np.asarray(u, dtype=np.float32)
    x = dequant_act(*quantize_act_1x128(u32))
    return layer_forward(u32, idx, gate, routed_q, shared_q, ffn=swiglu_ffn_fp8, x=x, map=map)


# ----------------------------------------------------------------------------- FP8 backward (R16)

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) through fp32, returned as float64."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def quantize_runs_of_rows(x: np.ndarray) -> np.ndarray:
    """Fake-quantise [rows, C] along the rows: each column is cut into runs of 128 consecutive
    rows (the last run zero-padded), and each run is one 1x128 tile of R8.  Returns the
    dequantised values, float64 [rows, C]."""
    x32 = np.asarray(x, dtype=np.float32)
    r, c = x32.shape
    rp = -(-r // 128) * 128
    t = np.zeros((c, rp), dtype=np.float32)
    t[:, :r] = x32.T
    return dequant_act(*quantize_act_1x128(t))[:, :r].T


class ExactPolicy:
    """Every quantiser and storage rounding of R16 replaced by the identity: the steps of
    layer_backward_steps then state the R14 backward."""

    @staticmethod
    def tiles(x):          # 1x128 tiles along the last axis
        return np.asarray(x, dtype=np.float64)

    @staticmethod
    def runs(x):           # runs of 128 rows
        return np.asarray(x, dtype=np.float64)

    @staticmethod
    def held(x):           # storage between steps
        return np.asarray(x, dtype=np.float64)

    @staticmethod
    def scaled(g, x):      # gate * dout
        return np.asarray(g, dtype=np.float64)[:, None] * np.asarray(x, dtype=np.float64)

    @staticmethod
    def saved(x):          # the SwiGLU inputs a, b as the backward reads them
        return np.asarray(x, dtype=np.float64)


class Fp8Policy:
    """The quantisers and storage precisions of R16."""

    @staticmethod
    def tiles(x):
        return dequant_act(*quantize_act_1x128(np.asarray(x, dtype=np.float32)))

    runs = staticmethod(quantize_runs_of_rows)
    held = staticmethod(bf16_round)

    @staticmethod
    def scaled(g, x):      # one fp32 product per element
        return (np.asarray(g, dtype=np.float32)[:, None] * np.asarray(x, dtype=np.float32)).astype(np.float64)

    saved = ExactPolicy.saved   # a, b recomputed in the backward


class Bf16Policy:
    """The storage precisions of R17: no quantiser, held tensors in bf16, gate * dout rounded
    once to bf16 from its fp32 product, a and b recomputed."""

    tiles = ExactPolicy.tiles
    runs = ExactPolicy.runs
    held = staticmethod(bf16_round)
    saved = ExactPolicy.saved

    @staticmethod
    def scaled(g, x):
        return bf16_round(np.asarray(g, dtype=np.float32)[:, None] * np.asarray(x, dtype=np.float32))


class Bf16SavedPolicy(Bf16Policy):
    """R17 with a and b held in bf16 from the forward (the saved-input variant)."""

    saved = staticmethod(bf16_round)


class Fp8SavedPolicy(Fp8Policy):
    """R16 with a and b held in bf16 from the forward (the saved-input variant of R17)."""

    saved = staticmethod(bf16_round)


def expert_backward(x, dy, u_rows, dout_rows, g, wg, wu, wd, q):
    """One expert's part of layer_backward_steps over its rows (token order): x = tiles(u) and
    dy = tiles(dout) of those rows, their held u and dout, and their gates g.
    Returns (dx [rows, d], dg [rows], (dWg, dWu, dWd))."""
    wg, wu, wd = (np.asarray(w, dtype=np.float64) for w in (wg, wu, wd))
    g = np.asarray(g, dtype=np.float64)
    a = q.saved(x @ wg.T)
    b = q.saved(x @ wu.T)
    dh_pre = q.held(dy @ wd)
    sg = 1.0 / (1.0 + np.exp(-a))
    h = a * sg * b
    dg = np.sum(dh_pre * h, axis=1)
    dh = g[:, None] * dh_pre
    da = q.held(dh * b * sg * (1.0 + a * (1.0 - sg)))
    db = q.held(dh * a * sg)
    dx = q.tiles(np.concatenate([da, db], axis=1)) @ np.concatenate([wg, wu], axis=0)
    uo = q.runs(u_rows)
    dwd = q.runs(q.scaled(g, dout_rows)).T @ q.runs(q.held(h))
    return dx, dg, (q.runs(da).T @ uo, q.runs(db).T @ uo, dwd)


def layer_backward_steps(u, centroids, idx, routed, shared, dout, q, map=map):
    """The R14 backward taken step by step, each GEMM operand passed through policy q (R16).

    routed(e) / shared[i] give float64 (w_gate [I, d], w_up [I, d], w_down [d, I]); for the FP8
    backward these are the dequantised 128x128-block weights.  Per expert, with its rows in
    token order and gate column g (1 for a shared expert), x = tiles(u), dy = tiles(dout):
      a = x Wg^T, b = x Wu^T, dH = held(dy Wd), h = SiLU(a) b, dg = sum dH h,
      dA = held(g dH b SiLU'(a)), dB = held(g dH SiLU(a)), dx = tiles([dA dB]) [Wg; Wu],
      dWd = runs(scaled(g, dout))^T runs(held(h)), dWg = runs(dA)^T runs(u), dWu = runs(dB)^T runs(u).
    The router part and the residual follow layer_backward.  Returns the same tuple; map as
    in layer_backward.
    """
    u = np.asarray(u, dtype=np.float64)
    e = np.asarray(centroids, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    idx = np.asarray(idx)
    t_n, k_n = idx.shape
    s = affinity64(u, e)
    ssel = np.take_along_axis(s, idx, axis=1)
    ssum = ssel.sum(axis=1, keepdims=True)
    gate = ssel / ssum
    xq = q.tiles(u)
    dyq = q.tiles(dout)

    def expert(rows, g, wg, wu, wd):
        return expert_backward(xq[rows], dyq[rows], u[rows], dout[rows], g, wg, wu, wd, q)

    du = dout.copy()
    d_shared = []
    all_rows = np.arange(t_n)
    for wg, wu, wd in shared:
        dx, _, grads = expert(all_rows, np.ones(t_n), wg, wu, wd)
        du += dx
        d_shared.append(grads)
    dg = np.zeros((t_n, k_n))
    d_routed = {}

    def term(ex):
        rows, slots = np.nonzero(idx == ex)          # rows ascend: token order
        return (int(ex), rows, slots, *expert(rows, gate[rows, slots], *routed(int(ex))))

    for ex, rows, slots, dx, dg_e, grads in map(term, np.unique(idx)):
        dg[rows, slots] = dg_e
        du[rows] += dx
        d_routed[ex] = grads
    ds = dg / ssum - np.sum(dg * ssel, axis=1, keepdims=True) / ssum ** 2
    dz = ds * ssel * (1.0 - ssel)
    de = np.zeros_like(e)
    for k in range(k_n):
        du += dz[:, k:k + 1] * e[idx[:, k]]
        np.add.at(de, idx[:, k], dz[:, k:k + 1] * u)
    return du, de, d_routed, d_shared


def layer_backward_fp8(u, centroids, idx, routed_q, shared_q, dout, saved=False, map=map):
    """FP8 backward of R16.  routed_q(e) / shared_q entries are ((codes, scale) x 3) from
    quantize_weight_128x128 of (w_gate, w_up, w_down); u and dout as held (bf16 values).
    saved: a and b held in bf16 from the forward (R17's saved-input variant)."""
    deq = lambda ws: tuple(dequant_weight(*w) for w in ws)  # noqa: E731
    return layer_backward_steps(u, centroids, idx, lambda ex: deq(routed_q(ex)), [deq(w) for w in shared_q], dout,
                                Fp8SavedPolicy if saved else Fp8Policy, map=map)
