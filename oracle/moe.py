"""Expert FFN (GMM1, activation, requantization, GMM2) and the weighted combine.

MegaMoE page, "A8W8-FP quantization scenario":
  stage 1  X_e, S_X,e = Q_MX(X[T_e])                (routing.gather_rows)
  stage 2  G_e = DQ(X_e) . DQ(W1_e^(G)),  U_e = DQ(X_e) . DQ(W1_e^(U)),
           A_e = Activation(G_e, U_e),  A^_e, S_A,e = Q_MX(A_e)  (same FP8 type)
  stage 3  O_e = DQ(A^_e) . DQ(W2_e)
  stage 4  Y[i] = sum_k W[i,k] O[pi(i,k)] + sum_s O_s^shared[i],  Y is BF16
"Activation function formulas": sigma(z) = 1/(1+e^-z), SiLU(z) = z sigma(z); with
the clamp c (+inf when not configured or 0), G_c = min(G, c), U_c = clip(U, -c, c):
  swiglu      A = SiLU(G_c) * U_c
  swiglustep  A = min(SiLU(G), c) * U_c
  swigluoai   A = G_c * sigma(alpha G_c) * (U_c + beta)
  situglu     A = beta tanh(G / beta) * sigma(G) * L(U), L(U) = U, or
              lb tanh(U / lb) when linear_beta lb is configured
  gelu        A = Z * sigma(sqrt(8/pi) (Z + 0.044715 Z^3)) on the whole GMM1 output
              Z (no split, no clamp), so A and weight2's input are 2I wide.
Parameter lists and defaults (activation_params): swiglu / swiglustep [] or
[clamp]; swigluoai [] or [clamp, alpha, beta] with defaults alpha 1.702, beta 1.0;
situglu [], [beta] or [beta, linear_beta] with default beta 1.0; gelu takes none
(its placeholder [FLT_MAX] is ignored).
"MXFP quantization scenario constraints": weight1 (E, 2I, H) and weight2
(E, H, I), each output channel holding its K-contiguous inputs; G is the first
I output channels of weight1 and U the last I (the page splits the logical
H x 2I matrix into its first and second halves of columns).

Readings: accumulations are float64 on exact dequantized operands; the
activation is evaluated in float64 and rounded once to fp32 before the MX
requantization (the pages do not give A's precision); the combine sums in
float64 in k order, then the shared experts, and rounds once to bf16 (one GPU:
no bf16 wire format between expert output and combine).
"""

from __future__ import annotations

import numpy as np

from . import mxfp, routing


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):   # e^-z = inf for very negative z: the limit 0 is right
        return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    """A = SiLU(G) * U (no clamp)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


ACTIVATIONS = ("swiglu", "swiglustep", "swigluoai", "situglu", "gelu")


def activation_settings(kind, params=()):
    """The (clamp, alpha, beta, linear_beta) an activation uses, from its parameter list
    with the pages' defaults; clamp +inf = none (0 means none), linear_beta None = L(U) = U."""
    p = [float(v) for v in params]
    clamp, alpha, beta, lin = np.inf, 1.702, 1.0, None
    if kind in ("swiglu", "swiglustep"):
        assert len(p) in (0, 1)
        if p and p[0] > 0:
            clamp = p[0]
    elif kind == "swigluoai":
        assert len(p) in (0, 3)
        if p:
            clamp = p[0] if p[0] > 0 else np.inf
            alpha, beta = p[1], p[2]
    elif kind == "situglu":
        assert len(p) in (0, 1, 2) and all(v > 0 for v in p)
        if p:
            beta = p[0]
        if len(p) == 2:
            lin = p[1]
    else:
        assert kind == "gelu" and len(p) <= 1
    return clamp, alpha, beta, lin


def activate(h1, kind="swiglu", params=()):
    """Activation of GMM1's output h1 [m, 2I] (float64): gated kinds take G = h1[:, :I]
    and U = h1[:, I:] and return [m, I]; gelu returns [m, 2I]."""
    h1 = np.asarray(h1, dtype=np.float64)
    c, alpha, beta, lin = activation_settings(kind, params)
    if kind == "gelu":
        z = h1
        return z * sigmoid(np.sqrt(8.0 / np.pi) * (z + 0.044715 * z ** 3))
    inter = h1.shape[1] // 2
    g, u = h1[:, :inter], h1[:, inter:]
    gc, uc = np.minimum(g, c), np.clip(u, -c, c)
    if kind == "swiglu":
        return silu(gc) * uc
    if kind == "swiglustep":
        return np.minimum(silu(g), c) * uc
    if kind == "swigluoai":
        return gc * sigmoid(alpha * gc) * (uc + beta)
    if kind == "situglu":
        lu = u if lin is None else lin * np.tanh(u / lin)
        return beta * np.tanh(g / beta) * sigmoid(g) * lu
    raise ValueError(kind)


def gmm(aq, sa, wq, ws, fmt, wfmt=None):
    """DQ_MX(A) . DQ_MX(W)^T for W stored (out, in): float64 [m, out]. wfmt: the weights'
    element format when it differs from the activations' (A8W4-FP: "e2m1", codes two a
    byte as stored, element 2j in the low nibble)."""
    wfmt = fmt if wfmt is None else wfmt
    ad = mxfp.dequantize(aq, sa, fmt)
    wcodes = mxfp.unpack_fp4(wq) if wfmt == "e2m1" else wq
    wd = mxfp.dequantize(wcodes, ws, wfmt)
    return ad @ wd.T


def expert_ffn(xq, sx, w1q, w1s, w2q, w2s, fmt, act=("swiglu", ()), wfmt=None):
    """Stages 2-3 for the rows of one expert. xq/sx: [m, H] codes/scales;
    act = (activation kind, parameter list); wfmt = the weights' format (A8W4-FP: "e2m1",
    MegaMoE "A8W4-FP quantization scenario": X^ and A^ stay MXFP8, W1 and W2 MXFP4)."""
    h1 = gmm(xq, sx, w1q, w1s, fmt, wfmt)
    a = mxfp.fp32_round(activate(h1, *act))
    assert a.shape[1] == w2q.shape[1] * (2 if wfmt == "e2m1" else 1), "weight2's input width must equal A's"
    aq, sa = mxfp.quantize(a, fmt)
    o = gmm(aq, sa, w2q, w2s, fmt, wfmt)
    return dict(h1=h1, a=a, aq=aq, sa=sa, o=o)


def _getter(weights):
    """weights: either a tuple of stacked arrays (w1q, w1s, w2q, w2s) with a leading
    expert axis, or a callable e -> (w1q[e], w1s[e], w2q[e], w2s[e])."""
    if callable(weights):
        return weights
    w1q, w1s, w2q, w2s = weights
    return lambda e: (w1q[e], w1s[e], w2q[e], w2s[e])


def combine(o_rows, expanded_row_idx, topk_weights, shared_o=(), combine_comm_mode=0):
    """Stage 4: Y[t] = bf16( sum_k w[t,k] O[row(t,k)] + sum_s O_s[t] ), float64 sum.

    MegaMoE combineCommMode: with 0 (no deduplication, the default) each expert's output
    row is sent back as BF16, so every O row (routed and shared) is rounded to bf16
    before the weighted sum; with 1 a token's expert outputs on the card are summed in
    FP32 and converted to BF16 once, so the rows enter the sum unrounded."""
    if combine_comm_mode not in (0, 1):
        raise ValueError("combine_comm_mode must be 0 or 1 on one card")
    rows = mxfp.bf16_round if combine_comm_mode == 0 else (lambda v: np.asarray(v, dtype=np.float64))
    w = np.asarray(topk_weights, dtype=np.float64)
    n, k = w.shape
    idx = np.asarray(expanded_row_idx).reshape(n, k)
    o_rows = rows(o_rows)
    y = np.zeros((n, o_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * o_rows[idx[:, j]]
    for o_s in shared_o:
        y += rows(o_s)
    return mxfp.bf16_round(y)


def mega_moe(x, topk_ids, topk_weights, weights, fmt, num_experts, shared=(), act=("swiglu", ()), wfmt=None,
             shared_wfmt=None, combine_comm_mode=0, workers=1) -> dict:
    """The whole layer on all tokens, in the permuted (expert-contiguous) order.

    x: [N, H] values (bf16 as float64); topk_ids int [N, K]; topk_weights [N, K];
    weights: see _getter; shared: list of (w1q, w1s, w2q, w2s) per shared expert.
    workers > 1 evaluates the experts' FFNs (independent of one another) in that many
    threads; the results are the same.
    Returns routing, xq/sx (permuted), h1 [F, 2I], a, aq, sa, o [F, H],
    shared outputs, y (float64 bf16 values) and expert_token_nums (int32 [E])."""
    x = np.asarray(x, dtype=np.float64)
    get = _getter(weights)
    quant_mode = {"e5m2": 2, "e4m3": 3}[fmt]
    r = routing.init_routing(topk_ids, num_experts)
    k = r["topk"]
    xq, sx = routing.gather_rows(x, r["sorted_row_idx"], k, quant_mode)
    flat = xq.shape[0]
    busy = [e for e in range(num_experts) if r["offsets"][e + 1] > r["offsets"][e]]

    def run(e):
        lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
        return e, expert_ffn(xq[lo:hi], sx[lo:hi], *get(e), fmt, act, wfmt)

    if workers > 1 and len(busy) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            parts = dict(ex.map(run, busy))
    else:
        parts = dict(run(e) for e in busy)
    hidden = x.shape[1]
    shape_of = get(busy[0] if busy else 0)   # any expert's weights give the widths
    two_i = shape_of[0].shape[0]
    aw = shape_of[2].shape[1] * (2 if wfmt == "e2m1" else 1)   # width of A: I (gated) or 2I (gelu)
    out = dict(routing=r, xq=xq, sx=sx,
               h1=np.zeros((flat, two_i)), a=np.zeros((flat, aw)),
               aq=np.zeros((flat, aw), np.uint8),
               sa=np.zeros((flat, mxfp.scale_cols(aw)), np.uint8),
               o=np.zeros((flat, hidden)))
    for e, p in parts.items():
        lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
        for name in ("h1", "a", "aq", "sa", "o"):
            out[name][lo:hi] = p[name]
    shared_o = []
    if shared:
        xq_tok, sx_tok = mxfp.quantize(x, fmt)
        out["xq_tok"], out["sx_tok"] = xq_tok, sx_tok
        for sw in shared:
            shared_o.append(expert_ffn(xq_tok, sx_tok, *sw, fmt, act,
                                       wfmt if shared_wfmt is None else shared_wfmt)["o"])
    out["shared_o"] = shared_o
    full_scatter = routing.inverse(r["sorted_row_idx"])
    out["y"] = combine(out["o"], full_scatter, topk_weights, shared_o, combine_comm_mode)
    out["expert_token_nums"] = r["counts"].astype(np.int32)
    return out


def per_token(x, topk_ids, topk_weights, weights, fmt, tokens, shared=(), act=("swiglu", ()), wfmt=None,
              shared_wfmt=None, combine_comm_mode=0) -> dict:
    """The layer for selected tokens, one (token, k) at a time, with no permutation
    (the "brute force" form of stage 1-4: each expert receives a copy of x_t).

    Returns y [len(tokens), H] (bf16 values as float64) and, per (token, k), the
    expert's h1 and o rows: h1[j, k], o[j, k]."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_weights, dtype=np.float64)
    get = _getter(weights)
    tokens = list(tokens)
    k = ids.shape[1]
    cache = {}

    def expert(e):
        if e not in cache:
            if len(cache) >= 16:
                cache.clear()
            cache[e] = get(e)
        return cache[e]

    # combineCommMode 0: each expert's output row arrives at the combine as BF16
    rows = mxfp.bf16_round if combine_comm_mode == 0 else (lambda v: v)
    ys, h1s, os_ = [], [], []
    for t in tokens:
        xq_t, sx_t = mxfp.quantize(x[t:t + 1], fmt)
        acc = np.zeros((1, x.shape[1]))
        h1_t, o_t = [], []
        for j in range(k):
            r = expert_ffn(xq_t, sx_t, *expert(int(ids[t, j])), fmt, act, wfmt)
            acc = acc + w[t, j] * rows(r["o"])
            h1_t.append(r["h1"][0])
            o_t.append(r["o"][0])
        for sw in shared:
            acc = acc + rows(expert_ffn(xq_t, sx_t, *sw, fmt, act, wfmt if shared_wfmt is None else shared_wfmt)["o"])
        ys.append(mxfp.bf16_round(acc)[0])
        h1s.append(h1_t)
        os_.append(o_t)
    return dict(y=np.array(ys), h1=np.array(h1s), o=np.array(os_))
