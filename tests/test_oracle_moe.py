"""Pins for oracle.moe: activation, GEMMs, combine, the whole permuted layer.

Independent references: closed forms of SiLU/SwiGLU, an exact integer GEMM on
the same MX operands, a dense special case (one-hot input reproduces a weight
row), and the per-token brute force (no permutation) which must equal the
permuted layer bit for bit when the float64 GEMMs are exact.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs
from oracle import moe, mxfp, routing


def quantized_weights(cfg, n_experts=None, shared=False):
    n_experts = cfg.experts if n_experts is None else n_experts
    tag1, tag2 = ("sw1", "sw2") if shared else ("w1", "w2")
    w1q, w1s, w2q, w2s = [], [], [], []
    for e in range(n_experts):
        a = moe_inputs.weight_master(cfg, tag1, e).double().numpy()
        b = moe_inputs.weight_master(cfg, tag2, e).double().numpy()
        q1, s1 = mxfp.quantize(a, cfg.fmt)
        q2, s2 = mxfp.quantize(b, cfg.fmt)
        w1q.append(q1); w1s.append(s1); w2q.append(q2); w2s.append(s2)
    return tuple(np.stack(t) for t in (w1q, w1s, w2q, w2s))


def layer_inputs(cfg):
    x = moe_inputs.activations(cfg).double().numpy()
    return x, moe_inputs.expert_ids(cfg), moe_inputs.gate_weights(cfg)


def test_silu_closed_forms():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert moe.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert moe.silu(np.array([-2.0]))[0] == pytest.approx(-2.0 / (1.0 + math.exp(2.0)), rel=1e-15)
    assert moe.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-15)
    assert moe.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0


def _h1(g, u):
    return np.concatenate([np.atleast_2d(np.asarray(g, np.float64)), np.atleast_2d(np.asarray(u, np.float64))],
                          axis=1)


def test_activation_special_cases():
    """MegaMoE "Activation function formulas", checked through special cases that reduce
    to something else: no clamp gives the plain SwiGLU; a clamp saturates G from above and
    U on both sides; swigluoai with alpha = 1, beta = 0 is SwiGLU and with alpha = 0 is
    G (U + beta) / 2; situglu with a huge beta is SwiGLU; G = 0 gives 0 for every gated kind."""
    rng = np.random.default_rng(3)
    g, u = rng.normal(0, 2, (4, 64)), rng.normal(0, 2, (4, 64))
    h1 = np.concatenate([g, u], axis=1)
    plain = moe.swiglu(g, u)
    assert np.array_equal(moe.activate(h1, "swiglu"), plain)
    assert np.array_equal(moe.activate(h1, "swiglu", (0.0,)), plain)          # clamp 0 = none
    assert np.allclose(moe.activate(h1, "swigluoai", (0.0, 1.0, 0.0)), plain, rtol=1e-14, atol=0)
    assert np.allclose(moe.activate(h1, "situglu", (1e7,)), plain, rtol=1e-9, atol=1e-12)
    half = moe.activate(h1, "swigluoai", (0.0, 0.0, 0.75))
    assert np.allclose(half, g * (u + 0.75) / 2.0, rtol=1e-14, atol=0)
    for kind in ("swiglu", "swiglustep", "swigluoai", "situglu"):
        assert np.all(moe.activate(_h1(np.zeros(8), rng.normal(size=8)), kind) == 0.0)
    # clamp c = 1.5: G = 10 -> G_c = 1.5; U = -9 -> -1.5, U = 0.25 unchanged
    a = moe.activate(_h1([10.0, 10.0], [-9.0, 0.25]), "swiglu", (1.5,))[0]
    s15 = 1.5 / (1.0 + math.exp(-1.5))
    assert a[0] == pytest.approx(-1.5 * s15, rel=1e-15) and a[1] == pytest.approx(0.25 * s15, rel=1e-15)
    # swiglustep clamps SiLU(G) itself, not G: SiLU(10) ~ 10 -> 2; SiLU(1) < 2 untouched
    st = moe.activate(_h1([10.0, 1.0], [1.0, 1.0]), "swiglustep", (2.0,))[0]
    assert st[0] == 2.0 and st[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # situglu's linear beta: L(U) = lb tanh(U / lb) saturates at lb
    sl = moe.activate(_h1([50.0], [1e6]), "situglu", (3.0, 0.5))[0]
    assert sl[0] == pytest.approx(3.0 * 1.0 * 0.5, rel=1e-12)


def test_activation_defaults():
    """Empty parameter lists take the pages' defaults: swigluoai (no clamp, alpha 1.702,
    beta 1.0), situglu (beta 1.0, L(U) = U)."""
    rng = np.random.default_rng(4)
    h1 = rng.normal(0, 3, (3, 40))
    assert np.array_equal(moe.activate(h1, "swigluoai"), moe.activate(h1, "swigluoai", (0.0, 1.702, 1.0)))
    assert np.array_equal(moe.activate(h1, "situglu"), moe.activate(h1, "situglu", (1.0,)))
    assert np.array_equal(moe.activate(h1, "gelu"), moe.activate(h1, "gelu", (float(np.finfo(np.float32).max),)))


def test_gelu_tanh_form_and_width():
    """The page writes gelu two ways: Z (1 + tanh(sqrt(2/pi)(Z + 0.044715 Z^3))) / 2 and
    Z sigma(sqrt(8/pi)(...)); the oracle uses the second, the first must agree (since
    (1 + tanh x) / 2 = sigma(2x)). gelu keeps every channel: [m, 2I] in, [m, 2I] out,
    and gelu(0) = 0, gelu(Z) -> Z for large Z, -> 0 for very negative Z."""
    z = np.linspace(-8, 8, 321).reshape(3, 107)
    tanh_form = 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))
    got = moe.activate(z, "gelu")
    assert got.shape == z.shape
    assert np.allclose(got, tanh_form, rtol=1e-13, atol=1e-15)
    edge = moe.activate(np.array([[0.0, 30.0, -30.0]]), "gelu")[0]
    assert edge[0] == 0.0 and edge[1] == pytest.approx(30.0, rel=1e-15) and abs(edge[2]) < 1e-300


def test_gelu_layer_uses_all_channels():
    """A gelu expert: A = gelu(h1) over all 2I channels and weight2 has 2I inputs."""
    cfg = moe_inputs.config("tiny", tokens=16, hidden=64, inter=64, experts=2, topk=1, seed=5)
    x, ids, w = layer_inputs(cfg)
    w1q, w1s = mxfp.quantize(moe_inputs.weight_master(cfg, "w1", 0).double().numpy(), cfg.fmt)
    w2q, w2s = mxfp.quantize(moe_inputs.weight_master(cfg, "w2g", 0).double().numpy(), cfg.fmt)
    assert w2q.shape == (64, 128)
    xq, sx = mxfp.quantize(x, cfg.fmt)
    r = moe.expert_ffn(xq, sx, w1q, w1s, w2q, w2s, cfg.fmt, ("gelu", ()))
    assert r["a"].shape == (16, 128) and r["aq"].shape == (16, 128)
    assert np.array_equal(r["a"], mxfp.fp32_round(moe.activate(r["h1"], "gelu")))


def test_gate_is_first_half_up_is_second_half():
    """x one-hot at k=0 with value 1, all scales 2^0: G = W1[n, 0], U = W1[I + n, 0].
    With G=2, U=3 the activation is SiLU(2)*3 (swapping the halves would give SiLU(3)*2)."""
    fmt, h, inter = "e4m3", 32, 32
    one, two, three = 0x38, 0x40, 0x44
    xq = np.zeros((1, h), np.uint8); xq[0, 0] = one
    sx = np.full((1, 2), 127, np.uint8); sx[0, 1] = 0
    w1q = np.zeros((2 * inter, h), np.uint8); w1q[:inter, 0] = two; w1q[inter:, 0] = three
    w1s = np.full((2 * inter, 2), 127, np.uint8)
    w2q = np.zeros((h, inter), np.uint8); w2s = np.full((h, 2), 127, np.uint8)
    r = moe.expert_ffn(xq, sx, w1q, w1s, w2q, w2s, fmt)
    assert np.all(r["h1"][0, :inter] == 2.0) and np.all(r["h1"][0, inter:] == 3.0)
    expect = np.float32(2.0 / (1.0 + math.exp(-2.0)) * 3.0)
    assert np.all(r["a"][0] == expect)


def test_one_hot_input_reproduces_weight_row():
    rng = np.random.default_rng(1)
    fmt = "e5m2"
    wq = rng.integers(0, 0x7B, size=(48, 64)).astype(np.uint8)
    ws = rng.integers(110, 140, size=(48, 2)).astype(np.uint8)
    for k in (0, 17, 40, 63):
        aq = np.zeros((1, 64), np.uint8); aq[0, k] = 0x3C          # 1.0 in E5M2
        sa = np.full((1, 2), 127, np.uint8)
        out = moe.gmm(aq, sa, wq, ws, fmt)[0]
        assert np.array_equal(out, mxfp.dequantize(wq, ws, fmt)[:, k])


def exact_int_gemm(aq, sa, wq, ws, fmt):
    """The same product in exact integer arithmetic: every MX value is an integer
    multiple of 2^(esub + b - 127); scale everything to integers and use Python ints."""
    t = mxfp.decode_table(fmt)
    esub = {"e4m3": -9, "e5m2": -16}[fmt]
    ai = (t[aq] * 2.0 ** -esub).astype(np.int64)       # exact small integers
    wi = (t[wq] * 2.0 ** -esub).astype(np.int64)
    ga = np.repeat(sa[:, : aq.shape[1] // 32].astype(np.int64), 32, axis=1)
    gw = np.repeat(ws[:, : wq.shape[1] // 32].astype(np.int64), 32, axis=1)
    out = np.zeros((aq.shape[0], wq.shape[0]), dtype=object)
    emin = int(ga.min() + gw.min())
    for i in range(aq.shape[0]):
        sh_a = ga[i] - emin
        for n in range(wq.shape[0]):
            terms = [int(a) * int(w) << int(s1 + s2) for a, w, s1, s2 in zip(ai[i], wi[n], sh_a, gw[n]) if a and w]
            out[i, n] = sum(terms)
    scale = 2.0 ** (2 * esub + emin - 254)
    return out, scale


def test_float64_gemm_is_exact_on_small_shapes():
    cfg = moe_inputs.config("tiny")
    x, ids, _ = layer_inputs(cfg)
    w1q, w1s, _, _ = quantized_weights(cfg, n_experts=1)
    xq, sx = mxfp.quantize(x[:6], cfg.fmt)
    got = moe.gmm(xq, sx, w1q[0][:20], w1s[0][:20], cfg.fmt)
    ints, scale = exact_int_gemm(xq, sx, w1q[0][:20], w1s[0][:20], cfg.fmt)
    for i in range(6):
        for n in range(20):
            assert got[i, n] == float(ints[i, n]) * scale


@pytest.mark.parametrize("mode", [0, 1])
def test_brute_force_equals_permuted_layer_bitwise(mode):
    cfg = moe_inputs.config("tiny", shared=1)
    x, ids, w = layer_inputs(cfg)
    weights = quantized_weights(cfg)
    shared = [tuple(a[0] for a in quantized_weights(cfg, 1, shared=True))]
    full = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, shared=shared, combine_comm_mode=mode)
    bf = moe.per_token(x, ids, w, weights, cfg.fmt, range(cfg.tokens), shared=shared, combine_comm_mode=mode)
    assert np.array_equal(full["y"], bf["y"])
    inv = routing.inverse(full["routing"]["sorted_row_idx"]).reshape(cfg.tokens, cfg.topk)
    for t in range(cfg.tokens):
        for k in range(cfg.topk):
            assert np.array_equal(full["h1"][inv[t, k]], bf["h1"][t, k])
            assert np.array_equal(full["o"][inv[t, k]], bf["o"][t, k])
    assert full["expert_token_nums"].sum() == cfg.flat
    assert np.array_equal(full["y"], mxfp.bf16_round(full["y"]))


def test_sub_batch_and_threaded_experts_match_the_whole_layer():
    """The layer on a subset of the tokens gives those tokens' Y of the whole layer bit
    for bit (each token depends only on its own row and experts), and evaluating the
    experts in threads changes nothing: the full-size GPU tests use both."""
    cfg = moe_inputs.config("tiny", tokens=96, experts=8, topk=3, shared=1, seed=77)
    x, ids, w = layer_inputs(cfg)
    weights = quantized_weights(cfg)
    shared = [tuple(a[0] for a in quantized_weights(cfg, 1, shared=True))]
    full = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, shared=shared)
    threaded = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, shared=shared, workers=4)
    for key in ("y", "h1", "a", "aq", "sa", "o"):
        assert np.array_equal(full[key], threaded[key]), key
    tokens = np.array([3, 17, 40, 41, 95])
    sub = moe.mega_moe(x[tokens], ids[tokens], w[tokens], weights, cfg.fmt, cfg.experts, shared=shared, workers=3)
    assert np.array_equal(sub["y"], full["y"][tokens])
    # a getter that knows only the experts the sub-batch uses
    used = set(int(e) for e in ids[tokens].reshape(-1))
    only = {e: tuple(a[e] for a in weights) for e in used}
    sub2 = moe.mega_moe(x[tokens], ids[tokens], w[tokens], lambda e: only[e], cfg.fmt, cfg.experts, shared=shared)
    assert np.array_equal(sub2["y"], full["y"][tokens])


@pytest.mark.parametrize("mode", [0, 1])
def test_topk_one_unit_weight_is_plain_unpermute(mode):
    """K = 1, w = 1, no shared expert: Y is the unpermuted O rounded to bf16 in both
    combine modes (rounding a row to bf16 twice changes nothing)."""
    cfg = moe_inputs.config("tiny", topk=1)
    x, ids, _ = layer_inputs(cfg)
    weights = quantized_weights(cfg)
    w = np.ones((cfg.tokens, 1), np.float32)
    full = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, combine_comm_mode=mode)
    inv = routing.inverse(full["routing"]["sorted_row_idx"])
    assert np.array_equal(full["y"], mxfp.bf16_round(full["o"][inv]))


def test_combine_comm_mode_worked_example():
    """MegaMoE combineCommMode: BF16 rows per expert (0) against one FP32 merge (1), on a
    hand-derived two-expert example (tests/golden/combine_comm_mode.json)."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "combine_comm_mode.json")))
    o = np.array(g["expert_rows"], np.float64)[:, None]
    w = np.array(g["topk_weights"], np.float64)
    for mode, want in g["y"].items():
        y = moe.combine(o, np.array([0, 1]), w, combine_comm_mode=int(mode))
        assert y.shape == (1, 1) and y[0, 0] == want, (mode, y)
    with pytest.raises(ValueError):
        moe.combine(o, np.array([0, 1]), w, combine_comm_mode=2)


def test_zero_gate_weights_leave_the_shared_expert():
    cfg = moe_inputs.config("tiny", shared=1)
    x, ids, _ = layer_inputs(cfg)
    weights = quantized_weights(cfg)
    shared = [tuple(a[0] for a in quantized_weights(cfg, 1, shared=True))]
    w = np.zeros((cfg.tokens, cfg.topk), np.float32)
    full = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, shared=shared)
    xq, sx = mxfp.quantize(x, cfg.fmt)
    dense = moe.expert_ffn(xq, sx, *shared[0], cfg.fmt)["o"]
    assert np.array_equal(full["y"], mxfp.bf16_round(dense))


def test_a8w4_gemm_equals_the_same_weights_in_fp8():
    """A8W4-FP (MegaMoE "A8W4-FP quantization scenario"): FP8 activations times MXFP4
    weights. Every E2M1 value is exact in E4M3, so the same dequantized weights written
    as E4M3 codes under the same E8M0 scales must give the identical float64 product;
    this pins the nibble order and the FP4 dequantization against the FP8 path."""
    rng = np.random.default_rng(12)
    m, n, k = 5, 48, 256
    xq, sx = mxfp.quantize(rng.normal(size=(m, k)), "e4m3")
    w4, ws = mxfp.quantize(rng.normal(size=(n, k)) / 16, "e2m1")
    w4p = mxfp.pack_fp4(w4)
    w8 = mxfp.round_to_format(mxfp.decode_table("e2m1")[w4], "e4m3")
    assert np.array_equal(mxfp.decode_table("e4m3")[w8], mxfp.decode_table("e2m1")[w4])
    got = moe.gmm(xq, sx, w4p, ws, "e4m3", "e2m1")
    assert np.array_equal(got, moe.gmm(xq, sx, w8, ws, "e4m3"))
    # one-hot: x = 1.0 at k = 3 (scale 2^0), weight row 7 = 6.0 at k = 3 (code 7, scale 2^-1)
    xq = np.zeros((1, 64), np.uint8); xq[0, 3] = 0x38
    sx = np.full((1, 2), 127, np.uint8)
    w = np.zeros((16, 64), np.uint8); w[7, 3] = 7
    ws = np.full((16, 2), 126, np.uint8)
    h = moe.gmm(xq, sx, mxfp.pack_fp4(w), ws, "e4m3", "e2m1")
    assert h[0, 7] == 3.0 and np.count_nonzero(h) == 1
