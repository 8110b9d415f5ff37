"""The grouped-GEMM stages on the GPU against the oracle, on identical operands.

GMM1 + SwiGLU + MX requantization (MegaMoE A8W8-FP stage 2): h1 within 2e-3
normwise of the oracle's exact product; the requantized activations compared
code by code (unique where the rounding is decided with margin, a neighbouring
code otherwise). In an exact regime (integer sums, SiLU(G) = G in fp32) the
requantization must match bit for bit.
GMM2 + combine (stages 3-4) fed the oracle's own requantized activations: O
within 2e-3 normwise, the weighted accumulation within the Y tolerance."""
import numpy as np
import pytest
import torch

import moe_inputs
import routing_permute_mxfp8_amd as rp
from oracle import moe, mxfp, routing
from gpu_support import (DEV, FP8, abs_gmm, check_gemm_elementwise, check_requant, normwise_err, oracle_weights,
                         say, swiglu_delta, to_dev, y_errors)

pytestmark = pytest.mark.gpu


def grouped_operands(cfg):
    """Oracle stage-1 operands of a workload: routing + gathered MX rows."""
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg).double().numpy()
    r = routing.init_routing(ids, cfg.experts)
    xq, sx = routing.gather_rows(x, r["sorted_row_idx"], cfg.topk, {"e4m3": 3, "e5m2": 2}[cfg.fmt])
    return ids, x, r, xq, sx


CASES = [
    dict(name="tiny"),
    dict(name="tiny", tokens=300, hidden=384, inter=256, experts=13, topk=3, seed=21),   # ragged groups
    dict(name="skewed", tokens=700, hidden=512, inter=384, experts=24, topk=4, seed=22),  # zipf, E5M2, big groups
    dict(name="tiny", tokens=16, hidden=256, inter=128, experts=64, topk=6, seed=23),    # many empty groups
    dict(name="tiny", tokens=512, hidden=256, inter=128, experts=8, topk=4, seed=24),    # ~256 rows a group, odd K steps
    dict(name="tiny", tokens=600, hidden=512, inter=512, experts=5, topk=3, seed=25),    # LDS-streaming: 2 chunks a group
    dict(name="skewed", tokens=900, hidden=1024, inter=512, experts=12, topk=2, seed=26),  # LDS-streaming, skewed groups
]


def device_weights(wq, ws, wf):
    """Oracle-quantized ND weights on the GPU, packed by the library when wf is PACKED."""
    q, s = to_dev(wq), to_dev(ws)
    if wf == rp.WEIGHTS_PACKED:
        return rp.pack_weights(q, s)
    return q, s


WF = [rp.WEIGHTS_ND, rp.WEIGHTS_PACKED]


@pytest.mark.parametrize("wf", WF, ids=["nd", "packed"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['name']}-{c.get('tokens', '')}")
def test_gmm1_swiglu_quant(case, wf):
    case = dict(case)
    cfg = moe_inputs.config(case.pop("name"), **case)
    say(f"gmm1 N={cfg.tokens} H={cfg.hidden} I={cfg.inter} E={cfg.experts} K={cfg.topk} fmt={cfg.fmt}")
    ids, x, r, xq, sx = grouped_operands(cfg)
    w1q, w1s, w2q, w2s = oracle_weights(cfg)
    offs = to_dev(r["offsets"].astype(np.int32))
    dw, dws = device_weights(w1q, w1s, wf)
    aq, sa, h1 = rp.gmm1_swiglu_quant(to_dev(xq), to_dev(sx), offs, dw, dws, FP8[cfg.fmt], True, weight_format=wf)
    torch.cuda.synchronize()
    h1_ref = np.zeros((xq.shape[0], 2 * cfg.inter))
    h1_abs = np.zeros_like(h1_ref)
    for e in range(cfg.experts):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        if hi > lo:
            h1_ref[lo:hi] = moe.gmm(xq[lo:hi], sx[lo:hi], w1q[e], w1s[e], cfg.fmt)
            h1_abs[lo:hi] = abs_gmm(xq[lo:hi], sx[lo:hi], w1q[e], w1s[e], cfg.fmt)
    h1_got = h1.cpu().numpy()
    err = normwise_err(h1_got, h1_ref)
    ex = check_gemm_elementwise(h1_got, h1_ref, h1_abs, cfg.hidden)
    say(f"  h1 normwise err {err:.3g}, elementwise bound use {ex:.3g}")
    assert err <= 2e-3
    a_ref = mxfp.fp32_round(moe.swiglu(h1_ref[:, :cfg.inter], h1_ref[:, cfg.inter:]))
    delta = swiglu_delta(h1_ref, h1_abs, cfg.hidden, cfg.inter)
    codes, scales = check_requant(aq.cpu().numpy(), sa.cpu().numpy(), a_ref, delta, cfg.fmt)
    say(f"  requant: codes differing from the oracle {codes:.3g}, scales {scales:.3g}")


@pytest.mark.parametrize("wf", WF, ids=["nd", "packed"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_gmm1_requant_exact_regime(fmt, wf):
    """Integer-valued operands: every fp32 sum is exact whatever its order, G >= 256 so
    1 + exp(-G) rounds to 1 and A = G*U exactly on both sides -> bit-exact requant."""
    say(f"gmm1 exact regime fmt={fmt}")
    rng = np.random.default_rng(31)
    rows, h, inter, groups = 93, 256, 256, 5
    one, two = {"e4m3": (0x38, 0x40), "e5m2": (0x3C, 0x40)}[fmt]
    xq = np.full((rows, h), one, np.uint8)
    sx = rng.integers(127, 129, size=(rows, h // 32)).astype(np.uint8)
    w1q = np.empty((groups, 2 * inter, h), np.uint8)
    w1q[:, :inter] = rng.choice([one, two], size=(groups, inter, h))                 # gate: 1 or 2 -> G >= 256
    w1q[:, inter:] = rng.choice([0, one, two, one | 0x80, two | 0x80, 0, 0, 0], size=(groups, inter, h))
    w1s = np.full((groups, 2 * inter, h // 32), 127, np.uint8)
    offs = np.array([0, 10, 10, 41, 90, 93], np.int32)
    dw, dws = device_weights(w1q, w1s, wf)
    aq, sa, h1 = rp.gmm1_swiglu_quant(to_dev(xq), to_dev(sx), to_dev(offs), dw, dws, FP8[fmt], True, weight_format=wf)
    torch.cuda.synchronize()
    h1_ref = np.zeros((rows, 2 * inter))
    for e in range(groups):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            h1_ref[lo:hi] = moe.gmm(xq[lo:hi], sx[lo:hi], w1q[e], w1s[e], fmt)
    assert np.array_equal(h1.cpu().numpy().astype(np.float64), h1_ref)
    assert h1_ref[:, :inter].min() >= 256
    a_ref = mxfp.fp32_round(moe.swiglu(h1_ref[:, :inter], h1_ref[:, inter:]))
    assert np.array_equal(a_ref, h1_ref[:, :inter] * h1_ref[:, inter:])
    aq_o, sa_o = mxfp.quantize(a_ref, fmt)
    assert np.array_equal(sa.cpu().numpy(), sa_o)
    assert np.array_equal(aq.cpu().numpy(), aq_o)


@pytest.mark.parametrize("wf", WF, ids=["nd", "packed"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['name']}-{c.get('tokens', '')}")
def test_gmm2_combine(case, wf):
    case = dict(case)
    cfg = moe_inputs.config(case.pop("name"), **case)
    say(f"gmm2 N={cfg.tokens} H={cfg.hidden} I={cfg.inter} E={cfg.experts} K={cfg.topk} fmt={cfg.fmt}")
    ids, x, r, xq, sx = grouped_operands(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = oracle_weights(cfg)
    full = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts)
    aq_o, sa_o = full["aq"], full["sa"]
    srt = r["sorted_row_idx"]
    row_token = (srt // cfg.topk).astype(np.int32)
    row_weight = w.reshape(-1)[srt].astype(np.float32)
    y_acc = torch.zeros((cfg.tokens, cfg.hidden), dtype=torch.float32, device=DEV)
    dw, dws = device_weights(weights[2], weights[3], wf)
    o = rp.gmm2_combine(to_dev(aq_o), to_dev(sa_o), to_dev(r["offsets"].astype(np.int32)), dw, dws,
                        to_dev(row_token), to_dev(row_weight), y_acc, FP8[cfg.fmt], True, weight_format=wf)
    y = rp.combine_finalize(y_acc)
    torch.cuda.synchronize()
    o_got = o.cpu().numpy()
    err = normwise_err(o_got, full["o"])
    o_abs = np.zeros_like(full["o"])
    for e in range(cfg.experts):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        if hi > lo:
            o_abs[lo:hi] = abs_gmm(aq_o[lo:hi], sa_o[lo:hi], weights[2][e], weights[3][e], cfg.fmt)
    ex = check_gemm_elementwise(o_got, full["o"], o_abs, cfg.inter)
    say(f"  O normwise err {err:.3g}, elementwise bound use {ex:.3g}")
    assert err <= 2e-3
    mx, mean = y_errors(y.cpu().double().numpy(), full["y"])
    say(f"  Y max err {mx:.3g} mean rel {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


def packed_reference(codes, scales):
    """The packed layout of include/moe_mx.h re-stated with numpy index arithmetic."""
    g, n, k = codes.shape
    ks, kq = k // 128, (k // 128 + 3) // 4
    c = codes.reshape(g, n // 16, 16, ks, 2, 4, 16)          # (g, tile, r, s, h, lanegroup, byte)
    pc = c.transpose(0, 1, 3, 4, 5, 2, 6).reshape(-1)         # (g, tile, s, h, lanegroup, r, byte)
    sc = np.zeros((g, n // 16, kq, 4, 16, 4), np.uint8)       # (g, tile, q, lanegroup, r, j)
    sv = scales.reshape(g, n // 16, 16, ks, 4)                # (g, tile, r, s, block g)
    for s_ in range(ks):
        sc[:, :, s_ // 4, :, :, s_ % 4] = sv[:, :, :, s_, :].transpose(0, 1, 3, 2)
    return pc, sc.reshape(-1)


@pytest.mark.parametrize("shape", [(2, 32, 256), (3, 48, 640), (1, 16, 128)])
def test_pack_weights_layout(shape):
    say(f"pack_weights {shape}")
    rng = np.random.default_rng(sum(shape))
    g, n, k = shape
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    scales = rng.integers(0, 255, size=(g, n, k // 32)).astype(np.uint8)
    pc, ps = rp.pack_weights(to_dev(codes), to_dev(scales))
    torch.cuda.synchronize()
    rc, rs = packed_reference(codes, scales)
    assert np.array_equal(pc.cpu().numpy().reshape(-1), rc)
    assert np.array_equal(ps.cpu().numpy(), rs)
