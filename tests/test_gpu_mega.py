"""mega_moe on the GPU against the oracle (MegaMoE A8W8-FP stages 1-4, all experts local).

Small layers are compared whole: routing and stage-1 operands bit for bit, h1
within 2e-3 normwise, the requantized activations code by code, Y within
max|dY| <= 2e-2 max|Y| and sum|dY| <= 5e-3 sum|Y|. The full-size decode,
prefill and skewed layers run in the benchmark's configuration (weights made on
the GPU and quantized by the library) and are checked on the rows of their
special experts and on sampled tokens: the oracle requantizes the experts'
masters itself (and the library's weight bytes must equal its), then computes
those rows and tokens from its own operands."""
import os

import numpy as np
import pytest
import torch

import moe_inputs
import routing_permute_mxfp8_amd as rp
from oracle import moe, mxfp, routing
from gpu_support import (DEV, FP8, QMODE, abs_gmm, act_delta, check_gemm_elementwise, check_requant, library_weights,
                         normwise_err,
                         oracle_expert_from_gpu_masters, oracle_experts_parallel, oracle_weights, say, swiglu_delta,
                         to_dev, y_errors)

pytestmark = pytest.mark.gpu

SMALL = [
    dict(name="tiny"),
    dict(name="tiny", shared=1, seed=41),
    dict(name="tiny", tokens=333, hidden=512, inter=256, experts=16, topk=4, shared=2, seed=42),
    dict(name="skewed", tokens=500, hidden=384, inter=384, experts=20, topk=5, seed=43),
    dict(name="tiny", tokens=5, hidden=256, inter=128, experts=32, topk=8, seed=44),
    # ~256 rows per expert, inter 128 (an odd number of 128-wide K steps in GMM2): 128-row chunks
    dict(name="tiny", tokens=512, hidden=256, inter=128, experts=8, topk=4, shared=1, seed=45),
    # LDS-streaming GEMMs (more than 128 rows per expert, K steps a multiple of 4): ~350 rows per expert
    # (two chunks each), partial last channel blocks in both GEMMs (GMM1 2 of 6 gate tiles,
    # GMM2 8 of 12 output tiles), a shared expert over all tokens
    dict(name="tiny", tokens=700, hidden=512, inter=512, experts=6, topk=3, shared=1, seed=57),
    # LDS-streaming, Zipf-skewed: experts from a few rows (token tiles some waves do not
    # own) to several chunks
    dict(name="skewed", tokens=1500, hidden=1024, inter=512, experts=16, topk=2, seed=58),
]


def device_weights(arrays, wf):
    d = [to_dev(a) for a in arrays]
    if wf == rp.WEIGHTS_PACKED:
        return [*rp.pack_weights(d[0], d[1]), *rp.pack_weights(d[2], d[3])]
    return d


def assert_same_layer(y_fast, etn_fast, y_dbg, etn_dbg):
    """The call without parity outputs runs other kernel instances than the debug call
    (GMM2 stores bf16 O rows instead of the fp32 rows the debug output needs, and the
    combine reads them as bf16 instead of rounding fp32 rows as it reads them): the two
    must give the same Y bit for bit, so the instances a plain call runs are checked
    against the oracle through the debug call's comparison."""
    assert torch.equal(etn_fast, etn_dbg)
    if not torch.equal(y_fast, y_dbg):
        d = (y_fast.float() - y_dbg.float()).abs()
        raise AssertionError(f"plain and debug calls differ: {int((d > 0).sum())} elements, max {float(d.max()):.3g}")


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c['name']}-{c.get('tokens', '')}-{c.get('shared', 0)}")
@pytest.mark.parametrize("wdtype,wf", [(torch.float32, rp.WEIGHTS_ND), (torch.bfloat16, rp.WEIGHTS_PACKED),
                                       (torch.float32, rp.WEIGHTS_PACKED)], ids=["fp32-nd", "bf16-packed", "fp32-packed"])
def test_small_layers(case, wdtype, wf):
    case = dict(case)
    cfg = moe_inputs.config(case.pop("name"), **case)
    say(f"mega_moe N={cfg.tokens} H={cfg.hidden} I={cfg.inter} E={cfg.experts} K={cfg.topk} S={cfg.shared} "
        f"fmt={cfg.fmt} weights={wdtype}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    x = x_t.double().numpy()
    w = moe_inputs.gate_weights(cfg)
    w_t = torch.from_numpy(w).to(wdtype)
    w_used = w_t.double().numpy()
    weights = oracle_weights(cfg)
    shared = None
    shared_np = ()
    if cfg.shared:
        sh = oracle_weights(cfg, cfg.shared, shared=True)
        shared_np = [tuple(a[s] for a in sh) for s in range(cfg.shared)]
        shared = tuple(device_weights(sh, wf))
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), w_t.to(DEV), *device_weights(weights, wf))
    kw = dict(shared=shared, quant_out_dtype=FP8[cfg.fmt], weight_format=wf)
    y, etn, dbg = rp.mega_moe(*args, debug=True, **kw)
    y_fast, etn_fast = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    assert_same_layer(y_fast, etn_fast, y, etn)
    ref = moe.mega_moe(x, ids, w_used, weights, cfg.fmt, cfg.experts, shared=shared_np)
    assert np.array_equal(etn.cpu().numpy(), ref["expert_token_nums"])
    assert np.array_equal(dbg["sorted_row_idx"].cpu().numpy(), ref["routing"]["sorted_row_idx"])
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    assert np.array_equal(dbg["sx"].cpu().numpy(), ref["sx"])
    h1_got = dbg["h1"].cpu().numpy()
    err = normwise_err(h1_got, ref["h1"])
    assert err <= 2e-3, err
    offs = ref["routing"]["offsets"]
    h1_abs = np.zeros_like(ref["h1"])
    for e in range(cfg.experts):
        if offs[e + 1] > offs[e]:
            h1_abs[offs[e]:offs[e + 1]] = abs_gmm(ref["xq"][offs[e]:offs[e + 1]], ref["sx"][offs[e]:offs[e + 1]],
                                                  weights[0][e], weights[1][e], cfg.fmt)
    check_gemm_elementwise(h1_got, ref["h1"], h1_abs, cfg.hidden)
    delta = swiglu_delta(ref["h1"], h1_abs, cfg.hidden, cfg.inter)
    codes, scales = check_requant(dbg["aq"].cpu().numpy(), dbg["sa"].cpu().numpy(), ref["a"], delta, cfg.fmt)
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  h1 err {err:.3g} requant codes differing {codes:.3g} scales {scales:.3g} Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.parametrize("mode", [0, 1])
def test_combine_comm_modes(mode):
    """MegaMoE combineCommMode with every expert on the card: 0 rounds each expert output
    row (routed and shared) to bf16 before the fp32 weighted sum, 1 sums fp32 rows; each
    against the oracle's same mode. Y is the same bit for bit whether the fp32 o parity
    output is requested (rows rounded as the combine reads them) or not (GMM2 stores
    bf16 rows in mode 0)."""
    cfg = moe_inputs.config("tiny", tokens=333, hidden=512, inter=256, experts=16, topk=4, shared=2, seed=46)
    say(f"mega_moe combine_comm_mode {mode} N={cfg.tokens} H={cfg.hidden} E={cfg.experts} S={cfg.shared}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = oracle_weights(cfg)
    sh = oracle_weights(cfg, cfg.shared, shared=True)
    wf = rp.WEIGHTS_PACKED
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights(weights, wf))
    kw = dict(shared=tuple(device_weights(sh, wf)), quant_out_dtype=FP8[cfg.fmt], weight_format=wf,
              combine_comm_mode=mode)
    y_dbg, _, dbg = rp.mega_moe(*args, debug=True, **kw)
    y, etn = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_dbg)
    shared_np = [tuple(a[s] for a in sh) for s in range(cfg.shared)]
    ref = moe.mega_moe(x_t.double().numpy(), ids, w, weights, cfg.fmt, cfg.experts, shared=shared_np,
                       combine_comm_mode=mode)
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3
    with pytest.raises(rp.MoeError):
        rp.mega_moe(*args, **dict(kw, combine_comm_mode=2))


def test_stage1_quantize_then_gather():
    """A layer large enough (topk >= 3, tokens x hidden >= 2^22) for stage 1 to quantize
    each token once and then gather codes (routed rows and the shared expert's token-order
    rows): the gathered X^ / S_X bit for bit and Y against the oracle."""
    cfg = moe_inputs.config("tiny", tokens=1024, hidden=4096, inter=128, experts=16, topk=4, shared=1, seed=55)
    say(f"mega_moe two-pass stage 1 N={cfg.tokens} H={cfg.hidden} E={cfg.experts} K={cfg.topk}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = oracle_weights(cfg)
    sh = oracle_weights(cfg, cfg.shared, shared=True)
    wf = rp.WEIGHTS_PACKED
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights(weights, wf),
                              shared=tuple(device_weights(sh, wf)), quant_out_dtype=FP8[cfg.fmt], debug=True,
                              weight_format=wf)
    torch.cuda.synchronize()
    ref = moe.mega_moe(x_t.double().numpy(), ids, w, weights, cfg.fmt, cfg.experts,
                       shared=[tuple(a[0] for a in sh)])
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    assert np.array_equal(dbg["sx"].cpu().numpy(), ref["sx"])
    assert np.array_equal(etn.cpu().numpy(), ref["expert_token_nums"])
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


def test_empty_layer():
    """No tokens: y is empty, expert_token_nums all zero, nothing else is launched."""
    cfg = moe_inputs.config("tiny")
    say("mega_moe with no tokens")
    weights = oracle_weights(cfg)
    sh = oracle_weights(cfg, 1, shared=True)
    wf = rp.WEIGHTS_PACKED
    x = torch.zeros((0, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((0, cfg.topk), dtype=torch.int32, device=DEV)
    w = torch.zeros((0, cfg.topk), dtype=torch.float32, device=DEV)
    y, etn = rp.mega_moe(x, ids, w, *device_weights(weights, wf), shared=tuple(device_weights(sh, wf)),
                         quant_out_dtype=FP8[cfg.fmt], weight_format=wf)
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.hidden)
    assert np.array_equal(etn.cpu().numpy(), np.zeros(cfg.experts, np.int32))


@pytest.mark.parametrize("experts,topk,shared", [(8, 1, 1), (1, 1, 0), (1, 1, 2)])
def test_topk_one_and_single_expert(experts, topk, shared):
    """topK = 1 (each token's row is its expert's output, weighted) and a single routed
    expert, with and without shared experts, against the oracle."""
    cfg = moe_inputs.config("tiny", tokens=77, experts=experts, topk=topk, shared=shared, seed=56)
    say(f"mega_moe E={experts} K={topk} S={shared}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = oracle_weights(cfg)
    wf = rp.WEIGHTS_PACKED
    shared_np, shared_dev = (), None
    if shared:
        sh = oracle_weights(cfg, shared, shared=True)
        shared_np = [tuple(a[s] for a in sh) for s in range(shared)]
        shared_dev = tuple(device_weights(sh, wf))
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights(weights, wf),
                              shared=shared_dev, quant_out_dtype=FP8[cfg.fmt], debug=True, weight_format=wf)
    torch.cuda.synchronize()
    ref = moe.mega_moe(x_t.double().numpy(), ids, w, weights, cfg.fmt, cfg.experts, shared=shared_np)
    assert np.array_equal(etn.cpu().numpy(), ref["expert_token_nums"])
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    assert normwise_err(dbg["h1"].cpu().numpy(), ref["h1"]) <= 2e-3
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


ACTS = [("swiglu", (0.8,)), ("swiglustep", (0.6,)), ("swiglustep", ()), ("swigluoai", ()),
        ("swigluoai", (0.9, 1.2, 0.5)), ("situglu", (2.0,)), ("situglu", (1.5, 0.7)), ("situglu", ()),
        ("gelu", ()), ("gelu", (float(np.finfo(np.float32).max),))]
ACT_KIND = {"swiglu": rp.ACT_SWIGLU, "swiglustep": rp.ACT_SWIGLUSTEP, "swigluoai": rp.ACT_SWIGLUOAI,
            "situglu": rp.ACT_SITUGLU, "gelu": rp.ACT_GELU}


@pytest.mark.parametrize("kind,params", ACTS, ids=lambda v: str(v))
@pytest.mark.parametrize("tt", ["small", "wide", "long"])
def test_activations(kind, params, tt):
    """MegaMoE "Activation function formulas": every activation and parameter list, routed
    and shared experts, in 1-tile (small), 16-tile (wide) and 18-tile (long) chunks;
    clamps that bite."""
    if tt == "small":
        cfg = moe_inputs.config("tiny", tokens=96, hidden=256, inter=256, experts=8, topk=2, shared=1, seed=47)
    elif tt == "wide":
        cfg = moe_inputs.config("tiny", tokens=600, hidden=256, inter=128, experts=4, topk=2, shared=1, seed=48)
    else:
        cfg = moe_inputs.config("tiny", tokens=520, hidden=256, inter=256, experts=4, topk=2, shared=1, seed=49)
    say(f"mega_moe activation {kind} {params} N={cfg.tokens} I={cfg.inter} E={cfg.experts}")
    gelu = kind == "gelu"
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    x = x_t.double().numpy()
    w = moe_inputs.gate_weights(cfg)
    weights = oracle_weights(cfg, gelu=gelu)
    sh = oracle_weights(cfg, cfg.shared, shared=True, gelu=gelu)
    wf = rp.WEIGHTS_PACKED
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights(weights, wf))
    kw = dict(shared=tuple(device_weights(sh, wf)), quant_out_dtype=FP8[cfg.fmt], weight_format=wf,
              activation=ACT_KIND[kind], activation_params=params)
    y, etn, dbg = rp.mega_moe(*args, debug=True, **kw)
    y_fast, etn_fast = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    assert_same_layer(y_fast, etn_fast, y, etn)
    act = (kind, params)
    ref = moe.mega_moe(x, ids, w, weights, cfg.fmt, cfg.experts, shared=[tuple(a[0] for a in sh)], act=act)
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    h1_got = dbg["h1"].cpu().numpy()
    err = normwise_err(h1_got, ref["h1"])
    assert err <= 2e-3, err
    offs = ref["routing"]["offsets"]
    h1_abs = np.zeros_like(ref["h1"])
    for e in range(cfg.experts):
        if offs[e + 1] > offs[e]:
            h1_abs[offs[e]:offs[e + 1]] = abs_gmm(ref["xq"][offs[e]:offs[e + 1]], ref["sx"][offs[e]:offs[e + 1]],
                                                  weights[0][e], weights[1][e], cfg.fmt)
    delta = act_delta(ref["h1"], h1_abs, cfg.hidden, kind, params)
    aq, sa = dbg["aq"].cpu().numpy(), dbg["sa"].cpu().numpy()
    assert aq.shape[1] == (2 * cfg.inter if gelu else cfg.inter)
    codes, scales = check_requant(aq, sa, ref["a"], delta, cfg.fmt)
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  h1 err {err:.3g} requant codes differing {codes:.3g} scales {scales:.3g} Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


def fp4_weights(cfg, n_experts=None, shared=False):
    """MXFP4 (E2M1) weights quantized by the oracle from the bf16 masters, codes two a byte."""
    n_experts = cfg.experts if n_experts is None else n_experts
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    out = [[], [], [], []]
    for e in range(n_experts):
        q1, s1 = mxfp.quantize(moe_inputs.weight_master(cfg, t1, e).double().numpy(), "e2m1")
        q2, s2 = mxfp.quantize(moe_inputs.weight_master(cfg, t2, e).double().numpy(), "e2m1")
        for lst, v in zip(out, (mxfp.pack_fp4(q1), s1, mxfp.pack_fp4(q2), s2)):
            lst.append(v)
    return tuple(np.stack(v) for v in out)


def device_weights_fp4(arrays, wf):
    d = [to_dev(a) for a in arrays]
    if wf == rp.WEIGHTS_PACKED:
        return [*rp.pack_weights(d[0], d[1], fp4=True), *rp.pack_weights(d[2], d[3], fp4=True)]
    return d


@pytest.mark.parametrize("wf", [rp.WEIGHTS_ND, rp.WEIGHTS_PACKED], ids=["nd", "packed"])
@pytest.mark.parametrize("case", [dict(tokens=96, inter=256, experts=8, topk=2, seed=51, shared="fp8"),
                                  dict(tokens=600, inter=128, experts=4, topk=2, seed=52, shared="fp4"),
                                  dict(tokens=333, inter=256, experts=16, topk=4, seed=53, shared=None),
                                  dict(tokens=512, inter=256, experts=4, topk=2, seed=54, shared="fp4")],
                         ids=["2tile-shared8", "16tile-shared4", "4tile", "18tile-shared4"])
def test_a8w4(case, wf):
    """A8W4-FP: E4M3 activations, MXFP4 routed weights (and MXFP4 or FP8 shared weights),
    A requantized to E4M3; h1 and O from FP8 x FP4 products on the matrix cores."""
    case = dict(case)
    sh_kind = case.pop("shared")
    cfg = moe_inputs.config("tiny", hidden=256, shared=0 if sh_kind is None else 1, **case)
    say(f"mega_moe A8W4 N={cfg.tokens} I={cfg.inter} E={cfg.experts} K={cfg.topk} shared={sh_kind} wf={wf}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    x = x_t.double().numpy()
    w = moe_inputs.gate_weights(cfg)
    weights = fp4_weights(cfg)
    shared_dev, shared_np, swd = None, (), 0
    if sh_kind == "fp4":
        sh = fp4_weights(cfg, 1, shared=True)
        shared_dev, swd = tuple(device_weights_fp4(sh, wf)), rp.FP4_E2M1
    elif sh_kind == "fp8":
        sh = oracle_weights(cfg, 1, shared=True)
        shared_dev, swd = tuple(device_weights(sh, wf)), rp.FP8_E4M3
    if sh_kind:
        shared_np = [tuple(a[0] for a in sh)]
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights_fp4(weights, wf))
    kw = dict(shared=shared_dev, quant_out_dtype=rp.FP8_E4M3, weight_format=wf, weight_dtype=rp.FP4_E2M1,
              shared_weight_dtype=swd)
    y, etn, dbg = rp.mega_moe(*args, debug=True, **kw)
    y_fast, etn_fast = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    assert_same_layer(y_fast, etn_fast, y, etn)
    ref = moe.mega_moe(x, ids, w, weights, "e4m3", cfg.experts, shared=shared_np, wfmt="e2m1",
                       shared_wfmt="e4m3" if sh_kind == "fp8" else "e2m1")
    assert np.array_equal(dbg["xq"].cpu().numpy(), ref["xq"])
    h1_got = dbg["h1"].cpu().numpy()
    err = normwise_err(h1_got, ref["h1"])
    assert err <= 2e-3, err
    offs = ref["routing"]["offsets"]
    h1_abs = np.zeros_like(ref["h1"])
    for e in range(cfg.experts):
        if offs[e + 1] > offs[e]:
            h1_abs[offs[e]:offs[e + 1]] = np.abs(mxfp.dequantize(ref["xq"][offs[e]:offs[e + 1]],
                                                                 ref["sx"][offs[e]:offs[e + 1]], "e4m3")) @ \
                np.abs(mxfp.dequantize(mxfp.unpack_fp4(weights[0][e]), weights[1][e], "e2m1")).T
    check_gemm_elementwise(h1_got, ref["h1"], h1_abs, cfg.hidden)
    delta = swiglu_delta(ref["h1"], h1_abs, cfg.hidden, cfg.inter)
    codes, scales = check_requant(dbg["aq"].cpu().numpy(), dbg["sa"].cpu().numpy(), ref["a"], delta, "e4m3")
    mx, mean = y_errors(y.cpu().double().numpy(), ref["y"])
    say(f"  h1 err {err:.3g} requant codes differing {codes:.3g} scales {scales:.3g} Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_prequantized_passthrough(fmt):
    """MegaMoE dispatchQuantMode 0: x already MX-quantized (codes + E8M0 scales) skips the
    stage-1 quantization. Given the library's own quantization of x the layer must be the
    same bit for bit as with bf16 x quantized inside (routed and shared experts)."""
    cfg = moe_inputs.config("tiny", tokens=200, hidden=512, inter=256, experts=16, topk=4, shared=1, seed=61,
                            fmt=fmt)
    say(f"mega_moe pre-quantized x fmt={fmt}")
    ids = to_dev(moe_inputs.expert_ids(cfg).astype(np.int32))
    x = moe_inputs.activations(cfg).to(DEV)
    w = to_dev(moe_inputs.gate_weights(cfg))
    wts = device_weights(oracle_weights(cfg), rp.WEIGHTS_PACKED)
    sh = tuple(device_weights(oracle_weights(cfg, 1, shared=True), rp.WEIGHTS_PACKED))
    q = FP8[cfg.fmt]
    y0, e0, d0 = rp.mega_moe(x, ids, w, *wts, shared=sh, quant_out_dtype=q, debug=True,
                             weight_format=rp.WEIGHTS_PACKED)
    codes, scales = rp.mx_quantize(x, QMODE[cfg.fmt])
    y1, e1, d1 = rp.mega_moe(codes, ids, w, *wts, shared=sh, quant_out_dtype=q, debug=True,
                             weight_format=rp.WEIGHTS_PACKED, x_scales=scales)
    torch.cuda.synchronize()
    assert torch.equal(d0["xq"], d1["xq"]) and torch.equal(d0["sx"], d1["sx"])
    assert torch.equal(y0, y1) and torch.equal(e0, e1)
    ref = moe.mega_moe(x.cpu().double().numpy(), moe_inputs.expert_ids(cfg), moe_inputs.gate_weights(cfg),
                       oracle_weights(cfg), cfg.fmt, cfg.experts,
                       shared=[tuple(a[0] for a in oracle_weights(cfg, 1, shared=True))])
    assert np.array_equal(d1["xq"].cpu().numpy(), ref["xq"])
    mx, mean = y_errors(y1.cpu().double().numpy(), ref["y"])
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.parametrize("tokens,hidden,inter", [(64, 256, 128), (200, 512, 256), (40, 7168, 2048)])
def test_shared_expert_alone(tokens, hidden, inter):
    """All gate weights 0: Y is the shared expert's dense FFN over every token."""
    cfg = moe_inputs.config("tiny", tokens=tokens, hidden=hidden, inter=inter, shared=1, seed=46)
    say(f"mega_moe shared expert alone N={tokens} H={hidden} I={inter}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = np.zeros((cfg.tokens, cfg.topk), np.float32)
    weights = oracle_weights(cfg, 1)
    weights = tuple(np.repeat(a, cfg.experts, axis=0) for a in weights)
    sh = oracle_weights(cfg, 1, shared=True)
    y, _ = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *[to_dev(a) for a in weights],
                       shared=tuple(to_dev(a) for a in sh), quant_out_dtype=FP8[cfg.fmt])
    torch.cuda.synchronize()
    x = x_t.double().numpy()
    xq, sx = mxfp.quantize(x, cfg.fmt)
    ref = mxfp.bf16_round(moe.expert_ffn(xq, sx, *[a[0] for a in sh], cfg.fmt)["o"])
    mx, mean = y_errors(y.cpu().double().numpy(), ref)
    say(f"  Y max {mx:.3g} mean {mean:.3g}")
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.parametrize("name", ["tiny", "wide"])
def test_repeated_calls_reuse_workspace(name):
    """Two calls on one preallocated workspace (the second finds the first's leftovers in
    it) give the same Y bit for bit: the layer has no atomics and a fixed summation order."""
    if name == "tiny":
        cfg = moe_inputs.config("tiny", seed=45)
    else:   # 18-tile chunks and a shared expert
        cfg = moe_inputs.config("tiny", tokens=512, hidden=256, inter=128, experts=8, topk=4, shared=1, seed=45)
    say(f"mega_moe repeated calls on one workspace ({name})")
    ids = to_dev(moe_inputs.expert_ids(cfg).astype(np.int32))
    x = moe_inputs.activations(cfg).to(DEV)
    w = to_dev(moe_inputs.gate_weights(cfg))
    weights = device_weights(oracle_weights(cfg), rp.WEIGHTS_PACKED)
    shared = tuple(device_weights(oracle_weights(cfg, cfg.shared, shared=True), rp.WEIGHTS_PACKED)) \
        if cfg.shared else None
    kw = dict(shared=shared, weight_format=rp.WEIGHTS_PACKED)
    ws = torch.empty(rp.mega_moe_workspace_bytes(x, ids, w, *weights, **kw), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)
    y1, e1 = rp.mega_moe(x, ids, w, *weights, workspace=ws, **kw)
    y1 = y1.clone()
    y2, e2 = rp.mega_moe(x, ids, w, *weights, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(e1, e2)
    assert torch.equal(y1, y2)


ORACLE_THREADS = min(16, os.cpu_count() or 1)


def sample_tokens(ids, counts, n_random, special, seed):
    """n_random tokens at random plus, for each special expert, the first token routed to it
    that is not chosen yet (so every special expert's rows reach the sampled Y)."""
    rng = np.random.default_rng(seed)
    chosen = [int(t) for t in rng.choice(ids.shape[0], size=n_random, replace=False)]
    for e in special:
        for t in np.nonzero((ids == e).any(axis=1))[0]:
            if int(t) not in chosen:
                chosen.append(int(t))
                break
    return np.array(sorted(chosen))


def check_expert_rows(cfg, e, lo, hi, q, x, r, dbg):
    """Every row of expert e: X^ / S_X bit for bit, h1 within 2e-3 normwise and the
    elementwise bound, the requantized A^ a valid MX quantization of the oracle's A.
    Returns the oracle's A^ / S_A and O of the rows (oracle operands only)."""
    xq_rows = dbg["xq"][lo:hi].cpu().numpy()
    sx_rows = dbg["sx"][lo:hi].cpu().numpy()
    src = r["sorted_row_idx"][lo:hi] // cfg.topk
    xq_o, sx_o = mxfp.quantize(x[src], cfg.fmt)
    assert np.array_equal(xq_rows, xq_o) and np.array_equal(sx_rows, sx_o)
    ffn = moe.expert_ffn(xq_o, sx_o, *q, cfg.fmt)
    h1_abs = abs_gmm(xq_o, sx_o, q[0], q[1], cfg.fmt)
    h1_got = dbg["h1"][lo:hi].cpu().numpy()
    err_e = normwise_err(h1_got, ffn["h1"])
    check_gemm_elementwise(h1_got, ffn["h1"], h1_abs, cfg.hidden)
    delta = swiglu_delta(ffn["h1"], h1_abs, cfg.hidden, cfg.inter)
    codes, scales = check_requant(dbg["aq"][lo:hi].cpu().numpy(), dbg["sa"][lo:hi].cpu().numpy(), ffn["a"], delta,
                                  cfg.fmt)
    say(f"  expert {e} ({hi - lo} rows): h1 err {err_e:.3g}, requant codes differing {codes:.3g} "
        f"scales {scales:.3g}")
    assert err_e <= 2e-3
    return ffn


def check_gmm2_rows(cfg, experts, ffns, cache, wf):
    """GMM2 on the oracle's own A^ of every row of `experts` (stage entry point, the same
    kernels as the layer): O row by row within 2e-3 normwise and the elementwise bound,
    every output channel included (the partial last channel block of hidden 7168)."""
    aq = np.concatenate([ffns[e]["aq"] for e in experts])
    sa = np.concatenate([ffns[e]["sa"][:, :cfg.inter // 32] for e in experts])
    o_ref = np.concatenate([ffns[e]["o"] for e in experts])
    offs = np.zeros(len(experts) + 1, np.int32)
    offs[1:] = np.cumsum([ffns[e]["aq"].shape[0] for e in experts])
    w2q = to_dev(np.stack([cache[e][2] for e in experts]))
    w2s = to_dev(np.stack([cache[e][3] for e in experts]))
    if wf == rp.WEIGHTS_PACKED:
        w2q, w2s = rp.pack_weights(w2q, w2s)
    rows = aq.shape[0]
    y_acc = torch.zeros((rows, cfg.hidden), dtype=torch.float32, device=DEV)
    o = rp.gmm2_combine(to_dev(aq), to_dev(sa), to_dev(offs), w2q, w2s, to_dev(np.arange(rows, dtype=np.int32)),
                        to_dev(np.ones(rows, np.float32)), y_acc, FP8[cfg.fmt], True, weight_format=wf)
    torch.cuda.synchronize()
    o_got = o.cpu().numpy()
    o_abs = np.concatenate([abs_gmm(ffns[e]["aq"], ffns[e]["sa"], cache[e][2], cache[e][3], cfg.fmt)
                            for e in experts])
    err = normwise_err(o_got, o_ref)
    worst = max(normwise_err(o_got[offs[j]:offs[j + 1]], o_ref[offs[j]:offs[j + 1]]) for j in range(len(experts)))
    ex = check_gemm_elementwise(o_got, o_ref, o_abs, cfg.inter)
    say(f"  GMM2 on the oracle's A^ of experts {list(experts)} ({rows} rows): O err {err:.3g} "
        f"(worst expert {worst:.3g}), elementwise bound use {ex:.3g}")
    assert err <= 2e-3 and worst <= 2e-3


def full_size_check(name, n_random, wf=rp.WEIGHTS_ND, seed=7, plain_packed=False):
    """The layer at full size in the benchmark's configuration (weights made on the GPU
    and quantized by the library):
    * the plain call (the kernel instances the benchmark times) equals the debug call
      bit for bit; with plain_packed, so does a plain call on the packed copy of ND
      weights (the packed layout's kernels, one instance per chunk-size class, against
      the ND debug call's);
    * routing, counts and the sampled rows' X^ / S_X exact;
    * the special experts (the busiest one, every expert whose rows take more than one
      GEMM chunk, the least busy one): all their rows through GMM1 (h1, A^) and GMM2 (O
      from the oracle's A^);
    * Y of the sampled tokens (random ones plus one routed to each special expert) from
      the oracle's layer on those tokens."""
    cfg = moe_inputs.config(name)
    say(f"mega_moe full size {name}: N={cfg.tokens} H={cfg.hidden} I={cfg.inter} E={cfg.experts} K={cfg.topk} "
        f"S={cfg.shared} fmt={cfg.fmt}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = library_weights(cfg)
    shared = library_weights(cfg, cfg.shared, shared=True) if cfg.shared else None
    say("  weights ready")
    dev_w = list(weights)
    dev_sh = shared
    if wf == rp.WEIGHTS_PACKED:
        dev_w = [*rp.pack_weights(weights[0], weights[1]), *rp.pack_weights(weights[2], weights[3])]
        if shared is not None:
            dev_sh = (*rp.pack_weights(shared[0], shared[1]), *rp.pack_weights(shared[2], shared[3]))
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *dev_w)
    kw = dict(shared=dev_sh, quant_out_dtype=FP8[cfg.fmt], weight_format=wf)
    y, etn, dbg = rp.mega_moe(*args, debug=True, **kw)
    y_fast, etn_fast = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    say("  layer done (plain and debug calls)")
    assert_same_layer(y_fast, etn_fast, y, etn)
    del y_fast
    if plain_packed:
        assert wf == rp.WEIGHTS_ND and shared is None
        packed = [*rp.pack_weights(weights[0], weights[1]), *rp.pack_weights(weights[2], weights[3])]
        y_p, etn_p = rp.mega_moe(*args[:3], *packed, quant_out_dtype=FP8[cfg.fmt], weight_format=rp.WEIGHTS_PACKED)
        torch.cuda.synchronize()
        say("  plain call on packed weights done")
        assert_same_layer(y_p, etn_p, y, etn)
        del y_p, packed
    r = routing.init_routing(ids, cfg.experts)
    counts = r["counts"]
    assert np.array_equal(etn.cpu().numpy(), counts.astype(np.int32))
    assert np.array_equal(dbg["sorted_row_idx"].cpu().numpy(), r["sorted_row_idx"])
    busiest = int(np.argmax(counts))
    nonempty = np.nonzero(counts)[0]
    least = int(nonempty[np.argmin(counts[nonempty])])
    multi = [int(e) for e in np.argsort(-counts, kind="stable")[:8] if counts[e] > 256]
    special = sorted(set([busiest, least] + multi))
    tokens = sample_tokens(ids, counts, n_random, special, seed)
    needed = sorted(set(int(e) for e in ids[tokens].reshape(-1)) | set(special))
    cache = oracle_experts_parallel(cfg, needed, workers=ORACLE_THREADS)
    for e in needed:   # the library's weight bytes equal the oracle's quantization of the same masters
        for j in range(4):
            assert np.array_equal(weights[j][e].cpu().numpy(), cache[e][j]), (e, j)
    shared_np = [oracle_expert_from_gpu_masters(cfg, s, shared=True) for s in range(cfg.shared)]
    say(f"  oracle weights ready ({len(needed)} experts); special experts {special} "
        f"with {[int(counts[e]) for e in special]} rows")
    x = x_t.double().numpy()
    ffns = {}
    for e in special:
        lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
        ffns[e] = check_expert_rows(cfg, e, lo, hi, cache[e], x, r, dbg)
    check_gmm2_rows(cfg, special, ffns, cache, wf)
    # Y of the sampled tokens: the oracle's layer on those tokens alone (each token's Y
    # depends only on its own row and experts)
    ref = moe.mega_moe(x[tokens], ids[tokens], w[tokens], lambda e: cache[e], cfg.fmt, cfg.experts,
                       shared=shared_np, workers=ORACLE_THREADS)
    y_got = y[torch.from_numpy(tokens).to(DEV)].cpu().double().numpy()
    mx, mean = y_errors(y_got, ref["y"])
    # h1 / X^ rows of the sampled tokens: position in the full layer vs in the sub-layer
    inv = routing.inverse(r["sorted_row_idx"])
    inv_sub = routing.inverse(ref["routing"]["sorted_row_idx"])
    flat_full = (tokens[:, None] * cfg.topk + np.arange(cfg.topk)[None, :]).reshape(-1)
    pos = inv[flat_full]
    pos_sub = inv_sub[np.arange(len(tokens) * cfg.topk)]
    idx = torch.from_numpy(pos).to(DEV)
    assert np.array_equal(dbg["xq"][idx].cpu().numpy(), ref["xq"][pos_sub])
    assert np.array_equal(dbg["sx"][idx].cpu().numpy(), ref["sx"][pos_sub])
    err = normwise_err(dbg["h1"][idx].cpu().numpy(), ref["h1"][pos_sub])
    say(f"  {len(tokens)} sampled tokens: Y max {mx:.3g} mean {mean:.3g}, h1 err {err:.3g}")
    assert err <= 2e-3
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.timeout(900)
def test_full_size_decode_a8w4():
    """The decode-shaped layer with MXFP4 weights (A8W4-FP) in the benchmark's configuration
    (library-quantized, packed): routing exact, the library's MXFP4 weight bytes equal the
    oracle's, sampled tokens' Y and h1 within the layer tolerances."""
    cfg = moe_inputs.config("decode")
    say(f"mega_moe full size decode A8W4: N={cfg.tokens} H={cfg.hidden} I={cfg.inter} E={cfg.experts}")
    ids = moe_inputs.expert_ids(cfg)
    x_t = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    weights = library_weights(cfg, fp4=True)
    dev_w = [*rp.pack_weights(weights[0], weights[1], fp4=True), *rp.pack_weights(weights[2], weights[3], fp4=True)]
    say("  weights ready")
    args = (x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *dev_w)
    kw = dict(quant_out_dtype=rp.FP8_E4M3, weight_format=rp.WEIGHTS_PACKED, weight_dtype=rp.FP4_E2M1)
    y, etn, dbg = rp.mega_moe(*args, debug=True, **kw)
    y_fast, etn_fast = rp.mega_moe(*args, **kw)
    torch.cuda.synchronize()
    assert_same_layer(y_fast, etn_fast, y, etn)
    r = routing.init_routing(ids, cfg.experts)
    assert np.array_equal(dbg["sorted_row_idx"].cpu().numpy(), r["sorted_row_idx"])
    rng = np.random.default_rng(8)
    tokens = rng.choice(cfg.tokens, size=4, replace=False)
    needed = sorted(set(int(e) for e in ids[tokens].reshape(-1)))
    cache = oracle_experts_parallel(cfg, needed, fp4=True, workers=ORACLE_THREADS)
    for e in needed:
        for j in range(4):
            assert np.array_equal(weights[j][e].cpu().numpy(), cache[e][j]), (e, j)
    x = x_t.double().numpy()
    ref = moe.per_token(x, ids, w, lambda e: cache[e], "e4m3", tokens, wfmt="e2m1")
    y_got = y[torch.from_numpy(tokens).to(DEV)].cpu().double().numpy()
    mx, mean = y_errors(y_got, ref["y"])
    inv = routing.inverse(r["sorted_row_idx"]).reshape(cfg.tokens, cfg.topk)
    pos = inv[tokens].reshape(-1)
    h1_got = dbg["h1"][torch.from_numpy(pos).to(DEV)].cpu().numpy()
    err = normwise_err(h1_got, ref["h1"].reshape(len(pos), -1))
    say(f"  sampled tokens {tokens.tolist()}: Y max {mx:.3g} mean {mean:.3g}, h1 err {err:.3g}")
    assert err <= 2e-3
    assert mx <= 2e-2 and mean <= 5e-3


@pytest.mark.timeout(900)
def test_full_size_decode():
    full_size_check("decode", n_random=128, wf=rp.WEIGHTS_PACKED)   # every token


@pytest.mark.timeout(900)
def test_full_size_skewed():
    full_size_check("skewed", n_random=64, plain_packed=True)


@pytest.mark.timeout(900)
def test_full_size_prefill():
    full_size_check("prefill", n_random=64, wf=rp.WEIGHTS_PACKED)
