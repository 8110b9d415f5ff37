"""mega_moe on the GPU against the oracle (MegaMoE A8W8-FP stages 1-4, all experts local).

Small layers are compared whole: routing and stage-1 operands bit for bit, h1
within 2e-3 normwise, the requantized activations code by code, Y within
max|dY| <= 2e-2 max|Y| and sum|dY| <= 5e-3 sum|Y|. The full-size decode,
prefill and skewed layers run in the benchmark's configuration (weights made on
the GPU and quantized by the library) and are checked on sampled tokens: the
oracle requantizes the sampled experts' masters itself (and the library's weight
bytes must equal its), then computes those tokens one (token, k) at a time."""
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
    # ~256 rows per expert: both GEMMs in 288-row chunks (GMM2 with 48 channels a wave, a partial last block)
    dict(name="tiny", tokens=512, hidden=256, inter=128, experts=8, topk=4, shared=1, seed=45),
]


def device_weights(arrays, wf):
    d = [to_dev(a) for a in arrays]
    if wf == rp.WEIGHTS_PACKED:
        return [*rp.pack_weights(d[0], d[1]), *rp.pack_weights(d[2], d[3])]
    return d


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
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), w_t.to(DEV),
                              *device_weights(weights, wf), shared=shared, quant_out_dtype=FP8[cfg.fmt], debug=True,
                              weight_format=wf)
    torch.cuda.synchronize()
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
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights(weights, wf),
                              shared=tuple(device_weights(sh, wf)), quant_out_dtype=FP8[cfg.fmt], debug=True,
                              weight_format=wf, activation=ACT_KIND[kind], activation_params=params)
    torch.cuda.synchronize()
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
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *device_weights_fp4(weights, wf),
                              shared=shared_dev, quant_out_dtype=rp.FP8_E4M3, debug=True, weight_format=wf,
                              weight_dtype=rp.FP4_E2M1, shared_weight_dtype=swd)
    torch.cuda.synchronize()
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


def test_repeated_calls_reuse_workspace():
    cfg = moe_inputs.config("tiny", seed=45)
    say("mega_moe repeated calls")
    ids = to_dev(moe_inputs.expert_ids(cfg).astype(np.int32))
    x = moe_inputs.activations(cfg).to(DEV)
    w = to_dev(moe_inputs.gate_weights(cfg))
    weights = [to_dev(a) for a in oracle_weights(cfg)]
    y1, e1 = rp.mega_moe(x, ids, w, *weights)
    y2, e2 = rp.mega_moe(x, ids, w, *weights)
    torch.cuda.synchronize()
    assert torch.equal(e1, e2)
    d = (y1.float() - y2.float()).abs().max().item()
    assert d <= 2e-2 * y1.float().abs().max().item()


def full_size_check(name, n_tokens_sampled=1, check_expert_rows=True, wf=rp.WEIGHTS_ND):
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
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *dev_w, shared=dev_sh,
                              quant_out_dtype=FP8[cfg.fmt], debug=True, weight_format=wf)
    torch.cuda.synchronize()
    say("  layer done")
    r = routing.init_routing(ids, cfg.experts)
    assert np.array_equal(etn.cpu().numpy(), r["counts"].astype(np.int32))
    assert np.array_equal(dbg["sorted_row_idx"].cpu().numpy(), r["sorted_row_idx"])
    rng = np.random.default_rng(7)
    tokens = rng.choice(cfg.tokens, size=n_tokens_sampled, replace=False)
    busiest = int(np.argmax(r["counts"]))
    needed = sorted(set(int(e) for e in ids[tokens].reshape(-1)) | {busiest})
    cache = oracle_experts_parallel(cfg, needed)
    for e in needed:   # the library's weight bytes equal the oracle's quantization of the same masters
        for j in range(4):
            assert np.array_equal(weights[j][e].cpu().numpy(), cache[e][j]), (e, j)

    def expert(e):
        return cache[e]

    shared_np = [oracle_expert_from_gpu_masters(cfg, s, shared=True) for s in range(cfg.shared)]
    say(f"  oracle weights ready ({len(needed)} experts)")
    x = x_t.double().numpy()
    ref = moe.per_token(x, ids, w, expert, cfg.fmt, tokens, shared=shared_np)
    y_got = y[torch.from_numpy(tokens).to(DEV)].cpu().double().numpy()
    mx, mean = y_errors(y_got, ref["y"])
    inv = routing.inverse(r["sorted_row_idx"]).reshape(cfg.tokens, cfg.topk)
    pos = inv[tokens].reshape(-1)
    h1_got = dbg["h1"][torch.from_numpy(pos).to(DEV)].cpu().numpy()
    err = normwise_err(h1_got, ref["h1"].reshape(len(pos), -1))
    xq_ref, sx_ref = mxfp.quantize(x[tokens], cfg.fmt)
    assert np.array_equal(dbg["xq"][torch.from_numpy(pos).to(DEV)].cpu().numpy(), np.repeat(xq_ref, cfg.topk, axis=0))
    assert np.array_equal(dbg["sx"][torch.from_numpy(pos).to(DEV)].cpu().numpy(), np.repeat(sx_ref, cfg.topk, axis=0))
    say(f"  sampled tokens {tokens.tolist()}: Y max {mx:.3g} mean {mean:.3g}, h1 err {err:.3g}")
    assert err <= 2e-3
    assert mx <= 2e-2 and mean <= 5e-3
    if check_expert_rows:
        # every row of the busiest expert: h1 of the whole group (largest tile count)
        e = busiest
        lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
        q = expert(e)
        xq_rows = dbg["xq"][lo:hi].cpu().numpy()
        sx_rows = dbg["sx"][lo:hi].cpu().numpy()
        src = r["sorted_row_idx"][lo:hi] // cfg.topk
        xq_o, sx_o = mxfp.quantize(x[src], cfg.fmt)
        assert np.array_equal(xq_rows, xq_o) and np.array_equal(sx_rows, sx_o)
        h1_ref = moe.gmm(xq_o, sx_o, q[0], q[1], cfg.fmt)
        h1_abs = abs_gmm(xq_o, sx_o, q[0], q[1], cfg.fmt)
        h1_got = dbg["h1"][lo:hi].cpu().numpy()
        err_e = normwise_err(h1_got, h1_ref)
        check_gemm_elementwise(h1_got, h1_ref, h1_abs, cfg.hidden)
        a_ref = mxfp.fp32_round(moe.swiglu(h1_ref[:, :cfg.inter], h1_ref[:, cfg.inter:]))
        delta = swiglu_delta(h1_ref, h1_abs, cfg.hidden, cfg.inter)
        codes, scales = check_requant(dbg["aq"][lo:hi].cpu().numpy(), dbg["sa"][lo:hi].cpu().numpy(), a_ref, delta,
                                      cfg.fmt)
        say(f"  expert {e} ({hi - lo} rows): h1 err {err_e:.3g}, requant codes differing {codes:.3g} "
            f"scales {scales:.3g}")
        assert err_e <= 2e-3


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
    y, etn, dbg = rp.mega_moe(x_t.to(DEV), to_dev(ids.astype(np.int32)), to_dev(w), *dev_w,
                              quant_out_dtype=rp.FP8_E4M3, debug=True, weight_format=rp.WEIGHTS_PACKED,
                              weight_dtype=rp.FP4_E2M1)
    torch.cuda.synchronize()
    r = routing.init_routing(ids, cfg.experts)
    assert np.array_equal(dbg["sorted_row_idx"].cpu().numpy(), r["sorted_row_idx"])
    rng = np.random.default_rng(8)
    tokens = rng.choice(cfg.tokens, size=4, replace=False)
    needed = sorted(set(int(e) for e in ids[tokens].reshape(-1)))
    cache = oracle_experts_parallel(cfg, needed, fp4=True)
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
    full_size_check("decode", n_tokens_sampled=4, wf=rp.WEIGHTS_PACKED)


@pytest.mark.timeout(900)
def test_full_size_skewed():
    full_size_check("skewed", n_tokens_sampled=6)


@pytest.mark.timeout(900)
def test_full_size_prefill():
    full_size_check("prefill", n_tokens_sampled=3, wf=rp.WEIGHTS_PACKED)
