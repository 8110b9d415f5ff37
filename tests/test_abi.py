"""The C-ABI library: it loads, exports every function include/moe_mx.h declares, and
its host-side validation rejects bad arguments before any launch (MegaMoE README,
Constraints: errors raised up front with the required bytes, no silent fallback).
No call here reaches a kernel, so these run without a GPU."""
import ctypes

import numpy as np
import os
import re

import pytest

import routing_permute_mxfp8_amd as rp
from routing_permute_mxfp8_amd import MegaArgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mx.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rp.lib_path()):
        from routing_permute_mxfp8_amd import build
        build.build()
    return rp.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*((?:moe|mega)_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in rp._SIGS, f"binding does not declare {n}"


def test_helpers(lib):
    assert lib.moe_version() >= 100
    assert rp.mx_scale_cols(128) == 4 and rp.mx_scale_cols(7168) == 224 and rp.mx_scale_cols(96) == 4
    for n_out, m in [(None, 8), (0, 8), (6, 6), (100, 8), (-2, 6), (-100, 0)]:
        assert rp.token_permute_out_rows(8, n_out) == m


def ws_size(fn, *args):
    b = ctypes.c_size_t()
    st = fn(*args, ctypes.byref(b))
    return st, b.value


def test_workspace_queries(lib):
    st, a = ws_size(lib.moe_init_routing_workspace_size, 32768, 8, 256)
    assert st == 0 and a > 32768 * 8 * 4
    st, b = ws_size(lib.moe_token_permute_workspace_size, 1024, 256)
    assert st == 0 and b > 0
    st, _ = ws_size(lib.moe_init_routing_workspace_size, 10, 2, 0)
    assert st == 2
    # rows restaged in the tiled layout, each of the 4 groups padded to 16 rows
    st, c = ws_size(lib.moe_gmm_workspace_size, 100, 4, 256, 128)
    assert st == 0 and c >= (100 + 15 * 4) * (256 + 128)
    st, _ = ws_size(lib.moe_gmm_workspace_size, 100, 4, 200, 128)
    assert st == 2


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def init_routing(lib, **kw):
    a = dict(x=FAKE, x_dtype=2, num_rows=16, hidden=256, expert_idx=FAKE, k=2, expert_num=8, s=0, e=8, quant=3,
             row_idx_type=1, tokens_type=1, ex=FAKE, idx=FAKE, tok=FAKE, sc=FAKE, avail=FAKE, ws=FAKE,
             ws_bytes=0)
    a.update(kw)
    return lib.moe_init_routing(a["x"], a["x_dtype"], a.get("scale"), a["num_rows"], a["hidden"], a["expert_idx"], a["k"],
                                a["expert_num"], a["s"], a["e"], a["quant"], a["row_idx_type"], a["tokens_type"],
                                a["ex"], a["idx"], a["tok"], a["sc"], a["avail"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), 2), (dict(expert_num=0), 2), (dict(expert_num=20000), 2), (dict(s=5, e=3), 2),
    (dict(e=9), 2), (dict(s=-1), 2), (dict(quant=1), 4), (dict(quant=9), 5), (dict(quant=16), 4),
    (dict(hidden=100), 2), (dict(row_idx_type=2), 1), (dict(tokens_type=2), 5), (dict(tokens_type=5), 1),
    (dict(tokens_type=2, expert_num=6000, e=100), 2), (dict(tokens_type=2, s=3, e=3, tok=None), 1),
    (dict(x_dtype=8), 3), (dict(avail=None), 1), (dict(sc=None), 1), (dict(num_rows=1 << 23, k=2), 2),
    # x of MX codes ([V3] quantMode -1 with an FP8/FP4 x): quant -1 only, scale only with codes
    (dict(x_dtype=6), 4), (dict(x_dtype=6, quant=-1), 5), (dict(x_dtype=7, quant=-1, hidden=255), 2),
    (dict(scale=FAKE, quant=-1), 1), (dict(x_dtype=5, quant=-1, scale=FAKE, hidden=48), 2),
    (dict(x_dtype=7, quant=-1, scale=FAKE, sc=None), 1), (dict(x_dtype=7, quant=-1, scale=FAKE), 5),
    (dict(), 5),  # valid arguments, but no workspace: MOE_ERR_WORKSPACE names the byte count
])
def test_init_routing_validation(lib, kw, status):
    assert init_routing(lib, **kw) == status
    msg = lib.moe_last_error().decode()
    assert msg
    if status == 5:
        assert "bytes required" in msg


def test_token_permute_validation(lib):
    def call(**kw):
        a = dict(tokens=FAKE, dtype=2, n=4, hidden=128, indices=FAKE, idt=3, topk=2, ne=2, nout=0, padded=0,
                 quant=3, out=FAKE, srt=FAKE, sc=FAKE, ws=FAKE, wsb=0)
        a.update(kw)
        return lib.moe_token_permute(a["tokens"], a["dtype"], a["n"], a["hidden"], a["indices"], a["idt"],
                                     a["topk"], a["ne"], a["nout"], a["padded"], a["quant"], a["out"], a["srt"],
                                     a["sc"], a["ws"], a["wsb"], None)
    assert call(padded=1) == 4
    assert call(idt=2) == 3
    assert call(dtype=0) == 3          # MX modes take fp16/bf16 tokens only
    assert call(hidden=100) == 2
    assert call(quant=9) == 5          # MXFP4 output is supported: fails on the workspace
    assert call(quant=16) == 4
    assert call(n=1 << 24, topk=1) == 2
    assert call() == 5


def test_mega_moe_validation(lib):
    def args(**kw):
        a = MegaArgs()
        a.x, a.num_tokens, a.hidden, a.topk_ids, a.topk = FAKE, 8, 256, FAKE, 2
        a.topk_weights, a.topk_weights_dtype, a.num_experts, a.inter = FAKE, 0, 8, 128
        a.w1, a.w1_scales, a.w2, a.w2_scales = FAKE, FAKE, FAKE, FAKE
        a.quant_out_dtype, a.activation, a.y = 24, 0, FAKE
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    def status(**kw):
        b = ctypes.c_size_t()
        return lib.mega_moe_workspace_size(ctypes.byref(args(**kw)), ctypes.byref(b))

    assert status() == 0
    assert status(hidden=192) == 2
    assert status(inter=96) == 2
    assert status(topk=0) == 2 and status(topk=33) == 2 and status(topk=9) == 2
    assert status(num_experts=2000) == 2
    assert status(quant_out_dtype=1) == 3
    assert status(activation=5) == 1 and status(activation=-1) == 1

    def act(kind, *vals):
        a = args(activation=kind, num_activation_params=len(vals))
        for j, v in enumerate(vals):
            a.activation_params[j] = v
        b = ctypes.c_size_t()
        return lib.mega_moe_workspace_size(ctypes.byref(a), ctypes.byref(b))

    flt_max = float(np.finfo(np.float32).max)
    assert act(0) == 0 and act(0, 7.0) == 0 and act(0, 0.0) == 0       # swiglu, clamp 0 = none
    assert act(0, -1.0) == 1 and act(0, float("nan")) == 1 and act(0, 1.0, 2.0) == 1
    assert act(1, 3.0) == 0 and act(1, 1.0, 1.0) == 1                   # swiglustep
    assert act(2) == 0 and act(2, 7.0, 1.702, 1.0) == 0 and act(2, 7.0) == 1
    assert act(2, 7.0, float("inf"), 1.0) == 1                          # swigluoai alpha finite
    assert act(3) == 0 and act(3, 2.0) == 0 and act(3, 2.0, 4.0) == 0   # situglu
    assert act(3, 0.0) == 1 and act(3, 2.0, -1.0) == 1
    assert act(4) == 0 and act(4, flt_max) == 0 and act(4, 5.0) == 1     # gelu: no clamp
    assert status(x_is_quantized=1) == 1                       # pre-quantized x needs x_scales
    assert status(x_scales=FAKE) == 1                          # scales only with pre-quantized x
    assert status(x_is_quantized=1, x_scales=FAKE) == 0
    assert status(x_is_quantized=2, x_scales=FAKE) == 1
    assert status(weight_dtype=296) == 0 and status(weight_dtype=296, quant_out_dtype=23) == 4
    assert status(weight_dtype=23) == 4 and status(weight_dtype=7) == 3 and status(shared_weight_dtype=296) == 0
    assert status(topk_weights_dtype=1) == 3
    assert status(combine_comm_mode=1) == 0 and status(combine_comm_mode=2) == 4 and status(combine_comm_mode=-1) == 4
    # combineCommMode 0 keeps bf16 expert rows: half the O bytes of the fp32 merge (mode 1)
    ws = {}
    for mode in (0, 1):
        b = ctypes.c_size_t()
        assert lib.mega_moe_workspace_size(ctypes.byref(args(combine_comm_mode=mode)), ctypes.byref(b)) == 0
        ws[mode] = b.value
    assert ws[1] - ws[0] >= 8 * 2 * 256 * 2 - 256
    assert status(num_shared=5) == 2
    assert status(num_shared=1) == 1   # shared weights missing
    assert status(w2=None) == 1
    assert status(weight_format=2) == 1
    a = args()
    assert lib.mega_moe(ctypes.byref(a), FAKE, 16, None) == 5
    assert "bytes required" in lib.moe_last_error().decode()


def test_probe_validation(lib):
    """The measurement probes reject bad arguments before any launch."""
    assert lib.moe_probe_stream(3, FAKE, FAKE, 1024, None) == 1          # mode
    assert lib.moe_probe_stream(-1, FAKE, FAKE, 1024, None) == 1
    assert lib.moe_probe_stream(0, FAKE, FAKE, 1000, None) == 2          # not a multiple of 16
    assert lib.moe_probe_stream(0, FAKE, FAKE, 0, None) == 2
    assert lib.moe_probe_stream(1, None, FAKE, 1024, None) == 1          # NULL buffer
    assert lib.moe_probe_mfma(0, None, None, None, None) == 2            # iters


def test_binding_rejects_dtypes_the_library_would_misread():
    """The C side reads int32 ids, fp32/bf16 gate weights and bf16 x: the binding rejects
    anything else (e.g. torch.topk's int64 ids) before any call (host-only check)."""
    import torch
    import routing_permute_mxfp8_amd as rp
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.zeros((4, 2), dtype=torch.float32)
    rp._check_layer_dtypes(x, ids, w)
    rp._check_layer_dtypes(x, ids, w.to(torch.bfloat16))
    rp._check_layer_dtypes(torch.zeros((4, 256), dtype=torch.uint8), ids, w, x_scales=torch.zeros((4, 8)))
    bad = [(x, ids.to(torch.int64), w, None), (x.float(), ids, w, None), (x, ids, w.double(), None),
           (x, ids, w[:, :1], None), (x[:3], ids, w, None), (x, ids, w, torch.zeros((4, 8)))]
    for args in bad:
        with pytest.raises(ValueError):
            rp._check_layer_dtypes(*args)


def test_noalloc_routing_rejects_oversized_calls_on_the_host(lib):
    """moe_init_routing_noalloc: a call whose scratch exceeds its static 8 MiB array is
    refused before the device is touched (MOE_ERR_SHAPE, bytes named); argument errors
    come first, as for moe_init_routing."""
    out = (FAKE, FAKE, FAKE, FAKE, FAKE)
    st = lib.moe_init_routing_noalloc(FAKE, 2, None, 1 << 19, 32, FAKE, 8, 4096, 0, 4096, -1, 0, 1, *out, None)
    assert st == 2 and "static scratch" in lib.moe_last_error().decode()
    st = lib.moe_init_routing_noalloc(FAKE, 2, None, 16, 32, FAKE, 8, 64, 5, 3, -1, 0, 1, *out, None)
    assert st == 2 and "active range" in lib.moe_last_error().decode()
    b = ctypes.c_size_t()
    assert lib.moe_init_routing_workspace_size(32768, 8, 256, ctypes.byref(b)) == 0 and b.value <= 8 << 20
