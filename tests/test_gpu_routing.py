"""Routing and permute on the GPU against the oracle, bit for bit: sorted/inverse
indices, counts / cumsum, availableIdxNum and the MX-quantized gathered rows,
for the named workloads at full size and for the edge cases (empty and one-expert
active ranges, gather-type index, 1-D and int64 indices, num_out_tokens, ragged
sizes, fp16/fp32 inputs, no quantization)."""
import numpy as np
import pytest
import torch

import moe_inputs
import routing_permute_mxfp8_amd as rp
from oracle import mxfp, routing
from gpu_support import DEV, QMODE, say, to_dev

pytestmark = pytest.mark.gpu


def run_init_routing(x_cpu, ids, e_num, active, quant_mode, row_idx_type=1, tokens_type=1, run_twice=False):
    x = x_cpu.to(DEV)
    ti = to_dev(ids.astype(np.int32))
    outs = rp.init_routing(x, ti, e_num, active, quant_mode, row_idx_type, tokens_type)
    if run_twice:
        again = rp.init_routing(x, ti, e_num, active, quant_mode, row_idx_type, tokens_type)
        a = int(outs[4][0].item())   # rows >= availableIdxNum of expanded_x / expanded_scale are not written
        for j, (u, v) in enumerate(zip(outs, again)):
            if u is not None:
                assert torch.equal(u[:a], v[:a]) if j in (0, 3) else torch.equal(u, v), "repeated call differs"
    torch.cuda.synchronize()
    return [None if o is None else (o.cpu().float().numpy() if o.dtype in (torch.bfloat16, torch.float16)
                                    else o.cpu().numpy()) for o in outs]


def check_init_routing(x_cpu, ids, e_num, active, quant_mode, row_idx_type=1, tokens_type=1, run_twice=False):
    ex, idx, tok, sc, avail = run_init_routing(x_cpu, ids, e_num, active, quant_mode, row_idx_type, tokens_type,
                                               run_twice)
    ref = routing.init_routing(ids, e_num, active, row_idx_type, tokens_type)
    assert int(avail[0]) == ref["avail"]
    assert np.array_equal(idx, ref["expanded_row_idx"])
    assert np.array_equal(tok, ref["expert_tokens"])
    a = ref["avail"]
    k = ids.shape[1]
    srt = ref["sorted_row_idx"][ref["active_start"]:ref["active_start"] + a]
    if a * x_cpu.shape[1] > 20_000_000:   # full-size workloads: every index above, a row sample here
        pos = np.sort(np.random.default_rng(0).choice(a, size=4096, replace=False))
    else:
        pos = np.arange(a)
    src = srt[pos] // k
    x64 = x_cpu[torch.from_numpy(src)].double().numpy()
    if quant_mode == -1:
        assert np.array_equal(ex[pos].astype(np.float64), x64)
    else:
        codes, scales = mxfp.quantize(x64, routing.quant_mode_format(quant_mode))
        if quant_mode == rp.QUANT_MXFP4:
            codes = mxfp.pack_fp4(codes)
        assert np.array_equal(ex[pos], codes)
        assert np.array_equal(sc[pos], scales)
    return ref


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "routing"])
def test_named_workloads(name):
    cfg = moe_inputs.config(name)
    say(f"init_routing full workload {name}: N={cfg.tokens} H={cfg.hidden} E={cfg.experts} K={cfg.topk}")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg)
    q = QMODE[cfg.fmt]
    ref = check_init_routing(x, ids, cfg.experts, cfg.active_range, q, run_twice=(name == "routing"))
    assert ref["avail"] == int(((ids >= cfg.active_range[0]) & (ids < cfg.active_range[1])).sum())


@pytest.mark.parametrize("active", [(0, 8), (3, 3), (0, 1), (7, 8), (2, 6)])
@pytest.mark.parametrize("row_idx_type,tokens_type", [(1, 1), (0, 0), (0, 1), (1, 0), (1, 2), (0, 2)])
def test_ranges_and_index_types(active, row_idx_type, tokens_type):
    cfg = moe_inputs.config("tiny", tokens=203, hidden=96, topk=3, seed=77)
    say(f"init_routing active={active} row_idx_type={row_idx_type} tokens_type={tokens_type}")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg)
    check_init_routing(x, ids, cfg.experts, active, rp.QUANT_E4M3, row_idx_type, tokens_type)


@pytest.mark.parametrize("quant_mode,dtype", [(-1, torch.bfloat16), (-1, torch.float32), (-1, torch.float16),
                                              (2, torch.float16), (3, torch.float32), (2, torch.bfloat16),
                                              (9, torch.bfloat16), (9, torch.float16), (9, torch.float32)])
def test_dtypes_and_modes(quant_mode, dtype):
    cfg = moe_inputs.config("tiny", tokens=77, hidden=160, topk=4, experts=16, seed=5)
    say(f"init_routing quant_mode={quant_mode} dtype={dtype}")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg).to(dtype)
    check_init_routing(x, ids, cfg.experts, (1, 13), quant_mode)


def test_many_experts_and_chunks():
    # more chunks than one wave, many buckets, heavy ties (E = 5000, K = 1 ... 7)
    cfg = moe_inputs.config("tiny", tokens=30000, hidden=64, topk=7, experts=5000, seed=9)
    say("init_routing E=5000 K=7 N=30000")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg)
    check_init_routing(x, ids, cfg.experts, (100, 4000), rp.QUANT_E5M2, 0, 0)


@pytest.mark.parametrize("tokens,topk,experts,active,row_idx_type,tokens_type,quant",
                         [(10000, 8, 600, (50, 550), 0, 0, 2),     # 1024-row chunks, 500 buckets, gather index
                          (9000, 4, 64, (0, 64), 1, 1, 3),         # 256-row chunks, every expert active
                          (1111, 16, 300, (17, 290), 0, 2, 3),     # ragged last chunk, K = 16, key_value
                          (5000, 5, 40, (3, 37), 1, 0, 2),         # K = 5: tokens straddle chunks
                          (3000, 8, 256, (32, 64), 1, 1, 9)])      # MXFP4 output
def test_chunked_routing_shapes(tokens, topk, experts, active, row_idx_type, tokens_type, quant):
    # several hundred chunks, hundreds of buckets, ragged last chunk, K = 16 and odd K
    cfg = moe_inputs.config("tiny", tokens=tokens, hidden=256, topk=topk, experts=experts, seed=tokens)
    say(f"init_routing chunked N={tokens} K={topk} E={experts} active={active}")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg)
    check_init_routing(x, ids, cfg.experts, active, quant, row_idx_type, tokens_type, run_twice=True)


def test_empty_input():
    say("init_routing empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16)
    ids = np.zeros((0, 2), np.int32)
    ex, idx, tok, sc, avail = run_init_routing(x, ids, 8, (0, 8), rp.QUANT_E4M3)
    assert int(avail[0]) == 0 and np.all(tok == 0) and idx.size == 0


def check_permute(tokens_cpu, indices, num_out, quant_mode, num_experts):
    out, srt, sc = rp.token_permute(tokens_cpu.to(DEV), torch.from_numpy(indices).to(DEV), num_out, False,
                                    quant_mode, num_experts=num_experts)
    torch.cuda.synchronize()
    ref = routing.token_permute(tokens_cpu.double().numpy(), indices, num_out, quant_mode)
    assert np.array_equal(srt.cpu().numpy(), ref["sorted_indices"])
    assert out.shape[0] == ref["rows_out"]
    if quant_mode == -1:
        assert np.array_equal(out.cpu().double().numpy(), ref["permuted"])
        assert sc.numel() == 0
    else:
        assert np.array_equal(out.cpu().numpy(), ref["permuted"])
        assert np.array_equal(sc.cpu().numpy(), ref["scales"])


def test_permute_worked_example_shapes():
    say("token_permute worked example")
    tokens = torch.randn(4, 128).to(torch.float16)
    idx = np.array([[1, 0], [0, 1], [1, 0], [0, 1]], dtype=np.int32)
    out, srt, sc = rp.token_permute(tokens.to(DEV), torch.from_numpy(idx).to(DEV), 6, num_experts=2)
    assert tuple(out.shape) == (6, 128) and tuple(srt.shape) == (8,) and tuple(sc.shape) == (0,)
    assert srt.cpu().tolist() == [4, 0, 1, 5, 6, 2, 3, 7]
    out, srt, sc = rp.token_permute(tokens.to(DEV), torch.from_numpy(idx).to(DEV), quant_mode=2, num_experts=2)
    assert tuple(out.shape) == (8, 128) and tuple(sc.shape) == (8, 4)
    check_permute(tokens, idx, 6, -1, 2)
    check_permute(tokens, idx, None, 2, 2)
    out, srt, sc = rp.token_permute(tokens.to(DEV), torch.from_numpy(idx).to(DEV), quant_mode=9, num_experts=2)
    assert tuple(out.shape) == (8, 64) and tuple(sc.shape) == (8, 4)   # MXFP4: H / 2 bytes a row
    check_permute(tokens, idx, 5, 9, 2)


@pytest.mark.parametrize("num_out", [None, 0, 1000, 311, -5, -100000])
@pytest.mark.parametrize("int64", [False, True])
def test_permute_num_out_tokens(num_out, int64):
    rng = np.random.default_rng(3)
    n, k, e = 150, 3, 37
    idx = rng.integers(0, e, size=(n, k)).astype(np.int64 if int64 else np.int32)  # duplicates allowed here
    tokens = torch.from_numpy(rng.standard_normal((n, 64)).astype(np.float32)).to(torch.bfloat16)
    say(f"token_permute num_out={num_out} int64={int64}")
    check_permute(tokens, idx, num_out, 3, e)
    check_permute(tokens, idx, num_out, -1, e)


def test_permute_one_dimensional_indices():
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 5, size=(99,)).astype(np.int32)
    tokens = torch.from_numpy(rng.standard_normal((99, 32)).astype(np.float32)).to(torch.bfloat16)
    say("token_permute 1-D indices")
    check_permute(tokens, idx, None, 2, 5)
    check_permute(tokens, idx, -7, 9, 5)


@pytest.mark.parametrize("fmt,x_codes", [("e4m3", rp.DTYPE_FP8_E4M3), ("e5m2", rp.DTYPE_FP8_E5M2),
                                         ("e2m1", rp.DTYPE_FP4_E2M1)])
@pytest.mark.parametrize("with_scale", [True, False])
@pytest.mark.parametrize("row_idx_type", [1, 0])
def test_init_routing_passthrough(fmt, x_codes, with_scale, row_idx_type):
    """MoeInitRoutingV3 quantMode -1 with an x of FP8/FP4 codes and scaleOptional: the code
    rows and scale rows gathered as they are, bit for bit against the oracle's gather (the
    codes and scales are the oracle's quantization of bf16 x), with an active range."""
    cfg = moe_inputs.config("tiny", tokens=301, hidden=256, topk=3, experts=12, seed=78)
    active = (2, 9)
    say(f"init_routing pass-through {fmt} scale={with_scale} row_idx_type={row_idx_type}")
    ids = moe_inputs.expert_ids(cfg)
    x = moe_inputs.activations(cfg).double().numpy()
    codes, scales = mxfp.quantize(x, fmt)
    if fmt == "e2m1":
        codes = mxfp.pack_fp4(codes)
    ex, idx, tok, sc, avail = rp.init_routing(to_dev(codes), to_dev(ids.astype(np.int32)), cfg.experts, active,
                                              rp.QUANT_NONE, row_idx_type, 1, x_codes=x_codes,
                                              scale=to_dev(scales) if with_scale else None)
    torch.cuda.synchronize()
    ref = routing.init_routing(ids, cfg.experts, active, row_idx_type, 1)
    a = ref["avail"]
    assert int(avail.item()) == a
    assert np.array_equal(idx.cpu().numpy(), ref["expanded_row_idx"])
    assert np.array_equal(tok.cpu().numpy(), ref["expert_tokens"])
    want_c, want_s = routing.gather_passthrough(codes, scales if with_scale else None, ref["sorted_row_idx"],
                                                cfg.topk, ref["active_start"], a)
    assert np.array_equal(ex.cpu().numpy()[:a], want_c)
    if with_scale:
        assert np.array_equal(sc.cpu().numpy()[:a], want_s)
    else:
        assert sc is None
