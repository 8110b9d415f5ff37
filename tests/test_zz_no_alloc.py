"""moe_init_routing_noalloc (the allocation-free variant of moe_init_routing) against
moe_init_routing itself: the same outputs bit for bit on two calls in a row, the second
one smaller (so it runs on the scratch the first left behind), through the C ABI."""
import numpy as np
import pytest
import torch

import moe_inputs
import routing_permute_mxfp8_amd as rp
from gpu_support import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def both(x, ids, experts, active, quant, row_idx_type, tokens_type):
    ref = rp.init_routing(x, ids, experts, active, quant, row_idx_type, tokens_type)
    got = rp.init_routing_noalloc(x, ids, experts, active, quant, row_idx_type, tokens_type)
    torch.cuda.synchronize()
    return ref, got


def assert_same(ref, got):
    avail = int(ref[4].item())
    assert int(got[4].item()) == avail
    # rows >= availableIdxNum of expanded_x / expanded_scale are not written by either call
    assert torch.equal(ref[0][:avail], got[0][:avail])
    assert torch.equal(ref[1], got[1])
    assert torch.equal(ref[2], got[2])
    if ref[3] is not None:
        assert torch.equal(ref[3][:avail], got[3][:avail])


def test_noalloc_matches_init_routing_on_two_calls():
    # call 1: the routing workload (32768 tokens x 7168, topK 8 of 256, experts [32, 64),
    # scatter index, counts, MXFP8 E4M3)
    cfg = moe_inputs.config("routing")
    say(f"noalloc routing call 1: N={cfg.tokens} H={cfg.hidden} K={cfg.topk} E={cfg.experts} {cfg.active_range}")
    x = moe_inputs.activations(cfg).to(DEV)
    ids = to_dev(moe_inputs.expert_ids(cfg).astype(np.int32))
    ref, got = both(x, ids, cfg.experts, cfg.active_range, rp.QUANT_E4M3, 1, 1)
    assert_same(ref, got)
    del x, ids, ref, got
    # call 2, smaller: 300 tokens, gather index (scatter index in the scratch), cumsum,
    # E5M2, another active range
    cfg2 = moe_inputs.config("tiny", tokens=300, hidden=512, experts=24, topk=3, seed=91)
    say(f"noalloc routing call 2: N={cfg2.tokens} H={cfg2.hidden} K={cfg2.topk} E={cfg2.experts}")
    x = moe_inputs.activations(cfg2).to(DEV)
    ids = to_dev(moe_inputs.expert_ids(cfg2).astype(np.int32))
    ref, got = both(x, ids, cfg2.experts, (3, 17), rp.QUANT_E5M2, 0, 0)
    assert_same(ref, got)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A call whose scratch would exceed the static array fails before any launch."""
    n, k, e = 1 << 19, 8, 4096
    x = torch.zeros((n, 32), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((n, k), dtype=torch.int32, device=DEV)
    with pytest.raises(rp.MoeError, match="static scratch"):
        rp.init_routing_noalloc(x, ids, e, (0, e), rp.QUANT_NONE, 0, 1)
