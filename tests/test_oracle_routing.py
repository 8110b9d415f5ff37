"""Pins for oracle.routing: stable sort, inverse, histogram, active range, permute.

Independent references: Python's built-in stable sorted() on small inputs with
heavy ties, the moe_token_permute worked example (tests/golden), and the
invariants the pages state (inverse permutation, availableIdxNum = count in range,
counts summing to N*K).
"""
import json
import os

import numpy as np
import pytest

from oracle import mxfp, routing


def py_stable_order(keys):
    return sorted(range(len(keys)), key=keys.__getitem__)


@pytest.mark.parametrize("n,k,e,seed", [(1, 1, 1, 0), (5, 3, 4, 1), (37, 4, 3, 2), (64, 8, 16, 3), (100, 2, 2, 4)])
def test_sort_matches_python_sorted(n, k, e, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, e, size=(n, k))
    r = routing.init_routing(ids, e)
    keys = ids.reshape(-1).tolist()
    assert r["sorted_row_idx"].tolist() == py_stable_order(keys)
    assert r["sorted_keys"].tolist() == sorted(keys)
    # inverse: expandedRowIdx[sortedRowIdx[i]] = i
    inv = r["expanded_row_idx"]
    assert sorted(inv.tolist()) == list(range(n * k))
    for i, row in enumerate(r["sorted_row_idx"]):
        assert inv[row] == i
    assert r["counts"].sum() == n * k
    assert r["counts"].tolist() == [keys.count(x) for x in range(e)]
    assert r["avail"] == n * k


def test_permute_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "permute_worked_example.json")))
    tokens = np.arange(4 * g["hidden"], dtype=np.float64).reshape(4, g["hidden"])
    out = routing.token_permute(tokens, np.array(g["indices"]), num_out_tokens=g["num_out_tokens"])
    assert out["first"].tolist() == g["sorted_indices_first"]
    assert out["sorted_indices"].tolist() == g["sorted_indices"]
    assert list(out["permuted"].shape) == g["printed_shapes_plain"]["permuted_tokens"]
    assert list(out["sorted_indices"].shape) == g["printed_shapes_plain"]["sorted_indices"]
    assert out["scales"] is None
    assert np.array_equal(out["permuted"], tokens[g["source_tokens"][:g["num_out_tokens"]]])
    q = routing.token_permute(tokens / 100.0, np.array(g["indices"]), quant_mode=2)
    assert list(q["permuted"].shape) == g["printed_shapes_mxfp8"]["permuted_tokens"]
    assert list(q["scales"].shape) == g["printed_shapes_mxfp8"]["expanded_scale"]
    for n_out, m in g["num_out_tokens_rule"]:
        assert routing.actual_num_out_tokens(8, n_out) == m


def test_one_dimensional_indices_mean_topk_one():
    ids = np.array([3, 1, 3, 0, 1])
    out = routing.token_permute(np.eye(5), ids)
    assert out["topk"] == 1
    assert out["first"].tolist() == py_stable_order(ids.tolist())
    assert np.array_equal(out["permuted"], np.eye(5)[out["first"]])


@pytest.mark.parametrize("s,e", [(0, 8), (2, 5), (3, 3), (0, 1), (7, 8)])
def test_active_range(s, e):
    rng = np.random.default_rng(s * 10 + e)
    n, k, ne = 50, 3, 8
    ids = np.stack([rng.permutation(ne)[:k] for _ in range(n)])
    keys = ids.reshape(-1)
    in_range = (keys >= s) & (keys < e)
    sc = routing.init_routing(ids, ne, active=(s, e), row_idx_type=1, tokens_num_type=1)
    ga = routing.init_routing(ids, ne, active=(s, e), row_idx_type=0, tokens_num_type=0)
    avail = int(in_range.sum())
    assert sc["avail"] == avail == ga["avail"]
    idx = sc["expanded_row_idx"]
    assert np.all(idx[~in_range] == -1)
    assert sorted(idx[in_range].tolist()) == list(range(avail))
    # scatter position p of flat row r: expert-major, then ascending r
    order = py_stable_order([int(x) if lo else 10 ** 9 for x, lo in zip(keys, in_range)])[:avail]
    for p, r in enumerate(order):
        assert idx[r] == p
    gi = ga["expanded_row_idx"]
    assert gi[:avail].tolist() == order and np.all(gi[avail:] == -1)
    assert sc["expert_tokens"].tolist() == [int((keys == x).sum()) for x in range(s, e)]
    assert ga["expert_tokens"].tolist() == np.cumsum([int((keys == x).sum()) for x in range(s, e)]).tolist()
    if e > s:
        assert ga["expert_tokens"][-1] == avail


def test_gather_rows_quant_is_row_local():
    rng = np.random.default_rng(9)
    x = mxfp.bf16_round(rng.standard_normal((6, 64)))
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0], [1, 2]])
    r = routing.init_routing(ids, 3)
    codes, scales = routing.gather_rows(x, r["sorted_row_idx"], 2, 3)
    allq, alls = mxfp.quantize(x, "e4m3")
    src = r["sorted_row_idx"] // 2
    assert np.array_equal(codes, allq[src]) and np.array_equal(scales, alls[src])


def test_key_value_counts():
    """expertTokensNumType 2: (expert, count) rows of the active experts with rows, ascending,
    zero rows after them; hand-derived for the moe_token_permute example ids and checked
    against a brute-force count on random ids."""
    ids = np.array([[1, 0], [0, 1], [1, 0], [0, 1]])
    r = routing.init_routing(ids, 4, (0, 4), 1, 2)
    assert r["expert_tokens"].tolist() == [[0, 4], [1, 4], [0, 0], [0, 0]]
    r = routing.init_routing(ids, 4, (1, 3), 1, 2)
    assert r["expert_tokens"].tolist() == [[1, 4], [0, 0], [0, 0], [0, 0]]
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 50, (300, 3))
    kv = routing.init_routing(ids, 50, (7, 41), 1, 2)["expert_tokens"]
    want = [(e, int((ids == e).sum())) for e in range(7, 41) if (ids == e).sum() > 0]
    assert kv.shape == (50, 2)
    assert [tuple(v) for v in kv[:len(want)].tolist()] == want
    assert np.all(kv[len(want):] == 0)


@pytest.mark.parametrize("mode", [2, 3, 9])
def test_passthrough_gather_equals_quantize_then_gather(mode):
    """MoeInitRoutingV3 quantMode -1 with an x of MX codes and scaleOptional: gathering
    already-quantized rows and their scales gives what the MX modes give from bf16 x,
    because Q_MX is row-local ([V3] 计算公式 5 quantizes x before the gather)."""
    rng = np.random.default_rng(7 + mode)
    n, k, e, h = 37, 3, 9, 128
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)])
    x = mxfp.bf16_round(rng.normal(0, 1, (n, h)))
    r = routing.init_routing(ids, e, active=(2, 7))
    fmt = routing.quant_mode_format(mode)
    codes, scales = mxfp.quantize(x, fmt)
    if fmt == "e2m1":
        codes = mxfp.pack_fp4(codes)
    got_c, got_s = routing.gather_passthrough(codes, scales, r["sorted_row_idx"], k, r["active_start"], r["avail"])
    want_c, want_s = routing.gather_rows(x, r["sorted_row_idx"], k, mode, r["active_start"], r["avail"])
    assert got_c.dtype == np.uint8 and np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s)
    only_c, no_s = routing.gather_passthrough(codes, None, r["sorted_row_idx"], k, r["active_start"], r["avail"])
    assert no_s is None and np.array_equal(only_c, want_c)
