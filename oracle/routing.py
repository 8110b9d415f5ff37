"""Routing: stable key-value sort, inverse index, histogram, active range, gather.

MoeInitRoutingV3 README, 计算公式:
  1. sortedExpertIdx, sortedRowIdx = keyValueSort(expertIdx, rowIdx)
  2. expandedRowIdxOut[sortedRowIdx[i]] = i
  3. per-expert histogram of sortedExpertIdx
  5. expandedXOut[i] = quantResult[source row of sortedRowIdx[i]]
  6. availableIdxNum = #{x in expertIdx : expert_start <= x < expert_end}
moe_token_permute article, 功能说明: sortedIndicesFirst = stable argSort of the
flattened indices, sortedIndicesOut = its inverse, permuted row i is
tokens[sortedIndicesFirst[i] // topK].

Readings taken where the pages are silent or disagree:
* flat row numbering is token-major, r = t*K + k, and the source token of flat
  row r is r // K (the permute article's prose and golden reference); the
  "% NUM_ROWS" in the V3 gather formula is a different numbering and not used.
* the sort is stable: equal experts keep ascending r.
* with an active expert range [s, e), positions are relative to the start of
  the active segment; entries outside the range get -1 in both index types
  (the V3 page leaves scatter-type entries uninitialised; -1 is a superset).
* expertTokensNumType 1 (count) = per-expert counts of the active experts,
  0 (cumsum) = their inclusive prefix sum, both int64 [e - s].
"""

from __future__ import annotations

import numpy as np

from . import mxfp


def flatten_ids(expert_idx) -> tuple[np.ndarray, int]:
    """[N] or [N, K] ids -> (flat keys [N*K] in token-major order, K)."""
    ids = np.asarray(expert_idx)
    if ids.ndim == 1:
        return ids.astype(np.int64), 1
    assert ids.ndim == 2
    return ids.reshape(-1).astype(np.int64), ids.shape[1]


def key_value_sort(keys: np.ndarray):
    """keyValueSort(expertIdx, rowIdx) with rowIdx = 0..F-1: a stable sort by key.
    Returns (sorted keys, sorted row indices), both int64 [F]."""
    keys = np.asarray(keys, dtype=np.int64)
    order = np.argsort(keys, kind="stable")        # library stable sort
    return keys[order], order.astype(np.int64)


def inverse(sorted_row_idx: np.ndarray) -> np.ndarray:
    """expandedRowIdx[sortedRowIdx[i]] = i."""
    inv = np.empty_like(sorted_row_idx)
    inv[sorted_row_idx] = np.arange(sorted_row_idx.size, dtype=sorted_row_idx.dtype)
    return inv


def histogram(sorted_keys: np.ndarray, num_experts: int) -> np.ndarray:
    """counts[e] = number of flat rows routed to expert e (int64 [E])."""
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in range(num_experts):
        counts[e] = np.count_nonzero(sorted_keys == e)
    return counts


def init_routing(expert_idx, num_experts: int, active=None, row_idx_type: int = 1,
                 tokens_num_type: int = 1) -> dict:
    """MoeInitRoutingV3 index outputs (dropless).

    Returns a dict with
      sorted_row_idx   int64 [F]  full stable sort (all experts)
      sorted_keys      int64 [F]
      counts           int64 [E]  all experts
      offsets          int64 [E+1] exclusive prefix of counts
      active_start     int        offsets[s]
      avail            int        availableIdxNum
      expanded_row_idx int32 [F]  per row_idx_type (1 scatter, 0 gather)
      expert_tokens    int64 [e-s] per tokens_num_type (1 count, 0 cumsum), or
                       [E, 2] (expert, count) rows for 2 (key_value)
    """
    keys, k = flatten_ids(expert_idx)
    assert keys.size == 0 or (keys.min() >= 0 and keys.max() < num_experts)
    s, e = (0, num_experts) if active is None else active
    assert 0 <= s <= e <= num_experts
    sorted_keys, sorted_row_idx = key_value_sort(keys)
    counts = histogram(sorted_keys, num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    off0 = int(offsets[s])
    avail = int(np.count_nonzero((keys >= s) & (keys < e)))
    assert avail == int(offsets[e] - offsets[s])
    full_inv = inverse(sorted_row_idx)
    if row_idx_type == 1:
        in_range = (keys >= s) & (keys < e)
        idx = np.where(in_range, full_inv - off0, -1)
    elif row_idx_type == 0:
        idx = np.full(keys.size, -1, dtype=np.int64)
        idx[:avail] = sorted_row_idx[off0:off0 + avail]
    else:
        raise ValueError("row_idx_type must be 0 (gather) or 1 (scatter)")
    active_counts = counts[s:e]
    if tokens_num_type == 1:
        tok = active_counts.copy()
    elif tokens_num_type == 0:
        tok = np.cumsum(active_counts)
    elif tokens_num_type == 2:
        # key_value (README, expertTokensCountOrCumsumOut): shape [num_experts, 2], one row
        # (expert id, its row count) per active expert with a non-zero count, in ascending
        # expert order. Reading: the rows past them are 0 (the pages leave them open).
        tok = np.zeros((num_experts, 2), dtype=np.int64)
        row = 0
        for j, c in enumerate(active_counts):
            if c > 0:
                tok[row] = (s + j, c)
                row += 1
    else:
        raise ValueError("tokens_num_type must be 0 (cumsum), 1 (count) or 2 (key_value)")
    return dict(sorted_row_idx=sorted_row_idx, sorted_keys=sorted_keys, counts=counts,
                offsets=offsets, active_start=off0, avail=avail, topk=k,
                expanded_row_idx=idx.astype(np.int32), expert_tokens=tok.astype(np.int64))


def quant_mode_format(quant_mode: int):
    """quantMode 2 -> E5M2, 3 -> E4M3FN, 9 -> E2M1 (MXFP4), -1 -> no quantization (None)."""
    return {-1: None, 2: "e5m2", 3: "e4m3", 9: "e2m1"}[quant_mode]


def gather_rows(x, sorted_row_idx, topk: int, quant_mode: int, start: int = 0, count=None):
    """expandedX[i] = Q(x[sortedRowIdx[start + i] // K]) for i < count.

    x: float array [N, H] (bf16 values as float64). quant_mode -1 returns the
    rows unchanged (float64) and scales None; 2/3/9 return (codes, scales) of the
    MX quantization of each gathered row (Q_MX is row-local, so quantizing then
    gathering is the same as gathering then quantizing); for 9 the codes come
    packed two per byte ([count, H / 2], mxfp.pack_fp4)."""
    x = np.asarray(x, dtype=np.float64)
    if count is None:
        count = sorted_row_idx.size - start
    src = sorted_row_idx[start:start + count] // topk
    rows = x[src]
    fmt = quant_mode_format(quant_mode)
    if fmt is None:
        return rows, None
    codes, scales = mxfp.quantize(rows, fmt)
    if fmt == "e2m1":
        codes = mxfp.pack_fp4(codes)
    return codes, scales


def gather_passthrough(codes, scales, sorted_row_idx, topk: int, start: int = 0, count=None):
    """MoeInitRoutingV3 with quantMode -1 and an x already holding MX codes (FLOAT8_E4M3FN,
    FLOAT8_E5M2 or FLOAT4_E2M1 bytes) and, optionally, their FLOAT8_E8M0 scales
    (scaleOptional): expandedX[i] = codes[sortedRowIdx[start + i] // K] and
    expandedScaleOut[i] = scales[sortedRowIdx[start + i] // K], the rows taken as they are.
    Returns (code rows, scale rows or None)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if count is None:
        count = sorted_row_idx.size - start
    src = sorted_row_idx[start:start + count] // topk
    return codes[src], None if scales is None else np.asarray(scales, dtype=np.uint8)[src]


def actual_num_out_tokens(flat: int, num_out_tokens) -> int:
    """moe_token_permute 参数说明: None or 0 -> F; > 0 -> min(n, F); < 0 -> max(F + n, 0)."""
    if num_out_tokens is None or num_out_tokens == 0:
        return flat
    if num_out_tokens > 0:
        return min(num_out_tokens, flat)
    return max(flat + num_out_tokens, 0)


def token_permute(tokens, indices, num_out_tokens=None, quant_mode: int = -1) -> dict:
    """moe_token_permute (padded_mode False).

    Returns permuted (rows or codes) [M, H], scales [M, AlignUp(CeilDiv(H,32),2)]
    or None, sorted_indices int32 [F] (the inverse of the stable argsort, never
    truncated), and first (the stable argsort itself)."""
    keys, k = flatten_ids(indices)
    _, first = key_value_sort(keys)
    inv = inverse(first)
    m = actual_num_out_tokens(keys.size, num_out_tokens)
    rows, scales = gather_rows(tokens, first, k, quant_mode, 0, m)
    return dict(permuted=rows, scales=scales, sorted_indices=inv.astype(np.int32),
                first=first, rows_out=m, topk=k)
