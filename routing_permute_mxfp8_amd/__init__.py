"""Python binding of the MI355X MoE-layer hot path (libmoe_mx.so, C ABI in include/moe_mx.h).

Argument marshalling only: outputs and workspaces are allocated with torch on the
tensors' device, pointers and the current HIP stream are passed to the library,
and every step of the computation runs in the library's HIP kernels. If the
library has not been built (python -m routing_permute_mxfp8_amd.build, or
__graft_entry__.build()) the calls raise; there is no fallback path.

Byte conventions: FP8 codes and E8M0 scales are returned as torch.uint8 tensors
(view them as torch.float8_e4m3fn / float8_e5m2 / float8_e8m0fnu if wanted);
inputs may be uint8 or the matching float8 dtype.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import lib_path

__all__ = [
    "MoeError", "load", "QUANT_NONE", "QUANT_E5M2", "QUANT_E4M3", "QUANT_MXFP4", "FP8_E5M2", "FP8_E4M3",
    "mx_scale_cols", "token_permute_out_rows", "mx_quantize", "init_routing", "init_routing_noalloc", "token_permute",
    "mega_moe", "mega_moe_workspace_bytes", "gmm1_swiglu_quant", "gmm2_combine", "combine_finalize",
    "pack_weights", "WEIGHTS_ND", "WEIGHTS_PACKED", "DTYPE_FP8_E5M2", "DTYPE_FP8_E4M3", "DTYPE_FP4_E2M1",
]

QUANT_NONE, QUANT_E5M2, QUANT_E4M3, QUANT_MXFP4 = -1, 2, 3, 9
FP8_E5M2, FP8_E4M3 = 23, 24
WEIGHTS_ND, WEIGHTS_PACKED = 0, 1
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.int32: 3, torch.int64: 4}
# x dtypes of MX codes for init_routing's pass-through (one FP8 code a byte, two FP4 codes a byte)
DTYPE_FP8_E5M2, DTYPE_FP8_E4M3, DTYPE_FP4_E2M1 = 5, 6, 7
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "SHAPE", 3: "DTYPE", 4: "UNSUPPORTED", 5: "WORKSPACE", 6: "HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class MegaArgs(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
        ("topk_ids", ctypes.c_void_p), ("topk", ctypes.c_int64),
        ("topk_weights", ctypes.c_void_p), ("topk_weights_dtype", ctypes.c_int),
        ("num_experts", ctypes.c_int64), ("inter", ctypes.c_int64),
        ("w1", ctypes.c_void_p), ("w1_scales", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scales", ctypes.c_void_p),
        ("num_shared", ctypes.c_int64),
        ("shared_w1", ctypes.c_void_p), ("shared_w1_scales", ctypes.c_void_p),
        ("shared_w2", ctypes.c_void_p), ("shared_w2_scales", ctypes.c_void_p),
        ("quant_out_dtype", ctypes.c_int), ("activation", ctypes.c_int), ("weight_format", ctypes.c_int),
        ("y", ctypes.c_void_p), ("expert_token_nums", ctypes.c_void_p),
        ("xq", ctypes.c_void_p), ("sx", ctypes.c_void_p), ("h1", ctypes.c_void_p),
        ("aq", ctypes.c_void_p), ("sa", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("sorted_row_idx", ctypes.c_void_p),
        ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
        ("num_activation_params", ctypes.c_int), ("activation_params", ctypes.c_float * 3),
        ("weight_dtype", ctypes.c_int), ("shared_weight_dtype", ctypes.c_int),
        ("x_is_quantized", ctypes.c_int), ("x_scales", ctypes.c_void_p),
        ("combine_comm_mode", ctypes.c_int),
    ]

MEGA_STAGE_EVENTS = 7
# activation kinds of mega_moe (MegaMoE "Activation function formulas")
ACT_SWIGLU, ACT_SWIGLUSTEP, ACT_SWIGLUOAI, ACT_SITUGLU, ACT_GELU = 0, 1, 2, 3, 4
FP4_E2M1 = 296   # MXFP4 weights (A8W4-FP)
MEGA_STAGES = ["routing", "permute_quant", "gmm1_swiglu_quant", "gmm2", "shared_experts", "combine"]


_lib = None

_I64, _INT, _VP, _SZ = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_version": ([], _INT),
    "moe_mx_scale_cols": ([_I64], _I64),
    "moe_token_permute_out_rows": ([_I64, _I64], _I64),
    "moe_mx_quantize": ([_VP, _INT, _I64, _I64, _INT, _VP, _VP, _VP], _INT),
    "moe_mx_packed_scale_bytes": ([_I64, _I64, _I64], _I64),
    "moe_mx_pack_weights": ([_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP], _INT),
    "moe_mx_pack_weights_fp4": ([_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP], _INT),
    "moe_init_routing_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "moe_init_routing": ([_VP, _INT, _VP, _I64, _I64, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _INT,
                          _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], _INT),
    "moe_init_routing_noalloc": ([_VP, _INT, _VP, _I64, _I64, _VP, _I64, _I64, _I64, _I64, _INT, _INT, _INT,
                                  _VP, _VP, _VP, _VP, _VP, _VP], _INT),
    "moe_token_permute_workspace_size": ([_I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "moe_token_permute": ([_VP, _INT, _I64, _I64, _VP, _INT, _I64, _I64, _I64, _INT, _INT,
                           _VP, _VP, _VP, _VP, _SZ, _VP], _INT),
    "mega_moe_workspace_size": ([ctypes.POINTER(MegaArgs), ctypes.POINTER(_SZ)], _INT),
    "mega_moe": ([ctypes.POINTER(MegaArgs), _VP, _SZ, _VP], _INT),
    "moe_gmm_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "moe_gmm1_swiglu_quant": ([_VP, _VP, _I64, _I64, _I64, _VP, _I64, _VP, _VP, _INT, _INT, _VP, _VP, _VP,
                               _VP, _SZ, _VP], _INT),
    "moe_gmm2_combine": ([_VP, _VP, _I64, _I64, _I64, _VP, _I64, _VP, _VP, _INT, _INT, _VP, _VP, _I64, _VP,
                          _VP, _VP, _SZ, _VP], _INT),
    "moe_combine_finalize": ([_VP, _I64, _I64, _VP, _VP], _INT),
    "moe_probe_stream": ([_INT, _VP, _VP, _I64, _VP], _INT),
    "moe_probe_mfma": ([_INT, _VP, ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double), _VP], _INT),
}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmoe_mx.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run routing_permute_mxfp8_amd/build.py "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, _lib.moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _u8(t):
    if t is None:
        return None
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def mx_scale_cols(cols: int) -> int:
    return int(load().moe_mx_scale_cols(cols))


def token_permute_out_rows(flat: int, num_out_tokens) -> int:
    return int(load().moe_token_permute_out_rows(flat, 0 if num_out_tokens is None else int(num_out_tokens)))


def mx_quantize(x: torch.Tensor, quant_mode: int = QUANT_E4M3):
    """MX-quantize the rows of a 2-D bf16/fp16/fp32 tensor: (codes uint8 [R, C] ([R, C/2] packed
    for QUANT_MXFP4), scales uint8 [R, AlignUp(C/32, 2)])."""
    lib = load()
    _need_gpu(x)
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2 if quant_mode == QUANT_MXFP4 else cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, mx_scale_cols(cols)), dtype=torch.uint8, device=x.device)
    _check(lib.moe_mx_quantize(_ptr(x), _DT[x.dtype], rows, cols, quant_mode, _ptr(codes), _ptr(scales),
                               _stream(x.device)))
    return codes, scales


def pack_weights(codes, scales, fp4: bool = False):
    """MX weights [G, N, K] codes + [G, N, K/32] scales (the pages' layout) -> the library's
    MFMA-native packed layout: (codes uint8 [G, N, K] in packed order, scales uint8 1-D).
    fp4: MXFP4 codes [G, N, K/2] (two a byte; K = 2 * the last dimension)."""
    lib = load()
    codes, scales = _u8(codes), _u8(scales)
    _need_gpu(codes, scales)
    g, n, kb = codes.shape
    k = 2 * kb if fp4 else kb
    pc = torch.empty_like(codes)
    ps = torch.empty((int(lib.moe_mx_packed_scale_bytes(g, n, k)),), dtype=torch.uint8, device=codes.device)
    fn = lib.moe_mx_pack_weights_fp4 if fp4 else lib.moe_mx_pack_weights
    _check(fn(_ptr(codes), _ptr(scales), g, n, k, _ptr(pc), _ptr(ps), _stream(codes.device)))
    return pc, ps


def init_routing_noalloc(x, expert_idx, expert_num: int, active_range=None, quant_mode: int = QUANT_NONE,
                         row_idx_type: int = 1, expert_tokens_num_type: int = 1):
    """init_routing through moe_init_routing_noalloc: the library takes no workspace (its
    scratch is a static per-GPU array of 8 MiB; larger calls raise MoeError). The outputs
    are allocated here, as for init_routing; the same results."""
    lib = load()
    _need_gpu(x, expert_idx)
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2 or expert_idx.shape[0] != x.shape[0]:
        raise ValueError("expert_idx must be int32 [N, K] with N = x.shape[0]")
    n, h = x.shape
    k = expert_idx.shape[1]
    s, e = (0, expert_num) if active_range is None else active_range
    ex, idx, tok, sc, avail = _routing_outputs(x, n, h, k, expert_num, s, e, quant_mode, expert_tokens_num_type)
    _check(lib.moe_init_routing_noalloc(_ptr(x), _DT[x.dtype], None, n, h, _ptr(expert_idx), k, expert_num, s, e,
                                        quant_mode, row_idx_type, expert_tokens_num_type, _ptr(ex), _ptr(idx),
                                        _ptr(tok), _ptr(sc), _ptr(avail), _stream(x.device)))
    return ex, idx, tok, sc, avail


def _routing_outputs(x, n, h, k, expert_num, s, e, quant_mode, expert_tokens_num_type):
    flat = n * k
    mx = quant_mode != QUANT_NONE
    dev = x.device
    ex = torch.empty((flat, h // 2 if quant_mode == QUANT_MXFP4 else h), dtype=torch.uint8 if mx else x.dtype,
                     device=dev)
    idx = torch.empty((flat,), dtype=torch.int32, device=dev)
    if expert_tokens_num_type == 2:   # key_value: (expert, count) rows
        tok = torch.empty((expert_num, 2), dtype=torch.int64, device=dev)
    else:
        tok = torch.empty((max(e - s, 0),), dtype=torch.int64, device=dev)
    sc = torch.empty((flat, mx_scale_cols(h)), dtype=torch.uint8, device=dev) if mx else None
    avail = torch.empty((1,), dtype=torch.int64, device=dev)
    return ex, idx, tok, sc, avail


def init_routing(x, expert_idx, expert_num: int, active_range=None, quant_mode: int = QUANT_NONE,
                 row_idx_type: int = 1, expert_tokens_num_type: int = 1, x_codes: int | None = None, scale=None):
    """MoeInitRoutingV3 (dropless). Returns (expanded_x, expanded_row_idx, expert_tokens,
    expanded_scale or None, available_idx_num) with expanded_x of shape [N*K, H].

    x_codes: DTYPE_FP8_E5M2 / DTYPE_FP8_E4M3 / DTYPE_FP4_E2M1 when x holds MX codes (uint8
    [N, H], or [N, H/2] for FP4, H the logical hidden size): the rows are gathered as they
    are (quant_mode -1), with their E8M0 scales [N, mx_scale_cols(H)] when scale is given."""
    lib = load()
    _need_gpu(x, expert_idx)
    if expert_idx.dtype != torch.int32 or expert_idx.dim() != 2 or expert_idx.shape[0] != x.shape[0]:
        raise ValueError(f"expert_idx must be int32 [N, K] with N = x.shape[0] (got {expert_idx.dtype} "
                         f"{tuple(expert_idx.shape)})")
    n, h = x.shape
    if x_codes is not None:
        return _init_routing_codes(lib, x, expert_idx, expert_num, active_range, row_idx_type,
                                   expert_tokens_num_type, x_codes, scale)
    k = expert_idx.shape[1]
    s, e = (0, expert_num) if active_range is None else active_range
    dev = x.device
    ex, idx, tok, sc, avail = _routing_outputs(x, n, h, k, expert_num, s, e, quant_mode, expert_tokens_num_type)
    nbytes = ctypes.c_size_t()
    _check(lib.moe_init_routing_workspace_size(n, k, expert_num, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    _check(lib.moe_init_routing(_ptr(x), _DT[x.dtype], None, n, h, _ptr(expert_idx), k, expert_num, s, e, quant_mode,
                                row_idx_type, expert_tokens_num_type, _ptr(ex), _ptr(idx), _ptr(tok), _ptr(sc),
                                _ptr(avail), _ptr(ws), ws.numel(), _stream(dev)))
    return ex, idx, tok, sc, avail


def _init_routing_codes(lib, x, expert_idx, expert_num, active_range, row_idx_type, expert_tokens_num_type,
                        x_codes, scale):
    n, row_bytes = x.shape
    h = 2 * row_bytes if x_codes == DTYPE_FP4_E2M1 else row_bytes
    k = expert_idx.shape[1]
    s, e = (0, expert_num) if active_range is None else active_range
    flat = n * k
    dev = x.device
    ex = torch.empty((flat, row_bytes), dtype=torch.uint8, device=dev)
    idx = torch.empty((flat,), dtype=torch.int32, device=dev)
    if expert_tokens_num_type == 2:
        tok = torch.empty((expert_num, 2), dtype=torch.int64, device=dev)
    else:
        tok = torch.empty((max(e - s, 0),), dtype=torch.int64, device=dev)
    sc = None
    if scale is not None:
        _need_gpu(scale)
        scale = _u8(scale)
        if tuple(scale.shape) != (n, mx_scale_cols(h)):
            raise ValueError(f"scale must be [N, {mx_scale_cols(h)}] E8M0 bytes")
        sc = torch.empty((flat, mx_scale_cols(h)), dtype=torch.uint8, device=dev)
    avail = torch.empty((1,), dtype=torch.int64, device=dev)
    nbytes = ctypes.c_size_t()
    _check(lib.moe_init_routing_workspace_size(n, k, expert_num, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    _check(lib.moe_init_routing(_ptr(_u8(x)), x_codes, _ptr(scale), n, h, _ptr(expert_idx), k, expert_num, s, e,
                                QUANT_NONE, row_idx_type, expert_tokens_num_type, _ptr(ex), _ptr(idx), _ptr(tok),
                                _ptr(sc), _ptr(avail), _ptr(ws), ws.numel(), _stream(dev)))
    return ex, idx, tok, sc, avail


def token_permute(tokens, indices, num_out_tokens=None, padded_mode: bool = False, quant_mode: int = QUANT_NONE,
                  *, num_experts: int):
    """moe_token_permute: (permuted_tokens [M, H], sorted_indices int32 [F], expanded_scale or empty).

    num_experts is the exclusive bound of the index values (the counting sort's bucket count)."""
    lib = load()
    _need_gpu(tokens, indices)
    n, h = tokens.shape
    topk = 1 if indices.dim() == 1 else indices.shape[1]
    flat = indices.numel()
    m = token_permute_out_rows(flat, num_out_tokens)
    mx = quant_mode != QUANT_NONE
    dev = tokens.device
    out = torch.empty((m, h // 2 if quant_mode == QUANT_MXFP4 else h), dtype=torch.uint8 if mx else tokens.dtype,
                      device=dev)
    srt = torch.empty((flat,), dtype=torch.int32, device=dev)
    sc = (torch.empty((m, mx_scale_cols(h)), dtype=torch.uint8, device=dev) if mx
          else torch.empty((0,), dtype=torch.float32, device=dev))
    nbytes = ctypes.c_size_t()
    _check(lib.moe_token_permute_workspace_size(flat, num_experts, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    _check(lib.moe_token_permute(_ptr(tokens), _DT[tokens.dtype], n, h, _ptr(indices), _DT[indices.dtype], topk,
                                 num_experts, 0 if num_out_tokens is None else int(num_out_tokens),
                                 int(bool(padded_mode)), quant_mode, _ptr(out), _ptr(srt),
                                 _ptr(sc) if mx else None, _ptr(ws), ws.numel(), _stream(dev)))
    return out, srt, sc


def _check_layer_dtypes(x, topk_ids, topk_weights, x_scales=None):
    """The C side reads int32 ids, fp32/bf16 gate weights and bf16 x (uint8 codes with
    x_scales): anything else would be misread, so it is rejected here."""
    if topk_ids.dtype != torch.int32:
        raise ValueError(f"topk_ids must be int32 (got {topk_ids.dtype}); convert e.g. torch.topk's int64 ids")
    if topk_weights.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"topk_weights must be float32 or bfloat16 (got {topk_weights.dtype})")
    if x_scales is None:
        if x.dtype != torch.bfloat16:
            raise ValueError(f"x must be bfloat16 (got {x.dtype})")
    elif x.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2):
        raise ValueError(f"pre-quantized x must hold FP8 codes (uint8 or float8), got {x.dtype}")
    if topk_ids.dim() != 2 or topk_ids.shape != topk_weights.shape or topk_ids.shape[0] != x.shape[0]:
        raise ValueError("topk_ids and topk_weights must both be [N, K] with N = x.shape[0]")


def _mega_struct(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales, shared, quant_out_dtype, y, etn,
                 debug, weight_format=WEIGHTS_ND, activation=ACT_SWIGLU, activation_params=(), weight_dtype=0,
                 shared_weight_dtype=0, x_scales=None, combine_comm_mode=0):
    n, h = x.shape
    k = topk_ids.shape[1]
    e, two_i, _ = w1.shape
    a = MegaArgs()
    a.x, a.num_tokens, a.hidden = _ptr(x), n, h
    a.topk_ids, a.topk = _ptr(topk_ids), k
    a.topk_weights, a.topk_weights_dtype = _ptr(topk_weights), _DT[topk_weights.dtype]
    a.num_experts, a.inter = e, two_i // 2
    a.w1, a.w1_scales, a.w2, a.w2_scales = _ptr(_u8(w1)), _ptr(_u8(w1_scales)), _ptr(_u8(w2)), _ptr(_u8(w2_scales))
    if shared is not None:
        sw1, ss1, sw2, ss2 = shared
        a.num_shared = sw1.shape[0]
        a.shared_w1, a.shared_w1_scales = _ptr(_u8(sw1)), _ptr(_u8(ss1))
        a.shared_w2, a.shared_w2_scales = _ptr(_u8(sw2)), _ptr(_u8(ss2))
    a.quant_out_dtype, a.activation, a.weight_format = quant_out_dtype, activation, weight_format
    if len(activation_params) > 3:
        raise ValueError("activation_params holds at most 3 values")
    a.num_activation_params = len(activation_params)
    a.weight_dtype, a.shared_weight_dtype = weight_dtype, shared_weight_dtype
    if x_scales is not None:   # pre-quantized pass-through: x holds FP8 codes
        a.x_is_quantized, a.x_scales = 1, _ptr(_u8(x_scales))
    a.combine_comm_mode = combine_comm_mode
    for j, v in enumerate(activation_params):
        a.activation_params[j] = float(v)
    a.y, a.expert_token_nums = _ptr(y), _ptr(etn)
    for name in ("xq", "sx", "h1", "aq", "sa", "o", "sorted_row_idx"):
        setattr(a, name, _ptr(debug.get(name)) if debug else None)
    return a


def mega_moe(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales, shared=None,
             quant_out_dtype: int = FP8_E4M3, debug: bool = False, workspace=None, stage_events=None,
             weight_format: int = WEIGHTS_ND, activation: int = ACT_SWIGLU, activation_params=(),
             weight_dtype: int = 0, shared_weight_dtype: int = 0, x_scales=None, combine_comm_mode: int = 0):
    """The MX MoE layer. Returns (y bf16 [N, H], expert_token_nums int32 [E]) and, with
    debug=True, a dict of the stage intermediates (xq, sx, h1, aq, sa, o, sorted_row_idx).

    shared: None or (shared_w1, shared_w1_scales, shared_w2, shared_w2_scales) stacked
    over the shared experts. workspace: optional preallocated uint8 device tensor.
    weight_format: WEIGHTS_ND (the pages' layout) or WEIGHTS_PACKED (w1/w2 and the
    shared weights as returned by pack_weights; the code tensors keep their [E, N, K] shape).
    stage_events: optional list of MEGA_STAGE_EVENTS torch.cuda.Event(enable_timing=True) or
    None entries, recorded by the library on the stream at the boundaries of MEGA_STAGES
    (a None entry is skipped; each record costs a few microseconds of GPU time).
    activation / activation_params: ACT_* and its parameter list as in the C header (gelu
    makes A, and w2's input width, 2 * inter).
    weight_dtype: 0 or the activations' FP8 type (FP8 weights), or FP4_E2M1 (MXFP4 codes
    two a byte, e.g. from mx_quantize(..., QUANT_MXFP4); pack_weights(..., fp4=True)).
    shared_weight_dtype: 0 = the same as weight_dtype, else one of the values above
    (e.g. FP8_E4M3 for FP8 shared experts beside MXFP4 routed experts).
    x_scales: pre-quantized pass-through: x holds FP8 codes of quant_out_dtype (uint8
    [N, H], e.g. from mx_quantize) and x_scales their E8M0 scales [N, H/32].
    combine_comm_mode: 0 (each expert output row rounded to bf16 before the weighted sum,
    MegaMoE's default) or 1 (a token's expert outputs summed in fp32, rounded once)."""
    lib = load()
    _need_gpu(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales)
    _check_layer_dtypes(x, topk_ids, topk_weights, x_scales)
    if x_scales is not None and x_scales.shape[1] != x.shape[1] // 32:
        x_scales = x_scales[:, :x.shape[1] // 32].contiguous()   # drop the AlignUp(.., 2) padding column
    n, h = x.shape
    k = topk_ids.shape[1]
    e, two_i, _ = w1.shape
    inter = two_i // 2
    aw = two_i if activation == ACT_GELU else inter   # width of A
    dev = x.device
    y = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    etn = torch.empty((e,), dtype=torch.int32, device=dev)
    dbg = None
    if debug:
        f = n * k
        dbg = dict(xq=torch.empty((f, h), dtype=torch.uint8, device=dev),
                   sx=torch.empty((f, h // 32), dtype=torch.uint8, device=dev),
                   h1=torch.empty((f, 2 * inter), dtype=torch.float32, device=dev),
                   aq=torch.empty((f, aw), dtype=torch.uint8, device=dev),
                   sa=torch.empty((f, aw // 32), dtype=torch.uint8, device=dev),
                   o=torch.empty((f, h), dtype=torch.float32, device=dev),
                   sorted_row_idx=torch.empty((f,), dtype=torch.int32, device=dev))
    a = _mega_struct(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales, shared, quant_out_dtype, y, etn, dbg,
                     weight_format, activation, activation_params, weight_dtype, shared_weight_dtype, x_scales,
                     combine_comm_mode)
    if stage_events is not None:
        if len(stage_events) != MEGA_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MEGA_STAGE_EVENTS} entries (events or None)")
        for ev in stage_events:
            if ev is not None and not ev.cuda_event:
                ev.record()   # torch creates the HIP event at its first record
        handles = (ctypes.c_void_p * MEGA_STAGE_EVENTS)(*[ev.cuda_event if ev is not None else None
                                                          for ev in stage_events])
        a.stage_events = ctypes.cast(handles, ctypes.POINTER(ctypes.c_void_p))
    nbytes = ctypes.c_size_t()
    _check(lib.mega_moe_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    ws = workspace if workspace is not None and workspace.numel() >= nbytes.value else _workspace(nbytes.value, dev)
    _check(lib.mega_moe(ctypes.byref(a), _ptr(ws), ws.numel(), _stream(dev)))
    if debug:
        return y, etn, dbg
    return y, etn


def mega_moe_workspace_bytes(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales, shared=None,
                             quant_out_dtype: int = FP8_E4M3, weight_format: int = WEIGHTS_ND,
                             activation: int = ACT_SWIGLU, activation_params=(), weight_dtype: int = 0,
                             shared_weight_dtype: int = 0, combine_comm_mode: int = 0) -> int:
    lib = load()
    _check_layer_dtypes(x, topk_ids, topk_weights)
    a = _mega_struct(x, topk_ids, topk_weights, w1, w1_scales, w2, w2_scales, shared, quant_out_dtype, x, x, None,
                     weight_format, activation, activation_params, weight_dtype, shared_weight_dtype,
                     combine_comm_mode=combine_comm_mode)
    nbytes = ctypes.c_size_t()
    _check(lib.mega_moe_workspace_size(ctypes.byref(a), ctypes.byref(nbytes)))
    return nbytes.value


def gmm1_swiglu_quant(xq, sx, group_offsets, w1, w1_scales, quant_out_dtype: int = FP8_E4M3, want_h1: bool = False,
                      weight_format: int = WEIGHTS_ND):
    """Stage 2 on given operands: (aq uint8 [rows, I], sa uint8 [rows, I/32], h1 fp32 [rows, 2I] or None)."""
    lib = load()
    xq, sx, w1, w1_scales = _u8(xq), _u8(sx), _u8(w1), _u8(w1_scales)
    _need_gpu(xq, sx, group_offsets, w1, w1_scales)
    rows, h = xq.shape
    g, two_i, _ = w1.shape
    inter = two_i // 2
    dev = xq.device
    aq = torch.empty((rows, inter), dtype=torch.uint8, device=dev)
    sa = torch.empty((rows, inter // 32), dtype=torch.uint8, device=dev)
    h1 = torch.empty((rows, two_i), dtype=torch.float32, device=dev) if want_h1 else None
    nbytes = ctypes.c_size_t()
    _check(lib.moe_gmm_workspace_size(rows, g, h, inter, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    _check(lib.moe_gmm1_swiglu_quant(_ptr(xq), _ptr(sx), rows, h, inter, _ptr(group_offsets), g, _ptr(w1),
                                     _ptr(w1_scales), weight_format, quant_out_dtype, _ptr(aq), _ptr(sa), _ptr(h1),
                                     _ptr(ws), ws.numel(), _stream(dev)))
    return aq, sa, h1


def gmm2_combine(aq, sa, group_offsets, w2, w2_scales, row_token, row_weight, y_accum,
                 quant_out_dtype: int = FP8_E4M3, want_o: bool = False, weight_format: int = WEIGHTS_ND):
    """Stages 3-4 on given operands: y_accum[row_token[r]] += row_weight[r] * O[r]; returns O (fp32) or None."""
    lib = load()
    aq, sa, w2, w2_scales = _u8(aq), _u8(sa), _u8(w2), _u8(w2_scales)
    _need_gpu(aq, sa, group_offsets, w2, w2_scales, row_token, row_weight, y_accum)
    rows, inter = aq.shape
    g, h, _ = w2.shape
    dev = aq.device
    o = torch.empty((rows, h), dtype=torch.float32, device=dev) if want_o else None
    nbytes = ctypes.c_size_t()
    _check(lib.moe_gmm_workspace_size(rows, g, h, inter, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    _check(lib.moe_gmm2_combine(_ptr(aq), _ptr(sa), rows, inter, h, _ptr(group_offsets), g, _ptr(w2),
                                _ptr(w2_scales), weight_format, quant_out_dtype, _ptr(row_token), _ptr(row_weight),
                                y_accum.shape[0], _ptr(y_accum), _ptr(o), _ptr(ws), ws.numel(), _stream(dev)))
    return o


def combine_finalize(y_accum):
    """bf16 (round to nearest even) of an fp32 accumulation buffer."""
    lib = load()
    _need_gpu(y_accum)
    n, h = y_accum.shape
    y = torch.empty((n, h), dtype=torch.bfloat16, device=y_accum.device)
    _check(lib.moe_combine_finalize(_ptr(y_accum), n, h, _ptr(y), _stream(y_accum.device)))
    return y


def probe_stream(src, dst=None, copy: bool = False, fill_caches: bool = False):
    """One launch of the library's streaming kernel: read src (uint8 device tensor, a
    multiple of 16 bytes), or copy it to dst, with non-temporal accesses; with
    fill_caches a read with plain loads (to evict other data from the caches). Returns
    None; time it with events."""
    lib = load()
    _need_gpu(src)
    if copy and (dst is None or dst.numel() < src.numel()):
        raise ValueError("probe_stream: copy needs a dst at least as large as src")
    if dst is None:
        dst = torch.empty(16, dtype=torch.uint8, device=src.device)
    mode = 1 if copy else (2 if fill_caches else 0)
    _check(lib.moe_probe_stream(mode, _ptr(src), _ptr(dst), src.numel(), _stream(src.device)))


def probe_mfma(iters: int, out=None, device="cuda"):
    """One launch of the library's MFMA loop; returns (out tensor, flops of the launch)."""
    lib = load()
    n = ctypes.c_int64()
    fl = ctypes.c_double()
    _check(lib.moe_probe_mfma(iters, None, ctypes.byref(n), ctypes.byref(fl), None))
    if out is None or out.numel() < n.value:
        out = torch.empty(n.value, dtype=torch.float32, device=device)
    _check(lib.moe_probe_mfma(iters, _ptr(out), None, None, _stream(out.device)))
    return out, fl.value
