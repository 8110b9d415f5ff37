"""Helpers for the GPU parity tests: device inputs and weight preparation.

Weights of small workloads are quantized by the oracle on the CPU and uploaded
(they are oracle outputs fed to the GPU). Weights of the full-size workloads are
generated on the GPU (torch's seeded generator) and quantized by the library,
exactly as the benchmark does; a test then regenerates the masters of the experts
it samples, quantizes them with the oracle, checks the library's bytes against
them and computes its expected values from the oracle's own bytes.
"""
import sys

import numpy as np
import torch

import moe_inputs
import routing_permute_mxfp8_amd as rp
from oracle import moe, mxfp

DEV = "cuda"
QMODE = {"e4m3": rp.QUANT_E4M3, "e5m2": rp.QUANT_E5M2, "e2m1": rp.QUANT_MXFP4}
FP8 = {"e4m3": rp.FP8_E4M3, "e5m2": rp.FP8_E5M2}


def say(msg):
    conftest = sys.modules.get("conftest")
    if conftest is not None and hasattr(conftest, "progress"):
        conftest.progress(msg)
    else:
        print(msg, flush=True)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def oracle_weights(cfg, n_experts=None, shared=False, gelu=False):
    """Oracle-quantized weights (numpy): w1q [E,2I,H], w1s [E,2I,H/32], w2q [E,H,I], w2s [E,H,I/32]
    (w2 [E,H,2I] for a gelu layer)."""
    n_experts = cfg.experts if n_experts is None else n_experts
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    if gelu:
        t2 += "g"
    out = [[], [], [], []]
    for e in range(n_experts):
        q1, s1 = mxfp.quantize(moe_inputs.weight_master(cfg, t1, e).double().numpy(), cfg.fmt)
        q2, s2 = mxfp.quantize(moe_inputs.weight_master(cfg, t2, e).double().numpy(), cfg.fmt)
        for lst, v in zip(out, (q1, s1, q2, s2)):
            lst.append(v)
    return tuple(np.stack(v) for v in out)


def library_weights(cfg, n_experts=None, shared=False, fp4=False):
    """Weights generated on the GPU and quantized by the library (the benchmark's recipe);
    MXFP4 codes two a byte with fp4."""
    n_experts = cfg.experts if n_experts is None else n_experts
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    h, i = cfg.hidden, cfg.inter
    cb = 2 if fp4 else 1
    q = rp.QUANT_MXFP4 if fp4 else QMODE[cfg.fmt]
    w1q = torch.empty((n_experts, 2 * i, h // cb), dtype=torch.uint8, device=DEV)
    w1s = torch.empty((n_experts, 2 * i, h // 32), dtype=torch.uint8, device=DEV)
    w2q = torch.empty((n_experts, h, i // cb), dtype=torch.uint8, device=DEV)
    w2s = torch.empty((n_experts, h, i // 32), dtype=torch.uint8, device=DEV)
    for e in range(n_experts):
        c, s = rp.mx_quantize(moe_inputs.weight_master(cfg, t1, e, device=DEV), q)
        w1q[e].copy_(c); w1s[e].copy_(s)
        c, s = rp.mx_quantize(moe_inputs.weight_master(cfg, t2, e, device=DEV), q)
        w2q[e].copy_(c); w2s[e].copy_(s)
    return w1q, w1s, w2q, w2s


def oracle_expert_from_gpu_masters(cfg, e, shared=False):
    """Oracle quantization of expert e's masters regenerated on the GPU (same seed)."""
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    m1 = moe_inputs.weight_master(cfg, t1, e, device=DEV).cpu().double().numpy()
    m2 = moe_inputs.weight_master(cfg, t2, e, device=DEV).cpu().double().numpy()
    q1, s1 = mxfp.quantize(m1, cfg.fmt)
    q2, s2 = mxfp.quantize(m2, cfg.fmt)
    return q1, s1, q2, s2


def normwise_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def y_errors(got, ref):
    """(max|dY| / max|Y_ref|, sum|dY| / sum|Y_ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-300)), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def abs_gmm(aq, sa, wq, ws, fmt):
    """sum_k |DQ(a)_k| |DQ(w)_k| for every output: the scale of the fp32 summation error."""
    a = np.abs(mxfp.dequantize(aq, sa, fmt))
    w = np.abs(mxfp.dequantize(wq, ws, fmt))
    return a @ w.T


def gemm_gamma(k_len):
    """Error factor of the GPU GEMMs: |dh| <= gamma * sum|a||b|. One scaled f8f6f4 MFMA
    (K = 128) was measured on gfx950 at up to 2^-12 of the sum of its product
    magnitudes, unbiased; 2^-11 allows twice that, plus fp32 adds across K steps."""
    return 2.0 ** -11 + (k_len / 128.0 + 2.0) * 2.0 ** -24


def check_gemm_elementwise(got, ref, abs_sum, k_len):
    bound = gemm_gamma(k_len) * abs_sum + 1e-30
    excess = np.abs(np.asarray(got, np.float64) - ref) / bound
    assert np.all(excess <= 1.0), float(excess.max())
    return float(excess.max())


def swiglu_delta(h1_ref, abs_h1, k_len, inter):
    """Bound on |A_gpu - A_ref| from the accumulation bounds of G and U (SiLU' <= 1.1)
    plus a few fp32 roundings in the activation itself."""
    g, u = h1_ref[:, :inter], h1_ref[:, inter:]
    gam = gemm_gamma(k_len)
    dg, du = gam * abs_h1[:, :inter], gam * abs_h1[:, inter:]
    silu = g / (1.0 + np.exp(-g))
    a = silu * u
    return 1.1 * dg * (np.abs(u) + du) + np.abs(silu) * du + np.abs(a) * 2.0 ** -20 + 1e-30


def act_delta(h1_ref, abs_h1, k_len, kind, params):
    """Bound on |A_gpu - A_ref| for any activation: the largest change of A over the box
    G +- dG, U +- dU (Z +- dZ for gelu) of GEMM errors, probed at its corners and centre
    lines, with a 25% margin, plus a few fp32 roundings in the activation itself."""
    gam = gemm_gamma(k_len)
    d = gam * np.asarray(abs_h1)
    a_ref = moe.activate(h1_ref, kind, params)
    if kind == "gelu":
        probes = [moe.activate(h1_ref + sz * d, kind, params) for sz in (-1.0, -0.5, 0.5, 1.0)]
    else:
        inter = h1_ref.shape[1] // 2
        probes = []
        for sg in (-1.0, 0.0, 1.0):
            for su in (-1.0, 0.0, 1.0):
                sh = np.concatenate([sg * d[:, :inter], su * d[:, inter:]], axis=1)
                probes.append(moe.activate(h1_ref + sh, kind, params))
    dev = np.max([np.abs(p - a_ref) for p in probes], axis=0)
    return 1.25 * dev + np.abs(a_ref) * 2.0 ** -18 + 1e-30


def check_requant(aq_gpu, sa_gpu, a_ref, delta, fmt, max_code_diff=0.02, max_scale_diff=0.01):
    """Requantized activations against the oracle's A (which the GPU reproduces only up to
    delta, its GEMM error): every GPU scale / code must be a valid MX quantization of a
    value within delta of A, and the share of codes differing from the oracle's must be small.

    Valid quantization, per element with the GPU's scale X: |DQ - A| <= half an FP8 ulp of
    |A| / X (relative 2^-(m+1), or half the subnormal quantum) + saturation above max*X
    + delta; the GPU scale must lie between the scales of the group amax -/+ delta."""
    a_ref = np.asarray(a_ref, np.float64)
    rows, cols = a_ref.shape
    ng = cols // 32
    mbits, esub = {"e4m3": (3, -9), "e5m2": (2, -16)}[fmt]
    top = mxfp.max_finite(fmt)
    sa_g = np.asarray(sa_gpu)[:, :ng].astype(np.int64)
    aq_g = np.asarray(aq_gpu)
    g_abs = np.abs(a_ref).reshape(rows, ng, 32)
    g_del = np.asarray(delta).reshape(rows, ng, 32)

    def scale_of(amax):
        _, e = np.frexp(np.where(amax > 0, amax, 1.0))
        b = np.clip(e.astype(np.int64) - 1 - mxfp.EMAX[fmt] + 127, 0, 254)
        return np.where(amax > 0, b, 0)

    lo_s = scale_of(np.maximum(g_abs - g_del, 0).max(axis=2))
    hi_s = scale_of((g_abs + g_del).max(axis=2))
    assert np.all((sa_g >= lo_s) & (sa_g <= hi_s)), "scale outside the valid range"
    x = mxfp.e8m0_value(np.repeat(sa_g, 32, axis=1))
    dq = mxfp.dequantize(aq_g, sa_g.astype(np.uint8), fmt)
    absa = np.abs(a_ref)
    tol = (2.0 ** -(mbits + 1)) * absa + 2.0 ** (esub - 1) * x + np.maximum(absa - top * x, 0) + delta
    assert np.all(np.abs(dq - a_ref) <= tol * (1 + 1e-12)), "code outside the valid range"
    aq_o, sa_o = mxfp.quantize(a_ref, fmt)
    code_diff = float(np.mean(aq_g != aq_o))
    scale_diff = float(np.mean(sa_g != sa_o[:, :ng]))
    assert code_diff <= max_code_diff, code_diff
    assert scale_diff <= max_scale_diff, scale_diff
    return code_diff, scale_diff


def oracle_experts_parallel(cfg, experts, shared=False, workers=8, fp4=False):
    """oracle_expert_from_gpu_masters for several experts: masters regenerated on the GPU
    one batch of `workers` experts at a time (so that only one batch of float masters is
    held), the oracle quantizations of a batch run in a thread pool (MXFP4, codes packed
    two a byte, with fp4)."""
    from concurrent.futures import ThreadPoolExecutor
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    experts = list(experts)
    out = {}

    def work(item):
        e, (m1, m2) = item
        q1, s1 = mxfp.quantize(m1.double().numpy(), "e2m1" if fp4 else cfg.fmt)
        q2, s2 = mxfp.quantize(m2.double().numpy(), "e2m1" if fp4 else cfg.fmt)
        if fp4:
            q1, q2 = mxfp.pack_fp4(q1), mxfp.pack_fp4(q2)
        return e, (q1, s1, q2, s2)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        for b in range(0, len(experts), workers):
            masters = [(e, (moe_inputs.weight_master(cfg, t1, e, device=DEV).cpu(),
                            moe_inputs.weight_master(cfg, t2, e, device=DEV).cpu()))
                       for e in experts[b:b + workers]]
            out.update(ex.map(work, masters))
            if len(experts) > 4 * workers and (b // workers) % 4 == 3:
                say(f"  oracle weights: {len(out)} of {len(experts)} experts")
    return out
