"""MX quantization on the GPU against the oracle, bit for bit: every finite bf16 value,
both FP8 formats and MXFP4 (E2M1), in two arrangements (random groups; groups of neighbouring
magnitudes, which sweeps every scale byte, saturation, subnormal elements and
subnormal amax). Plus fp16 / fp32 inputs and a ragged row count."""
import numpy as np
import pytest
import torch

import routing_permute_mxfp8_amd as rp
from oracle import mxfp
from gpu_support import DEV, QMODE, say

pytestmark = pytest.mark.gpu


def finite_bf16_bits():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return bits[np.isfinite(v)].astype(np.uint16)


def run(bits_2d, fmt):
    x = torch.from_numpy(bits_2d.astype(np.int16)).view(torch.bfloat16).to(DEV)
    codes, scales = rp.mx_quantize(x, QMODE[fmt])
    torch.cuda.synchronize()
    vals = mxfp.bf16_from_bits(bits_2d)
    oc, os_ = mxfp.quantize(vals, fmt)
    if fmt == "e2m1":   # MXFP4: two codes a byte, element 2j in the low nibble
        oc = mxfp.pack_fp4(oc)
    return codes.cpu().numpy(), scales.cpu().numpy(), oc, os_


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
@pytest.mark.parametrize("arrangement", ["random", "sorted"])
def test_all_bf16_values(fmt, arrangement):
    say(f"mx_quantize all bf16 fmt={fmt} arrangement={arrangement}")
    bits = finite_bf16_bits()
    rng = np.random.default_rng(0)
    if arrangement == "random":
        bits = rng.permutation(bits)
    else:
        mag = np.abs(mxfp.bf16_from_bits(bits))
        bits = bits[np.argsort(mag, kind="stable")]
    pad = (-bits.size) % 256
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(-1, 256)
    gc, gs, oc, os_ = run(bits, fmt)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_other_input_dtypes(dtype):
    say(f"mx_quantize dtype={dtype}")
    rng = np.random.default_rng(1)
    a = (rng.standard_normal((37, 96)) * np.exp(rng.uniform(-6, 6, (37, 1)))).astype(np.float32)
    x = torch.from_numpy(a).to(dtype)
    vals = x.double().numpy()
    codes, scales = rp.mx_quantize(x.to(DEV), rp.QUANT_E4M3)
    oc, os_ = mxfp.quantize(vals, "e4m3")
    assert scales.shape == (37, 4)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


@pytest.mark.gpu
def test_bandwidth_probes():
    """The roofline probes: the non-temporal copy copies every byte (a buffer whose size is
    not a multiple of the kernel's 4 KB step per thread group), the reads (non-temporal and
    cache-filling) and the MFMA loop run and report positive work."""
    n = (64 << 20) + 16 * 37
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n + 64, dtype=torch.uint8, device=DEV)
    rp.probe_stream(src, dst, copy=True)
    rp.probe_stream(src)
    rp.probe_stream(src, fill_caches=True)
    out, flops = rp.probe_mfma(10)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert int(dst[n:].count_nonzero()) == 0
    assert flops > 0 and out.numel() > 0
