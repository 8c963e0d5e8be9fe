"""Codec kernels in isolation, both codebooks (linear-square and dynamic tree): packed
codes and scales bit-exact against the oracle on identical float32 inputs;
dequantization bit-exact."""

import numpy as np
import pytest
import torch

from oracle import codec
from tests.gpu_util import announce, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _adversarial(rng, n):
    x = rng.standard_normal(n).astype(np.float32)
    x *= (10.0 ** rng.uniform(-3, 3, n)).astype(np.float32)
    return x


CODEBOOKS = ["ls", "dt"]


def _cases(cb="ls"):
    rng = np.random.default_rng(100)
    cases = {}
    for n in (1, 3, 63, 64, 65, 127, 1000, 4096, 64 * 64, 1024 * 1024 + 7):
        cases[f"normal_{n}"] = rng.standard_normal(n).astype(np.float32)
    cases["wide_range"] = _adversarial(rng, 50_000)
    # values exactly on the decision midpoints and their neighbours, absmax 1 per block
    m32 = codec.midpoints(cb)
    mids = np.concatenate([m32, np.nextafter(m32, np.float32(2)),
                           np.nextafter(m32, np.float32(-2))]).astype(np.float32)
    blocks = np.zeros((len(mids) // 63 + 1, 64), np.float32)
    blocks[:, 0] = 1.0
    flat = blocks[:, 1:].reshape(-1)
    flat[: len(mids)] = mids
    blocks[:, 1:] = flat.reshape(blocks.shape[0], 63)
    cases["midpoints"] = blocks.ravel()
    # every power-of-two eighth step from 2^-14 to 2 (the edges of the exponent /
    # top-mantissa-bit buckets a fast code lookup may key on), their neighbours, both
    # signs, in blocks of absmax 1
    edges = np.array([2.0 ** e * (1 + k / 8) for e in range(-14, 1) for k in range(8)], np.float32)
    edges = np.concatenate([edges, np.nextafter(edges, np.float32(0)), np.nextafter(edges, np.float32(4))])
    edges = edges[np.abs(edges) <= 1]
    edges = np.concatenate([edges, -edges]).astype(np.float32)
    eb = np.zeros((len(edges) // 63 + 1, 64), np.float32)
    eb[:, 0] = 1.0
    ef = eb[:, 1:].reshape(-1)
    ef[: len(edges)] = edges
    eb[:, 1:] = ef.reshape(eb.shape[0], 63)
    cases["bucket_edges"] = eb.ravel()
    cases["dense_sweep"] = np.linspace(-1, 1, 1 << 20, dtype=np.float32)
    # codebook values times scales
    codes = rng.integers(0, 16, (200, 64))
    codes[:, 0] = 15
    s = (10.0 ** rng.uniform(-5, 5, 200)).astype(np.float32)
    cases["codebook"] = (codec.levels(cb)[codes] * s[:, None]).astype(np.float32).ravel()
    z = np.zeros(64 * 5, np.float32)
    z[64:128] = -0.0
    z[130] = 1e-42
    z[131] = -3e-41
    z[200] = 7.0
    cases["zeros_subnormals"] = z
    cases["identity_1024"] = np.eye(1024, dtype=np.float32).ravel()
    # block scales from the subnormal range to 2^120, both sides of the range in which
    # the quantizer divides through one reciprocal per block (2^-60 .. 2^60), with
    # values on and next to the decision midpoints times each scale
    exps = np.concatenate([np.arange(-149, 121, 3), [-61, -60, -59, 59, 60, 61, -126, -127]])
    sb = np.zeros((exps.size, 64), np.float32)
    for i, e in enumerate(exps):
        base = np.concatenate([rng.uniform(-1, 1, 32), m32[rng.integers(0, 15, 31)]])
        sb[i, 0] = 1.0
        sb[i, 1:] = base
        sb[i] = (sb[i].astype(np.float64) * 2.0 ** float(e)).astype(np.float32)
    cases["scale_range"] = sb.ravel()
    return cases


@pytest.mark.parametrize("cb", CODEBOOKS)
@pytest.mark.parametrize("name", list(_cases().keys()))
def test_quantize_bit_exact(name, cb):
    require_gpu()
    from bit_quantized_shampoo_amd import dequantize, quantize
    x = _cases(cb)[name]
    announce(f"codec quantize {name} codebook={cb} n={x.size}")
    c_gpu, s_gpu = quantize(to_dev(x), codebook=cb)
    torch.cuda.synchronize()
    c_ref, s_ref = codec.quantize(x, 64, cb)
    assert np.array_equal(s_gpu.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(c_gpu.cpu().numpy(), c_ref)
    announce(f"codec dequantize {name} codebook={cb}")
    y_gpu = dequantize(c_gpu, s_gpu, x.size, codebook=cb)
    torch.cuda.synchronize()
    y_ref = codec.dequantize(c_ref, s_ref, x.size, 64, cb)
    assert np.array_equal(y_gpu.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("cb", CODEBOOKS)
def test_dequantize_random_codes_bit_exact(cb):
    require_gpu()
    from bit_quantized_shampoo_amd import dequantize
    rng = np.random.default_rng(101)
    n = 64 * 777 + 13
    nqb = (n + 63) // 64
    codes = rng.integers(0, 256, nqb * 32).astype(np.uint8)
    scales = (10.0 ** rng.uniform(-30, 30, nqb)).astype(np.float32)
    announce(f"codec dequantize random codes codebook={cb} n={n}")
    y = dequantize(to_dev(codes), to_dev(scales), n, codebook=cb)
    torch.cuda.synchronize()
    ref = codec.dequantize(codes, scales, n, 64, cb)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
