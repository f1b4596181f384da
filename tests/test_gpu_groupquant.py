"""GPU parity of the affine group quantization of values (tq_gq_encode / tq_gq_decode).

Every step is an IEEE float32 operation on the page, so the bar is bit-exactness: packed
codes, float16 scales and zeros, and the float32 reconstruction must equal the oracle's; a
16-bit output must equal the float32 reconstruction rounded to nearest even.
"""

import numpy as np
import pytest
import torch

import tq_inputs as ti
from oracle import groupquant as ogq
from parity import log

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _inputs(n, d, dtype, seed):
    x = ti.normal((n, d), seed) * torch.exp(ti.normal((n, 1), seed + 1))
    x[0] = 1.25                                   # constant row: the scale floor
    if n > 1:
        x[1, :32] = torch.tensor([0.0, 3.0, 0.5, 1.5, 2.5] + [1.0] * 27)   # ties at 2 bits
    return x.to(dtype)


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_bit_exact(dev, d, bits, dtype):
    n = 333
    x = _inputs(n, d, dtype, d * 10 + bits)
    log("case: gq d%d b%d %s" % (d, bits, dtype))
    packed, scales, zeros = tq.gq_encode(x.to(dev), bits)
    out = tq.gq_decode(packed, scales, zeros, bits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    x32 = x.float().numpy()
    pr, sr, zr = ogq.encode(x32, bits, 32)
    assert np.array_equal(packed.cpu().numpy(), pr)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), sr.view(np.uint16))
    assert np.array_equal(zeros.cpu().numpy().view(np.uint16), zr.view(np.uint16))
    ref = ogq.decode(pr, sr, zr, bits, d, 32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    for od in (torch.bfloat16, torch.float16):
        o16 = tq.gq_decode(packed, scales, zeros, bits, out_dtype=od)
        assert torch.equal(o16.cpu(), torch.from_numpy(ref).to(od))


def test_strided_rows_and_empty(dev):
    d, bits = 128, 4
    x = _inputs(70, 2 * d, torch.bfloat16, 5).to(dev)
    view = x[:, d:]                               # row stride 2d
    packed, scales, zeros = tq.gq_encode(view, bits)
    pr, sr, zr = ogq.encode(view.float().cpu().numpy(), bits, 32)
    assert np.array_equal(packed.cpu().numpy(), pr)
    p0, s0, z0 = tq.gq_encode(torch.empty(0, d, dtype=torch.bfloat16, device=dev), bits)
    assert p0.shape == (0, 64) and s0.shape == (0, 4)


def test_error_paths(dev):
    from kv_cache_vector_encode_amd import _lib
    L = _lib.lib()
    assert L.tq_gq_encode(100, 2, None, 1, 1, 100, None, None, None, None) == -1
    assert b"d = 100" in L.tq_last_error()
    assert L.tq_gq_encode(128, 5, None, 1, 1, 128, None, None, None, None) == -1
    assert b"bits = 5" in L.tq_last_error()
