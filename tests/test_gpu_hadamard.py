"""GPU parity of the Hadamard rotation and of the norm-corrected encode (through the C ABI).

Hadamard rotation: the library's Pi must equal the oracle's H_d diag(s) / sqrt(d) exactly,
and encode / decode / fused attention with it must meet the usual bars (tests/parity.py).
Norm correction: the codes are the plain encode's (bit for bit, same kernel), and the stored
scalar equals the oracle's n / ||c[idx]|| computed from the GPU's own codes, within the
kernel's float32 rounding: the sum of squares as in the plain encode ((d/4 + 4) 2^-24), the
sum of d code energies over two lanes (d/2 + 2) 2^-24, a square root and a division (2^-23),
so |n'_gpu - n'_ref| <= (3d/4 + 8) 2^-24 n'_ref.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt, codebook as ocb, codec as occ, rotation as orot
from parity import check_attention, check_decode, check_encode, log, to64

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _signs(d, n_rot, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (n_rot, d), generator=g) * 2 - 1).to(torch.int8).numpy()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_matrices_equal_the_oracle(dev, d):
    s = _signs(d, 3, d)
    rot = tq.Rotation.hadamard(d, s)
    got = rot.matrices()
    for r in range(3):
        assert np.array_equal(got[r], orot.hadamard_rotation(d, s[r]))
    plain = tq.Rotation.hadamard(d).matrices()[0]
    assert np.array_equal(plain, orot.hadamard_rotation(d))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_decode(dev, d, bits):
    n = 777
    s = _signs(d, 1, 100 + d + bits)
    rot, pi = tq.Rotation.hadamard(d, s), orot.hadamard_rotation(d, s[0])
    cb = tq.Codebook(d, bits)
    g = torch.Generator().manual_seed(d + bits)
    # outlier channels: what the Hadamard rotation is for
    x = torch.randn(n, d, generator=g)
    x[:, :4] *= 10.0
    xd = x.to(torch.bfloat16).to(dev)
    what = "hadamard d%d b%d" % (d, bits)
    log("case:", what)
    packed, norms = tq.encode(cb, rot, xd)
    out = tq.decode(cb, rot, packed, norms, out_dtype=torch.float32)
    torch.cuda.synchronize()
    pk, nm = packed.cpu().numpy(), norms.cpu().numpy()
    check_encode(to64(xd), pk, nm, pi, d, bits, what)
    check_decode(out, pk, nm, pi, d, bits, what)


@pytest.mark.parametrize("d,bk,bv", [(128, 4, 2), (64, 3, 3), (256, 2, 4)])
def test_attention_with_hadamard_rotations(dev, d, bk, bv):
    B, Hq, Hkv, T = 3, 8, 2, 300
    g = torch.Generator().manual_seed(17)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16).to(dev)
    sk, sv = _signs(d, 1, 1), _signs(d, 1, 2)
    rk, rv = tq.Rotation.hadamard(d, sk), tq.Rotation.hadamard(d, sv)
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kp, kn = tq.encode(ck, rk, k)
    vp, vn = tq.encode(cv, rv, v)
    kp, kn, vp, vn = kp.view(B, Hkv, T, -1), kn.view(B, Hkv, T), vp.view(B, Hkv, T, -1), vn.view(B, Hkv, T)
    lens = torch.tensor([300, 5, 129], dtype=torch.int32, device=dev)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, kp, kn, vp, vn, seq_lens=lens, out_dtype=torch.float32,
                            return_lse=True)
    torch.cuda.synchronize()
    pk, pv = orot.hadamard_rotation(d, sk[0]), orot.hadamard_rotation(d, sv[0])
    khat = oatt.decode_cache(kp.cpu().numpy(), kn.cpu().numpy(), pk, ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vp.cpu().numpy(), vn.cpu().numpy(), pv, ocb.codebook(d, bv).centroids, bv, d)
    check_attention(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), khat, vhat,
                    1 / math.sqrt(d), lens.cpu().numpy(), "hadamard attention d%d K%dV%d" % (d, bk, bv))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("hadamard", [False, True])
def test_norm_corrected_encode(dev, d, bits, hadamard):
    n = 1000
    g = torch.Generator().manual_seed(3 * d + bits)
    x = (torch.randn(n, d, generator=g) * torch.exp(torch.randn(n, 1, generator=g))).to(dev)
    x[5] = 0.0
    if hadamard:
        s = _signs(d, 1, bits)
        rot, pi = tq.Rotation.hadamard(d, s), orot.hadamard_rotation(d, s[0])
    else:
        gg = torch.randn(1, d, d, generator=torch.Generator().manual_seed(42))
        rot, pi = tq.Rotation.from_gaussian(gg), orot.haar_rotation(gg[0].numpy())
    cb = tq.Codebook(d, bits)
    what = "norm-corrected d%d b%d %s" % (d, bits, "hadamard" if hadamard else "haar")
    log("case:", what)
    p0, n0 = tq.encode(cb, rot, x)
    p1, n1 = tq.encode(cb, rot, x, norm_correction=True)
    out = tq.decode(cb, rot, p1, n1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(p0, p1)
    codes = occ.unpack_codes(p1.cpu().numpy(), bits, d)
    c = ocb.codebook(d, bits).centroids
    x64 = to64(x)
    nref = np.linalg.norm(x64, axis=1) / np.linalg.norm(c[codes.astype(np.int64)], axis=1)
    got = n1.cpu().numpy().astype(np.float64)
    bar = (0.75 * d + 8) * 2.0 ** -24
    err = np.abs(got - nref) / np.maximum(nref, 1e-300)
    assert got[5] == 0.0
    assert np.all((err <= bar) | (nref == 0)), float(np.max(err))
    # the decode keeps the input's length (to the decode's own 2e-3 bar)
    ln = np.linalg.norm(to64(out), axis=1)
    xn = np.linalg.norm(x64, axis=1)
    ok = xn > 0
    assert np.max(np.abs(ln[ok] / xn[ok] - 1.0)) <= 2e-3
    check_decode(out, p1.cpu().numpy(), n1.cpu().numpy(), pi, d, bits, what)
