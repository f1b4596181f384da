"""GPU parity of the Hadamard rotation and of the norm-corrected encode (through the C ABI).

Hadamard rotation: the library's Pi must equal the oracle's H_d diag(s) / sqrt(d) exactly,
and encode / decode / fused attention with it must meet the usual bars (tests/parity.py).
Norm correction: the codes are the plain encode's (bit for bit, same kernel), and for every
vector whose codes equal the oracle's, the stored scalar equals the oracle's n / ||c[idx]||
(oracle.codec.encode_codes_norm_corrected of the same x) within the kernel's float32 rounding:
the sum of squares as in the plain encode ((d/4 + 4) 2^-24), the sum of d code energies over
two lanes (d/2 + 2) 2^-24, a square root and a division (2^-23), so
|n'_gpu - n'_ref| <= (3d/4 + 8) 2^-24 n'_ref.
Decode and attention read caches made by the oracle's encode of the seeded inputs.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt, codebook as ocb, codec as occ, rotation as orot
import tq_inputs as ti
from parity import check_attention, check_decode, check_encode, log, oracle_encoded, to64, unpack, upload

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _signs(d, n_rot, seed):
    return ti.random_signs(n_rot, d, seed)


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
    # outlier channels: what the Hadamard rotation is for
    x = ti.normal((n, d), d + bits)
    x[:, :4] *= 10.0
    xd = x.to(torch.bfloat16).to(dev)
    what = "hadamard d%d b%d" % (d, bits)
    log("case:", what)
    packed, norms = tq.encode(cb, rot, xd)
    torch.cuda.synchronize()
    check_encode(to64(xd), packed.cpu().numpy(), norms.cpu().numpy(), pi, d, bits, what)
    pr, nr = oracle_encoded(to64(xd), pi, bits)
    out = tq.decode(cb, rot, upload(pr, dev), upload(nr, dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_decode(out, pr, nr, pi, d, bits, what)


@pytest.mark.parametrize("d,bk,bv", [(128, 4, 2), (64, 3, 3), (256, 2, 4)])
def test_attention_with_hadamard_rotations(dev, d, bk, bv):
    B, Hq, Hkv, T = 3, 8, 2, 300
    q = ti.normal((B, Hq, d), 17, dtype=torch.bfloat16, device=dev)
    k = ti.normal((B, Hkv, T, d), 18, dtype=torch.bfloat16)
    v = ti.normal((B, Hkv, T, d), 19, dtype=torch.bfloat16)
    sk, sv = _signs(d, 1, 1), _signs(d, 1, 2)
    rk, rv = tq.Rotation.hadamard(d, sk), tq.Rotation.hadamard(d, sv)
    pk, pv = orot.hadamard_rotation(d, sk[0]), orot.hadamard_rotation(d, sv[0])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kpn, knn = oracle_encoded(to64(k), pk, bk)
    vpn, vnn = oracle_encoded(to64(v), pv, bv)
    lens = torch.tensor([300, 5, 129], dtype=torch.int32, device=dev)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, upload(kpn, dev), upload(knn, dev), upload(vpn, dev), upload(vnn, dev),
                            seq_lens=lens, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    khat = oatt.decode_cache(kpn, knn, pk, ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vpn, vnn, pv, ocb.codebook(d, bv).centroids, bv, d)
    check_attention(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), khat, vhat,
                    1 / math.sqrt(d), lens.cpu().numpy(), "hadamard attention d%d K%dV%d" % (d, bk, bv))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("hadamard", [False, True])
def test_norm_corrected_encode(dev, d, bits, hadamard):
    n = 1000
    x = (ti.normal((n, d), 3 * d + bits) * torch.exp(ti.normal((n, 1), 3 * d + bits + 1))).to(dev)
    x[5] = 0.0
    if hadamard:
        s = _signs(d, 1, bits)
        rot, pi = tq.Rotation.hadamard(d, s), orot.hadamard_rotation(d, s[0])
    else:
        gg = ti.rotation_gaussian(d, 42)[None]
        rot, pi = tq.Rotation.from_gaussian(gg), orot.haar_rotation(gg[0].double().numpy())
    cb = tq.Codebook(d, bits)
    what = "norm-corrected d%d b%d %s" % (d, bits, "hadamard" if hadamard else "haar")
    log("case:", what)
    p0, n0 = tq.encode(cb, rot, x)
    p1, n1 = tq.encode(cb, rot, x, norm_correction=True)
    out = tq.decode(cb, rot, p1, n1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(p0, p1)
    x64 = to64(x)
    check_encode(x64, p0.cpu().numpy(), n0.cpu().numpy(), pi, d, bits, what)
    codes_ref, nref, _ = occ.encode_codes_norm_corrected(x64, pi, ocb.codebook(d, bits).centroids)
    same = np.all(unpack(p1.cpu().numpy(), bits, d) == codes_ref, axis=1)
    nref = nref.astype(np.float64)
    got = n1.cpu().numpy().astype(np.float64)
    bar = (0.75 * d + 8) * 2.0 ** -24
    err = np.abs(got - nref) / np.maximum(nref, 1e-300)
    assert got[5] == 0.0
    assert np.all(((err <= bar) | (nref == 0))[same]), float(np.max(err[same]))
    assert same.mean() > 0.95
    # the decode keeps the input's length (to the decode's own 2e-3 bar)
    ln = np.linalg.norm(to64(out), axis=1)
    xn = np.linalg.norm(x64, axis=1)
    ok = xn > 0
    assert np.max(np.abs(ln[ok] / xn[ok] - 1.0)) <= 2e-3
    # decode of the oracle's corrected (codes, norms), against the oracle's decode of them
    pr, nr32 = occ.pack_codes(codes_ref, bits), nref.astype(np.float32)
    out2 = tq.decode(cb, rot, upload(pr, dev), upload(nr32, dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_decode(out2, pr, nr32, pi, d, bits, what)
