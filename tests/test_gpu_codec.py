"""GPU parity of tq_encode / tq_decode against the float64 oracle (through the C ABI).

Encode: the GPU and the oracle encode the same seeded x. Decode: the GPU decodes the oracle's
own encode of x (or, at full size, tq_inputs' random code bytes and norms) and the oracle
decodes the same bytes; no GPU output is an oracle input."""

import ctypes as C

import numpy as np
import pytest
import torch

import tq_inputs as ti
from parity import check_decode, check_encode, log, oracle_encoded, rotation_pair, to64, unpack, upload

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")
from kv_cache_vector_encode_amd import _lib  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run(x_dev, d, bits, seed=42, out_dtype=None, what=""):
    rot, pis = rotation_pair(d, [seed])
    cb = tq.Codebook(d, bits)
    log("case:", what, "shape", tuple(x_dev.shape), x_dev.dtype, "bits", bits)
    packed, norms = tq.encode(cb, rot, x_dev)
    torch.cuda.synchronize()
    x64 = to64(x_dev.reshape(-1, d))
    flips = check_encode(x64, packed.cpu().numpy(), norms.cpu().numpy(), pis[0], d, bits, what)
    pr, nr = oracle_encoded(x64, pis[0], bits)
    out = tq.decode(cb, rot, upload(pr, x_dev.device), upload(nr, x_dev.device), out_dtype=out_dtype or x_dev.dtype)
    torch.cuda.synchronize()
    check_decode(out, pr, nr, pis[0], d, bits, what)
    return packed, norms, out, flips


def test_codec_check_workload(dev):
    """4096 float32 N(0,1) vectors from seed 0, d=128, 4 bits, rotation seed 42."""
    x = ti.codec_check_inputs()
    _, _, out, flips = _run(x.to(dev), 128, 4, out_dtype=torch.float32, what="codec-check")
    xh = to64(out)
    rel = np.linalg.norm(xh - x.numpy()) / np.linalg.norm(x.numpy())
    log("relative reconstruction error %.4f, flips %d" % (rel, flips))
    assert round(rel, 2) == 0.10


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_shapes_and_dtypes(dev, d, bits, dtype):
    n = 1000   # 31 full 32-vector tiles and a ragged tail of 8
    x = ti.normal((n, d), d * 10 + bits) * torch.exp(ti.normal((n, 1), d * 10 + bits + 1))
    _run(x.to(dtype).to(dev), d, bits, seed=7 + d, what="d%d b%d %s" % (d, bits, dtype))


def test_identity_rotation_is_scalar_quantization(dev):
    d, bits = 128, 3
    rot = tq.Rotation.from_matrix(np.eye(d))
    cb = tq.Codebook(d, bits)
    x = ti.codec_check_inputs(777, d, seed=5)
    packed, norms = tq.encode(cb, rot, x.to(dev))
    check_encode(x.numpy().astype(np.float64), packed.cpu().numpy(), norms.cpu().numpy(), np.eye(d), d, bits,
                 "identity rotation")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_extreme_coordinates(dev, d):
    """y = +-1 in one coordinate, the two ends of the encode's quantization table, and 0 in the
    others: signed basis vectors under the identity rotation, and signed rows of a Haar rotation
    (y = Pi x = +-e_i up to rounding), float32 inputs, every width."""
    eye = np.eye(d)
    rot_id = tq.Rotation.from_matrix(eye)
    rot, pis = rotation_pair(d, [d + 3])
    cases = [(rot_id, eye, np.concatenate([eye, -eye]) * 3.0, "basis"),
             (rot, pis[0], np.concatenate([pis[0], -pis[0]]) * 0.5, "rows")]
    for bits in (2, 3, 4):
        cb = tq.Codebook(d, bits)
        for r, pi, x, what in cases:
            xd = torch.from_numpy(x).float().to(dev)
            log("case: extreme coordinates", what, "d", d, "bits", bits)
            packed, norms = tq.encode(cb, r, xd)
            torch.cuda.synchronize()
            check_encode(to64(xd), packed.cpu().numpy(), norms.cpu().numpy(), pi, d, bits,
                         "extreme %s d%d b%d" % (what, d, bits))
            codes = unpack(packed.cpu().numpy(), bits, d)
            top = np.abs(x @ pi.T).argmax(axis=1)
            hit = codes[np.arange(2 * d), top]
            assert np.all(hit[:d] == 2 ** bits - 1) and np.all(hit[d:] == 0)


def test_zero_and_small_vectors(dev):
    d = 128
    x = torch.zeros(64, d)
    x[32:] = ti.codec_check_inputs(32, d, seed=11) * 1e-10
    for bits in (2, 3, 4):
        packed, norms, out, _ = _run(x.to(dev), d, bits, out_dtype=torch.float32, what="zero/small b%d" % bits)
        codes = unpack(packed[:32].cpu().numpy(), bits, d)
        assert np.all(codes == 2 ** (bits - 1) - 1)
        assert torch.all(norms[:32] == 0) and torch.all(out[:32] == 0)


def test_strided_rows(dev):
    d, bits = 128, 4
    big = ti.codec_check_inputs(600, d + 64, seed=3).to(torch.bfloat16).to(dev)
    view = big[:, :d]
    rot, pis = rotation_pair(d, [42])
    cb = tq.Codebook(d, bits)
    p1, n1 = tq.encode(cb, rot, view)
    p2, n2 = tq.encode(cb, rot, view.contiguous())
    assert torch.equal(p1, p2) and torch.equal(n1, n2)


def test_slot_mapping_scatter_and_gather(dev):
    d, bits, n = 128, 3, 500
    rot, pis = rotation_pair(d, [42])
    cb = tq.Codebook(d, bits)
    x = ti.codec_check_inputs(n, d, seed=21).to(torch.bfloat16).to(dev)
    slots = torch.randperm(800, generator=ti.generator("cpu", 4))[:n]
    slots[::7] = -1                                     # skipped vectors
    slots_d = slots.to(dev)
    row = tq.packed_row_bytes(d, bits)
    packed = torch.full((800, row), 0xAB, dtype=torch.uint8, device=dev)
    norms = torch.full((800,), -1.0, device=dev)
    tq.encode(cb, rot, x, packed=packed, norms=norms, slot_mapping=slots_d, num_slots=800)
    dense_p, dense_n = tq.encode(cb, rot, x)
    keep = slots >= 0
    assert torch.equal(packed[slots_d[keep.to(dev)]].cpu(), dense_p[keep.to(dev)].cpu())
    assert torch.equal(norms[slots_d[keep.to(dev)]].cpu(), dense_n[keep.to(dev)].cpu())
    untouched = torch.ones(800, dtype=torch.bool)
    untouched[slots[keep]] = False
    assert torch.all(packed[untouched.to(dev)] == 0xAB) and torch.all(norms[untouched.to(dev)] == -1.0)
    # gather decode: negative slots give zeros
    out = tq.decode(cb, rot, packed, norms, slot_mapping=slots_d, out_dtype=torch.float32)
    ref = tq.decode(cb, rot, dense_p, dense_n, out_dtype=torch.float32)
    assert torch.equal(out[keep.to(dev)], ref[keep.to(dev)])
    assert torch.all(out[~keep.to(dev)] == 0)


def test_rotation_stack(dev):
    d, bits, vpr, n = 128, 4, 700, 1900               # 3 rotations, ragged segment ends
    rot, pis = rotation_pair(d, [42, 49, 56])
    cb = tq.Codebook(d, bits)
    x = ti.codec_check_inputs(n, d, seed=8).to(torch.bfloat16).to(dev)
    packed, norms = tq.encode(cb, rot, x, vectors_per_rot=vpr)
    x64 = to64(x)
    enc = [oracle_encoded(x64[r * vpr:(r + 1) * vpr], pis[r], bits) for r in range(3)]
    pr, nr = np.concatenate([e[0] for e in enc]), np.concatenate([e[1] for e in enc])
    out = tq.decode(cb, rot, upload(pr, dev), upload(nr, dev), vectors_per_rot=vpr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for r in range(3):
        sl = slice(r * vpr, min(n, (r + 1) * vpr))
        check_encode(x64[sl], packed[sl].cpu().numpy(), norms[sl].cpu().numpy(), pis[r], d, bits, "stack r%d" % r)
        check_decode(out[sl], pr[sl], nr[sl], pis[r], d, bits, "stack r%d" % r)


def test_deterministic(dev):
    d, bits = 256, 3
    rot, _ = rotation_pair(d, [1])
    cb = tq.Codebook(d, bits)
    x = ti.codec_check_inputs(3000, d, seed=1).to(torch.bfloat16).to(dev)
    a = tq.encode(cb, rot, x)
    b = tq.encode(cb, rot, x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(tq.decode(cb, rot, *a), tq.decode(cb, rot, *b))


def test_power_of_two_scale_invariance(dev):
    d, bits = 128, 3
    rot, pis = rotation_pair(d, [42])
    cb = tq.Codebook(d, bits)
    x = ti.codec_check_inputs(2048, d, seed=13).to(torch.bfloat16).to(dev)
    p1, n1 = tq.encode(cb, rot, x)
    p2, n2 = tq.encode(cb, rot, x * 64)
    assert torch.equal(n2, n1 * 64)
    c1 = unpack(p1.cpu().numpy(), bits, d)
    c2 = unpack(p2.cpu().numpy(), bits, d)
    assert np.mean(c1 != c2) < 1e-5


def test_error_paths_on_device(dev):
    L = _lib.lib()
    d, bits = 128, 4
    rot, _ = rotation_pair(d, [42])
    cb = tq.Codebook(d, bits)
    cb64 = tq.Codebook(64, bits)
    x = torch.zeros(64, d, dtype=torch.bfloat16, device=dev)
    pk = torch.zeros(64, 64, dtype=torch.uint8, device=dev)
    nm = torch.zeros(64, device=dev)
    vp = C.c_void_p
    args = lambda xp, stride, n=64, vpr=0, c=cb: (c.handle, rot.handle, vpr, vp(xp), 1, n, stride, vp(pk.data_ptr()),
                                                  vp(nm.data_ptr()), None, None)
    assert L.tq_encode(*args(x.data_ptr() + 2, d)) == -3
    assert L.tq_encode(*args(x.data_ptr(), d + 1)) == -3
    assert L.tq_encode(*args(x.data_ptr(), d - 8)) == -1
    assert L.tq_encode(*args(x.data_ptr(), d, vpr=10)) == -1        # needs 7 rotations, has 1
    assert "rotations" in _lib.last_error()
    assert L.tq_encode(*args(x.data_ptr(), d, c=cb64)) == -1
    assert "does not match" in _lib.last_error()
    assert L.tq_encode(*args(x.data_ptr(), d, n=0)) == 0             # no-op
    assert L.tq_decode(cb.handle, rot.handle, 0, vp(pk.data_ptr()), vp(nm.data_ptr()), None, 64,
                       vp(x.data_ptr() + 8), 1, None) == -3


def _sample_rows(n_total, k, seed):
    return torch.randperm(n_total, generator=ti.generator("cpu", seed))[:k].sort().values


def test_llama_shaped_cache_full(dev):
    """32 layers x 8 KV heads x 8192 tokens x d=128 bf16, K4/V2, one launch per tensor over
    the 32-rotation stack (one shared rotation per layer); sampled oracle parity. The decode
    runs at the same size on random code bytes and norms (every code value occurs)."""
    shape = ti.LlamaCacheShape()
    L_, H, T, d = shape.layers, shape.kv_heads, shape.tokens, shape.head_dim
    K = torch.empty(L_, H, T, d, dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for l in range(L_):
        ti.llama_layer_kv(shape, l, device=dev, out_k=K[l], out_v=V[l])
    rot, pis = rotation_pair(d, [ti.key_seed(l) for l in range(L_)])
    ck, cv = tq.Codebook(d, 4), tq.Codebook(d, 2)
    vpr = H * T
    log("case: llama-shaped cache, encode K4 and V2 over 32 layers")
    kp, kn = tq.encode(ck, rot, K, vectors_per_rot=vpr)
    vp, vn = tq.encode(cv, rot, V, vectors_per_rot=vpr)
    N_ = L_ * vpr
    rkp, rvp = ti.random_bytes((N_, d * 4 // 8), 61, dev), ti.random_bytes((N_, d * 2 // 8), 62, dev)
    rkn, rvn = ti.random_norms((N_,), 63, device=dev), ti.random_norms((N_,), 64, device=dev)
    ko = tq.decode(ck, rot, rkp, rkn, vectors_per_rot=vpr)
    vo = tq.decode(cv, rot, rvp, rvn, vectors_per_rot=vpr)
    torch.cuda.synchronize()
    rows = _sample_rows(N_, 4096, 0)
    layer = (rows // vpr).numpy()
    Kf, Vf = K.view(-1, d), V.view(-1, d)
    for l in np.unique(layer)[:8]:
        sel = rows[layer == l].to(dev)
        for name, X, P, N, RP, RN, O, bits in (("K", Kf, kp, kn, rkp, rkn, ko, 4), ("V", Vf, vp, vn, rvp, rvn, vo, 2)):
            check_encode(to64(X[sel]), P[sel].cpu().numpy(), N[sel].cpu().numpy(), pis[l], d, bits,
                         "llama %s layer %d" % (name, l))
            check_decode(O[sel], RP[sel].cpu().numpy(), RN[sel].cpu().numpy(), pis[l], d, bits,
                         "llama %s layer %d" % (name, l))


@pytest.mark.parametrize("layer", [0, 79])
def test_long_cache_layer_full(dev, layer):
    """One layer of the 70B-class 128K-context cache: 8 x 131072 x 128 bf16, 3-bit K and V."""
    shape = ti.LongCacheShape()
    d = shape.head_dim
    K, V = ti.long_cache_layer_kv(shape, layer, device=dev)
    rk, pk = rotation_pair(d, [ti.key_seed(layer)])
    rv, pv = rotation_pair(d, [ti.value_seed(layer)])
    cb = tq.Codebook(d, 3)
    log("case: long cache layer %d" % layer)
    kp, kn = tq.encode(cb, rk, K)
    vp, vn = tq.encode(cb, rv, V)
    n = K.numel() // d
    rkp, rkn = ti.random_bytes((n, d * 3 // 8), 70 + layer, dev), ti.random_norms((n,), 71 + layer, device=dev)
    ko = tq.decode(cb, rk, rkp, rkn)
    torch.cuda.synchronize()
    rows = _sample_rows(n, 4096, layer).to(dev)
    Kf, Vf = K.view(-1, d), V.view(-1, d)
    check_encode(to64(Kf[rows]), kp[rows].cpu().numpy(), kn[rows].cpu().numpy(), pk[0], d, 3, "long K l%d" % layer)
    check_encode(to64(Vf[rows]), vp[rows].cpu().numpy(), vn[rows].cpu().numpy(), pv[0], d, 3, "long V l%d" % layer)
    check_decode(ko[rows], rkp[rows].cpu().numpy(), rkn[rows].cpu().numpy(), pk[0], d, 3, "long K l%d" % layer)


def test_gpu_codes_reach_the_distortion_integral(dev):
    """Statistical pin on the GPU's own codes: rotated-domain squared error = D_b(d)."""
    import math
    from oracle import codebook as ocb, codec as occ
    d = 128
    x = ti.codec_check_inputs()
    for bits in (2, 3, 4):
        rot, pis = rotation_pair(d, [42])
        cb = tq.Codebook(d, bits)
        packed, _ = tq.encode(cb, rot, x.to(dev))
        codes = unpack(packed.cpu().numpy(), bits, d).astype(np.int64)
        _, _, y = occ.encode_codes(x.numpy(), pis[0], ocb.codebook(d, bits).centroids)
        err = ((y - ocb.codebook(d, bits).centroids[codes]) ** 2).mean(axis=1)
        se = err.std(ddof=1) / math.sqrt(err.size)
        assert abs(err.mean() - ocb.codebook(d, bits).mse) <= 5 * se
