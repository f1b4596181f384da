"""GPU parity of the QJL residual stage (tq_qjl_encode, QJL scores and decode attention).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantCompressorV2 (compress and
asymmetric_attention_scores). Inputs are seeded and synthetic; the oracle never sees a GPU
output:
  * encode: the same x goes to tq_qjl_encode and to oracle.qjl.encode. Codes and norms follow
    the codec bars (bit-exact outside the 1e-5 window). For vectors whose codes all match, the
    signs are bit-exact except where the oracle's float64 projection lies within
    SIGN_WINDOW * ||S_i|| * ||x|| of zero (counted), and ||r|| agrees to 1e-5 * ||x||;
  * scores / attention: the compressed cache is uniform random bytes (codes and signs) with
    log-normal norms (tq_inputs), given to both sides. Score bar per entry:
    2e-3 * scale * (n_t ||q|| ||c[idx_t]|| + ||r_t|| sqrt(pi/2)/d ||S q||_1); attention bar as
    for plain keys (2e-3 * sum_t p_t ||v_hat_t||).
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_vector_encode_amd as tq
import tq_inputs as ti
from oracle import attention as oatt, codebook as ocb, codec as occ, qjl as oqjl
from parity import REL, WINDOW, check_attention, log, rotation_pair, to64

pytestmark = pytest.mark.gpu

SIGN_WINDOW = 1e-4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _sketches(d, seeds):
    return torch.stack([ti.qjl_sketch_gaussian(d, s) for s in seeds])


def _check_qjl_encode(x64, packed, norms, signs, rnorms, pi, S64, d, mbits, what):
    cb = ocb.codebook(d, mbits)
    codes_ref, n_ref, signs_ref, rn_ref, y, proj = oqjl.encode(x64, pi, S64, cb.centroids)
    codes = occ.unpack_codes(packed, mbits, d)
    delta = occ.boundary_distance(y, cb.thresholds)
    cdiff = codes != codes_ref
    assert not (cdiff & (delta >= WINDOW)).any(), "%s: codes differ outside the window" % what
    nr = np.sqrt(np.sum(x64 * x64, axis=1))
    assert np.all(np.abs(norms.astype(np.float64) - nr) <= (d / 4 + 4) * 2.0 ** -24 * nr), what
    clean = ~cdiff.any(axis=1)
    sg = oqjl.unpack_signs(signs, d)
    srow = np.linalg.norm(S64, axis=1)                     # ||S_i||
    near = np.abs(proj) <= SIGN_WINDOW * srow[None, :] * nr[:, None]
    sdiff = (sg != signs_ref) & clean[:, None]
    bad = sdiff & ~near
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d signs differ outside the window (vector %d row %d: proj %.3g, "
                             "||S_i|| ||x|| %.3g)" % (what, int(bad.sum()), i, j, proj[i, j], srow[j] * nr[i]))
    rerr = np.abs(rnorms.astype(np.float64) - rn_ref.astype(np.float64))[clean]
    assert np.all(rerr <= 1e-5 * nr[clean] + 1e-30), "%s: residual norm error %.3g" % (
        what, float(np.max(rerr / np.maximum(nr[clean], 1e-300))))
    log("%s: %d vectors, %d code flips, %d sign flips (%d projections in the window), %d vectors "
        "skipped for a code flip" % (what, x64.shape[0], int(cdiff.sum()), int(sdiff.sum()), int(near.sum()),
                                     int((~clean).sum())))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mbits", [1, 2, 3, 4])
def test_qjl_encode(dev, d, mbits):
    n = 777                                    # several 32-vector tiles and a ragged tail
    log("case: qjl encode d%d mse bits %d" % (d, mbits))
    x = ti.codec_check_inputs(n=n, d=d, seed=d + mbits).to(dev, torch.bfloat16)
    rot, pis = rotation_pair(d, [42])
    S = _sketches(d, [42])
    sk = tq.QJLSketch(rot, S)
    cb = tq.Codebook(d, mbits)
    pk, nm, sg, rn = tq.qjl_encode(cb, sk, x)
    torch.cuda.synchronize()
    _check_qjl_encode(to64(x), pk.cpu().numpy(), nm.cpu().numpy(), sg.cpu().numpy(), rn.cpu().numpy(), pis[0],
                      S[0].double().numpy(), d, mbits, "qjl d%d b%d" % (d, mbits))


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_qjl_encode_dtypes_stack_and_slots(dev, dtype, d):
    # two rotations (vectors_per_rot), a slot mapping that scatters and skips
    mbits, n, vpr = 3, 300, 150
    log("case: qjl encode %s d%d stack + slots" % (dtype, d))
    x = ti.codec_check_inputs(n=n, d=d, seed=7).to(dev, dtype)
    rot, pis = rotation_pair(d, [42, 49])
    S = _sketches(d, [42, 49])
    sk = tq.QJLSketch(rot, S)
    cb = tq.Codebook(d, mbits)
    perm = torch.randperm(n + 40, generator=ti.generator("cpu", 3))[:n]
    slots = perm.clone()
    slots[::17] = -1
    slots = slots.to(dev)
    rows = n + 40
    pk = torch.zeros(rows, d * mbits // 8, dtype=torch.uint8, device=dev)
    nm = torch.zeros(rows, dtype=torch.float32, device=dev)
    sg = torch.zeros(rows, d // 8, dtype=torch.uint8, device=dev)
    rn = torch.zeros(rows, dtype=torch.float32, device=dev)
    tq.qjl_encode(cb, sk, x, vectors_per_rot=vpr, packed=pk, norms=nm, signs=sg, rnorms=rn, slot_mapping=slots)
    torch.cuda.synchronize()
    x64 = to64(x)
    sl = slots.cpu().numpy()
    for r in range(2):
        idx = np.arange(r * vpr, (r + 1) * vpr)
        idx = idx[sl[idx] >= 0]
        dst = sl[idx]
        _check_qjl_encode(x64[idx], pk[dst].cpu().numpy(), nm[dst].cpu().numpy(), sg[dst].cpu().numpy(),
                          rn[dst].cpu().numpy(), pis[r], S[r].double().numpy(), d, mbits,
                          "qjl %s d%d rot %d" % (dtype, d, r))
    untouched = np.setdiff1d(np.arange(rows), sl[sl >= 0])
    assert torch.all(sg[untouched] == 0) and torch.all(rn[untouched] == 0)


def test_qjl_zero_vector(dev):
    # x = 0: codes of y = 0 (lower middle centroid), n = 0, residual 0, every projection 0 -> +1
    d, mbits = 128, 2
    rot, _ = rotation_pair(d, [42])
    sk = tq.QJLSketch(rot, _sketches(d, [42]))
    cb = tq.Codebook(d, mbits)
    x = torch.zeros(33, d, dtype=torch.bfloat16, device=dev)
    pk, nm, sg, rn = tq.qjl_encode(cb, sk, x)
    torch.cuda.synchronize()
    codes = occ.unpack_codes(pk.cpu().numpy(), mbits, d)
    assert np.all(codes == 2 ** (mbits - 1) - 1)
    assert torch.all(nm == 0) and torch.all(rn == 0) and torch.all(sg == 255)


def _qjl_cache(dev, B, Hkv, T, d, mbits, seed):
    rowb = d * mbits // 8
    return dict(kp=ti.random_bytes((B, Hkv, T, rowb), seed, dev), kn=ti.random_norms((B, Hkv, T), seed + 1, device=dev),
                ks=ti.random_bytes((B, Hkv, T, d // 8), seed + 2, dev),
                kr=ti.random_norms((B, Hkv, T), seed + 3, median=4.0, device=dev))


def _oracle_keys(c, d, mbits):
    codes = occ.unpack_codes(c["kp"].cpu().numpy().reshape(-1, c["kp"].shape[-1]), mbits, d)
    signs = oqjl.unpack_signs(c["ks"].cpu().numpy().reshape(-1, d // 8), d)
    shp = c["kn"].shape
    return (codes.reshape(*shp, d), c["kn"].cpu().numpy(), signs.reshape(*shp, d), c["kr"].cpu().numpy())


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("mbits", [1, 2, 3, 4])
def test_qjl_scores(dev, d, mbits):
    B, Hq, Hkv, T = 3, 8, 2, 200
    log("case: qjl scores d%d mse bits %d" % (d, mbits))
    q = ti.attn_inputs(ti.AttnShape(B, Hq, Hkv, 1, d, mbits, 2), device=dev, seed=5)[0]
    rot, pis = rotation_pair(d, [42])
    S = _sketches(d, [42])
    sk = tq.QJLSketch(rot, S)
    cb = tq.Codebook(d, mbits)
    c = _qjl_cache(dev, B, Hkv, T, d, mbits, 100 + d)
    lens = torch.tensor([200, 1, 77], dtype=torch.int32, device=dev)
    s = tq.scores_compressed(cb, rot, q, c["kp"], c["kn"], seq_lens=lens, qjl=sk, k_signs=c["ks"], k_rnorms=c["kr"])
    torch.cuda.synchronize()
    codes, norms, signs, rnorms = _oracle_keys(c, d, mbits)
    q64, S64 = to64(q), S[0].double().numpy()
    scale = 1 / math.sqrt(d)
    cbo = ocb.codebook(d, mbits)
    ref = oqjl.cache_scores(q64, codes, norms, signs, rnorms, pis[0], S64, cbo.centroids, scale, lens.cpu().numpy())
    G = Hq // Hkv
    cn = np.repeat(norms.astype(np.float64) * np.linalg.norm(cbo.centroids[codes.astype(np.int64)], axis=-1), G, 1)
    rr = np.repeat(rnorms.astype(np.float64), G, 1)
    sq1 = np.sum(np.abs(q64 @ S64.T), axis=-1)               # ||S q||_1 [B, Hq]
    bound = REL * scale * (cn * np.linalg.norm(q64, axis=-1)[:, :, None]
                           + rr * math.sqrt(math.pi / 2) / d * sq1[:, :, None])
    got = s.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b, L in enumerate(lens.tolist()):
        err = np.abs(got[b, :, :L] - ref[b, :, :L])
        worst = max(worst, float(np.max(err / bound[b, :, :L])))
        assert np.all(err <= bound[b, :, :L]), (b, float(np.max(err / bound[b, :, :L])))
        assert np.all(np.isnan(got[b, :, L:]))
        if L >= 32:
            rown = np.linalg.norm(got[b, :, :L] - ref[b, :, :L], axis=1) / np.linalg.norm(ref[b, :, :L], axis=1)
            assert np.all(rown <= REL), float(np.max(rown))
    log("qjl scores d%d b%d: worst error / bound %.3g" % (d, mbits, worst))


def _check_qjl_attention(o, lse, q64, keys, vhat, pi, S64, cbo, scale, lens, what):
    codes, norms, signs, rnorms = keys
    o_ref, lse_ref = oqjl.attention(q64, codes, norms, signs, rnorms, pi, S64, cbo.centroids, vhat, scale, lens)
    s_ref = oqjl.cache_scores(q64, codes, norms, signs, rnorms, pi, S64, cbo.centroids, scale, lens)
    B, Hq, d = q64.shape
    G = Hq // vhat.shape[1]
    worst = 0.0
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            if L == 0:
                assert np.all(o[b, h] == 0) and np.isneginf(lse[b, h]), (what, b, h)
                continue
            p = np.exp(s_ref[b, h, :L] - lse_ref[b, h])
            bound = REL * float(p @ np.linalg.norm(vhat[b, h // G, :L], axis=1))
            err = float(np.linalg.norm(o[b, h] - o_ref[b, h]))
            worst = max(worst, err / bound)
            assert err <= bound, "%s: b=%d h=%d error %.3g > %.3g" % (what, b, h, err, bound)
            assert abs(lse[b, h] - lse_ref[b, h]) <= 1e-3 * max(1.0, abs(lse_ref[b, h])), (what, b, h)
    log("%s: attention worst error / bound %.3g" % (what, worst))


@pytest.mark.parametrize("d,mbits,bv,Hq,Hkv", [(128, 3, 2, 32, 8), (128, 2, 3, 8, 8), (64, 2, 4, 16, 2),
                                               (128, 1, 2, 32, 8), (64, 1, 3, 8, 2), (256, 1, 4, 8, 4),
                                                (64, 3, 2, 16, 1), (256, 3, 3, 8, 2), (256, 2, 2, 4, 4)])
def test_qjl_attention_dense(dev, d, mbits, bv, Hq, Hkv):
    B, T = 4, 333
    log("case: qjl attention dense d%d K%d V%d Hq%d Hkv%d" % (d, mbits, bv, Hq, Hkv))
    q = ti.attn_inputs(ti.AttnShape(B, Hq, Hkv, 1, d, mbits, bv), device=dev, seed=6)[0]
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    S = _sketches(d, [42])
    sk = tq.QJLSketch(rk, S)
    ck, cv = tq.Codebook(d, mbits), tq.Codebook(d, bv)
    c = _qjl_cache(dev, B, Hkv, T, d, mbits, 200 + d)
    vp = ti.random_bytes((B, Hkv, T, d * bv // 8), 300 + d, dev)
    vn = ti.random_norms((B, Hkv, T), 301 + d, device=dev)
    lens = torch.tensor([333, 1, 0, 190], dtype=torch.int32, device=dev)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, c["kp"], c["kn"], vp, vn, seq_lens=lens, out_dtype=torch.float32,
                            return_lse=True, qjl=sk, k_signs=c["ks"], k_rnorms=c["kr"])
    torch.cuda.synchronize()
    vhat = oatt.decode_cache(vp.cpu().numpy(), vn.cpu().numpy(), pv[0], ocb.codebook(d, bv).centroids, bv, d)
    _check_qjl_attention(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), _oracle_keys(c, d, mbits),
                         vhat, pk[0], S[0].double().numpy(), ocb.codebook(d, mbits), 1 / math.sqrt(d),
                         lens.cpu().numpy(), "qjl dense d%d K%dV%d G%d" % (d, mbits, bv, Hq // Hkv))


@pytest.mark.parametrize("block_size", [16, 24])
def test_qjl_attention_paged(dev, block_size):
    d, mbits, bv, Hq, Hkv, S_ = 128, 3, 2, 16, 4, 5
    lens_l = [700, 33, 1, 0, 256]
    log("case: qjl attention paged block %d" % block_size)
    mb = max((L + block_size - 1) // block_size for L in lens_l)
    nblocks = S_ * mb + 3
    q = ti.attn_inputs(ti.AttnShape(S_, Hq, Hkv, 1, d, mbits, bv), device=dev, seed=8)[0]
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    S = _sketches(d, [42])
    sk = tq.QJLSketch(rk, S)
    ck, cv = tq.Codebook(d, mbits), tq.Codebook(d, bv)
    pool = _qjl_cache(dev, nblocks, Hkv, block_size, d, mbits, 400)
    vp = ti.random_bytes((nblocks, Hkv, block_size, d * bv // 8), 410, dev)
    vn = ti.random_norms((nblocks, Hkv, block_size), 411, device=dev)
    table = torch.randperm(nblocks, generator=ti.generator("cpu", 5))[:S_ * mb].view(S_, mb).to(torch.int32)
    lens = torch.tensor(lens_l, dtype=torch.int32)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, pool["kp"], pool["kn"], vp, vn, seq_lens=lens.to(dev),
                            max_seq_len=mb * block_size, block_table=table.to(dev), block_size=block_size,
                            out_dtype=torch.float32, return_lse=True, qjl=sk, k_signs=pool["ks"],
                            k_rnorms=pool["kr"], num_kv_heads=Hkv)
    torch.cuda.synchronize()
    # dense views of the pools per sequence, padded to the longest
    T = max(lens_l)
    codes, norms, signs, rnorms = _oracle_keys(pool, d, mbits)
    vhat_pool = oatt.decode_cache(vp.cpu().numpy(), vn.cpu().numpy(), pv[0], ocb.codebook(d, bv).centroids, bv, d)
    tab = table.numpy()
    dense = [np.zeros((S_, Hkv, T, d), np.uint8), np.zeros((S_, Hkv, T), np.float32),
             np.ones((S_, Hkv, T, d), np.int8), np.zeros((S_, Hkv, T), np.float32), np.zeros((S_, Hkv, T, d))]
    for s_, L in enumerate(lens_l):
        t = np.arange(L)
        blk, off = tab[s_, t // block_size], t % block_size
        for arr, src in zip(dense, (codes, norms, signs, rnorms, vhat_pool)):
            arr[s_, :, :L] = src[blk, :, off].swapaxes(0, 1)
    _check_qjl_attention(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), tuple(dense[:4]), dense[4],
                         pk[0], S[0].double().numpy(), ocb.codebook(d, mbits), 1 / math.sqrt(d), lens_l,
                         "qjl paged block %d" % block_size)


def test_qjl_error_paths(dev):
    d = 128
    rot, _ = rotation_pair(d, [42])
    with pytest.raises(ValueError):
        tq.QJLSketch(rot, torch.zeros(2, d, d))
    sk = tq.QJLSketch(rot, _sketches(d, [42]))
    cb1 = tq.Codebook(d, 1)
    x = torch.zeros(4, d, dtype=torch.bfloat16, device=dev)
    # 1-bit codes are a QJL key's MSE stage only: the plain encode refuses them
    with pytest.raises(tq.TQError, match="not supported on the GPU"):
        tq.encode(cb1, rot, x)
    cb64 = tq.Codebook(64, 2)
    with pytest.raises((ValueError, tq.TQError), match="does not match"):
        tq.qjl_encode(cb64, sk, x)
    cb = tq.Codebook(d, 2)
    sg = torch.empty(4 * 16 + 8, dtype=torch.uint8, device=dev)[8:].view(4, 16)   # misaligned signs
    with pytest.raises(tq.TQError, match="16-byte aligned"):
        tq.qjl_encode(cb, sk, x, signs=sg)
    other, _ = rotation_pair(d, [43])
    q = torch.zeros(1, 8, d, dtype=torch.bfloat16, device=dev)
    kp = torch.zeros(1, 2, 8, d * 2 // 8, dtype=torch.uint8, device=dev)
    kn = torch.zeros(1, 2, 8, device=dev)
    with pytest.raises((ValueError, tq.TQError), match="not created on rot_k"):
        tq.scores_compressed(cb, other, q, kp, kn, qjl=sk, k_signs=torch.zeros(1, 2, 8, 16, dtype=torch.uint8,
                                                                             device=dev), k_rnorms=kn)


def test_qjl_attention_with_window(dev):
    # QJL keys in the compressed part, the newest min(L, R) tokens exact in the rings: one softmax
    # over both (the window partial joins the merge like with plain keys)
    from oracle import window as ow
    d, mbits, bv, Hq, Hkv, B, T, R = 128, 3, 2, 8, 2, 3, 300, 40
    log("case: qjl attention with a %d-token window" % R)
    q = ti.attn_inputs(ti.AttnShape(B, Hq, Hkv, 1, d, mbits, bv), device=dev, seed=12)[0]
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    S = _sketches(d, [42])
    sk = tq.QJLSketch(rk, S)
    ck, cv = tq.Codebook(d, mbits), tq.Codebook(d, bv)
    c = _qjl_cache(dev, B, Hkv, T, d, mbits, 500)
    vp = ti.random_bytes((B, Hkv, T, d * bv // 8), 510, dev)
    vn = ti.random_norms((B, Hkv, T), 511, device=dev)
    kw = ti.normal((B, Hkv, R, d), 512, scale=4.0, dtype=torch.bfloat16, device=dev)
    vw = ti.normal((B, Hkv, R, d), 513, scale=4.0, dtype=torch.bfloat16, device=dev)
    lens = [300, 25, 41]
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, c["kp"], c["kn"], vp, vn,
                            seq_lens=torch.tensor(lens, dtype=torch.int32, device=dev), out_dtype=torch.float32,
                            return_lse=True, qjl=sk, k_signs=c["ks"], k_rnorms=c["kr"], k_window=kw, v_window=vw)
    torch.cuda.synchronize()
    codes, norms, signs, rnorms = _oracle_keys(c, d, mbits)
    vhat = oatt.decode_cache(vp.cpu().numpy(), vn.cpu().numpy(), pv[0], ocb.codebook(d, bv).centroids, bv, d)
    q64, S64, scale = to64(q), S[0].double().numpy(), 1 / math.sqrt(d)
    kw64, vw64 = to64(kw), to64(vw)
    cb = ocb.codebook(d, mbits)
    G = Hq // Hkv
    worst = 0.0
    for b, L in enumerate(lens):
        cpos, w = ow.split(L, R)
        for h in range(Hq):
            g = h // G
            s_c = oqjl.scores(q64[b, h][None], codes[b, g, :cpos], norms[b, g, :cpos], signs[b, g, :cpos],
                              rnorms[b, g, :cpos], pk[0], S64, cb.centroids, scale)[0] if cpos else np.zeros(0)
            kwin = np.stack([kw64[b, g, t % R] for t in range(cpos, L)])
            vwin = np.stack([vw64[b, g, t % R] for t in range(cpos, L)])
            s_all = np.concatenate([s_c, scale * (kwin @ q64[b, h])])
            vals = np.concatenate([vhat[b, g, :cpos], vwin])
            m = s_all.max()
            p = np.exp(s_all - m)
            o_ref = (p / p.sum()) @ vals
            lse_ref = m + math.log(p.sum())
            bound = REL * float((p / p.sum()) @ np.linalg.norm(vals, axis=1))
            err = float(np.linalg.norm(o[b, h].cpu().numpy().astype(np.float64) - o_ref))
            worst = max(worst, err / bound)
            assert err <= bound, (b, h, err, bound)
            assert abs(float(lse[b, h]) - lse_ref) <= 1e-3 * max(1.0, abs(lse_ref))
    log("qjl + window: worst error / bound %.3g" % worst)
