"""GPU parity of the recent-token window: attention over compressed + full-precision tokens,
and the append / flush that maintains the rings (through the C ABI).

Attention with a window must match oracle/window.py (the newest min(L, R) tokens exact, the
older ones decoded from a compressed cache the oracle's encode made of the same tokens) to the
usual bar ||do|| <= 2e-3 sum_t p_t ||v_t||.
Append: a prefill (one call with the whole prompt) and token-by-token appends must leave the
same state, bit for bit; the flushed rows must equal tq_encode of the same tokens (same
kernel) and meet the oracle's code parity; the rings must hold the newest tokens verbatim.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt, codebook as ocb, window as ow
import tq_inputs as ti
from parity import REL, check_encode, log, oracle_encoded, rotation_pair, to64, upload

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _check(o_gpu, lse_gpu, q64, khat, vhat, kw, vw, lens, R, scale, what):
    o_ref, lse_ref = ow.attention(q64, khat, vhat, kw, vw, lens, R, scale)
    B, Hq, d = q64.shape
    G = Hq // khat.shape[1]
    worst = 0.0
    for b in range(B):
        L = int(lens[b])
        c, w = ow.split(L, R)
        for h in range(Hq):
            if L == 0:
                assert np.all(o_gpu[b, h] == 0)
                continue
            g = h // G
            keys = np.concatenate([khat[b, g, :c], np.stack([kw[b, g, t % R] for t in range(c, L)])]) if w else \
                khat[b, g, :c]
            vals = np.concatenate([vhat[b, g, :c], np.stack([vw[b, g, t % R] for t in range(c, L)])]) if w else \
                vhat[b, g, :c]
            s = scale * (keys @ q64[b, h])
            p = np.exp(s - lse_ref[b, h])
            bound = REL * float(p @ np.linalg.norm(vals, axis=1))
            err = float(np.linalg.norm(o_gpu[b, h] - o_ref[b, h]))
            worst = max(worst, err / bound)
            assert err <= bound, "%s: b=%d h=%d error %.3g > %.3g" % (what, b, h, err, bound)
            lb = REL * scale * float(np.max(np.linalg.norm(keys, axis=1))) * float(np.linalg.norm(q64[b, h]))
            assert abs(lse_gpu[b, h] - lse_ref[b, h]) <= lb + 1e-6
    log("%s: worst error / bound %.3g" % (what, worst))


@pytest.mark.parametrize("d,bk,bv,R,wdt", [(128, 4, 2, 128, torch.bfloat16), (64, 3, 3, 16, torch.float16),
                                            (256, 2, 4, 40, torch.float32), (128, 3, 2, 300, torch.bfloat16)])
def test_attention_with_window(dev, d, bk, bv, R, wdt):
    B, Hq, Hkv, T = 5, 8, 2, 600
    sd = 10 * (d + R)
    q = ti.normal((B, Hq, d), sd, dtype=torch.bfloat16, device=dev)
    k = ti.normal((B, Hkv, T, d), sd + 1, dtype=torch.bfloat16)
    v = ti.normal((B, Hkv, T, d), sd + 2, dtype=torch.bfloat16)
    kw = ti.normal((B, Hkv, R, d), sd + 3, scale=1.5, dtype=wdt, device=dev)
    vw = ti.normal((B, Hkv, R, d), sd + 4, dtype=wdt, device=dev)
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kpn, knn = oracle_encoded(to64(k), pk[0], bk)
    vpn, vnn = oracle_encoded(to64(v), pv[0], bv)
    kp, kn, vp, vn = upload(kpn, dev), upload(knn, dev), upload(vpn, dev), upload(vnn, dev)
    lens = torch.tensor([600, 0, min(R, 600) // 2 + 1, R, R + 1], dtype=torch.int32, device=dev)
    what = "window d%d K%dV%d R%d %s" % (d, bk, bv, R, wdt)
    log("case:", what)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, kp, kn, vp, vn, seq_lens=lens, out_dtype=torch.float32,
                            return_lse=True, k_window=kw, v_window=vw)
    torch.cuda.synchronize()
    khat = oatt.decode_cache(kpn, knn, pk[0], ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vpn, vnn, pv[0], ocb.codebook(d, bv).centroids, bv, d)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), khat, vhat, to64(kw), to64(vw),
           lens.cpu().numpy(), R, 1 / math.sqrt(d), what)


def _state(dev, B, Hkv, S, R, d, bk, bv, wdt=torch.bfloat16, paged=None):
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    rowk, rowv = d * bk // 8, d * bv // 8
    if paged is None:
        shape_k, shape_n = (B, Hkv, S, rowk), (B, Hkv, S)
        shape_v = (B, Hkv, S, rowv)
    else:
        nb, bs = paged
        shape_k, shape_n, shape_v = (nb, Hkv, bs, rowk), (nb, Hkv, bs), (nb, Hkv, bs, rowv)
    st = dict(ck=ck, cv=cv, rk=rk, rv=rv, pk=pk[0], pv=pv[0],
              kp=torch.zeros(shape_k, dtype=torch.uint8, device=dev), kn=torch.zeros(shape_n, device=dev),
              vp=torch.zeros(shape_v, dtype=torch.uint8, device=dev), vn=torch.zeros(shape_n, device=dev),
              kw=torch.zeros(B, Hkv, max(R, 1), d, dtype=wdt, device=dev)[:, :, :R],
              vw=torch.zeros(B, Hkv, max(R, 1), d, dtype=wdt, device=dev)[:, :, :R],
              lens=torch.zeros(B, dtype=torch.int32, device=dev))
    return st


def _append(st, k_new, v_new, S, block_table=None, block_size=0):
    tq.window_append(st["ck"], st["rk"], st["cv"], st["rv"], k_new.contiguous(), v_new.contiguous(),
                     st["kw"], st["vw"], st["lens"], st["kp"], st["kn"], st["vp"], st["vn"], max_seq_len=S,
                     block_table=block_table, block_size=block_size)


@pytest.mark.parametrize("R,chunks", [(16, "prefill"), (16, "ones"), (16, [20, 1, 1, 28]), (0, [7, 1, 42]),
                                      (64, [3, 3, 44]), (16, [16, 1, 33])])
def test_append_streaming_equals_prefill(dev, R, chunks):
    B, Hkv, S, d, bk, bv = 3, 2, 50, 128, 4, 2
    K = ti.normal((B, Hkv, S, d), 100 + R, dtype=torch.bfloat16, device=dev)
    V = ti.normal((B, Hkv, S, d), 200 + R, dtype=torch.bfloat16, device=dev)
    if chunks == "prefill":
        chunks = [S]
    elif chunks == "ones":
        chunks = [1] * S
    log("case: append R%d chunks %s" % (R, chunks[:6]))
    st = _state(dev, B, Hkv, S, R, d, bk, bv)
    pos = 0
    for n in chunks:
        _append(st, K[:, :, pos:pos + n], V[:, :, pos:pos + n], S)
        pos += n
    torch.cuda.synchronize()
    assert st["lens"].tolist() == [S] * B
    c, w = ow.split(S, R)
    # rings: the newest w tokens verbatim at slot position mod R
    for t in range(c, S):
        assert torch.equal(st["kw"][:, :, t % R], K[:, :, t]) and torch.equal(st["vw"][:, :, t % R], V[:, :, t])
    # compressed rows [0, c): the encode of the same tokens, bit for bit
    if c:
        kp, kn = tq.encode(st["ck"], st["rk"], K[:, :, :c])
        vp, vn = tq.encode(st["cv"], st["rv"], V[:, :, :c])
        assert torch.equal(st["kp"][:, :, :c].reshape(-1, kp.shape[-1]), kp)
        assert torch.equal(st["kn"][:, :, :c].reshape(-1), kn)
        assert torch.equal(st["vp"][:, :, :c].reshape(-1, vp.shape[-1]), vp)
        assert torch.equal(st["vn"][:, :, :c].reshape(-1), vn)
        check_encode(to64(K[:, :, :c].reshape(-1, d)), kp.cpu().numpy(), kn.cpu().numpy(), st["pk"], d, bk,
                     "append K")
    # rows past the compressed count are untouched
    assert torch.count_nonzero(st["kn"][:, :, c:]) == 0


def test_append_ragged_lengths_paged_then_attention(dev):
    """Sequences at different lengths in a paged compressed cache: per-sequence prefills of
    0, 5 and 11 tokens (one-sequence sub-batches), then 60 batched single-token appends, then
    attention over compressed + window against the oracle. The append's compressed rows are
    checked bit for bit against tq_encode of the same tokens; for the attention check they are
    then replaced by the oracle's encode of those tokens, which both sides read."""
    B, Hkv, Hq, S, R, d, bk, bv, bs = 3, 2, 8, 96, 24, 64, 3, 2, 16
    nblk = B * (S // bs)
    perm = torch.randperm(nblk, generator=ti.generator("cpu", 4)).to(torch.int32)
    table = perm.view(B, S // bs).to(dev)
    K = ti.normal((B, Hkv, S, d), 9, dtype=torch.bfloat16, device=dev)
    V = ti.normal((B, Hkv, S, d), 10, dtype=torch.bfloat16, device=dev)
    st = _state(dev, B, Hkv, S, R, d, bk, bv, paged=(nblk, bs))
    L0 = [0, 5, 11]
    for b, n in enumerate(L0):
        if n == 0:
            continue
        sub = {k2: st[k2] for k2 in ("ck", "rk", "cv", "rv", "kp", "kn", "vp", "vn")}
        sub.update(kw=st["kw"][b:b + 1], vw=st["vw"][b:b + 1], lens=st["lens"][b:b + 1])
        _append(sub, K[b:b + 1, :, :n], V[b:b + 1, :, :n], S, table[b:b + 1], bs)
    steps = 60
    for j in range(steps):
        idx = torch.tensor([L0[b] + j for b in range(B)], device=dev)
        kj = K[torch.arange(B, device=dev), :, idx].unsqueeze(2)
        vj = V[torch.arange(B, device=dev), :, idx].unsqueeze(2)
        _append(st, kj, vj, S, table, bs)
    torch.cuda.synchronize()
    final = [L0[b] + steps for b in range(B)]
    assert st["lens"].tolist() == final
    q = ti.normal((B, Hq, d), 11, dtype=torch.bfloat16, device=dev)
    lens = torch.tensor(final, dtype=torch.int32, device=dev)
    # the append's state: compressed rows = tq_encode of the tokens at those positions, rings verbatim
    tb = table.cpu().numpy()
    gkp = st["kp"].cpu().numpy()[tb].transpose(0, 2, 1, 3, 4).reshape(B, Hkv, S, -1)
    gkn = st["kn"].cpu().numpy()[tb].transpose(0, 2, 1, 3).reshape(B, Hkv, S)
    for b in range(B):
        c, _ = ow.split(final[b], R)
        kp_b, kn_b = tq.encode(st["ck"], st["rk"], K[b, :, :c])
        assert np.array_equal(gkp[b, :, :c].reshape(-1, gkp.shape[-1]), kp_b.cpu().numpy())
        assert np.array_equal(gkn[b, :, :c].reshape(-1), kn_b.cpu().numpy())
        for t in range(c, final[b]):
            assert torch.equal(st["kw"][b, :, t % R], K[b, :, t])
    # attention input: the oracle's encode of every position, scattered into the same pages
    kpn, knn = oracle_encoded(to64(K), st["pk"], bk)           # [B, Hkv, S, row]
    vpn, vnn = oracle_encoded(to64(V), st["pv"], bv)
    def pages(a):   # [B, Hkv, S, ...] -> pool [nblk, Hkv, bs, ...] through the block table
        pool = np.zeros((nblk, Hkv, bs) + a.shape[3:], dtype=a.dtype)
        for b in range(B):
            for j in range(S // bs):
                pool[tb[b, j]] = a[b, :, j * bs:(j + 1) * bs]
        return upload(pool, dev)
    o, lse = tq.attn_decode(st["ck"], st["rk"], st["cv"], st["rv"], q, pages(kpn), pages(knn), pages(vpn),
                            pages(vnn), seq_lens=lens, max_seq_len=S, block_table=table, block_size=bs,
                            out_dtype=torch.float32, return_lse=True, num_kv_heads=Hkv, k_window=st["kw"],
                            v_window=st["vw"])
    torch.cuda.synchronize()
    khat = oatt.decode_cache(kpn, knn, st["pk"], ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vpn, vnn, st["pv"], ocb.codebook(d, bv).centroids, bv, d)
    # the oracle's rings are built from the appended tokens themselves (token t at slot t mod R)
    K64, V64 = to64(K), to64(V)
    kw_ref, vw_ref = np.zeros((B, Hkv, R, d)), np.zeros((B, Hkv, R, d))
    for b in range(B):
        c, _ = ow.split(final[b], R)
        for t in range(c, final[b]):
            kw_ref[b, :, t % R], vw_ref[b, :, t % R] = K64[b, :, t], V64[b, :, t]
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(q), khat, vhat, kw_ref, vw_ref, final, R,
           1 / math.sqrt(d), "append+paged attention")
