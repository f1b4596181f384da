"""GPU parity of tq_scores_compressed / tq_attn_decode against the float64 oracle.

The compressed cache both sides read is the oracle's encode of the seeded K and V (small
cases), or, at the full sizes, tq_inputs' random code bytes with norms taken from the seeded
tokens; the oracle never decodes a GPU-written row."""

import math

import numpy as np
import pytest
import torch

import tq_inputs as ti
from oracle import attention as oatt, codebook as ocb, codec as occ
from parity import (check_attention, check_decode, check_encode, log, oracle_encoded, rotation_pair, score_bounds,
                    to64, upload)

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _dense_cache(dev, B, Hq, Hkv, T, d, bk, bv, seed=11, kseed=42, vseed=542, qdtype=torch.bfloat16):
    q, k, v = ti.attn_inputs(ti.AttnShape(B, Hq, Hkv, T, d, bk, bv), device=dev, seed=seed)
    q = q.to(qdtype)
    rk, pk = rotation_pair(d, [kseed])
    rv, pv = rotation_pair(d, [vseed])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kpn, knn = oracle_encoded(to64(k), pk[0], bk)      # [B, Hkv, T, row], [B, Hkv, T]
    vpn, vnn = oracle_encoded(to64(v), pv[0], bv)
    return dict(q=q, k=k, v=v, rk=rk, rv=rv, pk=pk[0], pv=pv[0], ck=ck, cv=cv, kpn=kpn, knn=knn, vpn=vpn, vnn=vnn,
                kp=upload(kpn, dev), kn=upload(knn, dev), vp=upload(vpn, dev), vn=upload(vnn, dev))


def _oracle_cache(c, d, bk, bv):
    khat = oatt.decode_cache(c["kpn"], c["knn"], c["pk"], ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(c["vpn"], c["vnn"], c["pv"], ocb.codebook(d, bv).centroids, bv, d)
    return khat, vhat


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bk", [2, 3, 4])
def test_scores(dev, d, bk):
    B, Hq, Hkv, T = 3, 8, 2, 200
    log("case: scores d%d bk%d" % (d, bk))
    c = _dense_cache(dev, B, Hq, Hkv, T, d, bk, 2)
    lens = torch.tensor([200, 1, 77], dtype=torch.int32, device=dev)
    s = tq.scores_compressed(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], seq_lens=lens)
    torch.cuda.synchronize()
    khat, _ = _oracle_cache(c, d, bk, 2)
    q64 = to64(c["q"])
    scale = 1 / math.sqrt(d)
    ref = oatt.scores(q64, khat, scale, seq_lens=lens.cpu().numpy())
    codes = occ.unpack_codes(c["kpn"].reshape(-1, c["kpn"].shape[-1]), bk, d).reshape(B, Hkv, T, d)
    bound = score_bounds(q64, c["knn"], codes, ocb.codebook(d, bk), scale)
    got = s.cpu().numpy().astype(np.float64)
    for b, L in enumerate(lens.tolist()):
        err = np.abs(got[b, :, :L] - ref[b, :, :L])
        assert np.all(err <= bound[b, :, :L]), (b, float(np.max(err / bound[b, :, :L])))
        assert np.all(np.isnan(got[b, :, L:]))          # entries beyond len are left untouched
        # normwise per row (rows of a few tokens can have a near-zero norm: not a meaningful scale)
        if L >= 32:
            rown = np.linalg.norm(got[b, :, :L] - ref[b, :, :L], axis=1) / np.linalg.norm(ref[b, :, :L], axis=1)
            assert np.all(rown <= 2e-3), float(np.max(rown))


@pytest.mark.parametrize("d,bk,bv,Hq,Hkv", [
    (128, 4, 2, 32, 8), (128, 3, 3, 8, 8), (64, 2, 4, 16, 2), (64, 3, 2, 16, 1), (256, 4, 3, 8, 2),
    (256, 2, 2, 4, 4), (128, 2, 3, 12, 4)])
def test_attention_dense(dev, d, bk, bv, Hq, Hkv):
    B, T = 4, 333
    log("case: attention dense d%d K%dV%d Hq%d Hkv%d" % (d, bk, bv, Hq, Hkv))
    c = _dense_cache(dev, B, Hq, Hkv, T, d, bk, bv)
    lens = torch.tensor([333, 1, 0, 190], dtype=torch.int32, device=dev)
    o, lse = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                            seq_lens=lens, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    khat, vhat = _oracle_cache(c, d, bk, bv)
    check_attention(o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), to64(c["q"]), khat, vhat,
                    1 / math.sqrt(d), lens.cpu().numpy(), "dense d%d K%dV%d G%d" % (d, bk, bv, Hq // Hkv))


@pytest.mark.parametrize("splits", [1, 3, 40])
def test_attention_split_counts(dev, splits):
    d, bk, bv, B, Hq, Hkv, T = 128, 4, 2, 2, 8, 2, 1500
    c = _dense_cache(dev, B, Hq, Hkv, T, d, bk, bv, seed=5)
    o = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                       out_dtype=torch.float32, num_splits=splits)
    torch.cuda.synchronize()
    khat, vhat = _oracle_cache(c, d, bk, bv)
    check_attention(o.cpu().numpy().astype(np.float64), None, to64(c["q"]), khat, vhat, 1 / math.sqrt(d),
                    [T] * B, "splits %d" % splits)


def test_attention_bf16_output_and_scale(dev):
    d, bk, bv, B, Hq, Hkv, T = 128, 4, 2, 2, 8, 2, 257
    c = _dense_cache(dev, B, Hq, Hkv, T, d, bk, bv, seed=9, qdtype=torch.float16)
    o = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                       out_dtype=torch.bfloat16, scale=0.3)
    torch.cuda.synchronize()
    khat, vhat = _oracle_cache(c, d, bk, bv)
    check_attention(o.float().cpu().numpy().astype(np.float64), None, to64(c["q"]), khat, vhat, 0.3,
                    [T] * B, "bf16 out, scale 0.3")


def _paged(dev, S, max_len, Hkv, Hq, d, bk, bv, seed=7, oracle_rows=None, shape=None):
    """Paged pool [num_blocks, Hkv, block_size, row] of one layer's tokens, written by tq_encode
    through a slot mapping. oracle_rows: sequences whose rows are then replaced by oracle-side
    inputs (all sequences: the oracle's encode of their tokens; a list: random code bytes with
    the tokens' own norms, cheap at full size) so that the attention check reads no GPU-written
    row."""
    if shape is None:
        shape = ti.PagedShape(sequences=S, max_len=max_len, kv_heads=Hkv, q_heads=Hq)
    lay = ti.paged_layout(shape, seed=seed)
    total = int(lay.seq_starts[-1])
    k, v, _ = ti.paged_layer_tokens(shape, total, d, layer=seed, device=dev)
    bs = shape.block_size
    # slot of (token, head) in the pool [num_blocks, Hkv, bs, row]
    tok_slot = lay.token_slots                                   # block*bs + off
    blk, off = tok_slot // bs, tok_slot % bs
    heads = torch.arange(Hkv)
    slot = ((blk[:, None] * Hkv + heads[None, :]) * bs + off[:, None]).reshape(-1).to(dev)
    nslots = lay.num_blocks * Hkv * bs
    rk, pk = rotation_pair(d, [ti.key_seed(seed)])
    rv, pv = rotation_pair(d, [ti.value_seed(seed)])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kp, kn = tq.encode(ck, rk, k, slot_mapping=slot, num_slots=nslots)
    vp, vn = tq.encode(cv, rv, v, slot_mapping=slot, num_slots=nslots)
    q = ti.paged_queries(shape, S, d, seed, device=dev)
    c = dict(shape=shape, lay=lay, k=k, v=v, slot=slot, rk=rk, rv=rv, pk=pk[0], pv=pv[0], ck=ck, cv=cv, q=q,
             gkp=kp, gkn=kn)
    if oracle_rows is not None:
        seqs = range(S) if oracle_rows == "all" else oracle_rows
        starts = lay.seq_starts
        tok = torch.cat([torch.arange(int(starts[s_]), int(starts[s_ + 1])) for s_ in seqs])
        rows = (tok[:, None] * Hkv + heads[None, :]).reshape(-1)          # rows of k.view(-1, d)
        dst = slot[rows.to(dev)]
        if oracle_rows == "all":
            kr, knr = oracle_encoded(to64(k.view(-1, d)[rows.to(dev)]), pk[0], bk)
            vr, vnr = oracle_encoded(to64(v.view(-1, d)[rows.to(dev)]), pv[0], bv)
        else:
            n = rows.numel()
            kr = ti.random_bytes((n, d * bk // 8), 900 + seed, "cpu").numpy()
            vr = ti.random_bytes((n, d * bv // 8), 901 + seed, "cpu").numpy()
            knr = np.linalg.norm(to64(k.view(-1, d)[rows.to(dev)]), axis=1).astype(np.float32)
            vnr = np.linalg.norm(to64(v.view(-1, d)[rows.to(dev)]), axis=1).astype(np.float32)
        kp, kn, vp, vn = kp.clone(), kn.clone(), vp.clone(), vn.clone()
        kp[dst], kn[dst], vp[dst], vn[dst] = upload(kr, dev), upload(knr, dev), upload(vr, dev), upload(vnr, dev)
        pool = {}
        for name, arr, src in (("kp", kp, kr), ("kn", kn, knr), ("vp", vp, vr), ("vn", vn, vnr)):
            host = np.zeros(tuple(arr.shape), dtype=src.dtype)
            host[dst.cpu().numpy()] = src
            pool[name + "_host"] = host.reshape((lay.num_blocks, Hkv, bs) + tuple(arr.shape[1:]))
        c.update(pool)
    c.update(kp=kp.view(lay.num_blocks, Hkv, bs, -1), kn=kn.view(lay.num_blocks, Hkv, bs),
             vp=vp.view(lay.num_blocks, Hkv, bs, -1), vn=vn.view(lay.num_blocks, Hkv, bs))
    return c


def _check_paged(c, d, bk, bv, o, lse, seqs, what):
    lay, Hkv = c["lay"], c["shape"].kv_heads
    bs = c["shape"].block_size
    lens = lay.seq_lens.numpy()
    ck, cv = ocb.codebook(d, bk).centroids, ocb.codebook(d, bv).centroids
    q64 = to64(c["q"])
    kpn, knn, vpn, vnn = c["kp_host"], c["kn_host"], c["vp_host"], c["vn_host"]
    table = lay.block_table.numpy()
    worst = 0
    for s in seqs:
        L = int(lens[s])
        sub = np.array([s])
        kseq = oatt.gather_paged(kpn, table[sub], [L], bs)[0]
        knseq = oatt.gather_paged(knn, table[sub], [L], bs)[0]
        vseq = oatt.gather_paged(vpn, table[sub], [L], bs)[0]
        vnseq = oatt.gather_paged(vnn, table[sub], [L], bs)[0]
        khat = oatt.decode_cache(kseq, knseq, c["pk"], ck, bk, d)[None]
        vhat = oatt.decode_cache(vseq, vnseq, c["pv"], cv, bv, d)[None]
        worst = max(worst, check_attention(o[s:s + 1], None if lse is None else lse[s:s + 1], q64[s:s + 1], khat,
                                           vhat, 1 / math.sqrt(d), [L], "%s seq %d (len %d)" % (what, s, L)))
    return worst


@pytest.mark.parametrize("d,bk,bv", [(64, 3, 2), (128, 4, 2), (256, 2, 4)])
def test_attention_paged_small(dev, d, bk, bv):
    S, Hkv, Hq = 6, 2, 8
    log("case: paged small d%d K%dV%d" % (d, bk, bv))
    c = _paged(dev, S, 700, Hkv, Hq, d, bk, bv, oracle_rows="all")
    lay = c["lay"]
    # the slot-mapped GPU encode of every token meets the codec bar
    check_encode(to64(c["k"].view(-1, d)), c["gkp"][c["slot"]].cpu().numpy(), c["gkn"][c["slot"]].cpu().numpy(),
                 c["pk"], d, bk, "paged small K d%d" % d)
    o, lse = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                            seq_lens=lay.seq_lens.to(dev), max_seq_len=int(lay.seq_lens.max()),
                            block_table=lay.block_table.to(dev), block_size=16,
                            out_dtype=torch.float32, return_lse=True, num_kv_heads=Hkv)
    torch.cuda.synchronize()
    _check_paged(c, d, bk, bv, o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), range(S), "paged small")
    # scores from the paged cache, entry by entry against the oracle's scores over the gathered pages
    s = tq.scores_compressed(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], seq_lens=lay.seq_lens.to(dev),
                             max_seq_len=int(lay.seq_lens.max()), block_table=lay.block_table.to(dev),
                             block_size=16, num_kv_heads=Hkv)
    torch.cuda.synchronize()
    _check_paged_scores(c, d, bk, s.cpu().numpy().astype(np.float64), range(S), "paged small scores")


def _check_paged_scores(c, d, bk, got, seqs, what):
    """Paged tq_scores_compressed output `got` ([S, Hq, max_len], or a map from sequence to its
    [Hq, max_len] rows) against oracle.attention.scores over
    the sequence's gathered rows (the oracle-side pool copies), at the Cauchy-Schwarz bar; entries
    past a sequence's length are left untouched (NaN)."""
    lay = c["lay"]
    bs = c["shape"].block_size
    lens = lay.seq_lens.numpy()
    table = lay.block_table.numpy()
    cb = ocb.codebook(d, bk)
    q64 = to64(c["q"])
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for s_ in seqs:
        L = int(lens[s_])
        sub = np.array([s_])
        kseq = oatt.gather_paged(c["kp_host"], table[sub], [L], bs)[0]        # [Hkv, L, row]
        knseq = oatt.gather_paged(c["kn_host"], table[sub], [L], bs)[0]       # [Hkv, L]
        khat = oatt.decode_cache(kseq, knseq, c["pk"], cb.centroids, bk, d)[None]
        ref = oatt.scores(q64[s_:s_ + 1], khat, scale)[0]
        codes = occ.unpack_codes(kseq.reshape(-1, kseq.shape[-1]), bk, d).reshape(kseq.shape[0], L, d)
        bound = score_bounds(q64[s_:s_ + 1], knseq[None], codes[None], cb, scale)[0]
        g = got[s_]                                                            # [Hq, max_len]
        err = np.abs(g[:, :L] - ref)
        assert np.all(err <= bound), "%s seq %d: score error %.3g of the bound" % (what, s_, float(np.max(err / bound)))
        assert np.all(np.isnan(g[:, L:])), (what, s_)
        worst = max(worst, float(np.max(err / bound)))
    log("%s: %d sequences, worst score error / bound = %.3g" % (what, len(list(seqs)), worst))


@pytest.mark.parametrize("block", [12, 48])
def test_paged_any_block_size(dev, block):
    """Pages of 12 and 48 tokens: not a power of two, so every token's page is looked up on its own
    (the kernels' general paging path); scores and attention against the oracle."""
    d, bk, bv, S, Hkv, Hq = 128, 3, 2, 5, 2, 8
    log("case: paged block %d" % block)
    shape = ti.PagedShape(sequences=S, max_len=500, kv_heads=Hkv, q_heads=Hq, block_size=block)
    c = _paged(dev, S, 500, Hkv, Hq, d, bk, bv, seed=3, oracle_rows="all", shape=shape)
    lay = c["lay"]
    args = dict(seq_lens=lay.seq_lens.to(dev), max_seq_len=int(lay.seq_lens.max()),
                block_table=lay.block_table.to(dev), block_size=block, num_kv_heads=Hkv)
    s = tq.scores_compressed(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], **args)
    o, lse = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                            out_dtype=torch.float32, return_lse=True, **args)
    torch.cuda.synchronize()
    _check_paged_scores(c, d, bk, s.cpu().numpy().astype(np.float64), range(S), "paged block %d scores" % block)
    _check_paged(c, d, bk, bv, o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), range(S),
                 "paged block %d" % block)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bk", [2, 3, 4])
@pytest.mark.parametrize("bv", [2, 3, 4])
def test_paged_ragged_every_width_pair(dev, d, bk, bv):
    """Every (K, V) width pair of the paged ragged workload, per head size, through the paged
    path with its head shape (8 KV heads, 32 query heads, pages of 16) on a few ragged
    sequences: scores and attention against the oracle over every sequence."""
    S, Hkv, Hq = 5, 8, 32
    log("case: paged widths d%d K%dV%d" % (d, bk, bv))
    c = _paged(dev, S, 400, Hkv, Hq, d, bk, bv, seed=40 + 3 * bk + bv, oracle_rows="all")
    lay = c["lay"]
    args = dict(seq_lens=lay.seq_lens.to(dev), max_seq_len=int(lay.seq_lens.max()),
                block_table=lay.block_table.to(dev), block_size=16, num_kv_heads=Hkv)
    o, lse = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                            out_dtype=torch.float32, return_lse=True, **args)
    s = tq.scores_compressed(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], **args)
    torch.cuda.synchronize()
    _check_paged(c, d, bk, bv, o.cpu().numpy().astype(np.float64), lse.cpu().numpy(), range(S),
                 "paged widths d%d K%dV%d" % (d, bk, bv))
    _check_paged_scores(c, d, bk, s.cpu().numpy().astype(np.float64), range(S),
                        "paged widths d%d K%d scores" % (d, bk))


def test_fused_attention_workload_full(dev):
    """Batch 32, 32 query heads over 8 KV heads, context 32768, d=128, K4/V2, bf16 queries, in the
    launch configuration the bench times. The cache is random code bytes with log-normal norms
    (tq_inputs); oracle attention over the same bytes for 2 batch rows (all heads). The encode of
    the seeded K at this size is checked on 2048 sampled rows."""
    shape = ti.AttnShape()
    B, Hq, Hkv, T, d = shape.batch, shape.q_heads, shape.kv_heads, shape.tokens, shape.head_dim
    log("case: fused attention workload B%d Hq%d Hkv%d T%d" % (B, Hq, Hkv, T))
    q, k, _ = ti.attn_inputs(shape, device=dev, seed=11)
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    ck, cv = tq.Codebook(d, 4), tq.Codebook(d, 2)
    gkp, gkn = tq.encode(ck, rk, k)
    torch.cuda.synchronize()
    rows = torch.randperm(B * Hkv * T, generator=ti.generator("cpu", 3))[:2048].to(dev)
    check_encode(to64(k.view(-1, d)[rows]), gkp[rows].cpu().numpy(), gkn[rows].cpu().numpy(), pk[0], d, 4,
                 "attn workload K")
    del k, gkp, gkn
    kp = ti.random_bytes((B, Hkv, T, d * 4 // 8), 31)
    vp = ti.random_bytes((B, Hkv, T, d * 2 // 8), 32)
    kn = ti.random_norms((B, Hkv, T), 33)
    vn = ti.random_norms((B, Hkv, T), 34, median=11.0)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, kp.to(dev), kn.to(dev), vp.to(dev), vn.to(dev),
                            out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    rowsb = [0, 31]
    khat = oatt.decode_cache(kp[rowsb].numpy(), kn[rowsb].numpy(), pk[0], ocb.codebook(d, 4).centroids, 4, d)
    vhat = oatt.decode_cache(vp[rowsb].numpy(), vn[rowsb].numpy(), pv[0], ocb.codebook(d, 2).centroids, 2, d)
    check_attention(o[rowsb].cpu().numpy().astype(np.float64), lse[rowsb].cpu().numpy(), to64(q[rowsb]), khat, vhat,
                    1 / math.sqrt(d), [T, T], "attn workload")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_paged_ragged_workload(dev, d):
    """256 sequences, lengths U[1, 16384], block 16, 8 KV heads / 32 query heads, 1% of tokens
    x50; one layer per head size with its own (K, V) widths; sampled oracle checks."""
    layer = {64: 1, 128: 5, 256: 7}[d]
    bk, bv = ti.paged_layer_bits(layer)
    log("case: paged ragged workload d%d layer %d K%dV%d" % (d, layer, bk, bv))
    shape = ti.PagedShape()
    lay0 = ti.paged_layout(shape, seed=layer)
    lens = lay0.seq_lens.numpy()
    seqs = [int(np.argmin(lens)), int(np.argmax(lens)), 17, 100]
    c = _paged(dev, shape.sequences, shape.max_len, shape.kv_heads, shape.q_heads, d, bk, bv, seed=layer,
               oracle_rows=seqs)
    lay = c["lay"]
    o = tq.attn_decode(c["ck"], c["rk"], c["cv"], c["rv"], c["q"], c["kp"], c["kn"], c["vp"], c["vn"],
                       seq_lens=lay.seq_lens.to(dev), max_seq_len=int(lay.seq_lens.max()),
                       block_table=lay.block_table.to(dev), block_size=16, out_dtype=torch.float32,
                       num_kv_heads=shape.kv_heads)
    torch.cuda.synchronize()
    # codec parity on sampled (token, head) vectors of the GPU-written pool
    n = c["slot"].numel()
    idx = torch.randperm(n, generator=ti.generator("cpu", d))[:2048].to(dev)
    slots = c["slot"][idx]
    kflat = c["k"].view(-1, d)
    check_encode(to64(kflat[idx]), c["gkp"][slots].cpu().numpy(), c["gkn"][slots].cpu().numpy(), c["pk"], d, bk,
                 "paged K d%d" % d)
    # gather decode through a slot mapping, over the rows of the checked sequences (random bytes)
    kp_h = c["kp_host"].reshape(-1, c["kp_host"].shape[-1])
    kn_h = c["kn_host"].reshape(-1)
    lay_slots = torch.cat([c["slot"].view(-1, shape.kv_heads)[int(lay.seq_starts[s_]):int(lay.seq_starts[s_ + 1])]
                           .reshape(-1) for s_ in seqs[2:]])
    dec = tq.decode(c["ck"], c["rk"], c["kp"].view(-1, c["kp"].shape[-1]), c["kn"].view(-1),
                    slot_mapping=lay_slots, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ls = lay_slots.cpu().numpy()
    check_decode(dec, kp_h[ls], kn_h[ls], c["pk"], d, bk, "paged K gather decode d%d" % d)
    _check_paged(c, d, bk, bv, o.cpu().numpy().astype(np.float64), None, seqs, "paged ragged d%d" % d)
    # paged scores of the checked sequences (one query per sequence, all 32 heads)
    sc = tq.scores_compressed(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], seq_lens=lay.seq_lens.to(dev),
                              max_seq_len=int(lay.seq_lens.max()), block_table=lay.block_table.to(dev),
                              block_size=16, num_kv_heads=shape.kv_heads)
    torch.cuda.synchronize()
    got = {s_: sc[s_].cpu().numpy().astype(np.float64) for s_ in seqs}
    del sc
    _check_paged_scores(c, d, bk, got, seqs, "paged ragged d%d scores" % d)


def test_attention_softmax_margins(dev):
    # The fused kernel moves its running max and running value-norm max only past a margin and
    # folds 1/N into the exponent; these caches drive both paths hard: logits that keep growing
    # along the sequence, isolated large-logit spikes, value norms that grow 1.02x per token (many
    # 16x steps), leading blocks of zero value norms (N taken as 1), subnormal value norms, and a
    # head whose values are all zero. Codes are random bytes; norms and queries are seeded.
    d, bk, bv, B, Hq, Hkv, T = 128, 4, 2, 3, 8, 2, 700
    log("case: attention softmax margins")
    kp = ti.random_bytes((B, Hkv, T, d * bk // 8), 31, dev)
    vp = ti.random_bytes((B, Hkv, T, d * bv // 8), 32, dev)
    t = np.arange(T, dtype=np.float64)
    kn = np.ones((B, Hkv, T), np.float32)
    vn = np.ones((B, Hkv, T), np.float32)
    kn[0] = (1.0 + 0.05 * t).astype(np.float32)
    kn[1, :, ::50] = 40.0
    kn[2] = ti.random_norms((Hkv, T), 34).numpy()
    vn[0] = (1.02 ** t).astype(np.float32)
    vn[1, :, :64] = 0.0
    vn[2, 0, :32] = np.float32(1e-39)
    vn[2, 1, :] = 0.0
    q = ti.normal((B, Hq, d), 33, scale=4.0, dtype=torch.bfloat16, device=dev)
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    o, lse = tq.attn_decode(ck, rk, cv, rv, q, kp, upload(kn, dev), vp, upload(vn, dev), out_dtype=torch.float32,
                            return_lse=True)
    torch.cuda.synchronize()
    khat = oatt.decode_cache(kp.cpu().numpy(), kn, pk[0], ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vp.cpu().numpy(), vn, pv[0], ocb.codebook(d, bv).centroids, bv, d)
    s_ref = oatt.scores(to64(q), khat, 1 / math.sqrt(d))
    log("softmax margins: score range %.1f .. %.1f" % (float(s_ref.min()), float(s_ref.max())))
    o64 = o.cpu().numpy().astype(np.float64)
    assert np.all(o64[2, 4:] == 0.0)          # query heads of the all-zero value head
    check_attention(o64, lse.cpu().numpy(), to64(q), khat, vhat, 1 / math.sqrt(d), [T] * B, "softmax margins")


@pytest.mark.parametrize("splits", [0, 16])
def test_attention_one_round_and_more(dev, splits):
    # splits 0: the grid is one round of resident waves (issue priorities by progress);
    # 16 splits over 128 (sequence, KV head) pairs: more waves than fit at once (no priorities)
    d, bk, bv, B, Hq, Hkv, T = 128, 4, 2, 16, 32, 8, 512
    log("case: attention %s" % ("one round" if splits == 0 else "%d splits" % splits))
    kp = ti.random_bytes((B, Hkv, T, d * bk // 8), 41, dev)
    vp = ti.random_bytes((B, Hkv, T, d * bv // 8), 42, dev)
    kn = ti.random_norms((B, Hkv, T), 43, median=2.0, device=dev)
    vn = ti.random_norms((B, Hkv, T), 44, device=dev)
    q = ti.normal((B, Hq, d), 45, dtype=torch.bfloat16, device=dev)
    rk, pk = rotation_pair(d, [42])
    rv, pv = rotation_pair(d, [542])
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    lens = torch.tensor([(T * (i + 3)) // 19 for i in range(B)], dtype=torch.int32, device=dev)
    o = tq.attn_decode(ck, rk, cv, rv, q, kp, kn, vp, vn, seq_lens=lens, out_dtype=torch.float32, num_splits=splits)
    torch.cuda.synchronize()
    khat = oatt.decode_cache(kp.cpu().numpy(), kn.cpu().numpy(), pk[0], ocb.codebook(d, bk).centroids, bk, d)
    vhat = oatt.decode_cache(vp.cpu().numpy(), vn.cpu().numpy(), pv[0], ocb.codebook(d, bv).centroids, bv, d)
    check_attention(o.cpu().numpy().astype(np.float64), None, to64(q), khat, vhat, 1 / math.sqrt(d),
                    lens.cpu().numpy(), "splits %d" % splits)


def test_attention_dense_length_limit(dev):
    # dense caches are addressed with 32-bit byte offsets per (sequence, KV head): a row span of
    # 4 GiB or more is refused before any launch
    d = 128
    rk, _ = rotation_pair(d, [42])
    rv, _ = rotation_pair(d, [542])
    ck, cv = tq.Codebook(d, 4), tq.Codebook(d, 2)
    q = torch.zeros(1, 8, d, dtype=torch.bfloat16, device=dev)
    kp = torch.zeros(1, 2, 8, d * 4 // 8, dtype=torch.uint8, device=dev)
    vp = torch.zeros(1, 2, 8, d * 2 // 8, dtype=torch.uint8, device=dev)
    kn = torch.zeros(1, 2, 8, device=dev)
    p = tq._params(ck, rk, q, kp, kn, cv, rv, vp, kn)
    p.max_seq_len = 1 << 26                  # 64-byte key rows: exactly 4 GiB
    with pytest.raises(tq.TQError, match="too long for a dense cache"):
        tq.attn_workspace_size(p)
    p.max_seq_len = (1 << 26) - 1
    assert tq.attn_workspace_size(p) > 0
