"""tq_attn_decode_noalloc (static scratch, no allocation) against tq_attn_decode (caller workspace),
through the C ABI: two calls in a row, the second with a smaller input, each compared with the
workspace entry point's output on the same parameters (same kernels and split count, so the
outputs must be identical bit for bit); an oversized call is refused before any launch."""

import ctypes as C

import pytest
import torch

import tq_inputs as ti

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")
from kv_cache_vector_encode_amd import _lib  # noqa: E402


def _case(dev, B, Hq, Hkv, T, d, bk, bv, seed):
    rk = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 42 + seed))
    rv = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 542 + seed))
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kp = ti.random_bytes((B, Hkv, T, d * bk // 8), 31 + seed, dev)
    vp = ti.random_bytes((B, Hkv, T, d * bv // 8), 32 + seed, dev)
    kn = ti.random_norms((B, Hkv, T), 33 + seed, median=2.0, device=dev)
    vn = ti.random_norms((B, Hkv, T), 34 + seed, device=dev)
    q = ti.normal((B, Hq, d), 35 + seed, dtype=torch.bfloat16, device=dev)
    lens = torch.tensor([max(1, (T * (i + 2)) // (B + 1)) for i in range(B)], dtype=torch.int32, device=dev)
    return dict(ck=ck, rk=rk, cv=cv, rv=rv, q=q, kp=kp, kn=kn, vp=vp, vn=vn, lens=lens)


def _run_both(c, dev):
    B, Hq, d = c["q"].shape
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
        p = tq._params(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], c["cv"], c["rv"], c["vp"], c["vn"],
                       seq_lens=c["lens"], out=out, lse=lse)
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        if noalloc:
            st = _lib.lib().tq_attn_decode_noalloc(C.byref(p), stream)
        else:
            ws = torch.empty(tq.attn_workspace_size(p), dtype=torch.uint8, device=dev)
            p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
            st = _lib.lib().tq_attn_decode(C.byref(p), stream)
        _lib.check(st)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    return outs


def test_noalloc_matches_workspace_call_twice():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # first call: 4 sequences x 8 KV heads, 3000 tokens, d=128, K4/V2
    big = _case(dev, 4, 32, 8, 3000, 128, 4, 2, 0)
    (o1, l1), (o2, l2) = _run_both(big, dev)
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # second call, smaller: 2 sequences x 2 KV heads, 500 tokens, d=64, K3/V3 (the scratch still
    # holds the first call's partials; nothing in it has to start at zero)
    small = _case(dev, 2, 8, 2, 500, 64, 3, 3, 1)
    (o3, l3), (o4, l4) = _run_both(small, dev)
    assert torch.isfinite(o3).all() and torch.isfinite(l3).all()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_noalloc_refuses_oversized_calls():
    dev = torch.device("cuda:0")
    c = _case(dev, 2, 16, 4, 64, 128, 4, 2, 2)
    out = torch.empty(2, 16, 128, dtype=torch.float32, device=dev)
    p = tq._params(c["ck"], c["rk"], c["q"], c["kp"], c["kn"], c["cv"], c["rv"], c["vp"], c["vn"], out=out)
    p.num_splits = 4096          # 4096 partials x 2 x 16 heads x 130 floats: ~68 MB > 32 MiB
    assert tq.attn_workspace_size(p) > 32 << 20
    st = _lib.lib().tq_attn_decode_noalloc(C.byref(p), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -5 and "static scratch holds" in _lib.last_error()
