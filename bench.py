"""Benchmark of the TurboQuant KV-cache codec hot path on one MI355X.

Headline workload (N=1): a 70B-class GQA cache at 128K context - 80 layers x 8 KV heads x
131072 tokens x d=128, bf16, keys and values sigma * N(0,1) with a log-normal(0, 0.5)
per-channel sigma, 3-bit keys and values (codes packed across byte boundaries), one seeded key
rotation and one value rotation per layer. All inputs are synthetic and resident in HBM (40 GiB
of bf16 K and V) before timing.

One step = one pass of the whole hot path over the cache, streamed one layer at a time: for
each of the 80 layers, encode K and V (norm, rotation, Lloyd-Max quantization, 3-bit packing)
into the layer's compressed cache, decode K and V back to bf16, and run one fused decode
attention step (64 query heads over the 8 KV heads, GQA 8:1, one query per head) reading the
keys and values straight from the compressed cache.
value = fp16 bytes through the codec per second: every vector is encoded from 256 B of bf16 and
decoded to 256 B of bf16 once per step, so value = 2 x 80 x 2 x 1,048,576 x 256 B / step time
(GB/s, 1e9); the attention pass is inside the step time.

Printed: ONE JSON line with the driver's fields, a roofline object for the dominant kernel (its
algorithmic bytes / its mean duration from HIP events recorded inside the timed region on the
launch stream), the MFMA rate of the encode rotation, per-kernel figures, the other workloads
as separate keys (the Llama-3-8B-shaped cache, batch-32 fused attention at 32K context, the
paged ragged cache at d = 64/128/256, the 4096-vector codec check latency, the rows beside the
hot path), and the oracle timed on the host cores on a bounded sample (cpu_baseline: one core
and all cores, CPU model stated).
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import multiprocessing as mp
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV encode/decode GB/s in (fp16) + compressed-decode attn tokens/s; % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
Q_HEADS_70B = 64          # 70B-class GQA: 64 query heads over 8 KV heads


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the 70B-class headline step (for profiling runs)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the figures of the rows beside the hot path (window, Hadamard, QJL, group quant)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for scaling HBM byte counters)")
    ap.add_argument("--attention-32k-only", action="store_true",
                    help="profiling mode: time only the batch-32 x 32768-token fused decode attention and print "
                         "its record (not the bench line)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_vector_encode_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_70b_128k.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != src_hash:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def _frac(bytes_, ms):
    return round(bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)


def _gbs(bytes_, ms):
    return round(bytes_ / (ms * 1e-3) / 1e9, 1)


class Calls:
    """libtq calls with their ctypes arguments built once (marshalling only), so that the timed
    loop spends microseconds per launch on the host."""

    def __init__(self, tq, torch):
        self.lib = tq._lib.lib()
        self.check = tq._lib.check
        self.stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def encode(self, cb, rot, x, packed, norms):
        n, d = x.numel() // x.shape[-1], x.shape[-1]
        tq_dt = 1  # TQ_BF16
        a = (cb.handle, rot.handle, C.c_int64(0), C.c_void_p(x.data_ptr()), tq_dt, C.c_int64(n), C.c_int64(d),
             C.c_void_p(packed.data_ptr()), C.c_void_p(norms.data_ptr()), None, self.stream)
        fn, chk = self.lib.tq_encode, self.check
        return lambda: chk(fn(*a))

    def decode(self, cb, rot, packed, norms, out):
        n = out.shape[0]
        a = (cb.handle, rot.handle, C.c_int64(0), C.c_void_p(packed.data_ptr()), C.c_void_p(norms.data_ptr()), None,
             C.c_int64(n), C.c_void_p(out.data_ptr()), 1, self.stream)
        fn, chk = self.lib.tq_decode, self.check
        return lambda: chk(fn(*a))

    def attention(self, p):
        ref = C.byref(p)
        fn, chk, st = self.lib.tq_attn_decode, self.check, self.stream
        return lambda: chk(fn(ref, st))


def headline_70b(args, tq, ti, torch, dev):
    shape = ti.LongCacheShape()
    L, H, T, d = shape.layers, shape.kv_heads, shape.tokens, shape.head_dim
    bk, bv = shape.key_bits, shape.value_bits
    n = H * T                                   # vectors per layer and tensor
    print("bench: generating the %d-layer 70B-class cache on the GPU (%.1f GiB of bf16 K and V)"
          % (L, 2 * L * n * d * 2 / 2 ** 30), file=sys.stderr, flush=True)
    K = torch.empty(L, H, T, d, dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for l in range(L):
        ti.long_cache_layer_kv(shape, l, device=dev, out_k=K[l], out_v=V[l])
    torch.cuda.synchronize()
    rk = [tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.key_seed(l))) for l in range(L)]
    rv = [tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.value_seed(l))) for l in range(L)]
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    kp = torch.empty(L, H, T, d * bk // 8, dtype=torch.uint8, device=dev)
    vp = torch.empty(L, H, T, d * bv // 8, dtype=torch.uint8, device=dev)
    kn = torch.empty(L, H, T, device=dev)
    vn = torch.empty(L, H, T, device=dev)
    ko = torch.empty(n, d, dtype=torch.bfloat16, device=dev)     # decoded layer (reused per layer)
    vo = torch.empty_like(ko)
    Hq = Q_HEADS_70B
    q = ti.normal((L, 1, Hq, d), 7, dtype=torch.bfloat16, device=dev)
    ao = torch.empty(L, 1, Hq, d, dtype=torch.bfloat16, device=dev)
    c = Calls(tq, torch)
    params, keep = [], []
    for l in range(L):
        p = tq._params(ck, rk[l], q[l], kp[l:l + 1], kn[l:l + 1], cv, rv[l], vp[l:l + 1], vn[l:l + 1], out=ao[l])
        ws = torch.empty(tq.attn_workspace_size(p), dtype=torch.uint8, device=dev)
        p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
        params.append(p)
        keep.append(ws)
    layer_calls = []
    for l in range(L):
        layer_calls.append([
            c.encode(ck, rk[l], K[l], kp[l], kn[l]),
            c.encode(cv, rv[l], V[l], vp[l], vn[l]),
            c.decode(ck, rk[l], kp[l], kn[l], ko),
            c.decode(cv, rv[l], vp[l], vn[l], vo),
            c.attention(params[l]),
        ])
    # event pairs bracket the encode pair (K then V), the decode pair and the attention call of
    # every layer; the calibration pass uses them to find the dominant kind, the timed steps
    # record only the dominant kind's pair (a recorded event costs a few us of idle GPU time)
    kinds = ["encode", "decode", "attention"]
    spans = {"encode": (0, 2), "decode": (2, 4), "attention": (4, 5)}

    def step(ev=None, only=None):
        for l in range(L):
            calls = layer_calls[l]
            for kind in kinds:
                a, b = spans[kind]
                rec = ev is not None and (only is None or kind == only)
                if rec:
                    ev[kind][l][0].record()
                for i in range(a, b):
                    calls[i]()
                if rec:
                    ev[kind][l][1].record()

    def events(only=None):
        return {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
                for k in kinds if only is None or k == only}

    for _ in range(args.warmup):
        step()
    cal = [events() for _ in range(2)]
    for e in cal:
        step(e)
    torch.cuda.synchronize()
    per = {k: sum(sum(a.elapsed_time(b) for a, b in e[k]) for e in cal) / len(cal) for k in kinds}   # ms per step
    dom = max(kinds, key=lambda k: per[k])
    evs = [events(dom) for _ in range(args.steps)]
    print("bench: timing %d steps (dominant kind: %s)" % (args.steps, dom), file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s], only=dom)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    launches = {"encode": 2, "decode": 2, "attention": 1}[dom]
    dom_ms_launch = sum(sum(a.elapsed_time(b) for a, b in e[dom]) for e in evs) / (args.steps * L * launches)

    fp16_bytes = 2 * L * n * d * 2                       # K and V of all layers in 16-bit form
    value = 2 * fp16_bytes / (ms_step * 1e-3) / 1e9       # encoded + decoded
    enc_b = n * (d * 2 + d * bk // 8 + 4)                 # per launch (K; V is the same at 3 bits)
    dec_b = n * (d * bk // 8 + 4 + d * 2)
    att_b = n * (d * bk // 8 + 4) + n * (d * bv // 8 + 4) + 2 * Hq * d * 2
    alg = {"encode": enc_b, "decode": dec_b, "attention": att_b}
    kname = {"encode": "encode_kernel<128,3,bf16>", "decode": "decode_kernel<128,3,bf16>",
             "attention": "qrot + attn_kernel<128,3,3> + merge"}
    kernels = {}
    for k in kinds:
        ms_launch = per[k] / (L * {"encode": 2, "decode": 2, "attention": 1}[k])
        kernels[k] = {"ms_per_launch": round(ms_launch, 4), "alg_bytes_per_launch": alg[k],
                      "GB/s": _gbs(alg[k], ms_launch), "hbm_frac": _frac(alg[k], ms_launch),
                      "ms_per_step": round(per[k], 3)}
    kernels["attention"]["context_tokens_per_s"] = round(T / (kernels["attention"]["ms_per_launch"] * 1e-3), 1)
    kernels["encode"]["vectors_per_s"] = round(n / (kernels["encode"]["ms_per_launch"] * 1e-3), 1)
    kernels["decode"]["vectors_per_s"] = round(n / (kernels["decode"]["ms_per_launch"] * 1e-3), 1)
    # MFMA work of the encode rotation: 2 bf16 passes (Pi = Pi_hi + Pi_lo) x 2 d^2 flops per vector
    enc_ms = kernels["encode"]["ms_per_launch"]
    mfma_tf = n * 2 * 2 * d * d / (enc_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    achieved = alg[dom] / (dom_ms_launch * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(dom, src_hash),
                "kernel": kname[dom], "alg_bytes_per_launch": alg[dom], "mean_launch_ms": round(dom_ms_launch, 4)}
    res = {
        "value": round(value, 1), "ms_per_step": round(ms_step, 4), "roofline": roofline, "kernels": kernels,
        "mfma_rotation": {"kernel": kname["encode"], "TFLOP/s": round(mfma_tf, 1),
                          "frac_bf16_peak": round(mfma_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "flops_per_vector": 2 * 2 * d * d,
                          "note": "algorithmic MFMA flops (2 bf16 passes of 2 d^2) / event time; counter "
                                  "check in profiles/"},
        "encode_decode_GBps_fp16": round(2 * fp16_bytes / ((per["encode"] + per["decode"]) * 1e-3) / 1e9, 1),
        "attn_context_tokens_per_s": kernels["attention"]["context_tokens_per_s"],
        "ms_80_layers": {k: round(per[k], 3) for k in kinds},
        "source_hash": src_hash,
    }
    del K, V, kp, vp, kn, vn, ko, vo, keep, params, layer_calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _time(torch, fn, reps: int = 10):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def llama8b_cache(tq, ti, torch, dev, with_next: bool):
    """The Llama-3-8B-shaped cache: 32 layers x 8 KV heads x 8192 tokens x d=128 bf16, K4/V2, one
    shared rotation per layer; one launch per tensor over the 32-rotation stack, and one fused
    decode attention step (32 query heads per layer; the layers form the batch)."""
    shape = ti.LlamaCacheShape()
    L, H, T, d = shape.layers, shape.kv_heads, shape.tokens, shape.head_dim
    bk, bv = shape.key_bits, shape.value_bits
    Hq, N = 32, L * H * T
    K = torch.empty(L, H, T, d, dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for l in range(L):
        ti.llama_layer_kv(shape, l, device=dev, out_k=K[l], out_v=V[l])
    rot = tq.Rotation.from_gaussian(ti.rotation_gaussians(d, [ti.key_seed(l) for l in range(L)]))
    ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
    vpr = H * T
    kp = torch.empty(N, d * bk // 8, dtype=torch.uint8, device=dev)
    vp = torch.empty(N, d * bv // 8, dtype=torch.uint8, device=dev)
    kn = torch.empty(N, device=dev)
    vn = torch.empty(N, device=dev)
    ko = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    q = ti.normal((L, Hq, d), 7, dtype=torch.bfloat16, device=dev)
    ao = torch.empty(L, Hq, d, dtype=torch.bfloat16, device=dev)
    kp4, kn4 = kp.view(L, H, T, -1), kn.view(L, H, T)
    vp4, vn4 = vp.view(L, H, T, -1), vn.view(L, H, T)
    p = tq._params(ck, rot, q, kp4, kn4, cv, rot, vp4, vn4, batch_per_rot=1, out=ao)
    ws = torch.empty(tq.attn_workspace_size(p), dtype=torch.uint8, device=dev)
    calls = {
        "encode_k": lambda: tq.encode(ck, rot, K, vectors_per_rot=vpr, packed=kp, norms=kn),
        "encode_v": lambda: tq.encode(cv, rot, V, vectors_per_rot=vpr, packed=vp, norms=vn),
        "decode_k": lambda: tq.decode(ck, rot, kp, kn, vectors_per_rot=vpr, out=ko),
        "decode_v": lambda: tq.decode(cv, rot, vp, vn, vectors_per_rot=vpr, out=vo),
        "attention": lambda: tq.attn_decode(ck, rot, cv, rot, q, kp4, kn4, vp4, vn4, batch_per_rot=1, out=ao,
                                            workspace=ws),
    }
    alg = {
        "encode_k": N * (d * 2 + d * bk // 8 + 4), "encode_v": N * (d * 2 + d * bv // 8 + 4),
        "decode_k": N * (d * bk // 8 + 4 + d * 2), "decode_v": N * (d * bv // 8 + 4 + d * 2),
        "attention": N * (d * bk // 8 + 4) + N * (d * bv // 8 + 4) + 2 * L * Hq * d * 2,
    }
    # one pass in step order (warm), then per-call events over 5 steps, each call cold as in the step
    for f in calls.values():
        f()
    torch.cuda.synchronize()
    ev = {k: [] for k in calls}
    for _ in range(5):
        for k, f in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            ev[k].append((e0, e1))
    torch.cuda.synchronize()
    out = {"workload": "llama3-8b-shaped cache, 32 layers x 8 KV heads x 8192 tokens x d=128 bf16, K4/V2, "
                       "shared rotation per layer; one launch per tensor over the rotation stack"}
    for k in calls:
        ms = sorted(a.elapsed_time(b) for a, b in ev[k])[len(ev[k]) // 2]
        out[k] = {"ms": round(ms, 4), "GB/s": _gbs(alg[k], ms), "hbm_frac": _frac(alg[k], ms)}
    out["attention"]["context_tokens_per_s"] = round(L * T / (out["attention"]["ms"] * 1e-3), 1)
    nxt = None
    if with_next:
        nxt = next_rows(tq, ti, torch, dev, K, V, kp, kn, vp, vn, rot, ck, cv, q, kp4, kn4, vp4, vn4, ws, L, H, T,
                        d, out["attention"]["ms"])
    del K, V, ko, vo, kp, vp, kn, vn
    torch.cuda.empty_cache()
    return out, nxt


def next_rows(tq, ti, torch, dev, K, V, kp, kn, vp, vn, rot, ck, cv, q, kp4, kn4, vp4, vn4, ws, L, H, T, d,
              attn_ms):
    """Figures for the rows beside the hot path, on the Llama-3-8B-shaped cache: the recent-token
    window (attention over 8064 compressed + 128 full-precision tokens per sequence, and a
    one-token append that flushes one token per (layer, KV head)), the Hadamard rotation and the
    norm-corrected encode (keys, 4 bits), QJL keys at 4 bits (encode and decode attention), and
    affine group quantization of the values (2 bits, groups of 32)."""
    N = L * H * T
    out = {}
    rh = tq.Rotation.hadamard(d, ti.random_signs(L, d, 1))
    ms = _time(torch, lambda: tq.encode(ck, rh, K, vectors_per_rot=H * T, packed=kp, norms=kn))
    alg = N * (d * 2 + d // 2 + 4)
    out["hadamard_encode_k"] = {"ms": round(ms, 4), "GB/s": _gbs(alg, ms), "hbm_frac": _frac(alg, ms)}
    ms = _time(torch, lambda: tq.encode(ck, rot, K, vectors_per_rot=H * T, packed=kp, norms=kn,
                                        norm_correction=True))
    out["norm_corrected_encode_k"] = {"ms": round(ms, 4), "GB/s": _gbs(alg, ms), "hbm_frac": _frac(alg, ms)}
    tq.encode(ck, rot, K, vectors_per_rot=H * T, packed=kp, norms=kn)   # restore the keys' cache
    cq = tq.Codebook(d, 3)
    sk = tq.QJLSketch(rot, torch.stack([ti.qjl_sketch_gaussian(d, ti.key_seed(l)) for l in range(L)]))
    qp = torch.empty(N, d * 3 // 8, dtype=torch.uint8, device=dev)
    qn = torch.empty(N, device=dev)
    qs = torch.empty(N, d // 8, dtype=torch.uint8, device=dev)
    qr = torch.empty(N, device=dev)
    ms = _time(torch, lambda: tq.qjl_encode(cq, sk, K, vectors_per_rot=H * T, packed=qp, norms=qn, signs=qs,
                                            rnorms=qr))
    alg = N * (d * 2 + d * 3 // 8 + 4 + d // 8 + 4)
    flops = N * 5 * 2 * d * d    # MFMA work: rotation (2 bf16 passes) + sketch product (3 passes)
    out["qjl_encode_k4"] = {"ms": round(ms, 4), "GB/s": _gbs(alg, ms), "hbm_frac": _frac(alg, ms),
                            "mfma_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                            "mfma_frac_bf16": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    ao_q = torch.empty(L, q.shape[1], d, dtype=torch.bfloat16, device=dev)
    qv = dict(qjl=sk, k_signs=qs.view(L, H, T, -1), k_rnorms=qr.view(L, H, T))
    tq.attn_decode(cq, rot, cv, rot, q, qp.view(L, H, T, -1), qn.view(L, H, T), vp4, vn4, batch_per_rot=1, out=ao_q,
                   **qv)
    wsq = ao_q._tq_workspace
    ms = _time(torch, lambda: tq.attn_decode(cq, rot, cv, rot, q, qp.view(L, H, T, -1), qn.view(L, H, T), vp4, vn4,
                                             batch_per_rot=1, out=ao_q, workspace=wsq, **qv))
    alg = N * (d * 3 // 8 + 4 + d // 8 + 4) + N * (d * cv.bits // 8 + 4) + 2 * L * q.shape[1] * d * 2
    out["qjl_attention_k4v2"] = {"ms": round(ms, 4), "context_tokens_per_s": round(L * T / (ms * 1e-3), 1),
                                 "hbm_frac": _frac(alg, ms), "plain_k4_attention_ms": round(attn_ms, 4)}
    del qp, qn, qs, qr, ao_q, wsq
    gp = torch.empty(N, d // 4, dtype=torch.uint8, device=dev)
    gs = torch.empty(N, d // 32, dtype=torch.float16, device=dev)
    gz = torch.empty_like(gs)
    go = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    ms_e = _time(torch, lambda: tq.gq_encode(V, 2, packed=gp, scales=gs, zeros=gz))
    ms_d = _time(torch, lambda: tq.gq_decode(gp, gs, gz, 2, out=go))
    ae, ad = N * (d * 2 + d // 4 + 4 * (d // 32)), N * (d // 4 + 4 * (d // 32) + d * 2)
    out["group_quant_v2"] = {"encode_ms": round(ms_e, 4), "encode_hbm_frac": _frac(ae, ms_e),
                             "decode_ms": round(ms_d, 4), "decode_hbm_frac": _frac(ad, ms_d)}
    del gp, gs, gz, go
    R = 128
    kw = K[:, :, T - R:].contiguous()
    vw = V[:, :, T - R:].contiguous()
    ao = torch.empty(L, q.shape[1], d, dtype=torch.bfloat16, device=dev)
    lens = torch.full((L,), T, dtype=torch.int32, device=dev)
    ms = _time(torch, lambda: tq.attn_decode(ck, rot, cv, rot, q, kp4, kn4, vp4, vn4, seq_lens=lens, batch_per_rot=1,
                                             out=ao, k_window=kw, v_window=vw))
    out["window_attention"] = {"window": R, "ms": round(ms, 4), "without_window_ms": round(attn_ms, 4),
                               "context_tokens_per_s": round(L * T / (ms * 1e-3), 1)}
    kn1 = K[:, :, :1].contiguous()
    vn1 = V[:, :, :1].contiguous()
    alen = torch.full((L,), T - 64, dtype=torch.int32, device=dev)
    wsa = tq.window_append(ck, rot, cv, rot, kn1, vn1, kw, vw, alen, kp4, kn4, vp4, vn4, batch_per_rot=1)
    alen.fill_(T - 64)
    ms = _time(torch, lambda: tq.window_append(ck, rot, cv, rot, kn1, vn1, kw, vw, alen, kp4, kn4, vp4, vn4,
                                               batch_per_rot=1, workspace=wsa), reps=20)
    out["window_append_1_token"] = {"batch": L, "kv_heads": H, "us": round(ms * 1e3, 2)}
    return out


def hadamard_fast_transform(tq, ti, torch, dev, reps: int = 10):
    """A Hadamard rotation encodes and decodes by the fast Walsh-Hadamard transform (no
    MFMA), a Haar rotation by the dense MFMA kernels; 1,048,576 bf16 vectors at 3 bits (the 70B-class
    layer's keys at d=128, the same byte count at d=256), each call streaming from HBM."""
    res = {}
    for d in (128, 256):
        n = 1048576
        x = torch.randn(n, d, generator=ti.generator(dev, 77 + d), device=dev).to(torch.bfloat16)
        cb = tq.Codebook(d, 3)
        rots = {"haar_mfma": tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 42)),
                "hadamard_fwht": tq.Rotation.hadamard(d, ti.random_signs(1, d, 5))}
        pk = torch.empty(n, d * 3 // 8, dtype=torch.uint8, device=dev)
        nm = torch.empty(n, device=dev)
        out = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
        alg = n * (d * 2 + d * 3 // 8 + 4)
        rec = {}
        for name, rot in rots.items():
            ms_e = _time(torch, lambda: tq.encode(cb, rot, x, packed=pk, norms=nm), reps)
            ms_d = _time(torch, lambda: tq.decode(cb, rot, pk, nm, out=out), reps)
            rec[name] = {"encode_ms": round(ms_e, 4), "encode_hbm_frac": _frac(alg, ms_e),
                         "decode_ms": round(ms_d, 4), "decode_hbm_frac": _frac(alg, ms_d)}
            if name == "haar_mfma":
                rec[name]["encode_mfma_TFLOPs"] = round(n * 2 * 2 * d * d / (ms_e * 1e-3) / 1e12, 1)
                rec[name]["decode_mfma_TFLOPs"] = round(n * 3 * 2 * d * d / (ms_d * 1e-3) / 1e12, 1)
        res["d%d" % d] = rec
        del x, pk, nm, out
        torch.cuda.empty_cache()
    res["workload"] = "1,048,576 bf16 N(0,1) vectors, 3 bits, per d; Haar (dense MFMA) vs Hadamard (fast transform)"
    return res


def decode_attention_32k(tq, ti, torch, dev, reps: int = 10):
    """Fused decode attention over a long context: batch 32, 32 query heads over 8 KV heads, 32768
    tokens, d=128, K4/V2 (random code bytes with log-normal norms, as in the parity test of this
    size). The 832 MiB cache exceeds the last-level cache, so every call streams it from HBM."""
    shape = ti.AttnShape()
    B, Hq, Hkv, T, d = shape.batch, shape.q_heads, shape.kv_heads, shape.tokens, shape.head_dim
    rk = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 42))
    rv = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 542))
    ck, cv = tq.Codebook(d, 4), tq.Codebook(d, 2)
    kp = ti.random_bytes((B, Hkv, T, d * 4 // 8), 31, device=dev)
    vp = ti.random_bytes((B, Hkv, T, d * 2 // 8), 32, device=dev)
    kn = ti.random_norms((B, Hkv, T), 33, device=dev)
    vn = ti.random_norms((B, Hkv, T), 34, median=11.0, device=dev)
    q = ti.normal((B, Hq, d), 11, dtype=torch.bfloat16, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    tq.attn_decode(ck, rk, cv, rv, q, kp, kn, vp, vn, out=out)
    ws = out._tq_workspace
    ms = _time(torch, lambda: tq.attn_decode(ck, rk, cv, rv, q, kp, kn, vp, vn, out=out, workspace=ws), reps)
    alg = B * Hkv * T * (d * 4 // 8 + 4 + d * 2 // 8 + 4) + 2 * B * Hq * d * 2
    res = {"ms": round(ms, 4), "context_tokens_per_s": round(B * T / (ms * 1e-3), 1), "GB/s": _gbs(alg, ms),
           "hbm_frac": _frac(alg, ms), "decode_steps_per_s": round(1e3 / ms, 1),
           "workload": "batch 32 x 32 query heads over 8 KV heads x 32768 tokens x d=128, K4/V2"}
    del kp, vp, kn, vn
    torch.cuda.empty_cache()
    return res


def paged_ragged(tq, ti, torch, dev):
    """Paged ragged cache: 256 sequences with lengths U[1, 16384], pages of 16 tokens in a seeded
    random order, 8 KV heads, 32 query heads, bf16 N(0,1) tokens with 1% of tokens x50; for each
    head size the nine (K, V) width pairs. Per layer: encode K and V through the slot mapping
    (scatter into the pools), decode K and V back through a gather, and one paged decode
    attention step (one query per sequence)."""
    shape = ti.PagedShape()
    lay = ti.paged_layout(shape, seed=7)
    total = int(lay.seq_starts[-1])
    Hkv, Hq, bs = shape.kv_heads, shape.q_heads, shape.block_size
    heads = torch.arange(Hkv)
    blk, off = lay.token_slots // bs, lay.token_slots % bs
    slot = ((blk[:, None] * Hkv + heads[None, :]) * bs + off[:, None]).reshape(-1).to(dev)
    nslots = lay.num_blocks * Hkv * bs
    n = slot.numel()
    lens, table = lay.seq_lens.to(dev), lay.block_table.to(dev)
    res = {"workload": "256 sequences, lengths U[1,16384] (%d tokens), pages of 16, 8 KV / 32 query heads, "
                       "bf16 N(0,1) with 1%% of tokens x50; per head size the 9 (K,V) width pairs" % total}
    for d in shape.head_dims:
        k, v, _ = ti.paged_layer_tokens(shape, total, d, layer=0, device=dev)
        q = ti.paged_queries(shape, shape.sequences, d, 0, device=dev)
        rk = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.key_seed(0)))
        rv = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.value_seed(0)))
        dec = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
        ao = torch.empty(shape.sequences, Hq, d, dtype=torch.bfloat16, device=dev)
        t_enc = t_dec = t_att = 0.0
        b_enc = b_dec = b_att = 0
        for layer in range(shape.layers_per_dim):
            bk, bv = ti.paged_layer_bits(layer)
            ck, cv = tq.Codebook(d, bk), tq.Codebook(d, bv)
            kp = torch.empty(nslots, d * bk // 8, dtype=torch.uint8, device=dev)
            vp = torch.empty(nslots, d * bv // 8, dtype=torch.uint8, device=dev)
            kn = torch.empty(nslots, device=dev)
            vn = torch.empty(nslots, device=dev)
            enc = lambda: (tq.encode(ck, rk, k, packed=kp, norms=kn, slot_mapping=slot, num_slots=nslots),
                           tq.encode(cv, rv, v, packed=vp, norms=vn, slot_mapping=slot, num_slots=nslots))
            dcd = lambda: (tq.decode(ck, rk, kp, kn, slot_mapping=slot, out=dec),
                           tq.decode(cv, rv, vp, vn, slot_mapping=slot, out=dec))
            kp4, kn4 = kp.view(lay.num_blocks, Hkv, bs, -1), kn.view(lay.num_blocks, Hkv, bs)
            vp4, vn4 = vp.view(lay.num_blocks, Hkv, bs, -1), vn.view(lay.num_blocks, Hkv, bs)
            args = dict(seq_lens=lens, max_seq_len=int(lay.seq_lens.max()), block_table=table, block_size=bs,
                        num_kv_heads=Hkv, out=ao)
            enc()
            tq.attn_decode(ck, rk, cv, rv, q, kp4, kn4, vp4, vn4, **args)
            ws = ao._tq_workspace
            att = lambda: tq.attn_decode(ck, rk, cv, rv, q, kp4, kn4, vp4, vn4, workspace=ws, **args)
            t_enc += _time(torch, enc, 3)
            t_dec += _time(torch, dcd, 3)
            t_att += _time(torch, att, 3)
            b_enc += n * (2 * d * 2 + d * (bk + bv) // 8 + 8) + 2 * n * 8
            b_dec += n * (2 * d * 2 + d * (bk + bv) // 8 + 8) + 2 * n * 8
            b_att += n * (d * (bk + bv) // 8 + 8)
            del kp, vp, kn, vn, kp4, kn4, vp4, vn4, ws
        L9 = shape.layers_per_dim
        res["d%d" % d] = {
            "encode_ms_per_layer": round(t_enc / L9, 4), "encode_GBps_fp16": _gbs(L9 * n * 2 * d * 2, t_enc),
            "encode_hbm_frac": _frac(b_enc, t_enc),
            "decode_ms_per_layer": round(t_dec / L9, 4), "decode_GBps_fp16": _gbs(L9 * n * 2 * d * 2, t_dec),
            "decode_hbm_frac": _frac(b_dec, t_dec),
            "attention_ms_per_layer": round(t_att / L9, 4),
            "attention_context_tokens_per_s": round(L9 * total / (t_att * 1e-3), 1),
            "attention_hbm_frac": _frac(b_att, t_att),
        }
        del k, v, dec, ao
        torch.cuda.empty_cache()
    return res


def codec_check_latency(tq, ti, torch, dev, reps: int = 50):
    """The 4096-vector codec check (fp32 N(0,1), d=128, 4 bits): encode and fp32 decode latency.
    The 2 MiB input sits in the caches, so this is a latency figure, not an HBM one."""
    d = 128
    x = ti.codec_check_inputs().to(dev)
    rot = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, 42))
    cb = tq.Codebook(d, 4)
    pk, nm = tq.encode(cb, rot, x)
    out = torch.empty(4096, d, dtype=torch.float32, device=dev)
    ms_e = _time(torch, lambda: tq.encode(cb, rot, x, packed=pk, norms=nm), reps)
    ms_d = _time(torch, lambda: tq.decode(cb, rot, pk, nm, out=out), reps)
    return {"encode_us": round(ms_e * 1e3, 2), "decode_us": round(ms_d * 1e3, 2),
            "workload": "4096 vectors, d=128, fp32 in / fp32 out, 4 bits (cache-resident; back-to-back launches)"}


# ---- the oracle on the host ---------------------------------------------------------------

def _oracle_warm(_):
    """Imports the oracle's modules in a pool worker (so that the timed map measures work only)."""
    import numpy  # noqa: F401
    import torch  # noqa: F401

    import oracle  # noqa: F401
    import tq_inputs  # noqa: F401
    time.sleep(0.5)
    return os.getpid()


def _oracle_layer_share(args):
    """One process's share of the CPU baseline: encode + decode (to bf16) of the first `n` K and
    `n` V vectors of layer `layer` of the 70B-class cache, then attention (decode the compressed
    K/V, 64 query heads) over the first `tokens` tokens x 8 KV heads of them; float64 numpy on
    one thread. Returns seconds."""
    layer, n, tokens = args
    os.environ["OMP_NUM_THREADS"] = "1"
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import tq_inputs as ti
    from oracle import attention as oatt, codebook as ocb, codec as occ, rotation as orot
    torch.set_num_threads(1)
    shape = ti.LongCacheShape()
    d, H = shape.head_dim, shape.kv_heads
    with threadpool_limits(limits=1):
        k, v = ti.long_cache_layer_kv(shape, layer, device="cpu", tokens=n // H)
        x_k = k.reshape(-1, d).float().numpy().astype(np.float64)
        x_v = v.reshape(-1, d).float().numpy().astype(np.float64)
        pk_ = orot.haar_rotation(ti.rotation_gaussian(d, ti.key_seed(layer)).numpy())
        pv_ = orot.haar_rotation(ti.rotation_gaussian(d, ti.value_seed(layer)).numpy())
        cbk, cbv = ocb.codebook(d, shape.key_bits), ocb.codebook(d, shape.value_bits)
        t0 = time.perf_counter()
        kpk, knk = occ.encode(x_k, pk_, cbk.centroids, shape.key_bits)
        kpv, knv = occ.encode(x_v, pv_, cbv.centroids, shape.value_bits)
        kh = occ.decode(kpk, knk, pk_, cbk.centroids, shape.key_bits, d)
        vh = occ.decode(kpv, knv, pv_, cbv.centroids, shape.value_bits, d)
        occ.cast(kh, torch.bfloat16), occ.cast(vh, torch.bfloat16)
        T = min(tokens, n // H)
        # the cache is [H, tokens, row] per tensor: vectors are token-major within a head here
        khat = oatt.decode_cache(kpk.reshape(H, -1, kpk.shape[-1])[:, :T], knk.reshape(H, -1)[:, :T], pk_,
                                 cbk.centroids, shape.key_bits, d)[None]
        vhat = oatt.decode_cache(kpv.reshape(H, -1, kpv.shape[-1])[:, :T], knv.reshape(H, -1)[:, :T], pv_,
                                 cbv.centroids, shape.value_bits, d)[None]
        q = ti.normal((1, Q_HEADS_70B, d), 5 + layer, dtype=torch.bfloat16).float().numpy().astype(np.float64)
        oatt.attention(q, khat, vhat, 1 / math.sqrt(d))
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(n_vec: int = 262144, tokens: int = 16384, max_cores: int = 16):
    """The oracle as it stands (float64 numpy), on a bounded sample of the headline workload,
    in the headline's unit: fp16 bytes encoded + decoded per second, with an attention step
    inside the time as on the GPU. One core: n_vec K + n_vec V vectors of one layer encoded and
    decoded, plus attention of 64 query heads over `tokens` tokens x 8 KV heads. All cores: one
    such share (a different layer each) per core, all at once. The oracle's work per vector is
    constant, so the rate extrapolates linearly to the whole cache (stated, not measured)."""
    cores = max(1, min(len(os.sched_getaffinity(0)), max_cores))
    t1 = _oracle_layer_share((0, n_vec, tokens))
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_warm, range(cores), chunksize=1)
        t0 = time.perf_counter()
        pool.map(_oracle_layer_share, [(i % 80, n_vec, tokens) for i in range(cores)], chunksize=1)
        tall = time.perf_counter() - t0
    fp16 = 2 * n_vec * 2 * 128 * 2          # K and V vectors, each encoded from and decoded to 256 B
    v1 = fp16 / t1 / 1e9
    vall = cores * fp16 / tall / 1e9
    full = 80 * 2 * 1048576 * 2 * 128 * 2   # the headline step's fp16 bytes
    return {"value": round(v1, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d K + %d V vectors of one layer of the 70B-class cache encoded and decoded to bf16, plus "
                      "decode attention of 64 query heads over %d tokens x 8 KV heads (oracle decode + attend), "
                      "float64 numpy on 1 thread, %.1f s" % (n_vec, n_vec, tokens, t1),
            "all_cores": {"value": round(vall, 6), "unit": "GB/s", "cores": cores, "seconds": round(tall, 2),
                          "sample": "the same share (a different layer each) on %d processes at once" % cores},
            "cpu_model": cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0)),
            "extrapolated_step_s": {"1_core": round(full / (v1 * 1e9), 1),
                                    "%d_cores" % cores: round(full / (vall * 1e9), 1)}}


def copy_probe(torch, dev):
    """A plain 1 GiB device-to-device copy, three times: the reference for scaling the HBM byte
    counters of a profiling run."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def copy_bandwidth(torch, dev, reps: int = 10):
    """Measured HBM rate of a plain 1 GiB device-to-device copy (read + write bytes per copy /
    median event time): what streaming reaches on this machine, beside the 8 TB/s peak."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    ms = sorted(ts)[len(ts) // 2]
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "ms": round(ms, 4),
            "note": "1 GiB device-to-device copy, read + write bytes, median of %d" % reps}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the codec shards by layer or "
              "KV head with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_vector_encode_amd as tq
    import tq_inputs as ti

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.attention_32k_only:
        rec = decode_attention_32k(tq, ti, torch, dev, reps=args.steps)
        if args.copy_probe:
            copy_probe(torch, dev)
        rec["source_hash"] = kernel_source_hash()
        print(json.dumps(rec), flush=True)
        return
    head = headline_70b(args, tq, ti, torch, dev)
    show = lambda name, rec: print("bench: %s %s" % (name, json.dumps(rec)), file=sys.stderr, flush=True)
    show("headline", {k: head[k] for k in ("value", "ms_per_step", "roofline", "kernels", "mfma_rotation")})
    extra = {}
    if not args.headline_only:
        extra["llama8b_cache"], nxt = llama8b_cache(tq, ti, torch, dev, with_next=not args.no_next)
        show("llama8b_cache", extra["llama8b_cache"])
        extra["decode_attention_32k"] = decode_attention_32k(tq, ti, torch, dev)
        show("decode_attention_32k", extra["decode_attention_32k"])
        extra["paged_ragged"] = paged_ragged(tq, ti, torch, dev)
        show("paged_ragged", extra["paged_ragged"])
        extra["codec_check_4096"] = codec_check_latency(tq, ti, torch, dev)
        extra["hbm_copy"] = copy_bandwidth(torch, dev)
        show("hbm_copy", extra["hbm_copy"])
        if nxt is not None:
            nxt["hadamard_fast_transform"] = hadamard_fast_transform(tq, ti, torch, dev)
            show("hadamard_fast_transform", nxt["hadamard_fast_transform"])
        extra["next_rows"] = nxt
    if args.copy_probe:
        copy_probe(torch, dev)
    line = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "70B-class GQA KV cache at 128K context: 80 layers x 8 KV heads x 131072 tokens x "
                               "d=128 bf16, K3/V3 (3-bit codes across byte boundaries), log-normal(0,0.5) channel "
                               "scales, rotation per layer and tensor; step = per layer (streamed): encode K+V, "
                               "decode K+V to bf16, fused decode attention (64 query heads over 8 KV heads)",
                   "layers": 80, "kv_heads": 8, "tokens": 131072, "head_dim": 128, "key_bits": 3, "value_bits": 3,
                   "q_heads": Q_HEADS_70B},
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "kernels_note": "per-launch ms from an untimed calibration pass (2 steps, each layer's encode pair, "
                        "decode pair and attention call bracketed by events)",
        "mfma_rotation": head["mfma_rotation"],
        "encode_decode_GBps_fp16": head["encode_decode_GBps_fp16"],
        "attn_context_tokens_per_s": head["attn_context_tokens_per_s"],
        "ms_80_layers": head["ms_80_layers"],
        **extra,
        "source_hash": head["source_hash"],
    }
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
