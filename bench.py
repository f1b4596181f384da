"""Benchmark of the TurboQuant KV-cache codec hot path on one MI355X.

Workload (N=1): the Llama-3-8B-shaped cache - 32 layers x 8 KV heads x 8192 tokens x d=128,
bf16, keys N(0,1) with 4 of 128 channels x10, values N(0,1), one shared seeded rotation per
layer, keys at 4 bits and values at 2 bits. All inputs are synthetic and resident in HBM
before timing.

One step = one pass of the whole hot path over the cache:
  encode K (one launch over the 32-rotation stack), encode V, decode K -> bf16, decode V -> bf16,
  and one fused decode-attention step reading K and V straight from the compressed cache
  (32 query heads per layer over its 8 KV heads, GQA 4:1; the 32 layers form the batch, each
  with its own rotation).
value = fp16-equivalent KV bytes handled per second: the cache is 2 x 2,097,152 vectors x
256 B = 1 GiB in 16-bit form and each of the three passes (encode, decode, attention) handles
it once, so value = 3 x 1 GiB / step time (GB/s, 1e9).

Printed: ONE JSON line with the driver's fields plus a roofline object for the dominant kernel
(its algorithmic bytes / its mean duration from HIP events on the launch stream), per-kernel
figures, the 70B-class 128K-context per-layer encode/decode rates, and the oracle timed on the
host cores on a bounded sample (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV encode/decode GB/s in (fp16) + compressed-decode attn tokens/s; % HBM peak"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first; the GPU clocks take some tens of steps to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 70B-class per-layer figures")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the figures of the recent-token window, Hadamard rotation, norm-corrected encode "
                         "and group-quantized values")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for scaling HBM byte counters)")
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
    path = os.path.join(ROOT, "profiles", "traffic_llama8b.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != src_hash:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(sample_vectors: int = 327680, attn_tokens: int = 8192):
    """The oracle as it stands, one thread, on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import tq_inputs as ti
    from oracle import attention as oatt, codebook as ocb, codec as occ, rotation as orot

    shape = ti.LlamaCacheShape()
    d = shape.head_dim
    torch.set_num_threads(1)
    with threadpool_limits(limits=1):
        k, v = ti.llama_layer_kv(shape, 0, device="cpu", tokens=sample_vectors // shape.kv_heads)
        x_k = k.reshape(-1, d).float().numpy().astype(np.float64)
        x_v = v.reshape(-1, d).float().numpy().astype(np.float64)
        pi = orot.haar_rotation(ti.rotation_gaussian(d, ti.key_seed(0)).numpy())
        cbk, cbv = ocb.codebook(d, shape.key_bits), ocb.codebook(d, shape.value_bits)
        t0 = time.perf_counter()
        pk, nk = occ.encode(x_k, pi, cbk.centroids, shape.key_bits)
        pv, nv = occ.encode(x_v, pi, cbv.centroids, shape.value_bits)
        t_enc = time.perf_counter() - t0
        t0 = time.perf_counter()
        kh = occ.decode(pk, nk, pi, cbk.centroids, shape.key_bits, d)
        vh = occ.decode(pv, nv, pi, cbv.centroids, shape.value_bits, d)
        occ.cast(kh, torch.bfloat16), occ.cast(vh, torch.bfloat16)
        t_dec = time.perf_counter() - t0
        # attention (the oracle's definition: decode the cache, then attend): one layer's 32
        # query heads over its 8 KV heads, T tokens each
        T = min(attn_tokens, sample_vectors // shape.kv_heads)
        q = ti.normal((1, 32, d), 5, dtype=torch.bfloat16).float().numpy()
        t0 = time.perf_counter()
        khat = oatt.decode_cache(pk.reshape(shape.kv_heads, -1, pk.shape[-1])[:, :T],
                                 nk.reshape(shape.kv_heads, -1)[:, :T], pi, cbk.centroids, shape.key_bits, d)[None]
        vhat = oatt.decode_cache(pv.reshape(shape.kv_heads, -1, pv.shape[-1])[:, :T],
                                 nv.reshape(shape.kv_heads, -1)[:, :T], pi, cbv.centroids, shape.value_bits, d)[None]
        oatt.attention(q.astype(np.float64), khat, vhat, 1 / math.sqrt(d))
        t_att = time.perf_counter() - t0
    n2 = 2 * sample_vectors
    # same definition as the GPU value: each of the 3 passes handles the fp16-equivalent bytes
    secs_per_vec = t_enc / n2 + t_dec / n2 + t_att / (T * shape.kv_heads * 2)
    value = 3 * d * 2 / secs_per_vec / 1e9
    return {"value": round(value, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d K + %d V vectors of layer 0 encoded and decoded, plus attention of 32 query heads "
                      "over %d tokens x 8 KV heads (decode + attend), float64 numpy on 1 thread; rates "
                      "scaled per vector to the GPU value's definition" % (sample_vectors, sample_vectors, T),
            "seconds": round(t_enc + t_dec + t_att, 2)}


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
    shape = ti.LlamaCacheShape()
    L, H, T, d = shape.layers, shape.kv_heads, shape.tokens, shape.head_dim
    bk, bv = shape.key_bits, shape.value_bits
    Hq = 32
    N = L * H * T
    print("bench: generating the %d-layer cache on the GPU" % L, file=sys.stderr, flush=True)
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

    names = ["encode_k", "encode_v", "decode_k", "decode_v", "attention"]
    calls = [
        lambda: tq.encode(ck, rot, K, vectors_per_rot=vpr, packed=kp, norms=kn),
        lambda: tq.encode(cv, rot, V, vectors_per_rot=vpr, packed=vp, norms=vn),
        lambda: tq.decode(ck, rot, kp, kn, vectors_per_rot=vpr, out=ko),
        lambda: tq.decode(cv, rot, vp, vn, vectors_per_rot=vpr, out=vo),
        lambda: tq.attn_decode(ck, rot, cv, rot, q, kp4, kn4, vp4, vn4, batch_per_rot=1, out=ao, workspace=ws),
    ]

    def step(marks=None):
        # marks: {call index: (event before, event after)}; every event is recorded on the
        # stream the library launches on (torch's current stream)
        for i, c in enumerate(calls):
            if marks is not None and i in marks:
                marks[i][0].record()
            c()
            if marks is not None and i in marks:
                marks[i][1].record()

    def new_events(idx):
        return {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in idx}

    for _ in range(args.warmup):
        step()
    # calibration (untimed): every call bracketed by events, to find the dominant kernel and to
    # report the per-call breakdown; a recorded event costs a few us of idle GPU time, so the
    # timed steps below bracket only the dominant call
    cal = [new_events(range(len(calls))) for _ in range(3)]
    for m in cal:
        step(m)
    torch.cuda.synchronize()
    per = {n: sum(m[i][0].elapsed_time(m[i][1]) for m in cal) / len(cal) for i, n in enumerate(names)}
    dom_i = max(range(len(names)), key=lambda i: per[names[i]])
    dom = names[dom_i]
    evs = [new_events([dom_i]) for _ in range(args.steps)]
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    dom_ms = sum(e[dom_i][0].elapsed_time(e[dom_i][1]) for e in evs) / args.steps

    fp16_bytes = 2 * N * d * 2                  # K and V in 16-bit form
    value = 3 * fp16_bytes / (ms_step * 1e-3) / 1e9
    alg = {   # algorithmic HBM bytes per launch
        "encode_k": N * (d * 2 + d * bk // 8 + 4),
        "encode_v": N * (d * 2 + d * bv // 8 + 4),
        "decode_k": N * (d * bk // 8 + 4 + d * 2),
        "decode_v": N * (d * bv // 8 + 4 + d * 2),
        "attention": N * (d * bk // 8 + 4) + N * (d * bv // 8 + 4) + 2 * L * Hq * d * 2,
    }
    kernels = {}
    for n in names:
        gbs = alg[n] / (per[n] * 1e-3) / 1e9
        kernels[n] = {"ms": round(per[n], 4), "alg_bytes": alg[n], "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    kernels["attention"]["tokens_per_s"] = round(L * T / (per["attention"] * 1e-3), 1)
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(dom, src_hash)
    achieved = alg[dom] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "alg_bytes_per_launch": alg[dom], "mean_launch_ms": round(dom_ms, 4)}
    enc_dec_ms = per["encode_k"] + per["encode_v"] + per["decode_k"] + per["decode_v"]
    extra = {
        "encode_decode_GBps_fp16": round(2 * fp16_bytes / (enc_dec_ms * 1e-3) / 1e9, 1),
        "encode_decode_hbm_frac": round(sum(alg[n] for n in names[:4]) / (enc_dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "encode_vectors_per_s": round(2 * N / ((per["encode_k"] + per["encode_v"]) * 1e-3), 1),
        "attn_context_tokens_per_s": round(L * T / (per["attention"] * 1e-3), 1),
    }
    nxt = None if args.no_next else next_rows(tq, ti, torch, dev, K, V, kp, kn, vp, vn, rot, ck, cv, q, kp4, kn4,
                                              vp4, vn4, ws, L, H, T, d, per["attention"])
    del K, V, ko, vo
    torch.cuda.empty_cache()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    long = attn32k = None
    if not args.no_long:
        long = long_context_layer(tq, ti, torch, dev)
        attn32k = decode_attention_32k(tq, ti, torch, dev)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped KV cache, 32 layers x 8 KV heads x 8192 tokens x d=128 bf16, "
                               "K4/V2, one shared rotation per layer; step = encode K+V, decode K+V, fused decode "
                               "attention (32 query heads/layer)",
                   "layers": L, "kv_heads": H, "tokens": T, "head_dim": d, "key_bits": bk, "value_bits": bv,
                   "q_heads": Hq},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": "per-call ms from an untimed calibration pass (3 steps, every call bracketed by events)",
        **extra,
        "long_context_layer": long,
        "decode_attention_32k": attn32k,
        "next_rows": nxt,
        "source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


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


def next_rows(tq, ti, torch, dev, K, V, kp, kn, vp, vn, rot, ck, cv, q, kp4, kn4, vp4, vn4, ws, L, H, T, d,
              attn_ms):
    """Figures for the rows beside the hot path, on the same Llama-3-8B-shaped cache:
    the recent-token window (attention over 8064 compressed + 128 full-precision tokens per
    sequence, and a one-token append that flushes one token per (layer, KV head)), the Hadamard
    rotation and the norm-corrected encode (keys, 4 bits), QJL keys at 4 bits (encode and decode
    attention), and affine group quantization of the values (2 bits, groups of 32)."""
    N = L * H * T
    out = {}
    # Hadamard rotation: same encode kernel, a different Pi
    rh = tq.Rotation.hadamard(d, ti.random_signs(L, d, 1))
    ms = _time(torch, lambda: tq.encode(ck, rh, K, vectors_per_rot=H * T, packed=kp, norms=kn))
    alg = N * (d * 2 + d // 2 + 4)
    out["hadamard_encode_k"] = {"ms": round(ms, 4), "GB/s": round(alg / (ms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    ms = _time(torch, lambda: tq.encode(ck, rot, K, vectors_per_rot=H * T, packed=kp, norms=kn,
                                        norm_correction=True))
    out["norm_corrected_encode_k"] = {"ms": round(ms, 4), "GB/s": round(alg / (ms * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    tq.encode(ck, rot, K, vectors_per_rot=H * T, packed=kp, norms=kn)   # restore the keys' cache
    # QJL keys at 4 bits: 3-bit MSE codes + sign sketch of the residual + residual norm, then
    # decode attention over them (values as in the hot path)
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
    out["qjl_encode_k4"] = {"ms": round(ms, 4), "GB/s": round(alg / (ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "mfma_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                            "mfma_frac_bf16": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4)}
    ao_q = torch.empty(L, q.shape[1], d, dtype=torch.bfloat16, device=dev)
    qv = dict(qjl=sk, k_signs=qs.view(L, H, T, -1), k_rnorms=qr.view(L, H, T))
    tq.attn_decode(cq, rot, cv, rot, q, qp.view(L, H, T, -1), qn.view(L, H, T), vp4, vn4, batch_per_rot=1, out=ao_q, **qv)
    wsq = ao_q._tq_workspace
    ms = _time(torch, lambda: tq.attn_decode(cq, rot, cv, rot, q, qp.view(L, H, T, -1), qn.view(L, H, T), vp4, vn4,
                                             batch_per_rot=1, out=ao_q, workspace=wsq, **qv))
    alg = N * (d * 3 // 8 + 4 + d // 8 + 4) + N * (d * cv.bits // 8 + 4) + 2 * L * q.shape[1] * d * 2
    out["qjl_attention_k4v2"] = {"ms": round(ms, 4), "context_tokens_per_s": round(L * T / (ms * 1e-3), 1),
                                 "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "plain_k4_attention_ms": round(attn_ms, 4)}
    del qp, qn, qs, qr, ao_q, wsq
    # group-quantized values, 2 bits
    gp = torch.empty(N, d // 4, dtype=torch.uint8, device=dev)
    gs = torch.empty(N, d // 32, dtype=torch.float16, device=dev)
    gz = torch.empty_like(gs)
    go = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
    ms_e = _time(torch, lambda: tq.gq_encode(V, 2, packed=gp, scales=gs, zeros=gz))
    ms_d = _time(torch, lambda: tq.gq_decode(gp, gs, gz, 2, out=go))
    ae, ad = N * (d * 2 + d // 4 + 4 * (d // 32)), N * (d // 4 + 4 * (d // 32) + d * 2)
    out["group_quant_v2"] = {"encode_ms": round(ms_e, 4), "encode_hbm_frac": round(ae / (ms_e * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "decode_ms": round(ms_d, 4), "decode_hbm_frac": round(ad / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del gp, gs, gz, go
    # recent-token window of 128 tokens
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
    reps = 20
    alen.fill_(T - 64)
    ms = _time(torch, lambda: tq.window_append(ck, rot, cv, rot, kn1, vn1, kw, vw, alen, kp4, kn4, vp4, vn4,
                                               batch_per_rot=1, workspace=wsa), reps=reps)
    out["window_append_1_token"] = {"batch": L, "kv_heads": H, "us": round(ms * 1e3, 2)}
    return out


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
    res = {"ms": round(ms, 4), "context_tokens_per_s": round(B * T / (ms * 1e-3), 1),
           "GB/s": round(alg / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "workload": "batch 32 x 32 query heads over 8 KV heads x 32768 tokens x d=128, K4/V2"}
    del kp, vp, kn, vn
    torch.cuda.empty_cache()
    return res


def long_context_layer(tq, ti, torch, dev, reps: int = 10):
    """70B-class cache at 128K context, streamed per layer: encode and decode one layer's K and V
    (8 KV heads x 131072 tokens x d=128 bf16, 3 bits each)."""
    shape = ti.LongCacheShape()
    d = shape.head_dim
    K, V = ti.long_cache_layer_kv(shape, 0, device=dev)
    rk = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.key_seed(0)))
    rv = tq.Rotation.from_gaussian(ti.rotation_gaussian(d, ti.value_seed(0)))
    cb = tq.Codebook(d, 3)
    n = K.numel() // d
    kp = torch.empty(n, d * 3 // 8, dtype=torch.uint8, device=dev)
    vp = torch.empty_like(kp)
    kn = torch.empty(n, device=dev)
    vn = torch.empty(n, device=dev)
    ko = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)

    def enc():
        tq.encode(cb, rk, K, packed=kp, norms=kn)
        tq.encode(cb, rv, V, packed=vp, norms=vn)

    def dec():
        tq.decode(cb, rk, kp, kn, out=ko)
        tq.decode(cb, rv, vp, vn, out=vo)

    res = {}
    for name, fn in (("encode", enc), ("decode", dec)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        alg = 2 * n * (d * 2 + d * 3 // 8 + 4)
        res[name] = {"ms_per_layer": round(ms, 4), "GB/s_fp16_in": round(2 * n * d * 2 / (ms * 1e-3) / 1e9, 1),
                     "vectors_per_s": round(2 * n / (ms * 1e-3), 1),
                     "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "ms_80_layers": round(80 * ms, 3)}
    res["workload"] = "70B-class GQA cache at 128K context, one layer: 8 KV heads x 131072 tokens x d=128 bf16, K3/V3"
    return res


if __name__ == "__main__":
    main()
