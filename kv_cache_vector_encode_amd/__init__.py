"""TurboQuant KV-cache codec for AMD MI355X (gfx950): thin Python binding of libtq.

Every computation runs in libtq (C ABI, include/tq.h): the host float64 codebook solver and
QR, and the HIP kernels for encode, decode, compressed scores and fused decode attention.
This module only marshals arguments: torch supplies device memory and the current stream.
There is no CPU fallback; if libtq.so is missing the first call raises.
"""

from __future__ import annotations

import ctypes as C
import math

import numpy as np
import torch

from . import _lib
from ._lib import AttnParams, TQError, TQ_BF16, TQ_F16, TQ_F32, check, lib

__all__ = ["Codebook", "Rotation", "QJLSketch", "encode", "qjl_encode", "decode", "scores_compressed", "attn_decode",
           "attn_decode_noalloc",
           "attn_workspace_size", "packed_row_bytes", "TQError", "TQ_F32", "TQ_BF16", "TQ_F16",
           "dtype_code"]

_DT = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}
_DT_INV = {v: k for k, v in _DT.items()}


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError("unsupported dtype %s; use float32, bfloat16 or float16" % dt)
    return _DT[dt]


def packed_row_bytes(d: int, bits: int) -> int:
    return (d * bits + 7) // 8


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


# ---- argument checks: every tensor the kernels touch is checked before any launch (device,
# dtype, contiguity, shape or size). Values the host cannot see without a device sync (slot
# mapping entries, block table entries, sequence lengths) are the caller's to keep in range,
# as include/tq.h states.

def _tensor(t, name: str, device, dtypes=None, contiguous: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.device.type != "cuda":
        raise ValueError("%s must be a CUDA tensor (got device %s): the kernels read device memory" % (name, t.device))
    if device is not None and t.device.index != device:
        raise ValueError("%s is on cuda:%s but the rotation lives on cuda:%s" % (name, t.device.index, device))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s; accepted %s" % (name, t.dtype, ", ".join(str(d) for d in dtypes)))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _shape(t, name: str, shape):
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s has shape %s; expected %s" % (name, tuple(t.shape), tuple(int(v) for v in shape)))


def _rows(t, name: str, device, row_bytes: int, at_least: int = 0) -> int:
    """A contiguous uint8 tensor read or written as rows of row_bytes bytes; returns the row count."""
    _tensor(t, name, device, (torch.uint8,))
    if t.numel() % row_bytes:
        raise ValueError("%s has %d bytes, not a whole number of %d-byte rows" % (name, t.numel(), row_bytes))
    rows = t.numel() // row_bytes
    if rows < at_least:
        raise ValueError("%s holds %d rows of %d bytes; %d are needed" % (name, rows, row_bytes, at_least))
    return rows


def _floats(t, name: str, device, count: int):
    _tensor(t, name, device, (torch.float32,))
    if t.numel() != count:
        raise ValueError("%s has %d elements; expected %d (float32)" % (name, t.numel(), count))


def _pair(cb: "Codebook", rot: "Rotation", what: str):
    if cb.d != rot.d:
        raise ValueError("%s: codebook d = %d does not match rotation d = %d" % (what, cb.d, rot.d))


def _slots(slot_mapping, device, n: int):
    if slot_mapping is not None:
        _tensor(slot_mapping, "slot_mapping", device, (torch.int64,))
        if slot_mapping.numel() != n:
            raise ValueError("slot_mapping has %d entries; expected one per vector (%d)" % (slot_mapping.numel(), n))


class Codebook:
    """Lloyd-Max codebook for (head_dim d, bits), solved on the host by libtq."""

    def __init__(self, d: int, bits: int):
        h = lib().tq_codebook_init(int(d), int(bits))
        if not h:
            raise TQError(None, _lib.last_error())
        self._h = C.c_void_p(h)
        self.d, self.bits = int(d), int(bits)

    @property
    def handle(self):
        return self._h

    def get(self):
        L = 2 ** self.bits
        c = np.zeros(L)
        t = np.zeros(L - 1)
        m = C.c_double()
        check(lib().tq_codebook_get(self._h, c.ctypes.data_as(C.c_void_p), t.ctypes.data_as(C.c_void_p),
                                    C.byref(m)))
        return c, t, m.value

    @property
    def centroids(self):
        return self.get()[0]

    @property
    def thresholds(self):
        return self.get()[1]

    @property
    def mse(self):
        return self.get()[2]

    def __del__(self):
        h = getattr(self, "_h", None)
        try:
            if h is not None and _lib._LIB is not None:
                _lib._LIB.tq_codebook_free(h)
        except Exception:
            pass
        self._h = None


def rotation_compute(gaussian) -> np.ndarray:
    """Host-only float64 rotation for one float32 Gaussian draw [d, d] (no device)."""
    g = np.ascontiguousarray(np.asarray(gaussian, dtype=np.float32))
    d = g.shape[0]
    out = np.zeros((d, d))
    check(lib().tq_rotation_compute(d, g.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p)))
    return out


class Rotation:
    """A stack of n_rot Haar rotations uploaded to the current HIP device."""

    def __init__(self, handle, d: int, n_rot: int):
        self._h = C.c_void_p(handle)
        self.d, self.n_rot = d, n_rot
        # libtq uploads to the current device, which the handle is then bound to
        self.device = torch.cuda.current_device()

    @classmethod
    def from_gaussian(cls, gaussian):
        """gaussian: float32 [n_rot, d, d] (or [d, d]) standard-normal draws (CPU)."""
        g = torch.as_tensor(gaussian).detach().to("cpu", torch.float32).contiguous()
        if g.dim() == 2:
            g = g[None]
        n, d, _ = g.shape
        h = lib().tq_rotation_from_gaussian(d, n, C.c_void_p(g.data_ptr()))
        if not h:
            raise TQError(None, _lib.last_error())
        return cls(h, d, n)

    @classmethod
    def from_matrix(cls, pi):
        p = np.ascontiguousarray(np.asarray(pi, dtype=np.float64))
        if p.ndim == 2:
            p = p[None]
        n, d, _ = p.shape
        h = lib().tq_rotation_from_matrix(d, n, p.ctypes.data_as(C.c_void_p))
        if not h:
            raise TQError(None, _lib.last_error())
        return cls(h, d, n)

    @classmethod
    def hadamard(cls, d: int, signs=None, n_rot: int | None = None):
        """Pi_r = H_d diag(signs[r]) / sqrt(d) (signs: int8-convertible [n_rot, d] of +-1, or
        None for all +1 with n_rot rotations, default 1)."""
        if signs is None:
            n = 1 if n_rot is None else int(n_rot)
            ptr, keep = None, None
        else:
            keep = np.ascontiguousarray(np.asarray(signs).reshape(-1, d).astype(np.int8))
            n = keep.shape[0]
            ptr = keep.ctypes.data_as(C.c_void_p)
        h = lib().tq_rotation_hadamard(int(d), n, ptr)
        if not h:
            raise TQError(None, _lib.last_error())
        return cls(h, d, n)

    def matrices(self) -> np.ndarray:
        out = np.zeros((self.n_rot, self.d, self.d))
        check(lib().tq_rotation_get(self._h, out.ctypes.data_as(C.c_void_p)))
        return out

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        try:
            if h is not None and _lib._LIB is not None:
                _lib._LIB.tq_rotation_free(h)
        except Exception:
            pass
        self._h = None


class QJLSketch:
    """QJL sketch of a rotation stack: S_r (float32 [n_rot, d, d], one per rotation of `rot`),
    uploaded by libtq as the tiles of S_r Pi_r^T and S_r^T. Keeps `rot` alive."""

    def __init__(self, rot: Rotation, sketch):
        s = torch.as_tensor(sketch).detach().to("cpu", torch.float32).contiguous()
        if s.dim() == 2:
            s = s[None]
        if tuple(s.shape) != (rot.n_rot, rot.d, rot.d):
            raise ValueError("sketch must be [n_rot, d, d] = [%d, %d, %d]" % (rot.n_rot, rot.d, rot.d))
        h = lib().tq_qjl_create(rot.handle, C.c_void_p(s.data_ptr()))
        if not h:
            raise TQError(None, _lib.last_error())
        self._h = C.c_void_p(h)
        self.rot = rot
        self.d, self.n_rot = rot.d, rot.n_rot

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        try:
            if h is not None and _lib._LIB is not None:
                _lib._LIB.tq_qjl_free(h)
        except Exception:
            pass
        self._h = None


def qjl_encode(cb: Codebook, qjl: QJLSketch, x: torch.Tensor, vectors_per_rot: int = 0, packed=None, norms=None,
               signs=None, rnorms=None, slot_mapping=None, num_slots=None, stream=None):
    """QJL key encode of x [..., d] with the MSE codebook cb (max(b-1, 1) bits for b-bit keys).
    Returns (packed uint8 [rows, d*cb.bits/8], norms float32 [rows], signs uint8 [rows, d/8],
    rnorms float32 [rows]); rows as in encode()."""
    _pair(cb, qjl.rot, "qjl_encode")
    x2, n, rows = _encode_input(qjl.rot, x, slot_mapping, num_slots)
    d, dev = qjl.d, x.device
    rb = packed_row_bytes(d, cb.bits)
    if packed is None:
        packed = torch.empty(rows, rb, dtype=torch.uint8, device=dev)
    if norms is None:
        norms = torch.empty(rows, dtype=torch.float32, device=dev)
    if signs is None:
        signs = torch.empty(rows, d // 8, dtype=torch.uint8, device=dev)
    if rnorms is None:
        rnorms = torch.empty(rows, dtype=torch.float32, device=dev)
    rows = _encode_outputs(qjl.rot, packed, norms, rb, n, slot_mapping, num_slots)
    if _rows(signs, "signs", qjl.rot.device, d // 8) != rows:
        raise ValueError("signs must hold one %d-byte row per packed row (%d)" % (d // 8, rows))
    _floats(rnorms, "rnorms", qjl.rot.device, rows)
    check(lib().tq_qjl_encode(cb.handle, qjl.handle, int(vectors_per_rot), _ptr(x2), dtype_code(x2.dtype), n,
                              x2.stride(0), _ptr(packed), _ptr(norms), _ptr(signs), _ptr(rnorms),
                              _ptr(slot_mapping), _stream(stream)))
    return packed, norms, signs, rnorms


def _encode_input(rot: Rotation, x, slot_mapping, num_slots):
    """Checks the encode input x [..., d]; returns (x as [n, d] rows, n, rows of the outputs)."""
    _tensor(x, "x", rot.device, tuple(_DT), contiguous=False)
    if x.dim() < 1 or x.shape[-1] != rot.d:
        raise ValueError("x has shape %s; its last dimension must be the head dim %d" % (tuple(x.shape), rot.d))
    x2 = x.reshape(-1, rot.d) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()      # (row stride and alignment are checked by libtq)
    n = x2.shape[0]
    _slots(slot_mapping, rot.device, n)
    rows = n if slot_mapping is None else (int(num_slots) if num_slots is not None else n)
    return x2, n, rows


def _encode_outputs(rot: Rotation, packed, norms, rb: int, n: int, slot_mapping, num_slots) -> int:
    """Checks packed (rows of rb bytes) and norms (one float32 per row); without a slot mapping
    rows 0..n-1 are written. Returns the row count."""
    rows = _rows(packed, "packed", rot.device, rb, at_least=n if slot_mapping is None else 0)
    if slot_mapping is not None and num_slots is not None and rows != int(num_slots):
        raise ValueError("packed holds %d rows but num_slots = %d" % (rows, int(num_slots)))
    _floats(norms, "norms", rot.device, rows)
    return rows


def encode(cb: Codebook, rot: Rotation, x: torch.Tensor, vectors_per_rot: int = 0, packed=None, norms=None,
           slot_mapping=None, num_slots=None, stream=None, norm_correction: bool = False):
    """x: [..., d] on the GPU (float32/bfloat16/float16; rows may be strided).
    Returns (packed uint8 [rows, d*b/8], norms float32 [rows]); rows = N, or num_slots with a
    slot_mapping (int64 [N]: destination row of each vector, negative = skip).
    norm_correction: store ||x|| / ||c[codes]|| so that the decode keeps ||x||."""
    _pair(cb, rot, "encode")
    x2, n, rows = _encode_input(rot, x, slot_mapping, num_slots)
    rb = packed_row_bytes(rot.d, cb.bits)
    if packed is None:
        packed = torch.empty(rows, rb, dtype=torch.uint8, device=x.device)
    if norms is None:
        norms = torch.empty(rows, dtype=torch.float32, device=x.device)
    _encode_outputs(rot, packed, norms, rb, n, slot_mapping, num_slots)
    fn = lib().tq_encode_norm_corrected if norm_correction else lib().tq_encode
    check(fn(cb.handle, rot.handle, int(vectors_per_rot), _ptr(x2), dtype_code(x2.dtype), n,
             x2.stride(0), _ptr(packed), _ptr(norms), _ptr(slot_mapping), _stream(stream)))
    return packed, norms


def decode(cb: Codebook, rot: Rotation, packed: torch.Tensor, norms: torch.Tensor, n: int | None = None,
           out_dtype=torch.bfloat16, vectors_per_rot: int = 0, slot_mapping=None, out=None, stream=None):
    """Returns out [n, d] (out_dtype): row i decodes packed row slot_mapping[i] (or i)."""
    _pair(cb, rot, "decode")
    d, dev = rot.d, rot.device
    rb = packed_row_bytes(d, cb.bits)
    if slot_mapping is not None:
        _tensor(slot_mapping, "slot_mapping", dev, (torch.int64,))
    if n is None:
        n = slot_mapping.numel() if slot_mapping is not None else _rows(packed, "packed", dev, rb)
    n = int(n)
    rows = _rows(packed, "packed", dev, rb, at_least=n if slot_mapping is None else 0)
    _floats(norms, "norms", dev, rows)
    _slots(slot_mapping, dev, n)
    if out is None:
        out = torch.empty(n, d, dtype=out_dtype, device=packed.device)
    _tensor(out, "out", dev, tuple(_DT))
    if out.numel() != n * d:
        raise ValueError("out has %d elements; expected n * d = %d" % (out.numel(), n * d))
    check(lib().tq_decode(cb.handle, rot.handle, int(vectors_per_rot), _ptr(packed), _ptr(norms),
                          _ptr(slot_mapping), int(n), _ptr(out), dtype_code(out.dtype), _stream(stream)))
    return out


def _params(cb_k, rot_k, q, k_packed, k_norms, cb_v=None, rot_v=None, v_packed=None, v_norms=None,
            seq_lens=None, max_seq_len=None, block_table=None, block_size=0, batch_per_rot=0, scale=None,
            out=None, lse=None, num_splits=0, num_kv_heads=None, k_window=None, v_window=None, qjl=None,
            k_signs=None, k_rnorms=None):
    dev = rot_k.device
    _pair(cb_k, rot_k, "attention keys")
    _tensor(q, "q", dev, tuple(_DT))
    if q.dim() != 3 or q.shape[2] != rot_k.d:
        raise ValueError("q has shape %s; expected [batch, num_q_heads, %d]" % (tuple(q.shape), rot_k.d))
    B, Hq, d = q.shape
    _tensor(k_packed, "k_packed", dev, (torch.uint8,))
    if k_packed.dim() != 4:
        raise ValueError("k_packed must be 4-D: dense [batch, num_kv_heads, max_seq_len, row] or a paged pool "
                         "[num_blocks, num_kv_heads, block_size, row]")
    if num_kv_heads is None:
        num_kv_heads = k_packed.shape[1]
    Hkv = int(num_kv_heads)
    if max_seq_len is None:
        if block_table is not None:
            raise ValueError("a paged cache needs max_seq_len")
        max_seq_len = k_packed.shape[2]
    max_seq_len = int(max_seq_len)
    if block_table is not None:
        _tensor(block_table, "block_table", dev, (torch.int32,))
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table has shape %s; expected [batch = %d, max_blocks_per_seq]"
                             % (tuple(block_table.shape), B))
        lead = (k_packed.shape[0], Hkv, int(block_size))
    else:
        lead = (B, Hkv, max_seq_len)

    def cache(packed, norms, row, pname, nname):
        _tensor(packed, pname, dev, (torch.uint8,))
        _shape(packed, pname, lead + (row,))
        _tensor(norms, nname, dev, (torch.float32,))
        _shape(norms, nname, lead)

    cache(k_packed, k_norms, packed_row_bytes(d, cb_k.bits), "k_packed", "k_norms")
    if cb_v is not None:
        _pair(cb_v, rot_v, "attention values")
        if rot_v.device != dev:
            raise ValueError("the K and V rotations live on different devices")
        cache(v_packed, v_norms, packed_row_bytes(d, cb_v.bits), "v_packed", "v_norms")
    if seq_lens is not None:
        _tensor(seq_lens, "seq_lens", dev, (torch.int32,))
        _shape(seq_lens, "seq_lens", (B,))
    if out is not None:
        _tensor(out, "out", dev, tuple(_DT))
        _shape(out, "out", (B, Hq, d))
    if lse is not None:
        _tensor(lse, "lse", dev, (torch.float32,))
        _shape(lse, "lse", (B, Hq))
    if k_window is not None or v_window is not None:
        for name, w in (("k_window", k_window), ("v_window", v_window)):
            _tensor(w, name, dev, tuple(_DT))
            if w.dim() != 4 or tuple(w.shape[:2]) != (B, Hkv) or w.shape[3] != d:
                raise ValueError("%s has shape %s; expected [%d, %d, window, %d]" % (name, tuple(w.shape), B, Hkv, d))
        if k_window.shape != v_window.shape or k_window.dtype != v_window.dtype:
            raise ValueError("k_window and v_window must have the same shape and dtype")
    if qjl is not None:
        if qjl.rot is not rot_k:
            raise ValueError("qjl was not created on rot_k")
        cache(k_signs, k_rnorms, d // 8, "k_signs", "k_rnorms")
    p = AttnParams()
    p.cb_k, p.rot_k = cb_k.handle, rot_k.handle
    p.cb_v = cb_v.handle if cb_v is not None else None
    p.rot_v = rot_v.handle if rot_v is not None else None
    p.batch, p.num_q_heads = B, Hq
    p.num_kv_heads = Hkv
    p.q, p.q_dtype = q.data_ptr(), dtype_code(q.dtype)
    p.k_packed, p.k_norms = k_packed.data_ptr(), k_norms.data_ptr()
    p.v_packed = v_packed.data_ptr() if v_packed is not None else None
    p.v_norms = v_norms.data_ptr() if v_norms is not None else None
    p.seq_lens = seq_lens.data_ptr() if seq_lens is not None else None
    p.max_seq_len = max_seq_len
    p.block_table = block_table.data_ptr() if block_table is not None else None
    p.block_size = int(block_size)
    p.max_blocks_per_seq = int(block_table.shape[1]) if block_table is not None else 0
    p.batch_per_rot = int(batch_per_rot)
    p.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    p.out = out.data_ptr() if out is not None else None
    p.out_dtype = dtype_code(out.dtype) if out is not None else TQ_F32
    p.lse = lse.data_ptr() if lse is not None else None
    p.num_splits = int(num_splits)
    if k_window is not None:
        p.k_window, p.v_window = k_window.data_ptr(), v_window.data_ptr()
        p.window, p.window_dtype = int(k_window.shape[2]), dtype_code(k_window.dtype)
    if qjl is not None:
        p.qjl_k = qjl.handle
        p.k_signs, p.k_rnorms = k_signs.data_ptr(), k_rnorms.data_ptr()
    return p


def attn_workspace_size(p: AttnParams) -> int:
    n = lib().tq_attn_workspace_size(C.byref(p))
    if n == 0:
        raise TQError(None, _lib.last_error())
    return int(n)


def _workspace(p: AttnParams, device, workspace=None):
    need = attn_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return workspace


def scores_compressed(cb_k: Codebook, rot_k: Rotation, q: torch.Tensor, k_packed: torch.Tensor,
                      k_norms: torch.Tensor, seq_lens=None, max_seq_len=None, block_table=None, block_size=0,
                      batch_per_rot=0, scale=None, scores=None, num_kv_heads=None, workspace=None, stream=None,
                      qjl=None, k_signs=None, k_rnorms=None):
    """s[b, h, t] = scale * n_t <Pi_K q[b,h], c_K[idx_t]> for t < len_b, from the compressed keys.
    q: [B, Hq, d]; dense k_packed [B, Hkv, T, row] / k_norms [B, Hkv, T], or paged pools with a
    block_table [B, max_blocks] (int32) and block_size. Returns float32 [B, Hq, T].
    qjl (a QJLSketch) with k_signs [.., d/8] / k_rnorms in the layout of k_packed / k_norms: QJL
    keys, scored with the added term ||r_t|| sqrt(pi/2)/d <S q, signs_t>."""
    p = _params(cb_k, rot_k, q, k_packed, k_norms, seq_lens=seq_lens, max_seq_len=max_seq_len,
                block_table=block_table, block_size=block_size, batch_per_rot=batch_per_rot, scale=scale,
                num_kv_heads=num_kv_heads, qjl=qjl, k_signs=k_signs, k_rnorms=k_rnorms)
    if scores is None:
        scores = torch.full((q.shape[0], q.shape[1], p.max_seq_len), float("nan"), dtype=torch.float32,
                            device=q.device)
    _tensor(scores, "scores", rot_k.device, (torch.float32,))
    _shape(scores, "scores", (q.shape[0], q.shape[1], p.max_seq_len))
    ws = _workspace(p, q.device, workspace)
    check(lib().tq_scores_compressed(C.byref(p), _ptr(scores), _stream(stream)))
    scores._tq_workspace = ws
    return scores


def attn_decode(cb_k: Codebook, rot_k: Rotation, cb_v: Codebook, rot_v: Rotation, q: torch.Tensor,
                k_packed, k_norms, v_packed, v_norms, seq_lens=None, max_seq_len=None, block_table=None,
                block_size=0, batch_per_rot=0, scale=None, out=None, out_dtype=None, return_lse=False,
                num_splits=0, num_kv_heads=None, workspace=None, stream=None, k_window=None, v_window=None,
                qjl=None, k_signs=None, k_rnorms=None):
    """Fused decode attention over the compressed cache; returns out [B, Hq, d] (and lse).
    k_window / v_window: optional rings [B, Hkv, R, d] holding each sequence's newest
    min(len, R) tokens at full precision (token t in slot t % R); seq_lens are then total
    lengths and only the older positions are read from the compressed cache.
    qjl / k_signs / k_rnorms: QJL keys, as in scores_compressed."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
    p = _params(cb_k, rot_k, q, k_packed, k_norms, cb_v, rot_v, v_packed, v_norms, seq_lens, max_seq_len,
                block_table, block_size, batch_per_rot, scale, out, lse, num_splits, num_kv_heads, k_window,
                v_window, qjl, k_signs, k_rnorms)
    ws = _workspace(p, q.device, workspace)
    check(lib().tq_attn_decode(C.byref(p), _stream(stream)))
    out._tq_workspace = ws
    return (out, lse) if return_lse else out


def attn_decode_noalloc(cb_k: Codebook, rot_k: Rotation, cb_v: Codebook, rot_v: Rotation, q: torch.Tensor,
                        k_packed, k_norms, v_packed, v_norms, out: torch.Tensor, lse=None, seq_lens=None,
                        max_seq_len=None, block_table=None, block_size=0, batch_per_rot=0, scale=None, num_splits=0,
                        num_kv_heads=None, stream=None, k_window=None, v_window=None, qjl=None, k_signs=None,
                        k_rnorms=None):
    """attn_decode into caller-owned `out` (and `lse`) with libtq's static scratch as the
    workspace: the call allocates nothing. Calls that overlap on one GPU race on that scratch."""
    p = _params(cb_k, rot_k, q, k_packed, k_norms, cb_v, rot_v, v_packed, v_norms, seq_lens, max_seq_len,
                block_table, block_size, batch_per_rot, scale, out, lse, num_splits, num_kv_heads, k_window,
                v_window, qjl, k_signs, k_rnorms)
    check(lib().tq_attn_decode_noalloc(C.byref(p), _stream(stream)))
    return out


def window_append(cb_k: Codebook, rot_k: Rotation, cb_v: Codebook, rot_v: Rotation, k_new: torch.Tensor,
                  v_new: torch.Tensor, k_window: torch.Tensor, v_window: torch.Tensor, seq_lens: torch.Tensor,
                  k_packed, k_norms, v_packed, v_norms, max_seq_len=None, block_table=None, block_size=0,
                  batch_per_rot=0, workspace=None, stream=None):
    """Append n_new tokens per sequence (k_new / v_new [B, Hkv, n_new, d], the rings' dtype) to
    the full-precision rings [B, Hkv, R, d]; tokens leaving the window are encoded into the
    compressed cache (dense [B, Hkv, max_seq_len, row] or paged pools); seq_lens (device
    int32 [B]) is advanced by n_new on the stream."""
    dev = rot_k.device
    _pair(cb_k, rot_k, "window_append keys")
    _pair(cb_v, rot_v, "window_append values")
    _tensor(k_new, "k_new", dev, tuple(_DT))
    if k_new.dim() != 4 or k_new.shape[3] != rot_k.d:
        raise ValueError("k_new has shape %s; expected [batch, num_kv_heads, n_new, %d]" % (tuple(k_new.shape), rot_k.d))
    B, Hkv, n_new, d = k_new.shape
    _tensor(v_new, "v_new", dev, (k_new.dtype,))
    _shape(v_new, "v_new", k_new.shape)
    for name, w in (("k_window", k_window), ("v_window", v_window)):
        _tensor(w, name, dev, (k_new.dtype,), contiguous=w.numel() > 0)
        if w.dim() != 4 or tuple(w.shape[:2]) != (B, Hkv) or w.shape[3] != d:
            raise ValueError("%s has shape %s; expected [%d, %d, window, %d]" % (name, tuple(w.shape), B, Hkv, d))
    _tensor(seq_lens, "seq_lens", dev, (torch.int32,))
    _shape(seq_lens, "seq_lens", (B,))
    if max_seq_len is None:
        if block_table is not None:
            raise ValueError("a paged cache needs max_seq_len")
        max_seq_len = k_packed.shape[2]
    if block_table is not None:
        _tensor(block_table, "block_table", dev, (torch.int32,))
        lead = (k_packed.shape[0], Hkv, int(block_size))
    else:
        lead = (B, Hkv, int(max_seq_len))
    for pk_, nm_, bits, pn, nn in ((k_packed, k_norms, cb_k.bits, "k_packed", "k_norms"),
                                   (v_packed, v_norms, cb_v.bits, "v_packed", "v_norms")):
        _tensor(pk_, pn, dev, (torch.uint8,))
        _shape(pk_, pn, lead + (packed_row_bytes(d, bits),))
        _tensor(nm_, nn, dev, (torch.float32,))
        _shape(nm_, nn, lead)
    p = _lib.WindowAppendParams()
    p.cb_k, p.cb_v, p.rot_k, p.rot_v = cb_k.handle, cb_v.handle, rot_k.handle, rot_v.handle
    p.batch, p.num_kv_heads, p.n_new = B, Hkv, n_new
    p.k_new, p.v_new = k_new.data_ptr(), v_new.data_ptr()
    p.k_window, p.v_window = k_window.data_ptr(), v_window.data_ptr()
    p.window, p.window_dtype = int(k_window.shape[2]), dtype_code(k_window.dtype)
    p.seq_lens = seq_lens.data_ptr()
    p.k_packed, p.k_norms, p.v_packed, p.v_norms = (k_packed.data_ptr(), k_norms.data_ptr(), v_packed.data_ptr(),
                                                    v_norms.data_ptr())
    p.max_seq_len = int(max_seq_len)
    p.block_table = block_table.data_ptr() if block_table is not None else None
    p.block_size = int(block_size)
    p.max_blocks_per_seq = int(block_table.shape[1]) if block_table is not None else 0
    p.batch_per_rot = int(batch_per_rot)
    need = lib().tq_window_append_workspace_size(C.byref(p))
    if need == 0:
        raise TQError(None, _lib.last_error())
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_new.device)
    p.workspace, p.workspace_bytes = workspace.data_ptr(), int(workspace.numel())
    check(lib().tq_window_append(C.byref(p), _stream(stream)))
    return workspace


def _gq_buffers(packed, scales, zeros, n: int, d: int, bits: int, dev):
    if d % 32:
        raise ValueError("group quantization needs d a multiple of 32 (got %d)" % d)
    _tensor(packed, "packed", dev, (torch.uint8,))
    if packed.numel() != n * (d * bits // 8):
        raise ValueError("packed has %d bytes; expected n * d * bits / 8 = %d" % (packed.numel(), n * d * bits // 8))
    for name, t in (("scales", scales), ("zeros", zeros)):
        _tensor(t, name, dev, (torch.float16,))
        if t.numel() != n * (d // 32):
            raise ValueError("%s has %d elements; expected n * d / 32 = %d (float16)" % (name, t.numel(), n * d // 32))


def gq_encode(x: torch.Tensor, bits: int, stream=None, packed=None, scales=None, zeros=None):
    """Affine group quantization (groups of 32) of x [..., d] (float32/bfloat16/float16 on the GPU).
    Returns (packed uint8 [N, d*bits/8], scales float16 [N, d/32], zeros float16 [N, d/32])."""
    _tensor(x, "x", None, tuple(_DT), contiguous=False)
    d = x.shape[-1]
    x2 = x.reshape(-1, d) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    n = x2.shape[0]
    dev = x.device.index
    if packed is None:
        packed = torch.empty(n, d * bits // 8, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(n, d // 32, dtype=torch.float16, device=x.device)
    if zeros is None:
        zeros = torch.empty_like(scales)
    _gq_buffers(packed, scales, zeros, n, d, bits, dev)
    check(lib().tq_gq_encode(int(d), int(bits), _ptr(x2), dtype_code(x2.dtype), n, x2.stride(0), _ptr(packed),
                             _ptr(scales), _ptr(zeros), _stream(stream)))
    return packed, scales, zeros


def gq_decode(packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, bits: int,
              out_dtype=torch.float32, stream=None, out=None):
    _tensor(packed, "packed", None, (torch.uint8,))
    _tensor(scales, "scales", packed.device.index, (torch.float16,))
    n, d = packed.shape[0], scales.shape[-1] * 32
    _gq_buffers(packed, scales, zeros, n, d, bits, packed.device.index)
    if out is None:
        out = torch.empty(n, d, dtype=out_dtype, device=packed.device)
    _tensor(out, "out", packed.device.index, tuple(_DT))
    if out.numel() != n * d:
        raise ValueError("out has %d elements; expected %d" % (out.numel(), n * d))
    out_dtype = out.dtype
    check(lib().tq_gq_decode(int(d), int(bits), _ptr(packed), _ptr(scales), _ptr(zeros), n, _ptr(out),
                             dtype_code(out_dtype), _stream(stream)))
    return out
