"""C-ABI checks that need no GPU: the library loads, exports what include/tq.h declares,
the host codebook solver and QR agree with the oracle, and host-side validation rejects
bad arguments with a message naming them."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import tq_inputs as ti
from oracle import codebook as ocb, rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tq = pytest.importorskip("kv_cache_vector_encode_amd")
from kv_cache_vector_encode_amd import _lib  # noqa: E402


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtq.so is not built; run python -m kv_cache_vector_encode_amd.build_lib")
    return _lib.lib()


def test_exports_every_declared_function(L):
    header = open(os.path.join(ROOT, "include", "tq.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(tq_[a-z_]+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.tq_version() == 1


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_codebook_matches_oracle(L, d, b):
    cb = tq.Codebook(d, b)
    c, t, mse = cb.get()
    ref = ocb.codebook(d, b)
    assert np.max(np.abs(c - ref.centroids)) <= 1e-12
    assert np.max(np.abs(t - ref.thresholds)) <= 1e-12
    assert abs(mse - ref.mse) <= 1e-9 * ref.mse
    dd, bb = C.c_int(), C.c_int()
    assert L.tq_codebook_dims(cb.handle, C.byref(dd), C.byref(bb)) == 0
    assert (dd.value, bb.value) == (d, b)


@pytest.mark.parametrize("d,b", [(3, 2), (3, 4), (5, 1), (1024, 3)])
def test_codebook_other_sizes_match_oracle(L, d, b):
    c, t, _ = tq.Codebook(d, b).get()
    ref = ocb.lloyd_max(ocb.SphereCoordinate(d), b)
    assert np.max(np.abs(c - ref.centroids)) <= 1e-12


@pytest.mark.parametrize("d", [64, 128, 256])
def test_host_rotation_matches_oracle(L, d):
    g = ti.rotation_gaussian(d, 42).numpy()
    pi = tq.rotation_compute(g)
    assert np.max(np.abs(pi - orot.haar_rotation(g))) <= 1e-12


def test_codebook_rejects_bad_arguments(L):
    assert not L.tq_codebook_init(2, 3)
    assert "d = 2" in _lib.last_error()
    assert not L.tq_codebook_init(128, 5)
    assert "bits = 5" in _lib.last_error()
    with pytest.raises(tq.TQError, match="accepted 1..4"):
        tq.Codebook(128, 0)
    assert L.tq_codebook_get(None, None, None, None) == -2


def test_rotation_rejects_bad_arguments(L):
    g = np.zeros((100, 100), dtype=np.float32)
    assert not L.tq_rotation_from_gaussian(100, 1, g.ctypes.data_as(C.c_void_p))
    assert "accepted 64, 128, 256" in _lib.last_error()
    assert not L.tq_rotation_from_gaussian(128, 0, g.ctypes.data_as(C.c_void_p))
    assert "n_rot" in _lib.last_error()
    assert not L.tq_rotation_from_gaussian(128, 1, None)
    bad = np.eye(64) * 1.001
    assert not L.tq_rotation_from_matrix(64, 1, bad.ctypes.data_as(C.c_void_p))
    assert "not orthogonal" in _lib.last_error()
    assert L.tq_rotation_compute(2, g.ctypes.data_as(C.c_void_p), g.ctypes.data_as(C.c_void_p)) == -1


def test_rotation_without_a_device_fails_cleanly(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(tq.TQError, match="no HIP device"):
        tq.Rotation.from_gaussian(ti.rotation_gaussian(64, 1))


def test_hot_path_calls_validate_before_any_launch(L):
    cb = tq.Codebook(128, 4)
    assert L.tq_encode(None, None, 0, None, 1, 1, 128, None, None, None, None) == -2
    assert "cb is NULL" in _lib.last_error()
    assert L.tq_encode(cb.handle, None, 0, None, 1, 1, 128, None, None, None, None) == -2
    assert "rot is NULL" in _lib.last_error()
    assert L.tq_decode(cb.handle, None, 0, None, None, None, 1, None, 1, None) == -2
    assert L.tq_attn_workspace_size(None) == 0
    assert L.tq_attn_decode(None, None) == -2
    assert L.tq_scores_compressed(None, None, None) == -2


def test_hadamard_rejects_bad_arguments():
    from kv_cache_vector_encode_amd import _lib
    L = _lib.lib()
    assert not L.tq_rotation_hadamard(96, 1, None)
    assert b"d = 96" in L.tq_last_error()
    bad = (C.c_int8 * 64)(*([1] * 63 + [0]))
    assert not L.tq_rotation_hadamard(64, 1, C.cast(bad, C.c_void_p))
    assert b"signs[63]" in L.tq_last_error()


def test_qjl_calls_validate_before_any_launch(L):
    assert not L.tq_qjl_create(None, None)
    assert "rot is NULL" in _lib.last_error()
    cb = tq.Codebook(128, 3)
    assert L.tq_qjl_encode(cb.handle, None, 0, None, 1, 1, 128, None, None, None, None, None, None) == -2
    assert "qjl is NULL" in _lib.last_error()
    L.tq_qjl_free(None)   # freeing NULL is a no-op
