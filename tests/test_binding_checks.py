"""Host-only checks of the Python binding's argument validation: bad calls raise before any
kernel launch (no GPU needed: the checks run before libtq is asked to launch anything)."""

import pytest
import torch

import kv_cache_vector_encode_amd as tq


def _fake_rotation(d=128):
    # a Rotation object without a device upload; only its dimensions and device are read here
    r = tq.Rotation.__new__(tq.Rotation)
    r._h, r.d, r.n_rot, r.device = None, d, 1, 0
    return r


def test_host_tensors_are_refused():
    cb, rot = tq.Codebook(128, 4), _fake_rotation()
    x = torch.zeros(8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA tensor"):
        tq.encode(cb, rot, x)
    with pytest.raises(ValueError, match="CUDA tensor"):
        tq.decode(cb, rot, torch.zeros(8, 64, dtype=torch.uint8), torch.zeros(8))
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16)
    kp = torch.zeros(1, 2, 16, 64, dtype=torch.uint8)
    kn = torch.zeros(1, 2, 16)
    with pytest.raises(ValueError, match="CUDA tensor"):
        tq.attn_decode(cb, rot, cb, rot, q, kp, kn, kp, kn)
    with pytest.raises(ValueError, match="CUDA tensor"):
        tq.scores_compressed(cb, rot, q, kp, kn)
    with pytest.raises(ValueError, match="CUDA tensor"):
        tq.gq_encode(x, 2)


def test_mismatched_head_dims_are_refused():
    cb, rot = tq.Codebook(64, 4), _fake_rotation(128)
    with pytest.raises(ValueError, match="does not match"):
        tq.encode(cb, rot, torch.zeros(8, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="does not match"):
        tq.decode(cb, rot, torch.zeros(8, 32, dtype=torch.uint8), torch.zeros(8))
