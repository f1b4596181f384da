"""Bad calls on the GPU raise before any launch: the binding checks device, dtype, contiguity and
sizes of every tensor it hands to libtq."""

import pytest
import torch

import tq_inputs as ti

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("kv_cache_vector_encode_amd")


@pytest.fixture(scope="module")
def env():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    rot = tq.Rotation.from_gaussian(ti.rotation_gaussian(128, 42))
    return dev, rot, tq.Codebook(128, 4), tq.Codebook(128, 2)


def test_encode_checks(env):
    dev, rot, ck, _ = env
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="last dimension"):
        tq.encode(ck, rot, x[:, :64])                 # a [N, 64] view of 128-wide rows
    with pytest.raises(TypeError, match="dtype"):
        tq.encode(ck, rot, x.double())
    with pytest.raises(ValueError, match="rows"):
        tq.encode(ck, rot, x, packed=torch.empty(32, 64, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="whole number"):
        tq.encode(ck, rot, x, packed=torch.empty(4100, dtype=torch.uint8, device=dev))   # 4100 % 64 != 0
    with pytest.raises(ValueError, match="norms"):
        tq.encode(ck, rot, x, norms=torch.empty(63, device=dev))
    with pytest.raises(TypeError, match="slot_mapping"):
        tq.encode(ck, rot, x, slot_mapping=torch.zeros(64, dtype=torch.int32, device=dev))
    with pytest.raises(ValueError, match="slot_mapping"):
        tq.encode(ck, rot, x, slot_mapping=torch.zeros(63, dtype=torch.int64, device=dev))


def test_decode_checks(env):
    dev, rot, ck, _ = env
    p = torch.zeros(64, 64, dtype=torch.uint8, device=dev)
    n = torch.zeros(64, device=dev)
    with pytest.raises(ValueError, match="out"):
        tq.decode(ck, rot, p, n, out=torch.empty(64, 64, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="rows"):
        tq.decode(ck, rot, p, n, n=65)
    with pytest.raises(TypeError, match="norms"):
        tq.decode(ck, rot, p, n.half())


def test_attention_checks(env):
    dev, rot, ck, cv = env
    B, Hq, Hkv, T = 2, 8, 2, 32
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    kp = torch.zeros(B, Hkv, T, 64, dtype=torch.uint8, device=dev)
    vp = torch.zeros(B, Hkv, T, 32, dtype=torch.uint8, device=dev)
    kn = torch.zeros(B, Hkv, T, device=dev)
    ok = dict(out_dtype=torch.float32)
    with pytest.raises(TypeError, match="seq_lens"):
        tq.attn_decode(ck, rot, cv, rot, q, kp, kn, vp, kn, seq_lens=torch.full((B,), T, device=dev), **ok)
    with pytest.raises(ValueError, match="q must be contiguous"):
        tq.attn_decode(ck, rot, cv, rot, q.transpose(0, 1).contiguous().transpose(0, 1), kp, kn, vp, kn, **ok)
    with pytest.raises(ValueError, match="v_packed"):
        tq.attn_decode(ck, rot, cv, rot, q, kp, kn, kp, kn, **ok)          # 4-bit rows given as 2-bit values
    with pytest.raises(ValueError, match="out"):
        tq.attn_decode(ck, rot, cv, rot, q, kp, kn, vp, kn, out=torch.empty(B, Hq, 64, device=dev))
    with pytest.raises(ValueError, match="scores"):
        tq.scores_compressed(ck, rot, q, kp, kn, scores=torch.empty(B, Hq, T - 1, device=dev))
    with pytest.raises(ValueError, match="block_table"):
        tq.attn_decode(ck, rot, cv, rot, q, kp, kn, vp, kn, max_seq_len=T, block_size=T,
                       block_table=torch.zeros(B + 1, 1, dtype=torch.int32, device=dev), **ok)
