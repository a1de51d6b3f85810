"""The seeded input generators: deterministic, right shapes, planted and tie
structure as described."""
import torch

from block_sparse_attention_kv_amd import workloads as W


def test_deterministic_and_shapes():
    w = W.TINY_512
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.is_contiguous()
        assert torch.equal(x, y)
    q, k, v = a
    assert q.shape == (1, 2, 512, 64) and k.shape == (1, 1, 512, 64) and v.shape == k.shape


def test_planted_variant():
    w = W.STRUCTURED_8K.scaled(batch=1, seq_q=1024, seq_kv=1024)
    q, k, v = W.make_inputs(w)
    g = torch.Generator().manual_seed(w.seed)
    d = w.head_dim
    torch.randn((1, 32, 1024, d), generator=g)
    k0 = torch.randn((1, 2, 1024, d), generator=g)
    torch.randn((1, 2, 1024, d), generator=g)
    u = torch.randn((d,), generator=g)
    u = u / u.norm()
    shift = (k.float() - k0).reshape(1, 2, 16, 64, d).mean(dim=3) @ u   # per-block component along u
    planted = shift > 1.5
    assert 0 < int(planted.sum()) < 32
    assert torch.all((shift[planted] - 3.0).abs() < 0.05)
    assert torch.all(shift[~planted].abs() < 0.05)


def test_tie_variant_repeats_one_key_row():
    w = W.STRUCTURED_8K_TIE.scaled(batch=1, seq_q=256, seq_kv=256)
    q, k, v = W.make_inputs(w)
    assert torch.equal(k, k[:, :, :1].expand_as(k))
    assert not torch.equal(v, v[:, :, :1].expand_as(v))


def test_workload_table():
    assert W.PREFILL_8K.topk * W.PREFILL_8K.block == 1024          # 1024-token receptive field
    assert W.DECODE_32K.q_offset == 32767 and W.DECODE_32K.is_decode
    assert W.EXTRAP_32K.full_rows == (28672, 32768)
