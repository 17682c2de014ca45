"""The Python binding rejects malformed tensors before calling the library.

The C ABI takes raw pointers and cannot check a buffer's size, dtype or
device, so a wrong-shaped `out` or a host tensor would make the kernels write
out of bounds or fault.  Each case here must raise in the binding; the
tensors are host tensors, so a case that slipped through would reach the
shape-agnostic device check last -- the tests assert which check fired by
its message.  No kernel is launched (no GPU needed).
"""
from __future__ import annotations

import pytest
import torch


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


B, LQ, H, K = 1, 2, 8, 64


def good():
    return dict(q=torch.zeros(B, LQ, H, 576, dtype=torch.bfloat16),
                kv=torch.zeros(256, 576, dtype=torch.bfloat16),
                idx=torch.zeros(B, LQ, K, dtype=torch.int32),
                out=torch.zeros(B, LQ, H, 512, dtype=torch.bfloat16),
                lse=torch.zeros(B, LQ, H, dtype=torch.float32))


def decode(smla, **kw):
    a = good()
    a.update(kw)
    smla.smla_decode(a["q"], a["kv"], a["idx"], a["out"], a["lse"], 0.1, 1)


@pytest.mark.parametrize("kw,exc,msg", [
    (dict(q=torch.zeros(B, LQ, H, 576, dtype=torch.float16)), TypeError, "q must be"),
    (dict(q=torch.zeros(B, LQ, H, 512, dtype=torch.bfloat16)), ValueError, "q must be"),
    (dict(q=torch.zeros(B, LQ, 0, 576, dtype=torch.bfloat16)), ValueError, "heads"),
    (dict(q=torch.zeros(B, LQ, H, 1152, dtype=torch.bfloat16)[..., ::2]), ValueError, "contiguous"),
    (dict(kv=torch.zeros(256, 512, dtype=torch.bfloat16)), ValueError, "kv_cache must be"),
    (dict(kv=torch.zeros(256, 576, dtype=torch.float32)), TypeError, "kv_cache must be"),
    (dict(idx=torch.zeros(B, LQ, K, dtype=torch.int64)), TypeError, "topk_idx must be"),
    (dict(idx=torch.zeros(B, 1, K, dtype=torch.int32)), ValueError, "topk_idx must be"),
    # the write targets: a [B, H, 512] out with q_len 2, fewer heads, or the
    # wrong width would be written past its end
    (dict(out=torch.zeros(B, H, 512, dtype=torch.bfloat16)), ValueError, "out must be"),
    (dict(out=torch.zeros(B, LQ, H - 1, 512, dtype=torch.bfloat16)), ValueError, "out must be"),
    (dict(out=torch.zeros(B, LQ, H, 256, dtype=torch.bfloat16)), ValueError, "out must be"),
    (dict(out=torch.zeros(B, LQ, H, 512, dtype=torch.float32)), TypeError, "out must be"),
    (dict(lse=torch.zeros(B, H, dtype=torch.float32)), ValueError, "lse must be"),
    (dict(lse=torch.zeros(B, LQ, H, dtype=torch.bfloat16)), TypeError, "lse must be"),
    (dict(out=None), ValueError, "required"),
])
def test_decode_rejects(smla, kw, exc, msg):
    with pytest.raises(exc, match=msg):
        decode(smla, **kw)


def test_host_tensors_rejected(smla):
    # every shape right, but the tensors live in host memory
    with pytest.raises(ValueError, match="GPU"):
        decode(smla)


def test_fused_and_paged_and_dense_reject(smla):
    a = good()
    with pytest.raises(ValueError, match="out must be"):
        smla.smla_decode_fused(a["q"], a["kv"], a["idx"], a["out"][:, :1], a["lse"], 0.1, 2)
    with pytest.raises(TypeError, match="sync must be"):
        smla.smla_decode_fused(a["q"], a["kv"], a["idx"], a["out"], a["lse"], 0.1, 2,
                               sync=torch.zeros(4096, dtype=torch.int32))
    table = torch.zeros(B, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="lse must be"):
        smla.smla_decode_paged(a["q"], a["kv"], table, 64, a["idx"], a["out"], a["lse"][:, 0], 0.1)
    with pytest.raises(TypeError, match="block_table must be"):
        smla.smla_decode_paged(a["q"], a["kv"], table.long(), 64, a["idx"], a["out"], a["lse"], 0.1)
    ctx = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must be"):
        smla.smla_decode_dense(a["q"], a["kv"], ctx, 64, a["out"][..., :500], a["lse"], 0.1)
    with pytest.raises(ValueError, match="ctx_len must be"):
        smla.smla_decode_dense(a["q"], a["kv"], torch.zeros(B + 1, dtype=torch.int32), 64,
                               a["out"], a["lse"], 0.1)


def test_combine_rejects(smla):
    t, s, h = 3, 4, 8
    po = torch.zeros(t, s, h, 512, dtype=torch.float32)
    pl = torch.zeros(t, s, h, dtype=torch.float32)
    out = torch.zeros(t, h, 512, dtype=torch.bfloat16)
    lse = torch.zeros(t, h, dtype=torch.float32)
    with pytest.raises(TypeError, match="out must be"):
        smla.smla_combine(po, pl, out.float(), lse)
    with pytest.raises(ValueError, match="out must be"):
        smla.smla_combine(po, pl, out[:, :4], lse)
    with pytest.raises(ValueError, match="lse must be"):
        smla.smla_combine(po, pl, out, lse[:2])
    with pytest.raises(ValueError, match="part_o must be"):
        smla.smla_combine(po[:, :3], pl, out, lse)
    with pytest.raises(TypeError, match="part_lse must be"):
        smla.smla_combine(po, pl.double(), out, lse)
    with pytest.raises(ValueError, match="out must be"):
        smla.smla_combine(po, pl, out.view(1, t, h, 512)[:, :2], lse)
    with pytest.raises(ValueError, match="GPU"):
        smla.smla_combine(po, pl, out, lse)
    # [batch, q_len, heads, ...] outputs with batch * q_len tokens are accepted
    with pytest.raises(ValueError, match="GPU"):
        smla.smla_combine(po, pl, out.view(3, 1, h, 512), lse.view(1, 3, h))


def test_topk_rejects(smla):
    sc = torch.zeros(2, 1, 1000, dtype=torch.float32)
    out = torch.zeros(2, 1, 16, dtype=torch.int32)
    with pytest.raises(ValueError, match="out_pos must be"):
        smla.smla_topk(sc, 16, out[:1])
    with pytest.raises(TypeError, match="scores must be"):
        smla.smla_topk(sc.double(), 16, out)
    with pytest.raises(ValueError, match="ctx_len must be"):
        smla.smla_topk(sc, 16, out, ctx_len=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        smla.smla_topk(sc, 16, out)
