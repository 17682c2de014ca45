"""GPU parity of the paged and dense entry points (through the C ABI).

smla_decode_paged maps positions to cache rows through per-sequence page
tables inside the kernel; smla_decode_dense attends to every position of each
sequence's context.  Both are defined as smla_decode over the rows their
positions name (oracle.rows_of_positions, oracle.dense_positions), so each
case is checked twice: against the fp64 oracle on those rows (same tolerances
as the other parity tests), and bit for bit against smla_decode on the rows
the harness computed -- the same rows in the same order must give the same
bits.  For long contexts the dense entry point folds a sequence's query
tokens into the head dimension (they share one list); its bit-exact
reference is then smla_decode called the same folded way.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import (bf16_bits_to_f32, block_table, dense_inputs, flat_inputs, oracle_view,
                       to_device, torch_to_bits, workload)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def _outputs(inp, dev):
    import torch
    out = torch.empty((inp.batch, inp.q_len, inp.heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.q_len, inp.heads), dtype=torch.float32, device=dev)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    return out, lse


def _host(out, lse):
    return bf16_bits_to_f32(torch_to_bits(out)), lse.cpu().numpy()


def _parity(o_g, l_g, o_r, l_r, what):
    ok, m = check(o_g, l_g, o_r, l_r)
    print(f"{what}: max_abs={m['max_abs']:.3g} rel_l2={m['rel_l2']:.3g} "
          f"lse={m['lse_max_abs']:.3g} empty={m['empty']}", flush=True)
    assert ok, f"{what}: {m['reasons']}"


def _same_bits(a, b, what):
    import torch
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: out differs"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: lse differs"


def _rows_call(smla, inp, dev, idx_rows, nsplit, fold=False):
    """smla_decode on explicit rows; fold=True calls it the way the dense
    entry point does: the q_len tokens of a sequence as q_len*heads heads of
    one token over the sequence's shared list."""
    import torch
    out, lse = _outputs(inp, dev["q"].device)
    ix = torch.from_numpy(np.ascontiguousarray(idx_rows)).to(dev["q"].device)
    if fold:
        b, lq, h = inp.batch, inp.q_len, inp.heads
        assert (idx_rows == idx_rows[:, :1]).all(), "a folded call needs one list per sequence"
        used = smla.smla_decode(dev["q"].view(b, 1, lq * h, 576), dev["kv"], ix[:, :1].contiguous(),
                                out.view(b, 1, lq * h, 512), lse.view(b, 1, lq * h), inp.scale, nsplit)
    else:
        used = smla.smla_decode(dev["q"], dev["kv"], ix, out, lse, inp.scale, nsplit)
    torch.cuda.synchronize()
    return (out, lse), used


# ------------------------------------------------------------------ paged

@pytest.fixture(scope="module")
def batched(smla):
    import torch
    inp = workload("batched")
    dev = to_device(inp, "cuda")
    table = torch.from_numpy(block_table(inp)).cuda()
    pos = torch.from_numpy(np.ascontiguousarray(inp.pos)).cuda()
    return inp, dev, table, pos


@pytest.mark.parametrize("nsplit", [0, 1, 8])
def test_paged_batched_full_size(smla, batched, nsplit):
    import torch
    inp, dev, table, pos = batched
    out, lse = _outputs(inp, dev["q"].device)
    used = smla.smla_decode_paged(dev["q"], dev["kv"], table, 64, pos, out, lse, inp.scale, nsplit)
    torch.cuda.synchronize()
    ref, used_rows = _rows_call(smla, inp, dev, inp.idx, nsplit)
    assert used == used_rows
    _same_bits((out, lse), ref, f"paged batched nsplit={nsplit}")
    o_r, l_r = batched_ref(inp, dev)
    _parity(*_host(out, lse), o_r, l_r, f"paged batched nsplit={nsplit} (used {used}), all 64 sequences")


_REF = {}


def batched_ref(inp, dev):
    """The oracle over all 64 sequences (the rows the lists select, copied from
    the device), computed once."""
    if "batched" not in _REF:
        q_s, kv_s, idx_s = oracle_view(inp, dev["kv"])
        _REF["batched"] = oracle.decode(q_s, kv_s, idx_s, inp.scale)
    return _REF["batched"]


def test_paged_ragged_full_size(smla):
    """The ragged workload (128 x 128 heads, ~9.8 GB pool, page tables of up
    to 2048 pages: wider than the LDS stage) through the in-kernel page map,
    with -1 padding at shuffled positions in the first 16 lists."""
    import torch
    inp = workload("ragged", ragged_pad=True, pad_shuffle=True)
    dev = to_device(inp, "cuda")
    table = torch.from_numpy(block_table(inp)).cuda()
    pos = torch.from_numpy(np.ascontiguousarray(inp.pos)).cuda()
    out, lse = _outputs(inp, dev["q"].device)
    used = smla.smla_decode_paged(dev["q"], dev["kv"], table, 64, pos, out, lse, inp.scale, 0)
    torch.cuda.synchronize()
    ref, used_rows = _rows_call(smla, inp, dev, inp.idx, 0)
    assert used == used_rows
    _same_bits((out, lse), ref, "paged ragged")
    q_s, kv_s, idx_s = oracle_view(inp, dev["kv"])
    o_r, l_r = oracle.decode(q_s, kv_s, idx_s, inp.scale)
    _parity(*_host(out, lse), o_r, l_r, f"paged ragged (used {used}), all 128 sequences")
    del dev
    torch.cuda.empty_cache()


# heads, topk, pages per sequence, page ids drawn, pages inside the cache,
# NSPLITs.  24 heads: the 32-head block, which reads the table after each
# position.  64 and 72 heads: 64-head blocks, which stage a table of up to 512
# pages in LDS (5000 entries at NSPLIT 1: three staged list chunks, the table
# restaged for each; 72 heads: a second, partial head block).  600 pages: a
# table wider than the stage, read after each position.
PAGED_EDGES = [
    (24, 150, 12, 40, 30, (1, 3, 0)),
    (64, 5000, 12, 46, 30, (1, 2, 0)),
    (72, 300, 12, 46, 30, (1, 3, 0)),
    (64, 300, 600, 1810, 1700, (1, 3, 0)),
]


@pytest.mark.parametrize("case", PAGED_EDGES, ids=lambda c: f"h{c[0]}k{c[1]}p{c[2]}")
def test_paged_edges(smla, case):
    """Missing pages, positions beyond the table or negative, rows outside
    the cache, a 16-token page, three sequences of two query tokens."""
    import torch
    heads, topk, pages_per_seq, n_ids, kv_pages, nsplits = case
    rng = np.random.default_rng(31)
    page, batch, q_len = 16, 3, 2
    kv_rows = kv_pages * page  # page ids from kv_pages on point outside the cache
    inp = flat_inputs("paged_edges", 8100, batch, q_len, heads, kv_rows, min(topk, kv_rows))
    table = rng.permutation(n_ids)[: batch * pages_per_seq].reshape(batch, pages_per_seq).astype(np.int32)
    table[0, 3] = -1
    table[2, :] = -1
    table[2, 5] = 7
    pos = rng.integers(-20, pages_per_seq * page + 40, size=(batch, q_len, topk)).astype(np.int32)
    pos[1, 1, :] = -1
    rows = oracle.rows_of_positions(table, page, pos, kv_rows)
    assert (rows == -1).any() and (rows >= 0).any()
    dev = to_device(inp, "cuda")
    t_dev = torch.from_numpy(table).cuda()
    p_dev = torch.from_numpy(pos).cuda()
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    for nsplit in nsplits:
        out, lse = _outputs(inp, dev["q"].device)
        used = smla.smla_decode_paged(dev["q"], dev["kv"], t_dev, page, p_dev, out, lse, inp.scale,
                                      nsplit)
        torch.cuda.synchronize()
        _parity(*_host(out, lse), o_r, l_r, f"paged edges nsplit={nsplit} (used {used})")
        ref, _ = _rows_call(smla, inp, dev, rows, nsplit)
        _same_bits((out, lse), ref, f"paged edges nsplit={nsplit}")


# ------------------------------------------------------------------ dense

@pytest.mark.parametrize("ctx", [4096, 16384, 65536])
@pytest.mark.parametrize("nsplit", [16, 64, 0])
def test_dense_verify(smla, ctx, nsplit):
    """The verify shape: 9 query tokens, 8 heads, every row of a flat cache."""
    import torch
    inp = workload("verify", spec_ctx=ctx)
    dev = to_device(inp, "cuda")
    ctx_len = torch.tensor(inp.ctx, dtype=torch.int32, device="cuda")
    out, lse = _outputs(inp, dev["q"].device)
    used = smla.smla_decode_dense(dev["q"], dev["kv"], ctx_len, int(inp.ctx.max()), out, lse,
                                  inp.scale, nsplit)
    torch.cuda.synchronize()
    rows = oracle.rows_of_positions(None, 1, oracle.dense_positions(inp.ctx, ctx, inp.q_len),
                                    inp.kv_rows)
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    _parity(*_host(out, lse), o_r, l_r, f"dense verify ctx={ctx} nsplit={nsplit} (used {used})")
    ref, _ = _rows_call(smla, inp, dev, inp.idx, nsplit,
                        fold=smla.dense_folds(inp.q_len, inp.heads, ctx))
    _same_bits((out, lse), ref, f"dense verify ctx={ctx} nsplit={nsplit}")


@pytest.mark.parametrize("nsplit", [1, 4, 0])
def test_dense_paged_ragged(smla, nsplit):
    """Paged dense over ragged contexts, one of them empty."""
    import torch
    inp = dense_inputs("dense_paged", 8200, 4, 2, 40, [100, 0, 257, 1], paged=True)
    dev = to_device(inp, "cuda")
    table = torch.from_numpy(block_table(inp)).cuda()
    ctx_len = torch.tensor(inp.ctx, dtype=torch.int32, device="cuda")
    max_ctx = int(inp.ctx.max())
    out, lse = _outputs(inp, dev["q"].device)
    used = smla.smla_decode_dense(dev["q"], dev["kv"], ctx_len, max_ctx, out, lse, inp.scale,
                                  nsplit, block_table=table, page_size=64)
    torch.cuda.synchronize()
    rows = oracle.rows_of_positions(block_table(inp), 64,
                                    oracle.dense_positions(inp.ctx, max_ctx, inp.q_len), inp.kv_rows)
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    assert np.isneginf(l_r[1]).all()
    _parity(*_host(out, lse), o_r, l_r, f"dense paged nsplit={nsplit} (used {used})")
    ref, _ = _rows_call(smla, inp, dev, inp.idx, nsplit,
                        fold=smla.dense_folds(inp.q_len, inp.heads, max_ctx))
    _same_bits((out, lse), ref, f"dense paged nsplit={nsplit}")


@pytest.mark.parametrize("nsplit", [1, 2, 0])
def test_dense_paged_long_contexts(smla, nsplit):
    """Paged dense, 64 heads, contexts of thousands of positions (one slice
    streams its list through the stage in several refills, each position
    mapped through the page table inside the loop), one context empty."""
    import torch
    inp = dense_inputs("dense_paged_long", 8250, 3, 1, 64, [3000, 1500, 0], paged=True)
    dev = to_device(inp, "cuda")
    table = torch.from_numpy(block_table(inp)).cuda()
    ctx_len = torch.tensor(inp.ctx, dtype=torch.int32, device="cuda")
    max_ctx = int(inp.ctx.max())
    out, lse = _outputs(inp, dev["q"].device)
    used = smla.smla_decode_dense(dev["q"], dev["kv"], ctx_len, max_ctx, out, lse, inp.scale,
                                  nsplit, block_table=table, page_size=64)
    torch.cuda.synchronize()
    rows = oracle.rows_of_positions(block_table(inp), 64,
                                    oracle.dense_positions(inp.ctx, max_ctx, inp.q_len), inp.kv_rows)
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    assert np.isneginf(l_r[2]).all()
    _parity(*_host(out, lse), o_r, l_r, f"dense paged long nsplit={nsplit} (used {used})")
    ref, _ = _rows_call(smla, inp, dev, inp.idx, nsplit,
                        fold=smla.dense_folds(inp.q_len, inp.heads, max_ctx))
    _same_bits((out, lse), ref, f"dense paged long nsplit={nsplit}")


def test_dense_context_beyond_max(smla):
    """A context longer than max_ctx is attended only up to max_ctx."""
    import torch
    inp = dense_inputs("dense_cut", 8300, 2, 1, 8, [300, 120], paged=False)
    dev = to_device(inp, "cuda")
    ctx_len = torch.tensor([300, 120], dtype=torch.int32, device="cuda")
    out, lse = _outputs(inp, dev["q"].device)
    smla.smla_decode_dense(dev["q"], dev["kv"], ctx_len, 200, out, lse, inp.scale, 0)
    torch.cuda.synchronize()
    rows = oracle.rows_of_positions(None, 1, oracle.dense_positions([300, 120], 200, 1), inp.kv_rows)
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    _parity(*_host(out, lse), o_r, l_r, "dense ctx above max_ctx")
