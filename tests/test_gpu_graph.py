"""HIP-graph capture of the library's calls (include/smla.h promises that the
calls never synchronise the host, so they can be captured).

Each case captures one call on a side stream, then replays the graph several
times with the program's own eager work and device synchronisations between
replays (other calls on the same buffers, fills of the outputs with NaN),
and checks every replay bit for bit against the eager result of the same
call.  Covered: smla_decode at NSPLIT 1 and 4 (split and combine kernels),
and over 64-head slices long enough for the role-specialised kernel (its
list ring refilled during the call),
smla_decode_paged, smla_decode_dense (folded), smla_decode_fused (single
launch, with its synchronisation words) and smla_topk in each of its forms
(one workgroup per row; chunks in four launches; sampled, two launches).
"""
from __future__ import annotations

import numpy as np
import pytest

from tests.conftest import gpu_available
from workloads import block_table, dense_inputs, flat_inputs, index_scores, to_device, workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def _replays(fn, outs, disturb, n=4):
    """Eager result of fn(), then n replays of a captured fn() with disturb()
    run eagerly (and the outputs poisoned) before each; every replay must give
    the eager bits."""
    import torch
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.synchronize()
    for r in range(n):
        disturb()
        for o in outs:
            if o.dtype.is_floating_point:
                o.fill_(float("nan"))
            else:
                o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(_bits(o), _bits(w)), f"replay {r} differs from the eager result"


def _bits(t):
    import torch
    return {torch.bfloat16: lambda x: x.view(torch.int16),
            torch.float32: lambda x: x.view(torch.int32)}.get(t.dtype, lambda x: x)(t)


def _bufs(inp):
    import torch
    out = torch.empty((inp.batch, inp.q_len, inp.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, inp.q_len, inp.heads), dtype=torch.float32, device="cuda")
    return out, lse


@pytest.mark.parametrize("nsplit", [1, 4])
def test_graph_decode(smla, nsplit):
    inp = flat_inputs("graph", 9500, 2, 1, 24, 8192, 700)
    dev = to_device(inp, "cuda")
    out, lse = _bufs(inp)
    ws = smla.workspace(inp.batch, inp.q_len, inp.heads, nsplit, "cuda")
    other = flat_inputs("graph_other", 9501, 2, 1, 24, 8192, 700)
    odev = to_device(other, "cuda")
    oout, olse = _bufs(other)

    def fn():
        smla.smla_decode(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit, workspace_t=ws)

    def disturb():  # the same workspace used by an eager call on other inputs
        smla.smla_decode(odev["q"], odev["kv"], odev["idx"], oout, olse, other.scale, nsplit,
                         workspace_t=ws)
    _replays(fn, [out, lse], disturb)


def test_graph_decode_long_slices(smla):
    """64 heads over slices of 79 tiles: the role-specialised kernel (four
    tile buffers, refills past the last tile load the zero row, the list ring
    refilled every 16 tiles) replayed."""
    inp = flat_inputs("graph3", 9510, 1, 1, 64, 65536, 5000)
    dev = to_device(inp, "cuda")
    out, lse = _bufs(inp)
    ws = smla.workspace(inp.batch, inp.q_len, inp.heads, 2, "cuda")
    other = flat_inputs("graph3_other", 9511, 1, 1, 64, 65536, 5000)
    odev = to_device(other, "cuda")
    oout, olse = _bufs(other)

    def fn():
        smla.smla_decode(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, 2, workspace_t=ws)

    def disturb():
        smla.smla_decode(odev["q"], odev["kv"], odev["idx"], oout, olse, other.scale, 2,
                         workspace_t=ws)
    _replays(fn, [out, lse], disturb)


def test_graph_paged_and_fused(smla):
    import torch
    inp = workload("batched", batch=8)
    dev = to_device(inp, "cuda")
    table = torch.from_numpy(block_table(inp)).cuda()
    pos = torch.from_numpy(np.ascontiguousarray(inp.pos)).cuda()
    out, lse = _bufs(inp)
    out2, lse2 = _bufs(inp)
    ws = smla.workspace(inp.batch, inp.q_len, inp.heads, 4, "cuda")
    ws2 = smla.workspace(inp.batch, inp.q_len, inp.heads, 4, "cuda")
    sync = smla.fused_sync("cuda")

    def fn():
        smla.smla_decode_paged(dev["q"], dev["kv"], table, 64, pos, out, lse, inp.scale, 4, ws)
        smla.smla_decode_fused(dev["q"], dev["kv"], dev["idx"], out2, lse2, inp.scale, 4, ws2,
                               sync=sync)

    def disturb():
        smla.smla_decode_fused(dev["q"], dev["kv"], dev["idx"], out2, lse2, inp.scale, 4, ws2,
                               sync=sync)
    assert smla.smla_fused_in_launch(inp.batch, inp.q_len, inp.heads, 4)
    _replays(fn, [out, lse, out2, lse2], disturb)
    assert torch.count_nonzero(sync).item() == 0


def test_graph_dense(smla):
    import torch
    inp = dense_inputs("graph_dense", 9600, 1, 9, 8, [9000], paged=False)
    dev = to_device(inp, "cuda")
    ctx = torch.tensor(inp.ctx, dtype=torch.int32, device="cuda")
    out, lse = _bufs(inp)
    assert smla.dense_folds(9, 8, 9000)

    def fn():
        smla.smla_decode_dense(dev["q"], dev["kv"], ctx, 9000, out, lse, inp.scale, 0)
    _replays(fn, [out, lse], lambda: None)


def test_graph_topk(smla):
    import torch
    scores = torch.from_numpy(index_scores(9700, 4, 2, 20000)).cuda()
    other = torch.from_numpy(index_scores(9701, 4, 2, 20000)).cuda()
    ctx = torch.tensor([20000, 5000, 2047, 19999], dtype=torch.int32, device="cuda")
    pos = torch.empty((4, 2, 2048), dtype=torch.int32, device="cuda")
    pos2 = torch.empty_like(pos)

    def fn():
        smla.smla_topk(scores, 2048, pos, ctx)

    def disturb():
        smla.smla_topk(other, 2048, pos2, ctx)
    _replays(fn, [pos], disturb)


@pytest.mark.parametrize("form", ["auto", "chunks", "sampled"])
def test_graph_topk_multi(smla, form):
    """The multi-workgroup top-k forms captured: 4 rows of up to 65536
    positions (AUTO takes the sampled form), with one workspace that the
    disturbing calls between replays overwrite (the forms need no clearing)."""
    import torch
    scores = torch.from_numpy(index_scores(9710, 2, 2, 65536)).cuda()
    other = torch.from_numpy(index_scores(9711, 2, 2, 65536)).cuda()
    ctx = torch.tensor([65536, 30001], dtype=torch.int32, device="cuda")
    pos = torch.empty((2, 2, 2048), dtype=torch.int32, device="cuda")
    pos2 = torch.empty_like(pos)
    n = smla.smla_topk_workspace_bytes(2, 2, 65536)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    f = {"auto": smla.TOPK_AUTO, "chunks": smla.TOPK_CHUNKS, "sampled": smla.TOPK_SAMPLED}[form]

    def fn():
        smla.smla_topk(scores, 2048, pos, ctx, workspace_t=ws, form=f)

    def disturb():
        smla.smla_topk(other, 2048, pos2, ctx, workspace_t=ws, form=f)
    _replays(fn, [pos], disturb)
