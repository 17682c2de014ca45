"""GPU parity of the top-k producer (smla_topk, through the C ABI).

Positions are integers, so the bar is bit-exact: the GPU's output must equal
oracle.topk_positions element for element (selected set, ascending order and
-1 padding).  Scores: N(0,1), heavy ties, all equal, and a mix of special
values (+-0, +-inf, +-NaN, subnormals), over rows that are shorter than topk,
exactly topk, one longer, not a multiple of the workgroup width, with and
without per-sequence context lengths, with more equal keys than the LDS
candidate copy holds, with rows 16-byte aligned (16-byte loads) or not,
each through both work splits (one workgroup per row, and rows cut into
4096-position chunks over several workgroups, whose workspace starts as
garbage); then the full sizes of the batch-1
(65536) and batch-64 (32768) shapes and ragged contexts up to 131072,
compared on every row.  Last, the path end to end: scores -> smla_topk ->
smla_decode_paged against oracle.topk_positions -> rows_of_positions ->
oracle.decode.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import (PAGE, bf16_bits_to_f32, block_table, dense_inputs, index_scores, to_device,
                       torch_to_bits)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def _run(smla, scores, topk, ctx=None, multi=True):
    """multi: rows cut into 4096-position chunks over several workgroups
    (forced from two chunks on, with a workspace that starts as garbage),
    else one workgroup per row."""
    import torch
    s = torch.from_numpy(scores).cuda()
    out = torch.full((scores.shape[0], scores.shape[1], topk), 12345, dtype=torch.int32, device="cuda")
    c = None if ctx is None else torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws = None
    if multi:
        n = smla.smla_topk_workspace_bytes(scores.shape[0], scores.shape[1], scores.shape[2])
        ws = torch.full((max(n, 256),), 0xA5, dtype=torch.uint8, device="cuda")
    prev = smla.smla_set_topk_min_chunks(2 if multi else 0)
    try:
        smla.smla_topk(s, topk, out, c, workspace_t=ws)
        torch.cuda.synchronize()
    finally:
        smla.smla_set_topk_min_chunks(prev)
    return out.cpu().numpy()


def _same(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} positions differ, first at {bad[0].tolist()}"


CASES = [  # kind, batch, q_len, max_ctx, topk, ctx
    ("normal", 2, 3, 5000, 2048, None),
    ("normal", 3, 1, 3000, 2048, [2047, 2048, 2049]),
    ("normal", 2, 1, 1500, 2048, [1500, 0]),
    ("ties", 2, 2, 9000, 2048, None),
    ("ties", 1, 1, 4097, 1, None),
    ("equal", 2, 1, 7000, 2048, [7000, 3000]),
    ("special", 2, 2, 6000, 700, [6000, 5999]),
    ("normal", 1, 1, 20000, 5000, None),
    ("equal", 1, 2, 20000, 2048, None),      # > 8192 keys in the first digit's bin: no LDS copy
    ("normal", 2, 1, 5001, 2048, [5001, 4999]),  # rows not 16-byte aligned: 4-byte loads
    ("ties", 1, 1, 9001, 2048, None),
]


@pytest.mark.parametrize("multi", [True, False], ids=["chunks", "row"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-b{c[1]}q{c[2]}m{c[3]}k{c[4]}")
def test_topk_parity(smla, case, multi):
    kind, b, lq, m, k, ctx = case
    scores = index_scores(700 + m + k, b, lq, m, kind)
    got = _run(smla, scores, k, ctx, multi)
    _same(got, oracle.topk_positions(scores, ctx, k), f"{kind} b{b} q{lq} m{m} k{k} multi={multi}")


@pytest.mark.parametrize("multi", [True, False], ids=["chunks", "row"])
@pytest.mark.parametrize("shape", [(1, 1, 65536), (64, 1, 32768)], ids=["long", "batched"])
def test_topk_full_size(smla, shape, multi):
    b, lq, m = shape
    scores = index_scores(7100 + b, b, lq, m, "normal")
    got = _run(smla, scores, 2048, multi=multi)
    _same(got, oracle.topk_positions(scores, None, 2048), f"full size {shape} multi={multi}")


def test_topk_two_values(smla):
    """Half the scores 1.0, half 0.0, over 30000 positions: the threshold bin
    holds about 15000 keys (more than the LDS copy takes) and the ties at 1.0
    must go to the lowest positions."""
    rng = np.random.default_rng(7150)
    scores = (rng.random((2, 1, 30000)) < 0.5).astype(np.float32)
    for k in (2048, 15000, 29999):
        for multi in (True, False):
            _same(_run(smla, scores, k, multi=multi), oracle.topk_positions(scores, None, k),
                  f"two values k={k} multi={multi}")


def test_topk_ragged_contexts(smla):
    """Contexts of the ragged workload's range, up to 131072 positions."""
    rng = np.random.default_rng(7200)
    ctx = rng.integers(2048, 131073, size=8).tolist()
    ctx[0], ctx[1] = 131072, 1000  # the largest context, and one below topk
    scores = index_scores(7201, 8, 1, 131072, "normal")
    want = oracle.topk_positions(scores, ctx, 2048)
    for multi in (True, False):
        _same(_run(smla, scores, 2048, ctx, multi), want, f"ragged contexts multi={multi}")


def test_topk_feeds_paged_decode(smla):
    """scores -> smla_topk -> smla_decode_paged, against the oracle's own
    selection, page mapping and decode."""
    import torch
    ctx = [3000, 700, 5000]
    q_len, heads, k = 2, 16, 1024
    inp = dense_inputs("topk_e2e", 7300, len(ctx), q_len, heads, ctx, paged=True)
    max_ctx = int(max(ctx))
    scores = index_scores(7301, len(ctx), q_len, max_ctx, "normal")
    dev = to_device(inp, "cuda")
    table_np = block_table(inp)
    table = torch.from_numpy(table_np).cuda()
    pos = torch.empty((len(ctx), q_len, k), dtype=torch.int32, device="cuda")
    smla.smla_topk(torch.from_numpy(scores).cuda(), k, pos, torch.tensor(ctx, dtype=torch.int32,
                                                                          device="cuda"))
    out = torch.empty((len(ctx), q_len, heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(ctx), q_len, heads), dtype=torch.float32, device="cuda")
    smla.smla_decode_paged(dev["q"], dev["kv"], table, PAGE, pos, out, lse, inp.scale)
    torch.cuda.synchronize()
    pos_ref = oracle.topk_positions(scores, ctx, k)
    _same(pos.cpu().numpy(), pos_ref, "end-to-end positions")
    rows = oracle.rows_of_positions(table_np, PAGE, pos_ref, inp.kv_rows)
    o_r, l_r = oracle.decode(inp.q, inp.kv, rows, inp.scale)
    ok, m = check(bf16_bits_to_f32(torch_to_bits(out)), lse.cpu().numpy(), o_r, l_r)
    print(f"topk -> paged decode: max_abs={m['max_abs']:.3g} rel_l2={m['rel_l2']:.3g}", flush=True)
    assert ok, m["reasons"]
