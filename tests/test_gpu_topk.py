"""GPU parity of the top-k producer (smla_topk, through the C ABI).

Positions are integers, so the bar is bit-exact: the GPU's output must equal
oracle.topk_positions element for element (selected set, ascending order and
-1 padding).  Scores: N(0,1), heavy ties, all equal, and a mix of special
values (+-0, +-inf, +-NaN, subnormals), over rows that are shorter than topk,
exactly topk, one longer, not a multiple of the workgroup width, with and
without per-sequence context lengths, with more equal keys than the LDS
candidate copy holds, with rows 16-byte aligned (16-byte loads) or not,
each through the three work splits (one workgroup per row; rows cut into
4096-position chunks over several workgroups in four launches; and the
sampled two-launch form, whose candidate threshold comes from a sample of
the row, with the heavy-tie cases taking its fallback), the workspace
starting as garbage; then the full sizes of the batch-1
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


FORMS = ["chunks", "row", "sampled"]


def _run(smla, scores, topk, ctx=None, form="chunks"):
    """form: "chunks" (rows cut into 4096-position chunks, four launches) or
    "sampled" (two launches), each forced from two chunks on with a
    workspace that starts as garbage; "row": one workgroup per row."""
    import torch
    s = torch.from_numpy(scores).cuda()
    out = torch.full((scores.shape[0], scores.shape[1], topk), 12345, dtype=torch.int32, device="cuda")
    c = None if ctx is None else torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws = None
    if form != "row":
        n = smla.smla_topk_workspace_bytes(scores.shape[0], scores.shape[1], scores.shape[2])
        ws = torch.full((max(n, 256),), 0xA5, dtype=torch.uint8, device="cuda")
    f = {"chunks": smla.TOPK_CHUNKS, "row": smla.TOPK_ROWS, "sampled": smla.TOPK_SAMPLED}[form]
    smla.smla_topk(s, topk, out, c, workspace_t=ws, form=f)
    torch.cuda.synchronize()
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


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-b{c[1]}q{c[2]}m{c[3]}k{c[4]}")
def test_topk_parity(smla, case, form):
    kind, b, lq, m, k, ctx = case
    scores = index_scores(700 + m + k, b, lq, m, kind)
    got = _run(smla, scores, k, ctx, form)
    _same(got, oracle.topk_positions(scores, ctx, k), f"{kind} b{b} q{lq} m{m} k{k} form={form}")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("shape", [(1, 1, 65536), (64, 1, 32768)], ids=["long", "batched"])
def test_topk_full_size(smla, shape, form):
    b, lq, m = shape
    scores = index_scores(7100 + b, b, lq, m, "normal")
    got = _run(smla, scores, 2048, form=form)
    _same(got, oracle.topk_positions(scores, None, 2048), f"full size {shape} form={form}")


def test_topk_two_values(smla):
    """Half the scores 1.0, half 0.0, over 30000 positions: the threshold bin
    holds about 15000 keys (more than the LDS copy takes) and the ties at 1.0
    must go to the lowest positions."""
    rng = np.random.default_rng(7150)
    scores = (rng.random((2, 1, 30000)) < 0.5).astype(np.float32)
    for k in (2048, 15000, 29999):
        for form in FORMS:
            _same(_run(smla, scores, k, form=form), oracle.topk_positions(scores, None, k),
                  f"two values k={k} form={form}")


def test_topk_ragged_contexts(smla):
    """Contexts of the ragged workload's range, up to 131072 positions."""
    rng = np.random.default_rng(7200)
    ctx = rng.integers(2048, 131073, size=8).tolist()
    ctx[0], ctx[1] = 131072, 1000  # the largest context, and one below topk
    scores = index_scores(7201, 8, 1, 131072, "normal")
    want = oracle.topk_positions(scores, ctx, 2048)
    for form in FORMS:
        _same(_run(smla, scores, 2048, ctx, form), want, f"ragged contexts form={form}")


def _random_case(seed):
    """A seeded random shape: rows, length, ragged contexts (some below
    topk), topk and score kind."""
    rng = np.random.default_rng(seed)
    b, lq = int(rng.integers(1, 9)), int(rng.integers(1, 4))
    m = int(rng.integers(4097, 140000))
    k = int(rng.choice([1, 64, 2048, int(rng.integers(2, 6000))]))
    ctx = rng.integers(0, m + 1, size=b).tolist()
    ctx[0] = m
    kind = str(rng.choice(["normal", "normal", "ties", "special"]))
    return b, lq, m, k, ctx, kind


@pytest.mark.parametrize("seed", range(7500, 7508))
def test_topk_random_shapes(smla, seed):
    """Eight seeded random shapes, every form against the oracle."""
    b, lq, m, k, ctx, kind = _random_case(seed)
    scores = index_scores(seed, b, lq, m, kind)
    want = oracle.topk_positions(scores, ctx, k)
    for form in FORMS:
        _same(_run(smla, scores, k, ctx, form), want, f"seed {seed}: b{b} q{lq} m{m} k{k} {kind} form={form}")


def test_topk_rows_past_sampled_limit(smla):
    """Rows of 1100000 positions, past the 1048576 the sampled form takes:
    AUTO and the forced sampled form run the four launches there; two rows,
    one cut short by its context."""
    m = 1_100_000
    scores = index_scores(7450, 2, 1, m, "normal")
    ctx = [m, 700_001]
    want = oracle.topk_positions(scores, ctx, 2048)
    for form in ("chunks", "sampled"):
        _same(_run(smla, scores, 2048, ctx, form), want, f"1.1M positions form={form}")
    import torch
    s = torch.from_numpy(scores).cuda()
    out = torch.full((2, 1, 2048), 12345, dtype=torch.int32, device="cuda")
    n = smla.smla_topk_workspace_bytes(2, 1, m)
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    smla.smla_topk(s, 2048, out, torch.tensor(ctx, dtype=torch.int32, device="cuda"), workspace_t=ws,
                   form=smla.TOPK_AUTO)
    torch.cuda.synchronize()
    _same(out.cpu().numpy(), want, "1.1M positions form=auto")


def test_topk_sample_misleads(smla):
    """Scores large exactly on the sampled form's sample (256 blocks of 16
    positions at offsets floor(t n / 256) rounded down to a multiple of 4)
    and small elsewhere: its threshold then lands among the sampled keys,
    far fewer than topk keys reach it, and the row must take the exact
    fallback.  Rows of 65536 and 40000 positions, topk 2048 and 5000; every
    form must give the oracle's selection."""
    rng = np.random.default_rng(7400)
    lens = [65536, 40000]
    scores = rng.standard_normal((2, 1, 65536)).astype(np.float32) * 0.01
    for r, n in enumerate(lens):
        for t in range(256):
            s0 = (t * n // 256) & ~3
            scores[r, 0, s0:s0 + 16] = 10.0 + rng.random(16).astype(np.float32)
    for k in (2048, 5000):
        want = oracle.topk_positions(scores, lens, k)
        for form in FORMS:
            _same(_run(smla, scores, k, lens, form), want, f"misleading sample k={k} form={form}")


def test_topk_auto_many_long_rows(smla):
    """96 rows of ragged contexts up to 131072 positions through the
    automatic form (the sampled one here) and the forced four-launch form:
    with this many rows each chunk workgroup takes several 4096-position
    sub-chunks (three on a 256-CU device), including chunks that end inside
    a sub-chunk."""
    import torch
    rng = np.random.default_rng(7250)
    rows = 96
    ctx = rng.integers(2048, 131073, size=rows).tolist()
    ctx[0], ctx[1], ctx[2] = 131072, 1000, 4096 * 3 + 17
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert rows * (131072 // 4096) // (4 * cus) >= 2, "this shape must take more than one sub-chunk"
    scores = index_scores(7251, rows, 1, 131072, "normal")
    s = torch.from_numpy(scores).cuda()
    out = torch.full((rows, 1, 2048), 12345, dtype=torch.int32, device="cuda")
    n = smla.smla_topk_workspace_bytes(rows, 1, 131072)
    want = oracle.topk_positions(scores, ctx, 2048)
    for form in (smla.TOPK_AUTO, smla.TOPK_CHUNKS):
        ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
        out.fill_(12345)
        smla.smla_topk(s, 2048, out, torch.tensor(ctx, dtype=torch.int32, device="cuda"), workspace_t=ws,
                       form=form)
        torch.cuda.synchronize()
        _same(out.cpu().numpy(), want, f"96 long rows, form {form}")


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
