"""GPU edge cases: the HIP path (through the C ABI) against the fp64 oracle.

Same bar as the workload parity tests (oracle/compare.py).  Covered here:
head counts that leave partial head blocks (1, 17, 24, 33, 130, 1000), list
lengths that leave ragged tiles (1, 33, 100, 257) or span several staged list
chunks (5000); masked, out-of-range and duplicated indices; fully empty
selections and empty splits; topk == 0; the split kernel's partials against
the oracle's per-split results; seeded random shapes across the head
classes, list lengths and split counts; the combine kernel alone on synthetic
partials (both its few-pair and many-pair forms, with NaN in the slots of
empty splits); bit-exact repeatability; output and workspace buffers
poisoned with NaN beforehand; a non-default stream; the limits (4096 heads,
NSPLIT 1024, a list over all 65536 rows of a cache); outlier rows that raise
some heads' running maximum part-way through a slice, in either half of a
tile's rows.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import (bf16_bits_to_f32, edge_inputs, flat_inputs, partials_inputs, spike_inputs,
                       to_device, torch_to_bits, workload)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def _alloc(inp, dev, fill=None):
    import torch
    b, lq, h = inp.batch, inp.q_len, inp.heads
    out = torch.empty((b, lq, h, 512), dtype=torch.bfloat16, device=dev["q"].device)
    lse = torch.empty((b, lq, h), dtype=torch.float32, device=dev["q"].device)
    if fill is not None:
        out.fill_(fill)
        lse.fill_(fill)
    return out, lse


def _host(out, lse):
    return bf16_bits_to_f32(torch_to_bits(out)), lse.cpu().numpy()


def _parity(o_g, l_g, o_r, l_r, what):
    ok, m = check(o_g, l_g, o_r, l_r)
    print(f"{what}: max_abs={m['max_abs']:.3g} rel_l2={m['rel_l2']:.3g} "
          f"lse={m['lse_max_abs']:.3g} empty={m['empty']}", flush=True)
    assert ok, f"{what}: {m['reasons']}"


def _decode(smla, inp, dev, nsplit, fill=None, ws=None, stream=None):
    import torch
    out, lse = _alloc(inp, dev, fill)
    used = smla.smla_decode(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit,
                            workspace_t=ws, stream=stream)
    if stream is None:
        torch.cuda.synchronize()
    else:
        stream.synchronize()
    return out, lse, used


# ------------------------------------------------------------ shapes

SHAPES = [  # batch, q_len, heads, topk, kv_rows, nsplits
    (1, 1, 1, 1, 4096, [1, 0, 4]),
    (2, 1, 24, 33, 4096, [1, 2, 0]),
    (1, 2, 130, 100, 4096, [1, 4, 0]),
    (3, 1, 17, 100, 2000, [0, 7]),
    (2, 1, 33, 257, 4096, [0, 3, 9]),
    (1, 1, 8, 5000, 65536, [1, 2, 0]),
    (1, 1, 64, 5000, 65536, [1, 2]),
    (1, 1, 1000, 40, 4096, [1, 0, 2]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}q{}h{}k{}n{}".format(*s[:5]))
def test_shapes(smla, shape):
    b, lq, h, k, rows, nsplits = shape
    inp = flat_inputs("shape", 5000 + h * 7 + k, b, lq, h, rows, k)
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    for ns in nsplits:
        out, lse, used = _decode(smla, inp, dev, ns)
        _parity(*_host(out, lse), o_r, l_r, f"b{b} q{lq} h{h} k{k} nsplit={ns} (used {used})")


# The library's limits and the largest list: the most heads a call accepts
# (4096: 64 head blocks), the most splits (1024, with 2 and with 0.1 entries
# per split), and a list that is a permutation of a whole 65536-row cache
# (attention over every row: one split walks 2048 tiles and 64 staged list
# chunks, the planner's split count 256 of 8 tiles).
LIMITS = [  # batch, q_len, heads, topk, kv_rows, nsplits
    (1, 1, 4096, 300, 4096, [1, 0, 3]),
    (1, 1, 8, 2048, 4096, [1024]),
    (2, 1, 16, 100, 4096, [1024]),
    (1, 1, 8, 65536, 65536, [0, 1]),
]


@pytest.mark.parametrize("shape", LIMITS, ids=lambda s: "b{}q{}h{}k{}n{}".format(*s[:5]))
def test_limits(smla, shape):
    b, lq, h, k, rows, nsplits = shape
    inp = flat_inputs("limits", 7000 + h * 3 + k, b, lq, h, rows, k)
    if k == rows:  # a permutation of the whole cache
        assert (np.sort(inp.idx, axis=-1) == np.arange(rows)).all()
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    for ns in nsplits:
        out, lse, used = _decode(smla, inp, dev, ns)
        _parity(*_host(out, lse), o_r, l_r, f"b{b} q{lq} h{h} k{k} nsplit={ns} (used {used})")


# Seeded random shapes over every head class, list length and split count
# (including NSPLIT above the list length and the planner), each against the
# oracle: the fixed shapes above pin the known corners, these sample between.
def _random_shapes(n=10, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        h = int(rng.choice([1, 3, 8, 15, 16, 19, 32, 40, 63, 64, 65, 96, 129]))
        k = int(rng.integers(1, 3000))
        rows = int(rng.integers(k, 3 * k + 2))
        b, lq = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        ns = [0, int(rng.integers(1, 9)), int(rng.integers(9, 130))]
        out.append((b, lq, h, k, rows, ns))
    return out


@pytest.mark.parametrize("shape", _random_shapes(), ids=lambda s: "b{}q{}h{}k{}r{}".format(*s[:5]))
def test_random_shapes(smla, shape):
    b, lq, h, k, rows, nsplits = shape
    inp = flat_inputs("rand_shape", 6000 + h * 13 + k, b, lq, h, rows, k)
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    for ns in nsplits:
        out, lse, used = _decode(smla, inp, dev, ns)
        _parity(*_host(out, lse), o_r, l_r, f"b{b} q{lq} h{h} k{k} rows{rows} nsplit={ns} (used {used})")


# ------------------------------------------------------------ masking

@pytest.fixture(scope="module")
def edge(smla):
    inp = edge_inputs()
    dev = to_device(inp, "cuda")
    ref = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    return inp, dev, ref


@pytest.mark.parametrize("nsplit", [1, 2, 4, 0, 300, 301])
def test_masked_duplicate_out_of_range(smla, edge, nsplit):
    inp, dev, (o_r, l_r) = edge
    assert np.isneginf(l_r[0, 0]).all() and np.isfinite(l_r[1, 1]).all()
    out, lse, used = _decode(smla, inp, dev, nsplit)
    _parity(*_host(out, lse), o_r, l_r, f"edge nsplit={nsplit} (used {used})")


def test_topk_zero(smla):
    import torch
    inp = flat_inputs("k0", 77, 2, 1, 8, 512, 0)
    dev = to_device(inp, "cuda")
    out, lse, _ = _decode(smla, inp, dev, 0, fill=float("nan"))
    assert torch.all(out == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


# ------------------------------------------------------------ partials

@pytest.mark.parametrize("case", ["edge", "tiny"])
@pytest.mark.parametrize("nsplit", [3, 8, 128])
def test_split_partials(smla, case, nsplit):
    import torch
    inp = edge_inputs() if case == "edge" else workload("tiny")
    dev = to_device(inp, "cuda")
    out, lse = _alloc(inp, dev)
    used, ws = smla.smla_split(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit)
    torch.cuda.synchronize()
    assert used == nsplit
    po, pl = smla.partials_view(ws, inp.batch, inp.q_len, inp.heads, nsplit)
    po_r, pl_r = oracle.partial(inp.q, inp.kv, inp.idx, inp.scale, nsplit)
    _parity(po.cpu().numpy(), pl.cpu().numpy(), po_r, pl_r, f"partials {case} nsplit={nsplit}")


# ------------------------------------------------------------ combine alone

COMBINE = [  # tokens, nsplit, heads: few pairs (split-parallel form), many pairs (wide form)
    (2, 1, 8), (2, 2, 8), (2, 9, 8), (2, 33, 8), (1, 128, 8), (1, 1024, 4),
    (16, 1, 64), (16, 2, 64), (16, 8, 64), (16, 9, 64), (8, 20, 130),
]


@pytest.mark.parametrize("shape", COMBINE, ids=lambda s: "t{}s{}h{}".format(*s))
def test_combine_only(smla, shape):
    import torch
    t, s, h = shape
    po, pl = partials_inputs(900 + t * s + h, t, s, h)
    o_r, l_r = oracle.combine(po.astype(np.float64), pl.astype(np.float64))
    assert np.isneginf(l_r[-1, -1])
    out = torch.empty((t, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((t, h), dtype=torch.float32, device="cuda")
    smla.smla_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, lse)
    torch.cuda.synchronize()
    _parity(*_host(out, lse), o_r, l_r, f"combine t{t} s{s} h{h}")


# ------------------------------------------------------------ robustness

def test_repeatable_bit_exact(smla):
    import torch
    inp = workload("long")
    dev = to_device(inp, "cuda")
    first = None
    for i in range(20):
        out, lse, used = _decode(smla, inp, dev, 0)
        cur = (out.view(torch.int16).clone(), lse.view(torch.int32).clone())
        if first is None:
            first = cur
            continue
        assert torch.equal(cur[0], first[0]) and torch.equal(cur[1], first[1]), f"run {i}"
    print(f"20 runs bit-identical at nsplit {used}", flush=True)


@pytest.mark.parametrize("nsplit", [1, 4, 301])
def test_poisoned_buffers(smla, edge, nsplit):
    import torch
    inp, dev, (o_r, l_r) = edge
    ws = smla.workspace(inp.batch, inp.q_len, inp.heads, nsplit, "cuda")
    if ws is not None:
        ws.fill_(0xFF)  # every fp32 word of the partials is a NaN
    out, lse, _ = _decode(smla, inp, dev, nsplit, fill=float("nan"), ws=ws)
    _parity(*_host(out, lse), o_r, l_r, f"poisoned nsplit={nsplit}")


def test_side_stream(smla, edge):
    import torch
    inp, dev, (o_r, l_r) = edge
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = _alloc(inp, dev, float("nan"))
        smla.smla_decode(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, 0, stream=s)
    s.synchronize()
    _parity(*_host(out, lse), o_r, l_r, "side stream")


# Outlier rows (token, list position, head, factor): each raises that head's
# running maximum part-way through a long slice, most by far more than the
# lazy-rescale threshold (2^8), so the rescale of the accumulated O and sum
# runs after the first tile; factor 4 stays near the threshold, and factor 120
# lifts the score by 150-210 in base 2, past fp32's exp2 range for weights taken
# against the old maximum.  List position p sits in tile p // 32 at row
# p % 32: rows 0-15 and 16-31 of a tile are the two row halves of the 64-head
# blocks, whose waves must agree on the new maximum.  Positions 1500 and 1501
# spike two heads in one tile; head 3 and head 5 spike twice, the second time
# higher.
SPIKES = [(0, 610, 3, 4.0), (0, 700, 3, 14.0), (0, 1040, 17, 12.0), (0, 1500, 40, 12.0),
          (0, 1501, 41, 120.0), (0, 1999, 63, 12.0), (1, 33, 5, 12.0), (1, 1200, 5, 20.0)]


@pytest.mark.parametrize("heads", [8, 24, 64, 128])
@pytest.mark.parametrize("nsplit", [1, 2, 0])
def test_running_max_grows_mid_slice(smla, heads, nsplit):
    spikes = [(t, pos, h % heads, f) for t, pos, h, f in SPIKES]
    inp = spike_inputs(9800 + heads, 2, heads, 8192, 2048, spikes)
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    # each spiked head's LSE is about its outlier's score, above the ordinary ~8
    for t, _, h, _ in spikes:
        assert l_r[t, 0, h] > 10.0
    out, lse, used = _decode(smla, inp, dev, nsplit, fill=float("nan"))
    _parity(*_host(out, lse), o_r, l_r, f"spikes heads={heads} nsplit={nsplit} (used {used})")
