"""GPU parity of the single-launch merge (smla_decode_fused: the partials
merged inside the split launch) against the fp64 oracle and the two-launch
form.

The two-launch form (smla_split, then smla_combine) is the reference form of
the merge; both are held to the oracle with the tolerances of the other
parity tests.  Covered: NSPLIT 2 .. 64 on the 16-, 32- and 64-head kernels
(the last in both its forms: row halves and role-specialised), partial head blocks,
several tokens, splits that are empty, topk 0; the synchronisation words
back at zero after every call; one workspace and one set of synchronisation
words reused across shapes; the wait-free form (merge polls 0: the last
arriving workgroup merges every slice), which must give the same bits;
bit-exact repeats.
"""
from __future__ import annotations

import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import (bf16_bits_to_f32, flat_inputs, oracle_view, to_device, torch_to_bits,
                       workload)

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


def _sync_zero(sync, what):
    import torch
    assert torch.count_nonzero(sync).item() == 0, f"{what}: sync words left non-zero"


def _single(smla, inp, dev, nsplit, ws, sync, polls=2048):
    """smla_decode_fused with the partials area poisoned first (NaN words): a
    merge that read a partial before its writer's stores landed would show it."""
    import torch
    ws.fill_(0xFF)
    out, lse = _outputs(inp, dev["q"].device)
    smla.smla_decode_fused(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit,
                           workspace_t=ws, sync=sync, merge_polls=polls)
    torch.cuda.synchronize()
    return out, lse


def _two(smla, inp, dev, nsplit, ws):
    import torch
    out, lse = _outputs(inp, dev["q"].device)
    smla.smla_split(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit, workspace_t=ws)
    po, pl = smla.partials_view(ws, inp.batch, inp.q_len, inp.heads, nsplit)
    smla.smla_combine(po, pl, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _same_bits(a, b, what):
    import torch
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: out differs"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: lse differs"


CASES = [  # name, batch, q_len, heads, topk, kv_rows, nsplits
    ("h8", 1, 1, 8, 2048, 65536, [2, 3, 16, 64]),
    ("h8_ragged", 3, 1, 8, 1000, 8192, [7, 33]),
    ("h24", 2, 1, 24, 300, 4096, [4, 10]),
    ("h64", 4, 1, 64, 700, 16384, [2, 5]),
    ("h64_long", 1, 1, 72, 5000, 65536, [2, 3]),  # slices of 53-79 tiles: the role-specialised kernel
    ("h130", 1, 2, 130, 100, 4096, [4]),
    ("empty_splits", 2, 1, 8, 33, 4096, [64]),   # 1 entry per split: 31 empty splits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_single_launch_parity(smla, case):
    name, b, lq, h, k, rows, nsplits = case
    inp = flat_inputs("single_" + name, 9100 + h + k, b, lq, h, rows, k)
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    sync = smla.fused_sync("cuda")
    for ns in nsplits:
        assert smla.smla_fused_in_launch(b, lq, h, ns), f"{name} nsplit={ns} not single launch"
        ws = smla.workspace(b, lq, h, ns, "cuda")
        one = _single(smla, inp, dev, ns, ws, sync)
        _sync_zero(sync, f"{name} nsplit={ns}")
        _parity(*_host(*one), o_r, l_r, f"{name} single nsplit={ns}")
        two = _two(smla, inp, dev, ns, ws)
        _parity(*_host(*two), o_r, l_r, f"{name} two-launch nsplit={ns}")
        again = _single(smla, inp, dev, ns, ws, sync)
        _same_bits(one, again, f"{name} single nsplit={ns} repeat")


def test_topk_zero_forced_split(smla):
    import torch
    inp = flat_inputs("single_k0", 9300, 2, 1, 8, 512, 0)
    dev = to_device(inp, "cuda")
    ws = smla.workspace(2, 1, 8, 4, "cuda")
    sync = smla.fused_sync("cuda")
    out, lse = _single(smla, inp, dev, 4, ws, sync)
    assert torch.all(out == 0).item() and torch.all(torch.isneginf(lse)).item()
    _sync_zero(sync, "topk 0")


@pytest.mark.parametrize("name,nsplit", [("long", 64), ("batched", 4), ("spec", 0)])
def test_wait_free_merge_same_bits(smla, name, nsplit):
    """Merge polls 0: no workgroup waits, the last arriver merges every slice
    of its unit; the slices' arithmetic does not depend on who runs it."""
    inp = workload(name)
    dev = to_device(inp, "cuda")
    if nsplit == 0:
        nsplit = smla.smla_plan_nsplit(inp.batch, inp.q_len, inp.heads, inp.topk)
    assert smla.smla_fused_in_launch(inp.batch, inp.q_len, inp.heads, nsplit)
    ws = smla.workspace(inp.batch, inp.q_len, inp.heads, nsplit, "cuda")
    sync = smla.fused_sync("cuda")
    ref = _single(smla, inp, dev, nsplit, ws, sync)
    free = _single(smla, inp, dev, nsplit, ws, sync, polls=0)
    _sync_zero(sync, f"{name} wait-free")
    _same_bits(ref, free, f"{name} wait-free nsplit={nsplit}")
    seqs = list(range(min(inp.batch, 3)))
    q_s, kv_s, idx_s = oracle_view(inp, dev["kv"], seqs)
    o_r, l_r = oracle.decode(q_s, kv_s, idx_s, inp.scale)
    _parity(*_host(free[0][seqs], free[1][seqs]), o_r, l_r, f"{name} wait-free")


def test_workspace_reused_across_shapes(smla):
    """One workspace and one set of sync words, zeroed once, serve calls of
    different shapes in turn."""
    shapes = [(1, 1, 8, 2048, 65536, 64), (4, 1, 64, 700, 16384, 5), (2, 1, 24, 300, 4096, 4),
              (1, 1, 8, 2048, 65536, 64)]
    size = max(smla.smla_workspace_bytes(b, lq, h, ns) for b, lq, h, _, _, ns in shapes)
    import torch
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    sync = smla.fused_sync("cuda")
    for i, (b, lq, h, k, rows, ns) in enumerate(shapes):
        inp = flat_inputs("single_reuse", 9400 + i, b, lq, h, rows, k)
        dev = to_device(inp, "cuda")
        out = _single(smla, inp, dev, ns, ws[: smla.smla_workspace_bytes(b, lq, h, ns)], sync)
        _sync_zero(sync, f"reuse {i}")
        o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
        _parity(*_host(*out), o_r, l_r, f"reuse {i}: b{b} h{h} nsplit={ns}")
