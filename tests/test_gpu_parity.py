"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (oracle/compare.py): max-abs 1e-2 and relative L2 5e-3 on the bf16
output, 1e-3 absolute on LSE, -inf/0 exactly where the selection is empty.

Covered: the five workloads (tiny, long, batched, spec at three contexts,
ragged, plus ragged with -1 padding at the tail of the lists and at shuffled
positions) at the NSPLIT values the bench sweeps and the planner's choice.
Every workload runs at full size and is compared over its whole output
tensor: for the paged pools (2.4 GB and ~9.8 GB on the device) the oracle
receives host copies of exactly the rows the lists select.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import bf16_bits_to_f32, oracle_view, to_device, torch_to_bits, workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def run_gpu(smla, dev, inp, nsplit, sync=True):
    import torch
    b, lq, h = inp.batch, inp.q_len, inp.heads
    out = torch.empty((b, lq, h, 512), dtype=torch.bfloat16, device=dev["q"].device)
    lse = torch.empty((b, lq, h), dtype=torch.float32, device=dev["q"].device)
    used = smla.smla_decode(dev["q"], dev["kv"], dev["idx"], out, lse, inp.scale, nsplit)
    if sync:
        torch.cuda.synchronize()
    return out, lse, used


def host(out, lse):
    return bf16_bits_to_f32(torch_to_bits(out)), lse.cpu().numpy()


def assert_parity(out_g, lse_g, out_r, lse_r, what):
    ok, m = check(out_g, lse_g, out_r, lse_r)
    print(f"{what}: max_abs={m['max_abs']:.3g} rel_l2={m['rel_l2']:.3g} "
          f"lse={m['lse_max_abs']:.3g} empty={m['empty']}", flush=True)
    assert ok, f"{what}: {m['reasons']}"


# ---------------------------------------------------------------- workloads

@pytest.fixture(scope="module")
def tiny(smla):
    inp = workload("tiny")
    dev = to_device(inp, "cuda")
    ref = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    return inp, dev, ref


@pytest.mark.parametrize("nsplit", [1, 4, 0, 2, 3, 5, 8, 127, 128, 200])
def test_tiny(smla, tiny, nsplit):
    inp, dev, (o_r, l_r) = tiny
    out, lse, used = run_gpu(smla, dev, inp, nsplit)
    o_g, l_g = host(out, lse)
    assert_parity(o_g, l_g, o_r, l_r, f"tiny nsplit={nsplit} (used {used})")


@pytest.fixture(scope="module")
def long_ctx(smla):
    inp = workload("long")
    dev = to_device(inp, "cuda")
    ref = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    return inp, dev, ref


@pytest.mark.parametrize("nsplit", [1, 16, 64, 128, 0])
def test_long(smla, long_ctx, nsplit):
    inp, dev, (o_r, l_r) = long_ctx
    out, lse, used = run_gpu(smla, dev, inp, nsplit)
    o_g, l_g = host(out, lse)
    assert_parity(o_g, l_g, o_r, l_r, f"long nsplit={nsplit} (used {used})")


@pytest.mark.parametrize("ctx", [4096, 16384, 65536])
@pytest.mark.parametrize("nsplit", [16, 64, 0])
def test_spec(smla, ctx, nsplit):
    inp = workload("spec", spec_ctx=ctx)
    dev = to_device(inp, "cuda")
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    out, lse, used = run_gpu(smla, dev, inp, nsplit)
    o_g, l_g = host(out, lse)
    assert_parity(o_g, l_g, o_r, l_r, f"spec ctx={ctx} nsplit={nsplit} (used {used})")


@pytest.fixture(scope="module")
def batched(smla):
    inp = workload("batched")
    dev = to_device(inp, "cuda")
    q_s, kv_s, idx_s = oracle_view(inp, dev["kv"])  # all 64 sequences
    ref = oracle.decode(q_s, kv_s, idx_s, inp.scale)
    return inp, dev, ref


@pytest.mark.parametrize("nsplit", [0, 1, 2, 4, 8, 16])
def test_batched_full_size(smla, batched, nsplit):
    inp, dev, (o_r, l_r) = batched
    out, lse, used = run_gpu(smla, dev, inp, nsplit)
    o_g, l_g = host(out, lse)
    assert_parity(o_g, l_g, o_r, l_r, f"batched nsplit={nsplit} (used {used}), all 64 sequences")


@pytest.mark.parametrize("pad", ["none", "tail", "shuffled"])
def test_ragged_full_size(smla, pad):
    import torch
    inp = workload("ragged", ragged_pad=pad != "none", pad_shuffle=pad == "shuffled")
    dev = to_device(inp, "cuda")
    q_s, kv_s, idx_s = oracle_view(inp, dev["kv"])  # all 128 sequences
    o_r, l_r = oracle.decode(q_s, kv_s, idx_s, inp.scale)
    if pad == "none":  # NSPLIT 2: the 128-head partials through the combine
        out, lse, used = run_gpu(smla, dev, inp, 2)
        assert_parity(*host(out, lse), o_r, l_r, "ragged nsplit=2, all 128 sequences")
    out, lse, used = run_gpu(smla, dev, inp, 0)
    o_g, l_g = host(out, lse)
    if pad != "none":
        masked = inp.idx[:16] == -1
        assert masked.any(), "padded workload must hold -1 entries"
        if pad == "shuffled":  # some -1 entry sits before a valid one in its list
            first_masked = np.argmax(masked, axis=-1)
            assert (first_masked < (inp.idx[:16] >= 0).sum(-1) - 1).any()
    assert_parity(o_g, l_g, o_r, l_r, f"ragged pad={pad} planner nsplit={used}, all 128 sequences")
    del dev
    torch.cuda.empty_cache()
