"""smla_decode_noalloc (the partials in the library's static per-device
scratch array, nothing allocated) against smla_decode (a caller's workspace)
through the C ABI.

Same kernels, same arithmetic: the outputs must be bit-identical, and both
within the oracle tolerances.  Two calls in a row, the second on a smaller
input (the array keeps the first call's partials, which the second must not
read), then the first shape again; a shape whose partials exceed the array is
rejected before anything is launched.  Runs alone in a fresh process and
after the other GPU tests.
"""
from __future__ import annotations

import pytest

import oracle
from oracle.compare import check
from tests.conftest import gpu_available
from workloads import bf16_bits_to_f32, flat_inputs, to_device, torch_to_bits

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def _bufs(inp):
    import torch
    out = torch.full((inp.batch, inp.q_len, inp.heads, 512), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((inp.batch, inp.q_len, inp.heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    return out, lse


def _compare(smla, inp, dev, nsplit, what):
    import torch
    a_out, a_lse = _bufs(inp)
    used = smla.smla_decode_noalloc(dev["q"], dev["kv"], dev["idx"], a_out, a_lse, inp.scale, nsplit)
    torch.cuda.synchronize()
    b_out, b_lse = _bufs(inp)
    smla.smla_decode(dev["q"], dev["kv"], dev["idx"], b_out, b_lse, inp.scale, used)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16)), f"{what}: out differs"
    assert torch.equal(a_lse.view(torch.int32), b_lse.view(torch.int32)), f"{what}: lse differs"
    o_r, l_r = oracle.decode(inp.q, inp.kv, inp.idx, inp.scale)
    ok, m = check(bf16_bits_to_f32(torch_to_bits(a_out)), a_lse.cpu().numpy(), o_r, l_r)
    print(f"{what} nsplit={used}: max_abs={m['max_abs']:.3g} rel_l2={m['rel_l2']:.3g} "
          f"lse={m['lse_max_abs']:.3g}", flush=True)
    assert ok, f"{what}: {m['reasons']}"
    return used


def test_noalloc_matches_workspace_entry_point(smla):
    big = flat_inputs("noalloc_big", 9900, 4, 1, 64, 65536, 2048)
    small = flat_inputs("noalloc_small", 9901, 1, 2, 8, 4096, 300)
    dev_big, dev_small = to_device(big, "cuda"), to_device(small, "cuda")
    n1 = _compare(smla, big, dev_big, 0, "big (planner)")
    assert n1 > 1, "the first call must use the scratch array"
    _compare(smla, small, dev_small, 4, "small after big")
    _compare(smla, big, dev_big, 8, "big again")
    _compare(smla, small, dev_small, 1, "small, NSPLIT 1 (no partials)")


def test_noalloc_rejects_oversized_partials(smla):
    import torch
    # 64 tokens x 128 heads x 64 splits of fp32 partials: about 1 GiB > 64 MiB
    need = smla.smla_workspace_bytes(64, 1, 128, 64)
    assert need > smla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((4096, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((64, 1, 2048), dtype=torch.int32, device="cuda")
    out = torch.full((64, 1, 128, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((64, 1, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_decode_noalloc(q, kv, idx, out, lse, 0.1, 64)
    assert e.value.code == -4  # SMLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item() and torch.all(lse == 7.0).item()  # nothing written
