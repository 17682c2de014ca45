"""Host-side checks of the C-ABI library; no kernel is launched.

* the library loads after torch with a single HIP runtime in the process and
  exports every function include/smla.h declares (and nothing else);
* the planner is a deterministic pure function of (CUs, shape) with the
  documented bounds;
* workspace sizing follows the documented layout;
* invalid arguments return the documented status before anything launches.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    assert m.lib is not None  # the library loads (lazily) and binds every declared symbol
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_\w+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["smla_plan_nsplit", "smla_plan_nsplit_cus", "smla_workspace_bytes",
                            "smla_workspace_lse_offset", "smla_fused_in_launch",
                            "smla_decode", "smla_decode_fused", "smla_decode_noalloc",
                            "smla_topk", "smla_topk_workspace_bytes",
                            "smla_decode_paged",
                            "smla_decode_dense", "smla_plan_nsplit_dense", "smla_split",
                            "smla_combine", "smla_status_str"]), names


def test_library_exports_every_declared_symbol(smla):
    for name in declared_functions():
        assert hasattr(smla.lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", smla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines()
                       if ln.split()[1:2] == ["T"] and ln.split()[-1].startswith("smla_")})
    assert exported == declared_functions()


def test_single_hip_runtime_in_process(smla):
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths


def test_status_strings(smla):
    for code in range(0, -8, -1):
        assert smla.smla_status_str(code) not in ("", "unknown status")
    assert smla.smla_status_str(-99) == "unknown status"


# -------------------------------------------------------------------- planner

SHAPES = [(1, 1, 8, 128), (1, 1, 8, 2048), (64, 1, 64, 2048), (1, 9, 8, 2048),
          (128, 1, 128, 2048), (1, 1, 16, 2048), (32, 1, 8, 2048), (4, 2, 128, 100)]


TILE = 32  # list rows one split workgroup contracts per step


def _hpb(h):
    return 16 if h <= 16 else 32 if h <= 32 else 64


def _tiles(k, ns):
    return -(-(-(-k // ns)) // TILE)


@pytest.mark.parametrize("cus", [80, 188, 256, 304])
@pytest.mark.parametrize("shape", SHAPES)
def test_planner_bounds(smla, cus, shape):
    b, lq, h, k = shape
    ns = smla.smla_plan_nsplit_cus(cus, b, lq, h, k)
    assert ns == smla.smla_plan_nsplit_cus(cus, b, lq, h, k)  # deterministic
    assert 1 <= ns <= smla.MAX_NSPLIT
    per = -(-k // ns)
    assert ns == 1 or per >= TILE                # a split holds at least one tile
    assert -(-k // per) == ns                    # no trailing empty split
    units = b * lq * -(-h // _hpb(h))            # workgroups per split
    slots = cus                                  # one workgroup per CU
    assert ns == 1 or units * ns <= slots        # one wave of workgroups
    # no NSPLIT that still fits in one wave needs fewer tiles per split ...
    best = max(1, min(slots // units, k // TILE))
    assert _tiles(k, ns) == _tiles(k, best)
    # ... and none below ns keeps the same tile count
    assert ns == 1 or _tiles(k, ns - 1) > _tiles(k, ns)


def test_planner_fills_small_batches(smla):
    # batch 1, one head group: one 32-row tile per split
    assert smla.smla_plan_nsplit_cus(256, 1, 1, 8, 2048) == 64
    # 9 query tokens: 28 splits would fit, but 3 tiles each already needs only 22
    assert smla.smla_plan_nsplit_cus(256, 1, 9, 8, 2048) == 22
    # batch 64 x 64 heads: 64 workgroups per split, 4 splits fill 256 slots
    assert smla.smla_plan_nsplit_cus(256, 64, 1, 64, 2048) == 4
    # batch 128 x 128 heads: 256 workgroups per split already fill the device
    assert smla.smla_plan_nsplit_cus(256, 128, 1, 128, 2048) == 1
    # topk below one tile: no split
    assert smla.smla_plan_nsplit_cus(256, 1, 1, 8, 31) == 1
    # NSPLIT never grows with the batch
    prev = 10 ** 9
    for b in (1, 2, 4, 8, 16, 32, 64, 128):
        ns = smla.smla_plan_nsplit_cus(256, b, 1, 64, 2048)
        assert ns <= prev
        prev = ns


def test_planner_degenerate(smla):
    assert smla.smla_plan_nsplit_cus(256, 1, 1, 8, 0) == 1
    assert smla.smla_plan_nsplit_cus(256, 0, 1, 8, 2048) == 1
    assert smla.smla_plan_nsplit_cus(256, 1, 1, 8, 1) == 1
    for bad in [(0, 1, 1, 8, 2048), (256, -1, 1, 8, 2048), (256, 1, 1, 0, 2048),
                (256, 1, 1, 8, -1), (256, 1, 1, 5000, 2048)]:
        assert smla.lib.smla_plan_nsplit_cus(*bad) == -2, bad


# ------------------------------------------------------------------ workspace

@pytest.mark.parametrize("b,lq,h,s", [(1, 1, 8, 1), (1, 1, 8, 128), (64, 1, 64, 4), (1, 9, 8, 57),
                                      (3, 2, 5, 7)])
def test_workspace_layout(smla, b, lq, h, s):
    t = b * lq
    o_bytes = t * s * h * 512 * 4
    off = -(-o_bytes // 256) * 256  # part_o at 0, then part_lse at a 256-byte boundary
    assert smla.smla_workspace_lse_offset(b, lq, h, s) == off
    want = 0 if s <= 1 else off + t * s * h * 4
    assert smla.smla_workspace_bytes(b, lq, h, s) == want


def test_single_launch_query(smla):
    """When smla_decode_fused merges inside the split launch; the answers that
    need no device (NSPLIT 1 has no merge, NSPLIT above 64 exceeds the claim
    mask) and the argument errors."""
    q = smla.lib.smla_fused_in_launch
    assert q(1, 1, 8, 1) == 0
    assert q(1, 1, 8, 65) == 0 and q(4, 1, 128, 1024) == 0
    assert q(1, 1, 0, 4) == -2 and q(-1, 1, 8, 4) == -2 and q(1, 1, 4097, 4) == -2
    assert q(1, 1, 8, 0) == -3 and q(1, 1, 8, 1025) == -3


# ----------------------------------------------------------- argument errors

def _call(smla, fn="smla_decode", **kw):
    a = dict(q=0x10000, kv=0x20000, idx=0x30000, out=0x40000, lse=0x50000, scale=0.1,
             nsplit=1, batch=1, q_len=1, heads=8, topk=128, kv_rows=1024, ws=0, ws_bytes=0,
             sync=0x80000, sync_bytes=16384, polls=2048, stream=0)
    a.update(kw)
    f = getattr(smla.lib, fn)
    vp = ctypes.c_void_p
    args = [vp(a["q"]), vp(a["kv"]), vp(a["idx"]), vp(a["out"]), vp(a["lse"]), a["scale"],
            a["nsplit"], a["batch"], a["q_len"], a["heads"], a["topk"], a["kv_rows"],
            vp(a["ws"]), a["ws_bytes"]]
    if fn == "smla_decode_fused":
        args += [vp(a["sync"]), a["sync_bytes"], a["polls"]]
    return f(*args, vp(a["stream"]))


@pytest.mark.parametrize("fn", ["smla_decode", "smla_decode_fused", "smla_split"])
def test_invalid_arguments_rejected_before_launch(smla, fn):
    # pointers are fake: each call must fail validation and touch nothing
    assert _call(smla, fn, q=0) == -1
    assert _call(smla, fn, kv=0) == -1
    assert _call(smla, fn, idx=0) == -1
    assert _call(smla, fn, batch=-1) == -2
    assert _call(smla, fn, heads=0) == -2
    assert _call(smla, fn, heads=4097) == -2  # one above SMLA_MAX_HEADS
    assert _call(smla, fn, topk=-3) == -2
    assert _call(smla, fn, kv_rows=-1) == -2
    assert _call(smla, fn, nsplit=-1) == -3
    assert _call(smla, fn, nsplit=1025) == -3
    assert _call(smla, fn, q=0x10008) == -5
    assert _call(smla, fn, kv=0x20004) == -5
    assert _call(smla, fn, idx=0x30002) == -5
    # a split call needs a workspace of smla_workspace_bytes
    need = smla.smla_workspace_bytes(1, 1, 8, 4)
    assert _call(smla, fn, nsplit=4) == -4
    assert _call(smla, fn, nsplit=4, ws=0x60000, ws_bytes=need - 1) == -4
    assert _call(smla, fn, nsplit=4, ws=0x60008, ws_bytes=need) == -5


def test_fused_arguments(smla):
    # a negative poll bound is rejected whatever the shape
    assert _call(smla, "smla_decode_fused", polls=-1) == -2
    assert _call(smla, "smla_decode_fused", polls=-1, nsplit=4) == -2
    # NSPLIT 4 at one token x 8 heads merges in the launch: without a device the
    # question cannot be answered (SMLA_ERR_DEVICE); with one, the sync words
    # are checked (NULL, too small, misaligned) -- nothing is launched either way
    ws = dict(nsplit=4, ws=0x60000, ws_bytes=1 << 24)
    assert _call(smla, "smla_decode_fused", sync=0, **ws) in (-6, -1)
    assert _call(smla, "smla_decode_fused", sync_bytes=16383, **ws) in (-6, -4)
    assert _call(smla, "smla_decode_fused", sync=0x80002, **ws) in (-6, -5)


def test_noalloc_arguments(smla):
    """smla_decode_noalloc: errors before any launch and before the scratch
    array is looked up (fake pointers; nothing may be launched)."""
    f = smla.lib.smla_decode_noalloc
    vp = ctypes.c_void_p
    ok = (vp(0x10000), vp(0x20000), vp(0x30000), vp(0x40000), vp(0x50000), 0.1)
    assert f(*ok, -1, 1, 1, 8, 128, 1024, None) == -3
    assert f(*ok, 1025, 1, 1, 8, 128, 1024, None) == -3
    # partials above SMLA_NOALLOC_SCRATCH_BYTES (64 MiB): 64 tokens x 128 heads x 64 splits
    assert smla.smla_workspace_bytes(64, 1, 128, 64) > smla.NOALLOC_SCRATCH_BYTES
    assert f(*ok, 64, 64, 1, 128, 2048, 1024, None) == -4
    # NSPLIT 1 needs no scratch: plain argument errors come from the decode checks
    assert f(vp(0), *ok[1:], 1, 1, 1, 8, 128, 1024, None) == -1
    assert f(*ok, 1, 1, 1, 0, 128, 1024, None) == -2


def test_decode_needs_outputs(smla):
    assert _call(smla, "smla_decode", out=0) == -1
    assert _call(smla, "smla_decode", lse=0) == -1
    assert _call(smla, "smla_decode", out=0x40008) == -5
    # the split kernel with partials writes no final output: NULL out is fine
    # as far as validation goes (here it then fails on the missing workspace)
    assert _call(smla, "smla_split", out=0, lse=0, nsplit=4) == -4


def test_empty_batch_is_a_no_op(smla):
    # zero tokens: success with every pointer NULL and nothing launched
    assert _call(smla, "smla_decode", q=0, kv=0, idx=0, out=0, lse=0, batch=0) == 0
    assert _call(smla, "smla_decode", q=0, kv=0, idx=0, out=0, lse=0, q_len=0, nsplit=0) == 0


def test_combine_arguments(smla):
    f = smla.lib.smla_combine
    vp = ctypes.c_void_p
    ok = (vp(0x10000), vp(0x20000), vp(0x30000), vp(0x40000))
    assert f(vp(0), *ok[1:], 1, 8, 4, vp(0)) == -1
    assert f(*ok, 1, 0, 4, vp(0)) == -2
    assert f(*ok, -1, 8, 4, vp(0)) == -2
    assert f(*ok, 1, 8, 0, vp(0)) == -3
    assert f(*ok, 1, 8, 1025, vp(0)) == -3
    assert f(vp(0x10004), *ok[1:], 1, 8, 4, vp(0)) == -5
    assert f(*ok, 0, 8, 4, vp(0)) == 0


def _paged(smla, **kw):
    a = dict(q=0x10000, kv=0x20000, table=0x70000, max_pages=16, page=64, pos=0x30000, out=0x40000,
             lse=0x50000, scale=0.1, nsplit=1, batch=1, q_len=1, heads=8, topk=128, kv_rows=1024,
             ws=0, ws_bytes=0, stream=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return smla.lib.smla_decode_paged(vp(a["q"]), vp(a["kv"]), vp(a["table"]), a["max_pages"],
                                      a["page"], vp(a["pos"]), vp(a["out"]), vp(a["lse"]), a["scale"],
                                      a["nsplit"], a["batch"], a["q_len"], a["heads"], a["topk"],
                                      a["kv_rows"], vp(a["ws"]), a["ws_bytes"], vp(a["stream"]))


def _dense(smla, **kw):
    a = dict(q=0x10000, kv=0x20000, table=0, max_pages=0, page=1, ctx=0x30000, max_ctx=4096,
             out=0x40000, lse=0x50000, scale=0.1, nsplit=1, batch=1, q_len=9, heads=8,
             kv_rows=4096, ws=0, ws_bytes=0, stream=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return smla.lib.smla_decode_dense(vp(a["q"]), vp(a["kv"]), vp(a["table"]), a["max_pages"],
                                      a["page"], vp(a["ctx"]), a["max_ctx"], vp(a["out"]),
                                      vp(a["lse"]), a["scale"], a["nsplit"], a["batch"], a["q_len"],
                                      a["heads"], a["kv_rows"], vp(a["ws"]), a["ws_bytes"],
                                      vp(a["stream"]))


def test_paged_arguments(smla):
    # fake pointers: every call must fail validation and launch nothing
    assert _paged(smla, table=0) == -1          # the page table is required
    assert _paged(smla, pos=0) == -1
    assert _paged(smla, page=0) == -2
    assert _paged(smla, max_pages=-1) == -2
    assert _paged(smla, table=0x70002) == -5
    assert _paged(smla, pos=0x30002) == -5
    assert _paged(smla, nsplit=2000) == -3
    assert _paged(smla, nsplit=4) == -4          # no workspace
    assert _paged(smla, q=0, kv=0, pos=0, table=0, out=0, lse=0, batch=0) == 0


def test_dense_arguments(smla):
    assert _dense(smla, ctx=0) == -1            # context lengths are required
    assert _dense(smla, q=0) == -1
    assert _dense(smla, ctx=0x30002) == -5
    assert _dense(smla, max_ctx=-1) == -2
    assert _dense(smla, table=0x70000, max_pages=4, page=0) == -2
    assert _dense(smla, table=0x70000, max_pages=-4, page=64) == -2
    assert _dense(smla, nsplit=4) == -4
    # a flat cache needs no table; zero tokens launch nothing
    assert _dense(smla, q=0, kv=0, ctx=0, out=0, lse=0, batch=0) == 0


def test_planner_path_without_device(smla):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    # nsplit == 0 consults the device's CU count: no device -> SMLA_ERR_DEVICE
    assert _call(smla, "smla_decode", nsplit=0) == -6
    assert smla.lib.smla_plan_nsplit(1, 1, 8, 2048) == -6
    assert smla.lib.smla_fused_in_launch(1, 1, 8, 4) == -6
    # a valid fused call with NSPLIT > 1 asks the device whether to merge in-launch
    assert _call(smla, "smla_decode_fused", nsplit=4, ws=0x60000, ws_bytes=1 << 24) == -6
    # AUTO and CHUNKS with a workspace ask for the CU count (the sub-chunks per
    # chunk depend on it)
    f = smla.lib.smla_topk
    vp = ctypes.c_void_p
    assert f(vp(0x10000), None, 1, 1, 65536, 8, vp(0x30000), vp(0x40000), 1 << 30, 0, None) == -6
    assert f(vp(0x10000), None, 1, 1, 65536, 8, vp(0x30000), vp(0x40000), 1 << 30, 2, None) == -6


def test_topk_arguments(smla):
    """smla_topk validates before launching; empty calls launch nothing."""
    f = smla.lib.smla_topk
    vp = ctypes.c_void_p
    sc, ctx, out = vp(0x10000), vp(0x20000), vp(0x30000)
    assert f(sc, ctx, -1, 1, 100, 8, out, None, 0, 0, None) == -2
    assert f(sc, ctx, 1, -1, 100, 8, out, None, 0, 0, None) == -2
    assert f(sc, ctx, 1, 1, -5, 8, out, None, 0, 0, None) == -2
    assert f(sc, ctx, 1, 1, 100, -1, out, None, 0, 0, None) == -2
    assert f(sc, ctx, 1, 1, 100, (1 << 24) + 1, out, None, 0, 0, None) == -2
    assert f(sc, ctx, 1, 1, 100, 8, out, None, 0, 4, None) == -2   # unknown form
    assert f(sc, ctx, 1, 1, 100, 8, out, None, 0, -1, None) == -2
    assert f(sc, ctx, 1, 1, 100, 8, None, None, 0, 0, None) == -1
    assert f(None, ctx, 1, 1, 100, 8, out, None, 0, 0, None) == -1
    assert f(vp(0x10002), ctx, 1, 1, 100, 8, out, None, 0, 0, None) == -5
    assert f(sc, ctx, 1, 1, 100, 8, vp(0x30001), None, 0, 0, None) == -5
    assert f(sc, ctx, 1, 1, 100, 8, out, vp(0x40010), 1 << 20, 0, None) == -5  # workspace 256-aligned
    assert f(sc, ctx, 0, 1, 100, 8, out, None, 0, 0, None) == 0   # no rows
    assert f(sc, ctx, 1, 1, 100, 0, out, None, 0, 0, None) == 0   # topk 0


def test_topk_workspace_size(smla):
    """Per row: the candidate list (8192 x 8 B), 2048 bins per 4096-position
    chunk, chunk offsets and 4 words, rounded up to 256 B."""
    f = smla.lib.smla_topk_workspace_bytes
    for m in (0, 1, 4096, 4097, 65536, 131072):
        ch = -(-m // 4096)
        row = 8192 * 8 + (ch * 2048 + ch + 1 + 4) * 4
        assert f(3, 2, m) == 6 * (-(-row // 256) * 256), m
    assert f(-1, 1, 10) == 0

