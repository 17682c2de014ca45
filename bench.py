#!/usr/bin/env python3
"""Benchmark of sparse MLA decode (split-K over the top-k list) on one MI355X.

One step = one smla_decode call (split kernel + LSE-combine kernel when
NSPLIT > 1) over the workload's whole batch, i.e. one attention layer's
decode.  Default workload: the large ragged batch -- batch 128, q_len 1, 128
heads, top-2048 per sequence over contexts uniform in [2048, 131072] in a
paged pool of 64-token pages (the positions translated to rows by the
harness) -- with the planner's NSPLIT.

Timing protocol
  * inputs are resident in HBM before timing; successive steps rotate over
    (cache, index set) pairs whose distinct gathered rows exceed 512 MB (2x
    the Infinity Cache), so every step gathers rows from HBM (--warm turns the
    rotation off: a cache-resident figure, never an HBM one).  A workload
    whose rotation would need more than MAX_ROTATION steps (the tiny one: its
    whole 1.2 MB cache sits in one XCD's L2) is not rotated and is labelled
    warm;
  * steps/s: W warm-up steps, then untimed replays of the timed graph for at
    least --settle seconds (the GPU's clocks ramp up under load over tens of
    milliseconds), then exactly K steps -- HIP graphs of consecutive steps of
    the rotation, at most GRAPH_MAX steps each, replayed back to back --
    bracketed by device synchronisation;
  * per-kernel durations: an eager loop with HIP events recorded around each
    launch on the launch stream, queued behind a spin kernel so that host
    enqueue time cannot leak into the measured intervals;
  * roofline: gathered-KV bytes of one split launch (valid list entries x
    1152 B) / the split kernel's mean duration, against 8 TB/s HBM3E;
  * single_launch: the same step through smla_decode_fused, the merge inside
    the split launch (list workloads, when the shape allows it; skipped with
    --no-sweep, so that a profiled run holds only the two-launch kernels);
  * topk: the top-k producer (smla_topk) on synthetic N(0,1) index scores of
    the workload's shape (every context position of every query token),
    graph-timed, with the score bytes it must read per call against the
    HBM roofline (skipped with --no-sweep);
  * cpu_baseline: the fp64 oracle, as is, on the host cores, over a bounded
    sample of the same workload, scaled to steps/s (and on one core);
  * dispatch_floor_us: a graph of back-to-back empty kernel launches, the
    per-launch floor under every step (two launches per step);
  * nsplit_sweep: steps/s and the split kernel's gathered-KV rate of the same
    workload at each NSPLIT of its sweep (the planner's marked);
  * secondary: the same figures (steps/s, per-step and split-kernel gathered
    KV rate and roofline fraction) for every other workload at the planner's
    NSPLIT, and for the paged workloads with the page tables mapped in the
    kernel (skipped with --no-secondary or --no-sweep).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/s + gathered-KV HBM GB/s (% of roofline), sparse MLA topk=2048"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 1152
MIN_GRAPH_STEPS = 32  # steps per captured graph of the kernel timings, at least
GRAPH_MAX = 1024      # steps per captured graph of the headline timing, at most
MAX_ROTATION = 256    # rotation steps, at most (more: the workload runs warm)
KERNEL_SRC = os.path.join(ROOT, "sparse_mla_decode_amd", "csrc", "smla_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

DESCRIPTIONS = {
    "tiny": "batch 1, q_len 1, 8 heads, top-128 of a 1024-row cache",
    "long": "batch 1, q_len 1, 8 heads, top-2048 of a 65536-row cache (single request, long context)",
    "batched": "batch 64, q_len 1, 64 heads, top-2048 per sequence, 32768-token contexts in a paged pool of 32768 x 64-token pages",
    "spec": "batch 1, q_len 9 (9 verify tokens with their own lists), 8 heads, top-2048 of a {ctx}-row cache",
    "ragged": "batch 128, q_len 1, 128 heads, top-2048 per sequence, contexts uniform in [2048, 131072], paged 64-token pages",
    "verify": "dense verify: batch 1, q_len 9, 8 heads, every row of a {ctx}-row cache (no list)",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="ragged",
                    choices=["tiny", "long", "batched", "spec", "ragged", "verify"])
    ap.add_argument("--mode", default="rows", choices=["rows", "paged"],
                    help="paged: positions + page tables mapped in the kernel (batched, ragged)")
    ap.add_argument("--spec-ctx", type=int, default=65536)
    ap.add_argument("--nsplit", type=int, default=0, help="0 = the planner's choice")
    ap.add_argument("--warm", action="store_true", help="no input rotation (cache-resident figure)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--kernel-steps", type=int, default=512, help="launches per per-kernel timing")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed graph replays before the timed steps")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the NSPLIT sweep, the single-launch and top-k figures and the secondary workloads")
    ap.add_argument("--no-secondary", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--topk-only", action="store_true",
                    help="only time the top-k producer on the workload's shape (one JSON line) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain 1 GiB device-to-device copy (larger than the Infinity Cache),
    launched three times: the reference dispatch for scaling the HBM byte
    counters (it reads and writes exactly 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


SWEEPS = {"tiny": [1, 4], "long": [1, 16, 64, 128], "spec": [16, 64], "batched": [1, 2, 4, 8, 16],
          "ragged": [1, 2, 4], "verify": [16, 64]}


class Workload:
    """Device-resident inputs of one workload plus its rotation of
    (cache, index set) pairs, and the timing helpers over them."""

    def __init__(self, name, spec_ctx, warm, dev, mode="rows"):
        import numpy as np
        import torch

        import sparse_mla_decode_amd as smla
        import workloads as wl

        self.smla, self.torch, self.name, self.dev = smla, torch, name, dev
        inp = wl.workload(name, spec_ctx=spec_ctx, with_kv=False)
        self.inp = inp
        self.B, self.Lq, self.H, self.K = inp.batch, inp.q_len, inp.heads, inp.topk
        self.T = self.B * self.Lq
        self.kind = "dense" if inp.dense else mode
        if self.kind == "paged" and inp.pos is None:
            raise SystemExit(f"--mode paged needs a paged workload (batched, ragged), not {name}")
        self.pos_sets = None
        self.warm = warm
        if not warm:
            if self.kind == "dense":
                # no list to vary: rotate over caches whose rows together exceed 512 MB
                self.sets = [inp.idx]
                self.n_caches = max(1, -(-(512 << 20) // (inp.kv_rows * ROW_BYTES)))
            elif self.kind == "paged":
                self.n_caches, self.sets, self.pos_sets = wl.rotation(inp, positions=True)
            else:
                self.n_caches, self.sets = wl.rotation(inp)
            # a rotation longer than MAX_ROTATION steps (a cache this small
            # cannot be made cold in any useful sense) is not used
            self.warm = self.n_caches * len(self.sets) > MAX_ROTATION
        if self.warm:
            self.n_caches, self.sets = 1, [inp.idx]
            self.pos_sets = [inp.pos] if self.kind == "paged" else None
        self.q = wl.bits_to_torch(inp.q).to(dev)
        self.caches = [wl.device_pool(inp.kv_rows, (inp.pool_seed or 0) + 1000 * c, dev)
                       for c in range(self.n_caches)]
        self.idx_sets = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in self.sets]
        if self.kind == "paged":
            self.pos_dev = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in self.pos_sets]
            self.table = torch.from_numpy(wl.block_table(inp)).to(dev)
        if self.kind == "dense":
            self.ctx_len = torch.tensor(inp.ctx, dtype=torch.int32, device=dev)
            self.max_ctx = int(inp.ctx.max())
        self.out = torch.empty((self.B, self.Lq, self.H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.B, self.Lq, self.H), dtype=torch.float32, device=dev)
        self.n_rot = self.n_caches * len(self.sets)
        # steps per captured graph: whole rotation cycles, at least MIN_GRAPH_STEPS
        # (a graph of one step, as without rotation, would time the graph launch)
        self.graph_len = self.n_rot * max(1, -(-MIN_GRAPH_STEPS // self.n_rot))
        self.valid_rows = [int((x >= 0).sum()) for x in self.sets]  # every set points inside its cache
        if self.kind == "dense":
            # every query token of a sequence attends to the same context rows:
            # count each context row once (per query token it would exceed HBM)
            self.valid_rows = [int(np.minimum(inp.ctx, inp.idx.shape[-1]).sum())]
        self.mean_kv_bytes = self.kv_bytes(0, self.n_rot)
        self.stream = torch.cuda.Stream()
        self.ws = {}
        torch.cuda.synchronize()

    def kv_bytes(self, first, n):
        """Mean gathered-KV bytes per step over steps first .. first + n - 1."""
        return sum(self.valid_rows[(i // self.n_caches) % len(self.sets)] * ROW_BYTES
                   for i in range(first, first + n)) / n

    def flops(self):
        """Algorithmic flops of one step: tokens x heads x valid entries x 2 x (576 + 512)."""
        valid = self.valid_rows[0] if self.kind != "dense" else self.valid_rows[0] * self.Lq
        return self.H * valid * 2 * (576 + 512)

    def plan(self):
        if self.kind == "dense":
            return self.smla.smla_plan_nsplit_dense(self.B, self.Lq, self.H, self.K)
        return self.smla.smla_plan_nsplit(self.B, self.Lq, self.H, self.K)

    def workspace(self, nsplit):
        if nsplit not in self.ws:
            self.ws[nsplit] = self.smla.workspace(self.B, self.Lq, self.H, nsplit, self.dev)
        return self.ws[nsplit]

    def _args(self, i):
        return self.caches[i % self.n_caches], self.idx_sets[(i // self.n_caches) % len(self.sets)]

    def step_fn(self, nsplit):
        ws = self.workspace(nsplit)
        scale = self.inp.scale

        def rows(i, stream=None):
            c, ix = self._args(i)
            self.smla.smla_decode(self.q, c, ix, self.out, self.lse, scale, nsplit, ws, stream)

        def paged(i, stream=None):
            c = self.caches[i % self.n_caches]
            pos = self.pos_dev[(i // self.n_caches) % len(self.sets)]
            self.smla.smla_decode_paged(self.q, c, self.table, 64, pos, self.out, self.lse, scale,
                                        nsplit, ws, stream)

        def dense(i, stream=None):
            c = self.caches[i % self.n_caches]
            self.smla.smla_decode_dense(self.q, c, self.ctx_len, self.max_ctx, self.out, self.lse,
                                        scale, nsplit, workspace_t=ws, stream=stream)
        return {"rows": rows, "paged": paged, "dense": dense}[self.kind]

    def fused_in_launch(self, nsplit):
        return (self.kind == "rows" and nsplit > 1
                and self.smla.smla_fused_in_launch(self.B, self.Lq, self.H, nsplit))

    def fused_fn(self, nsplit):
        ws = self.workspace(nsplit)
        # one set of synchronisation words per workload, alive as long as the
        # graphs that use it (every call leaves it zero)
        if getattr(self, "sync", None) is None:
            self.sync = self.smla.fused_sync(self.dev)
        sync = self.sync

        def f(i):
            c, ix = self._args(i)
            self.smla.smla_decode_fused(self.q, c, ix, self.out, self.lse, self.inp.scale, nsplit, ws,
                                        sync=sync)
        return f

    def split_fn(self, nsplit):
        ws = self.workspace(nsplit)

        def f(i):
            c, ix = self._args(i)
            self.smla.smla_split(self.q, c, ix, self.out, self.lse, self.inp.scale, nsplit, ws)
        return f

    def combine_fn(self, nsplit):
        part = self.smla.partials_view(self.workspace(nsplit), self.B, self.Lq, self.H, nsplit)

        def f(i):
            self.smla.smla_combine(part[0], part[1], self.out, self.lse)
        return f

    def graph_of(self, fn, n=None, first=0):
        """n calls fn(first), fn(first + 1), ... captured in a HIP graph (by
        default graph_len calls: whole rotation cycles)."""
        torch = self.torch
        n = self.graph_len if n is None else n
        torch.cuda.synchronize()
        self.stream.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(first, first + n):
                    fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    def time_exact(self, fn, steps, settle):
        """Microseconds per step over exactly `steps` consecutive steps of the
        rotation: graphs of at most GRAPH_MAX steps replayed back to back
        between two events (after `settle` seconds of untimed replays)."""
        torch = self.torch
        graphs, first = [], 0
        while first < steps:
            n = min(GRAPH_MAX, steps - first)
            graphs.append(self.graph_of(fn, n, first))
            first += n
        t0 = time.time()
        while time.time() - t0 < settle:
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for g in graphs:
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / steps

    def time_graph(self, g, min_launches):
        """Mean microseconds per captured call over whole-cycle replays."""
        torch = self.torch
        reps = max(1, -(-min_launches // self.graph_len))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / (reps * self.graph_len), reps * self.graph_len

    def split_time(self, nsplit, kernel_steps, step_us):
        """The split kernel's time per launch: a graph of split-only launches
        (lists of rows), or for the paged and dense entry points, which have
        no split-only call, the step minus a graph of combine-only launches."""
        if self.kind == "rows":
            return self.time_graph(self.graph_of(self.split_fn(nsplit)), kernel_steps)[0]
        comb = self.time_graph(self.graph_of(self.combine_fn(nsplit)), kernel_steps)[0] if nsplit > 1 else 0.0
        return step_us - comb

    def settle(self, g, seconds):
        """Untimed replays of graph g for `seconds` (clocks ramp up under load)."""
        self.settle_graph(g, seconds, max(1, 64 // self.graph_len))

    def settle_graph(self, g, seconds, per_sync=1):
        t0 = time.time()
        while time.time() - t0 < seconds:
            for _ in range(per_sync):
                g.replay()
            self.torch.cuda.synchronize()

    def summary(self, nsplit, steps, kernel_steps, settle=0.1):
        """Steps/s and the split kernel's time and gathered-KV rate at nsplit."""
        g = self.graph_of(self.step_fn(nsplit))
        self.settle(g, settle)
        step_us, n = self.time_graph(g, steps)
        split_us = self.split_time(nsplit, kernel_steps, step_us)
        kv = self.mean_kv_bytes
        return {"nsplit": nsplit, "us_per_step": round(step_us, 3), "steps_per_s": round(1e6 / step_us, 2),
                "mfma_frac_split": round(self.flops() / (split_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "gathered_kv_gbps_per_step": round(kv / (step_us * 1e-6) / 1e9, 2),
                "roofline_frac_per_step": round(kv / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "split_us": round(split_us, 3),
                "split_kv_gbps": round(kv / (split_us * 1e-6) / 1e9, 2),
                "split_roofline_frac": round(kv / (split_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "kv_bytes_per_step": int(kv), "steps_timed": n,
                "cache_state": self.cache_state()}

    def cache_state(self):
        if self.warm:
            return "warm: one input set, no rotation (cache-resident)"
        return f"cold: rotation over {self.n_caches} caches x {len(self.sets)} disjoint index sets"


def topk_figure(w, steps):
    """smla_topk over index scores shaped like the workload: one row per
    query token over its whole context; rotation over score sets whose bytes
    exceed 512 MB when a set is smaller (cold reads)."""
    import numpy as np
    import torch

    import workloads as wl
    inp = w.inp
    max_ctx = int(inp.ctx.max()) if inp.ctx is not None else inp.kv_rows
    k = inp.topk
    set_bytes = w.B * w.Lq * max_ctx * 4
    n_sets = max(1, min(64, -(-(512 << 20) // set_bytes)))
    sets = [torch.from_numpy(wl.index_scores(9000 + i, w.B, w.Lq, max_ctx)).to(w.dev) for i in range(n_sets)]
    ctx = torch.tensor(inp.ctx, dtype=torch.int32, device=w.dev) if inp.ctx is not None else None
    out = torch.empty((w.B, w.Lq, k), dtype=torch.int32, device=w.dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    w.stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(w.stream):
        with torch.cuda.graph(g, stream=w.stream):
            for i in range(n_sets):
                w.smla.smla_topk(sets[i], k, out, ctx)
    torch.cuda.synchronize()
    w.settle_graph(g, 0.1)
    reps = max(1, -(-steps // n_sets))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / (reps * n_sets)
    valid = int(np.sum(np.minimum(inp.ctx, max_ctx))) * w.Lq if inp.ctx is not None else w.B * w.Lq * max_ctx
    read = valid * 4 + w.B * w.Lq * k * 4
    return {"us_per_call": round(us, 3), "rows": w.B * w.Lq, "positions_per_row": max_ctx, "topk": k,
            "bytes_per_call": read, "gbps": round(read / (us * 1e-6) / 1e9, 2),
            "roofline_frac": round(read / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "cache_state": f"rotation over {n_sets} score sets",
            "bytes": "valid scores x 4 B read + topk x 4 B written per row",
            "entry_point": "smla_topk"}


def split_kernel_name(w, nsplit):
    """The split kernel the library launches for this shape: blocks of more
    than 32 heads over slices of at least four 32-row tiles take the
    role-specialised 64-head kernel."""
    heads = w.H * (w.Lq if w.kind == "dense" and w.K >= 8192 else 1)  # dense verify folds tokens into heads
    per_split = -(-w.K // nsplit)
    return "split64_kernel" if heads > 32 and -(-per_split // 32) >= 4 else "split_kernel"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.time()
    w = Workload(args.workload, args.spec_ctx, args.warm, dev, args.mode)
    B, Lq, H, K, T = w.B, w.Lq, w.H, w.K, w.T
    log(f"[bench] workload={args.workload} B={B} Lq={Lq} H={H} K={K} kv_rows={w.inp.kv_rows} "
        f"caches={w.n_caches} index_sets={len(w.sets)}")
    if args.topk_only:
        tk = topk_figure(w, args.steps)
        print(json.dumps({"workload": args.workload, "topk_producer": tk}), flush=True)
        return
    nsplit = args.nsplit if args.nsplit > 0 else w.plan()
    rows_mode = w.kind == "rows"
    step = w.step_fn(nsplit)
    log(f"[bench] setup {time.time() - t_setup:.1f}s nsplit={nsplit} rotation={w.n_rot} steps")

    # ---- warm-up (eager), then the timed region: exactly K consecutive steps
    # of the rotation, replayed from HIP graphs
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = args.steps
    us_per_step = w.time_exact(step, steps, args.settle)
    ms_per_step = us_per_step * 1e-3
    steps_per_s = 1e6 / us_per_step
    log(f"[bench] timed: {steps} steps -> {us_per_step:.2f} us/step")
    # the same steps as whole rotation cycles of a graph of at least
    # MIN_GRAPH_STEPS steps, over many more launches (a steadier figure)
    long_us, long_n = w.time_graph(w.graph_of(step), max(args.kernel_steps, 256))
    log(f"[bench] whole-cycle graph replays: {long_n} steps -> {long_us:.2f} us/step")

    # ---- per-kernel durations (a): each kernel alone, one rotation cycle of
    # back-to-back launches per HIP graph, timed with events around replays
    combine_only = w.combine_fn(nsplit) if nsplit > 1 else None
    comb_us = w.time_graph(w.graph_of(combine_only), args.kernel_steps)[0] if nsplit > 1 else 0.0
    split_us = w.split_time(nsplit, args.kernel_steps, us_per_step)
    split_only = w.split_fn(nsplit) if rows_mode else step
    single_launch = None
    topk = None
    if not args.no_sweep and w.kind != "dense":
        topk = topk_figure(w, min(args.steps, 512))
        log(f"[bench] topk producer: {topk['us_per_call']:.2f} us per call ({topk['rows']} rows x "
            f"{topk['positions_per_row']} positions, k={topk['topk']}, {topk['gbps']:.0f} GB/s of scores)")
    if not args.no_sweep and w.fused_in_launch(nsplit):
        gf = w.graph_of(w.fused_fn(nsplit))
        w.settle(gf, 0.1)  # as the two-launch figures: clocks settled first
        fused_us = w.time_graph(gf, max(args.steps, 256))[0]
        single_launch = {"us_per_step": round(fused_us, 3), "steps_per_s": round(1e6 / fused_us, 2),
                         "entry_point": "smla_decode_fused",
                         "method": "graph replay of smla_decode_fused steps (one kernel per step)"}
        log(f"[bench] single launch (smla_decode_fused): {fused_us:.2f} us/step")

    # ---- per-kernel durations (b), diagnostic: events bracketing each eager
    # launch, queued behind a spin kernel so host enqueue time cannot leak in
    ks = min(args.kernel_steps, 4 * w.n_rot)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ks)]
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    for i in range(ks):
        ev[i][0].record()
        split_only(i)
        ev[i][1].record()
        if nsplit > 1 and rows_mode:
            combine_only(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    ev_split_us = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ev_comb_us = 1e3 * float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) if nsplit > 1 else 0.0
    eager_us = 1e3 * (ev[0][0].elapsed_time(ev[-1][2])) / ks
    log(f"[bench] kernels (graph, per launch): split {split_us:.2f} us, combine {comb_us:.2f} us; "
        f"(event-bracketed: split {ev_split_us:.2f} us, combine {ev_comb_us:.2f} us, eager step {eager_us:.2f} us)")

    kv_split = w.mean_kv_bytes
    kv_timed = w.kv_bytes(0, steps)  # the K timed steps' mean
    flops = w.flops()
    achieved = kv_split / (split_us * 1e-6) / 1e9
    traffic = None
    mfma_counters = None  # the profile's MFMA counters, while it matches this kernel
    prof_avg_ns = None    # the profile's trace-average split duration, likewise
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(profile_key(args.workload, args.spec_ctx, w.kind))
        if rec and rec.get("kernel_sha") == kernel_sha() and rec.get("nsplit") == nsplit and not w.warm:
            traffic = rec.get("bytes_per_launch")
            mfma_counters = rec
            prof_avg_ns = rec.get("split_trace_avg_ns")

    # ---- NSPLIT sweep of the same workload (graph timing only)
    sweep = []
    if not args.no_sweep:
        for ns in SWEEPS[args.workload] + ([] if nsplit in SWEEPS[args.workload] else [nsplit]):
            sweep.append(dict(w.summary(ns, min(args.steps, 1024), min(args.kernel_steps, 512)),
                              planner=(ns == w.plan())))
            log(f"[bench] sweep nsplit={ns}: {sweep[-1]['us_per_step']:.2f} us/step, "
                f"split {sweep[-1]['split_us']:.2f} us")
    # ---- every other workload at the planner's NSPLIT (graph timing only)
    secondary = {}
    if not args.no_sweep and not args.no_secondary:
        for name, mode in secondary_list(args.workload, w.kind):
            t0 = time.time()
            w2 = Workload(name, args.spec_ctx, args.warm, dev, mode)
            ns2 = w2.plan()
            key = name + ("_paged" if mode == "paged" else "")
            desc = DESCRIPTIONS[name].format(ctx=args.spec_ctx) + \
                ("; positions mapped through page tables in the kernel" if mode == "paged" else "")
            secondary[key] = dict(w2.summary(ns2, 512, 256), planner=True, workload=f"{name}: {desc}",
                                  entry_point=ENTRY[w2.kind])
            if w2.fused_in_launch(ns2):
                gf = w2.graph_of(w2.fused_fn(ns2))
                w2.settle(gf, 0.1)
                fu = w2.time_graph(gf, 512)[0]
                secondary[key]["single_launch"] = {
                    "us_per_step": round(fu, 3), "steps_per_s": round(1e6 / fu, 2),
                    "entry_point": "smla_decode_fused",
                    "method": "graph replay of smla_decode_fused steps (one kernel per step)"}
            log(f"[bench] secondary {key} (planner nsplit={ns2}): {secondary[key]['us_per_step']:.2f} us/step, "
                f"split {secondary[key]['split_us']:.2f} us ({secondary[key]['split_roofline_frac']:.3f} of HBM), "
                f"{time.time() - t0:.1f} s")
            del w2
            torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: " + DESCRIPTIONS[args.workload].format(ctx=args.spec_ctx)
                        + ("; positions mapped through page tables in the kernel" if w.kind == "paged" else ""),
            "entry_point": ENTRY[w.kind],
            "batch": B, "q_len": Lq, "heads": H, "topk": K, "kv_rows": w.inp.kv_rows,
            "nsplit": nsplit, "nsplit_from": "planner" if args.nsplit == 0 else "argument",
            "cache_state": w.cache_state(),
            "timing": (f"exactly {steps} consecutive steps replayed from HIP graphs of at most {GRAPH_MAX} "
                       f"steps, after {args.settle:g} s of untimed replays"),
        },
        "gathered_kv_gbps_per_step": round(kv_timed / (ms_per_step * 1e-3) / 1e9, 2),
        "whole_cycle_timing": {"us_per_step": round(long_us, 3), "steps": long_n,
                               "method": f"graph of {w.graph_len} steps (whole rotation cycles) replayed"},
        "kernels_us": {"split": round(split_us, 3), "combine": round(comb_us, 3),
                       "method": ("graph of back-to-back launches of one kernel, events around replays"
                                  if rows_mode else
                                  "split = graph step minus a graph of combine-only launches"),
                       "event_bracketed_split": round(ev_split_us, 3),
                       "event_bracketed_combine": round(ev_comb_us, 3),
                       "eager_step": round(eager_us, 3)},
        "roofline": {
            "bound": "hbm",
            "kernel": split_kernel_name(w, nsplit) + " (gather + QK^T + online softmax + PV)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(kv_split),
            "launch_us": round(split_us, 3),
            "launch_timing": "mean per launch over graph replays of back-to-back split launches (HIP events "
                             "on the launch stream)",
            "frac_per_step": round(kv_timed / (us_per_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "frac_from_profile": (None if not prof_avg_ns else
                                  round(kv_split / (prof_avg_ns * 1e-9) / 1e9 / HBM_PEAK_GBPS, 4)),
            "profile_avg_us": None if not prof_avg_ns else round(prof_avg_ns * 1e-3, 3),
            "bytes": ("context rows x 1152 B, each row once (all query tokens share them)"
                      if w.kind == "dense" else "valid list entries x 1152 B"),
        },
        "mfma": {"achieved_tflops": round(flops / (split_us * 1e-6) / 1e12, 3),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(flops / (split_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                 "flops": "algorithmic: tokens x heads x valid entries x 2 x (576 + 512)",
                 "counters": None if not mfma_counters or "mfma_flops_per_launch" not in mfma_counters else {
                     "executed_flops_per_launch": mfma_counters["mfma_flops_per_launch"],
                     "executed_tflops": round(mfma_counters["mfma_flops_per_launch"]
                                              / (split_us * 1e-6) / 1e12, 3),
                     "busy_frac": round(mfma_counters["mfma_busy_simd_cycles"]
                                        / (1024 * split_us * 1e-6 * 2.4e9), 5),
                     "source": mfma_counters.get("source"),
                     "note": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (heads padded to 16-head groups, "
                             "entries to 32-row tiles, and the QK^T both K-split pairs of a 16-head "
                             "block compute, included) and SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs "
                             "x the live split time x 2.4 GHz"}},
        "kernel_sha": kernel_sha(),
    }
    result["dispatch_floor_us"] = round(dispatch_floor_us(), 3)
    if single_launch:
        result["single_launch"] = single_launch
    if topk:
        result["topk_producer"] = topk
    if sweep:
        result["nsplit_sweep"] = sweep
    if secondary:
        result["secondary"] = secondary
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w.inp, w.caches[0], torch.from_numpy(w.sets[0]), args.cpu_seconds)
    print(json.dumps(result), flush=True)


ENTRY = {"rows": "smla_decode", "paged": "smla_decode_paged", "dense": "smla_decode_dense"}


def profile_key(name, spec_ctx, kind):
    """Key of a workload's record in profiles/traffic.json."""
    return name + (str(spec_ctx) if name in ("spec", "verify") else "") + ("_paged" if kind == "paged" else "")


def secondary_list(head, head_kind):
    """(workload, mode) of every figure besides the headline one."""
    figs = [(n, "rows") for n in ("tiny", "long", "batched", "spec", "ragged", "verify")]
    figs += [("batched", "paged"), ("ragged", "paged")]
    head_mode = "paged" if head_kind == "paged" else "rows"
    return [f for f in figs if f != (head, head_mode)]


def dispatch_floor_us(n=256):
    """Microseconds per launch of an empty kernel, back to back in a graph."""
    import torch
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(n):
                torch.cuda._sleep(0)
    torch.cuda.synchronize()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (10 * n)


def cpu_baseline(inp, kv_dev, idx0, seconds):
    """The fp64 oracle, as is, on a bounded sample of the workload: whole
    sequences of the first index set, added until `seconds` of CPU work are
    spent, scaled to steps/s of the whole batch."""
    import dataclasses

    import numpy as np

    import oracle
    import workloads as wl

    inp0 = dataclasses.replace(inp, idx=idx0.numpy())
    T_seq = inp.batch
    done_seqs, elapsed = 0, 0.0
    threads = oracle.threads()
    used = 0
    b = 0
    while elapsed < seconds:
        q_s, kv_s, idx_s = wl.oracle_view(inp0, kv_dev, [b % T_seq])
        t0 = time.perf_counter()
        oracle.decode(q_s, kv_s, idx_s, inp.scale)
        elapsed += time.perf_counter() - t0
        used = max(used, min(threads, inp.q_len * inp.heads))
        done_seqs += 1
        b += 1
    steps_per_s = (done_seqs / T_seq) / elapsed
    # the same on one core, over a quarter of the time budget
    q_s, kv_s, idx_s = wl.oracle_view(inp0, kv_dev, [0])
    one, t1 = 0, 0.0
    while t1 < seconds / 4:
        t0 = time.perf_counter()
        oracle.decode(q_s, kv_s, idx_s, inp.scale, nthreads=1)
        t1 += time.perf_counter() - t0
        one += 1
    return {"value": round(steps_per_s, 4), "unit": "steps/s", "cores": used, "kind": "oracle",
            "sample": f"{done_seqs} sequence(s) x {inp.q_len} token(s) x {inp.heads} heads of the first "
                      f"index set in {elapsed:.1f} s of fp64 oracle work, scaled to the {T_seq}-sequence step",
            "host_threads_available": threads,
            "single_core": {"value": round((one / T_seq) / t1, 4), "unit": "steps/s", "cores": 1,
                            "sample": f"sequence 0 {one} times in {t1:.1f} s, scaled to the step"}}


if __name__ == "__main__":
    main()
