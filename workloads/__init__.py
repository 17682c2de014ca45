"""Seeded synthetic inputs for sparse MLA decode.

This module only draws inputs: query vectors, latent cache rows, top-k index
lists and page tables.  It holds none of the attention arithmetic, and both
the HIP path's tests and the CPU oracle's tests consume what it produces.

Value recipe: every q and cache element is bf16_rne(0.5 * N(0, 1)).  Index
lists are drawn uniformly without replacement from each query token's own
context and left in sampled (random) order.  Paged pools use 64-token pages
whose physical order is a random permutation; logical positions are turned
into physical rows (page * 64 + slot) here, before the library sees them.

Seeds: workload k uses base seed 1000 * k, with sub-streams +0 q, +1 cache,
+2 index lists, +3 page permutation, +4 context lengths.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D = 576          # q / cache row width in bf16 elements (512 latent + 64 rope)
ROW_BYTES = D * 2
DV = 512         # value width: the first 512 columns of a row
PAGE = 64        # tokens per page in the paged pools
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))

SUB_Q, SUB_KV, SUB_IDX, SUB_PAGES, SUB_CTX, SUB_SCORES = 0, 1, 2, 3, 4, 5


# ----------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 0.5) -> np.ndarray:
    """bf16 bits of std * N(0, 1) samples."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ----------------------------------------------------------------- workloads

@dataclasses.dataclass
class Inputs:
    """One decode call's inputs, host side.

    q:   [B, Lq, H, 576] uint16 (bf16 bits)
    kv:  [N, 576] uint16, or None when the pool is generated on the device
    idx: [B, Lq, K] int32 physical row indices (-1 = masked)
    kv_rows: N
    pool_seed: seed of the device-side pool when kv is None
    """
    name: str
    q: np.ndarray
    kv: Optional[np.ndarray]
    idx: np.ndarray
    kv_rows: int
    scale: float = SCALE
    pool_seed: Optional[int] = None
    ctx: Optional[np.ndarray] = None          # per-sequence context lengths
    page_table: Optional[list] = None         # per-sequence physical page ids
    pos: Optional[np.ndarray] = None          # [B, Lq, K] positions behind idx (paged, dense)
    dense: bool = False                       # the list is every position of the context

    @property
    def batch(self): return self.q.shape[0]

    @property
    def q_len(self): return self.q.shape[1]

    @property
    def heads(self): return self.q.shape[2]

    @property
    def topk(self): return self.idx.shape[-1]


def sample_topk(rng: np.random.Generator, ctx: int, topk: int) -> np.ndarray:
    """`topk` distinct logical positions drawn uniformly from [0, ctx), in
    sampled order; when ctx < topk every position is taken and the rest of
    the list is -1."""
    k = min(ctx, topk)
    out = np.full(topk, -1, np.int32)
    if k > 0:
        out[:k] = rng.choice(ctx, size=k, replace=False).astype(np.int32)
    return out


def flat_inputs(name: str, seed: int, batch: int, q_len: int, heads: int, kv_rows: int,
                topk: int, ctx: Optional[int] = None, with_kv: bool = True) -> Inputs:
    """Flat cache [kv_rows, 576]; each query token draws its own list from [0, ctx)."""
    ctx = kv_rows if ctx is None else ctx
    q = normal_bf16(np.random.default_rng(seed + SUB_Q), (batch, q_len, heads, D))
    kv = normal_bf16(np.random.default_rng(seed + SUB_KV), (kv_rows, D)) if with_kv else None
    rng = np.random.default_rng(seed + SUB_IDX)
    idx = np.stack([np.stack([sample_topk(rng, ctx, topk) for _ in range(q_len)])
                    for _ in range(batch)]).astype(np.int32)
    return Inputs(name, q, kv, idx, kv_rows, pool_seed=None if with_kv else seed + SUB_KV)


def paged_inputs(name: str, seed: int, heads: int, topk: int, ctx: np.ndarray,
                 q_len: int = 1, with_kv: bool = False) -> Inputs:
    """Paged pool: sequence b owns ceil(ctx[b] / 64) pages scattered through a
    randomly permuted pool; its list holds physical rows of its own context."""
    ctx = np.asarray(ctx, np.int64)
    batch = len(ctx)
    pages = (ctx + PAGE - 1) // PAGE
    total_pages = int(pages.sum())
    perm = np.random.default_rng(seed + SUB_PAGES).permutation(total_pages).astype(np.int64)
    table, off = [], 0
    for b in range(batch):
        table.append(perm[off: off + pages[b]])
        off += pages[b]
    rng = np.random.default_rng(seed + SUB_IDX)
    idx = np.empty((batch, q_len, topk), np.int32)
    pos_all = np.empty((batch, q_len, topk), np.int32)
    for b in range(batch):
        for i in range(q_len):
            pos = sample_topk(rng, int(ctx[b]), topk).astype(np.int64)
            pos_all[b, i] = pos
            idx[b, i] = physical_rows(table[b], pos)
    kv_rows = total_pages * PAGE
    q = normal_bf16(np.random.default_rng(seed + SUB_Q), (batch, q_len, heads, D))
    kv = normal_bf16(np.random.default_rng(seed + SUB_KV), (kv_rows, D)) if with_kv else None
    return Inputs(name, q, kv, idx, kv_rows, pool_seed=None if with_kv else seed + SUB_KV,
                  ctx=ctx, page_table=table, pos=pos_all)


def physical_rows(pages: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rows of one sequence's positions in the pool (input construction: the
    harness's own page bookkeeping, -1 stays -1)."""
    pos = np.asarray(pos, np.int64)
    out = np.full(pos.shape, -1, np.int64)
    ok = pos >= 0
    if ok.any():
        out[ok] = np.asarray(pages, np.int64)[pos[ok] // PAGE] * PAGE + pos[ok] % PAGE
    return out.astype(np.int32)


def block_table(inp: Inputs) -> np.ndarray:
    """The paged workload's page tables as one int32 [B, max_pages] array,
    padded with -1 (no page)."""
    width = max(len(t) for t in inp.page_table)
    out = np.full((len(inp.page_table), width), -1, np.int32)
    for b, t in enumerate(inp.page_table):
        out[b, : len(t)] = t
    return out


def dense_inputs(name: str, seed: int, batch: int, q_len: int, heads: int, ctx,
                 paged: bool, with_kv: bool = True) -> Inputs:
    """Dense verify inputs: every token of sequence b attends to all ctx[b]
    positions of its context.  Flat (paged=False): one cache whose first
    ctx[b] rows are sequence b's context.  Paged: a permuted pool of 64-token
    pages as in paged_inputs.  idx holds the rows of positions 0..ctx[b]-1
    (then -1) up to max(ctx) entries, pos the positions themselves."""
    ctx = np.asarray(ctx, np.int64)
    max_ctx = int(ctx.max()) if len(ctx) else 0
    pos = np.full((batch, q_len, max_ctx), -1, np.int32)
    for b in range(batch):
        pos[b, :, : ctx[b]] = np.arange(ctx[b])
    if paged:
        pages = (ctx + PAGE - 1) // PAGE
        perm = np.random.default_rng(seed + SUB_PAGES).permutation(int(pages.sum())).astype(np.int64)
        table, off = [], 0
        for b in range(batch):
            table.append(perm[off: off + pages[b]])
            off += pages[b]
        kv_rows = int(pages.sum()) * PAGE
        idx = np.stack([np.stack([physical_rows(table[b], pos[b, i]) for i in range(q_len)])
                        for b in range(batch)]).astype(np.int32)
    else:
        table, kv_rows, idx = None, max_ctx, pos.copy()
    q = normal_bf16(np.random.default_rng(seed + SUB_Q), (batch, q_len, heads, D))
    kv = normal_bf16(np.random.default_rng(seed + SUB_KV), (kv_rows, D)) if with_kv else None
    return Inputs(name, q, kv, idx, kv_rows, pool_seed=None if with_kv else seed + SUB_KV,
                  ctx=ctx, page_table=table, pos=pos, dense=True)


def index_scores(seed: int, batch: int, q_len: int, max_ctx: int, kind: str = "normal") -> np.ndarray:
    """Synthetic index scores [batch, q_len, max_ctx] fp32 for the top-k
    producer (real ones come from a trained indexer, which the pages do not
    describe).  kind: "normal" N(0,1); "ties" multiples of 1/4 in [-1, 1]
    (every value repeats many times); "equal" all zero; "special" a mix of
    +-0, +-inf, +-NaN, subnormals and ordinary values."""
    rng = np.random.default_rng(seed + SUB_SCORES)
    shape = (batch, q_len, max_ctx)
    if kind == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if kind == "ties":
        return rng.integers(-4, 5, size=shape).astype(np.float32) * np.float32(0.25)
    if kind == "equal":
        return np.zeros(shape, np.float32)
    if kind == "special":
        pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 1e-40, -1e-40, 3.0, -3.0],
                        np.float32)
        s = rng.standard_normal(shape, dtype=np.float32)
        pick = rng.random(shape) < 0.3
        s[pick] = pool[rng.integers(0, len(pool), size=int(pick.sum()))]
        return s
    raise ValueError(kind)


# The five workload shapes: (1) tiny, (2) single request at long context,
# (3) batched decode over a paged pool, (4) speculative-verify shape (9 query
# tokens, each with its own list), (5) large ragged batch over a paged pool;
# and the dense verify shape: 9 query tokens over the whole context.
WORKLOADS = ("tiny", "long", "batched", "spec", "ragged", "verify")


def workload(name: str, *, spec_ctx: int = 65536, with_kv: Optional[bool] = None,
             ragged_pad: bool = False, pad_shuffle: bool = False,
             batch: Optional[int] = None) -> Inputs:
    """Inputs of a named workload.

    with_kv: build the cache on the host (default: only when it is small).
    batch: keep only the first `batch` sequences (sampling for the oracle).
    ragged_pad: the ragged workload with its first 16 sequences shorter than
      the list (contexts in [1, 2047]) so their lists end in -1 padding.
    pad_shuffle: with ragged_pad, each list of those 16 sequences is shuffled
      (seeded), so the -1 entries sit at random positions of the list rather
      than at its tail.
    """
    if name == "tiny":
        return flat_inputs(name, 1000, 1, 1, 8, 1024, 128, with_kv=True if with_kv is None else with_kv)
    if name == "long":
        return flat_inputs(name, 2000, 1, 1, 8, 65536, 2048, with_kv=True if with_kv is None else with_kv)
    if name == "batched":
        b = 64 if batch is None else batch
        ctx = np.full(64, 32768, np.int64)
        inp = paged_inputs(name, 3000, 64, 2048, ctx, with_kv=bool(with_kv))
        return _first_sequences(inp, b)
    if name == "spec":
        return flat_inputs(f"spec{spec_ctx}", 4000, 1, 9, 8, spec_ctx, 2048,
                           with_kv=True if with_kv is None else with_kv)
    if name == "verify":
        return dense_inputs(f"verify{spec_ctx}", 6000, 1, 9, 8, [spec_ctx], paged=False,
                            with_kv=True if with_kv is None else with_kv)
    if name == "ragged":
        rng = np.random.default_rng(5000 + SUB_CTX)
        ctx = rng.integers(2048, 131072, size=128, endpoint=True).astype(np.int64)
        if ragged_pad:
            ctx[:16] = rng.integers(1, 2047, size=16, endpoint=True)
        inp = paged_inputs("ragged_pad" if ragged_pad else name, 5000, 128, 2048, ctx,
                           with_kv=bool(with_kv))
        if ragged_pad and pad_shuffle:
            rng_s = np.random.default_rng(5000 + SUB_IDX + 100)
            for b in range(16):
                for i in range(inp.q_len):
                    order = rng_s.permutation(inp.topk)
                    inp.idx[b, i] = inp.idx[b, i, order]
                    inp.pos[b, i] = inp.pos[b, i, order]
            inp = dataclasses.replace(inp, name="ragged_pad_shuffled")
        return _first_sequences(inp, 128 if batch is None else batch)
    raise KeyError(name)


def _first_sequences(inp: Inputs, b: int) -> Inputs:
    if b >= inp.batch:
        return inp
    return dataclasses.replace(inp, q=inp.q[:b], idx=inp.idx[:b],
                               ctx=None if inp.ctx is None else inp.ctx[:b],
                               page_table=None if inp.page_table is None else inp.page_table[:b],
                               pos=None if inp.pos is None else inp.pos[:b])


def device_pool(kv_rows: int, seed: int, device, chunk_rows: int = 1 << 18):
    """Cache pool [kv_rows, 576] bf16 drawn on `device` with a seeded torch
    generator (for pools too large to build on the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    kv = torch.empty((kv_rows, D), dtype=torch.bfloat16, device=device)
    for r0 in range(0, kv_rows, chunk_rows):
        r1 = min(kv_rows, r0 + chunk_rows)
        kv[r0:r1] = (torch.randn((r1 - r0, D), generator=g, device=device, dtype=torch.float32) * 0.5
                     ).to(torch.bfloat16)
    return kv


def compact_rows(idx: np.ndarray, kv_rows: int):
    """Unique valid rows of a list set and the list remapped onto them.

    Returns (rows [U] int64, idx2 like idx) with idx2 = position of the row in
    `rows`, and -1 for every entry outside [0, kv_rows).  Lets the oracle read
    only the rows a call gathers instead of a multi-GB pool.
    """
    flat = idx.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < kv_rows)
    rows, inv = np.unique(flat[valid], return_inverse=True)
    idx2 = np.full(flat.shape, -1, np.int64)
    idx2[valid] = inv
    return rows, idx2.reshape(idx.shape).astype(np.int32)


# ------------------------------------------------------------ device helpers

def bits_to_torch(a: np.ndarray):
    """uint16 bf16 bits -> torch.bfloat16 CPU tensor (same bytes)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def torch_to_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor (any device) -> uint16 numpy bits (same bytes)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_device(inp: Inputs, device) -> dict:
    """q, kv, idx of `inp` as device tensors (the pool is drawn on the device
    when the host holds none)."""
    import torch
    q = bits_to_torch(inp.q).to(device)
    if inp.kv is not None:
        kv = bits_to_torch(inp.kv).to(device)
    else:
        kv = device_pool(inp.kv_rows, inp.pool_seed, device)
    idx = torch.from_numpy(np.ascontiguousarray(inp.idx)).to(device)
    return {"q": q, "kv": kv, "idx": idx}


def oracle_view(inp: Inputs, kv_dev=None, seqs=None):
    """Host copies of exactly what a call reads, for the CPU oracle.

    seqs: sequence indices to keep (default all).  When the pool lives on the
    device (or is large), only the rows the kept lists select are copied and
    the lists are remapped onto them (masked entries stay masked).
    Returns (q [b, Lq, H, 576] uint16, kv [U, 576] uint16, idx [b, Lq, K] int32).
    """
    import torch
    sel = np.arange(inp.batch) if seqs is None else np.asarray(seqs)
    q = inp.q[sel]
    idx = inp.idx[sel]
    if inp.kv is not None and inp.kv_rows <= (1 << 17):
        return q, inp.kv, idx
    rows, idx2 = compact_rows(idx, inp.kv_rows)
    if inp.kv is not None:
        return q, inp.kv[rows], idx2
    r = torch.from_numpy(rows).to(kv_dev.device)
    return q, torch_to_bits(kv_dev.index_select(0, r)), idx2


# ------------------------------------------------------------ bench rotation

def rotation(inp: Inputs, min_bytes: int = 512 << 20, seed: int = 77, positions: bool = False):
    """Input sets for timing with cold caches.

    Successive timed steps cycle through (cache, index set) pairs whose
    distinct gathered rows together exceed `min_bytes` (default 2x the
    256 MB Infinity Cache), so a row is never still cached from an earlier
    step.  Each index set keeps the workload's recipe (uniform, without
    replacement, from each token's own context); sets over one cache use
    disjoint rows while the context allows it.

    Returns (n_caches, sets): step i uses cache i % n_caches and
    sets[(i // n_caches) % len(sets)], each set an int32 [B, Lq, K] array.
    Paged workloads use their one pool (n_caches == 1); with positions=True
    they return (1, sets, position_sets), the positions behind each set.
    """
    rng = np.random.default_rng(seed)
    B, Lq, K = inp.idx.shape
    T = B * Lq
    if inp.page_table is None:
        ctx = inp.kv_rows
        distinct = min(T * K, ctx) * ROW_BYTES
        need = -(-min_bytes // distinct)
        n_sets = max(1, min(need, ctx // (T * K)))
        sets = []
        for _ in range(n_sets):
            if T * K <= ctx:
                perm = rng.permutation(ctx)[: T * K].astype(np.int32)
                sets.append(perm.reshape(B, Lq, K))
            else:
                sets.append(np.stack([np.stack([sample_topk(rng, ctx, K) for _ in range(Lq)])
                                      for _ in range(B)]).astype(np.int32))
        n_caches = max(1, -(-need // n_sets))
        return n_caches, sets
    ctx = np.asarray(inp.ctx)
    valid = int((inp.idx >= 0).sum())
    need = -(-min_bytes // max(1, valid * ROW_BYTES))
    # each sequence draws disjoint sets while its context allows it (a short
    # context repeats some rows across sets; the batch as a whole does not)
    n_sets = max(1, need)
    sets, pos_sets = [], []
    for s in range(n_sets):
        idx = np.empty((B, Lq, K), np.int32)
        pset = np.empty((B, Lq, K), np.int32)
        for b in range(B):
            perm = rng.permutation(int(ctx[b]))
            for i in range(Lq):
                j = s * Lq + i
                if (j + 1) * K <= ctx[b]:
                    pos = perm[j * K:(j + 1) * K].astype(np.int64)
                else:
                    pos = sample_topk(rng, int(ctx[b]), K).astype(np.int64)
                pset[b, i] = pos
                idx[b, i] = physical_rows(inp.page_table[b], pos)
        sets.append(idx)
        pos_sets.append(pset)
    return (1, sets, pos_sets) if positions else (1, sets)


def edge_inputs(seed: int = 4242, kv_rows: int = 4096, heads: int = 16, topk: int = 300) -> Inputs:
    """Index lists that exercise masking: [2, 3, topk] lists over a flat cache.

    (0,0) all -1; (0,1) first half -1; (0,2) one row repeated through most of
    the list; (1,0) out-of-range entries (kv_rows, kv_rows + 5, 2**31 - 1, -2,
    -2**31) mixed with valid ones; (1,1) a single valid entry, in the last
    slot; (1,2) an ordinary list.
    """
    inp = flat_inputs("edge", seed, 2, 3, heads, kv_rows, topk)
    idx = inp.idx
    idx[0, 0, :] = -1
    idx[0, 1, : topk // 2] = -1
    idx[0, 2, 5:] = idx[0, 2, 0]
    bad = np.array([kv_rows, kv_rows + 5, 2 ** 31 - 1, -2, -2 ** 31], np.int64)
    pos = np.random.default_rng(seed + 9).choice(topk, size=min(topk, 40), replace=False)
    idx[1, 0, pos] = bad[np.arange(len(pos)) % len(bad)].astype(np.int32)
    idx[1, 1, :] = -1
    idx[1, 1, -1] = kv_rows - 1
    return inp


def spike_inputs(seed: int, batch: int, heads: int, kv_rows: int, topk: int, spikes) -> Inputs:
    """A flat workload whose lists hold a few outlier rows.

    spikes: (token, list position, head, factor) tuples.  The cache row at that
    list position of that token gets rope part factor * q_rope[token, head]
    (bf16), so its score for that head rises by about
    factor * scale * |q_rope|^2 (|q_rope|^2 ~ 64) above the ordinary scores
    (standard deviation ~1) while its scores for the other heads stay
    ordinary.  Its latent part is the row's own, quartered, so the head's
    output (nearly that row's V) stays within [-2, 2], where bf16's rounding
    error is below 2^-8.  A later, larger spike for the same head raises the
    running maximum again part-way through a split's slice.
    """
    inp = flat_inputs("spikes", seed, batch, 1, heads, kv_rows, topk)
    q32 = bf16_bits_to_f32(inp.q)
    for tok, pos, head, factor in spikes:
        row = int(inp.idx[tok, 0, pos])
        lat = 0.25 * bf16_bits_to_f32(inp.kv[row, :DV])
        inp.kv[row, :DV] = f32_to_bf16_bits(lat)
        inp.kv[row, DV:] = f32_to_bf16_bits(np.float32(factor) * q32[tok, 0, head, DV:])
    return inp


def partials_inputs(seed: int, tokens: int, nsplit: int, heads: int, empty_frac: float = 0.2):
    """Synthetic combine inputs: part_o [T, S, H, 512] fp32 ~ N(0, 0.5) and
    part_lse [T, S, H] fp32 ~ U(-20, 20), with about `empty_frac` of the
    (token, split, head) slots empty (LSE = -inf, O slot filled with NaN) and
    the last (token, head) pair empty in every split."""
    rng = np.random.default_rng(seed)
    part_o = rng.normal(0.0, 0.5, (tokens, nsplit, heads, DV)).astype(np.float32)
    part_lse = rng.uniform(-20.0, 20.0, (tokens, nsplit, heads)).astype(np.float32)
    empty = rng.random((tokens, nsplit, heads)) < empty_frac
    empty[-1, :, -1] = True
    part_lse[empty] = -np.inf
    part_o[empty] = np.nan
    return part_o, part_lse

