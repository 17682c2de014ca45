"""fp64 CPU oracle for sparse MLA decode with split-K over the top-k list.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It is independent
of the HIP library: no shared code, headers, tables or constants, and neither
imports the other.

The arithmetic lives in ``smla_ref.c`` (plain C, fp64); this module only
marshals numpy arrays into it.  Inputs are the raw bf16 bit patterns
(``numpy.uint16``) the GPU consumes, so the oracle sees exactly the values
the kernel read.

Page citations (by title and section):
  [SPLITK] "The Moment of Truth: Validating Split-K Parallelization for
           Blackwell MLA Decode" -- "The Split-K Imperative".
  [NSPLIT] "The Occupancy Hypothesis: How One Kernel Parameter Unlocked 1.8x
           Decode Speedup on Blackwell" -- "The Occupancy Insight",
           "The Broader Context", "The Road to This Experiment".

  [BISECT] "The Negative Result That Refined the Hunt: Disabling the MMA
           FlashMLA Kernel" -- "The Context".

Paged and dense calls (``rows_of_positions``, ``dense_positions``) are
defined as a plain decode over the rows their positions name, so the oracle
for them is the index map below followed by ``decode``.  The top-k producer
(``topk_positions``) is a selection, defined by a sort.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla_ref.so")

D = 576   # row width of q and of a cache row (512 latent + 64 rope)
DV = 512  # value width: the first 512 columns of a row


class RefLib:
    """ctypes view of one build of smla_ref.c (the default build unless a path
    is given; the oracle's own tests also load deliberately mutated builds)."""

    def __init__(self, path: str = LIB_PATH):
        if path == LIB_PATH and not os.path.exists(path):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.smla_ref_decode.argtypes = [u16p, u16p, i64, i32p, i64, i32, i32, f32, f64p, f64p, i32]
        lib.smla_ref_partial.argtypes = [u16p, u16p, i64, i32p, i64, i32, i32, f32, i32, f64p,
                                         f64p, i32]
        lib.smla_ref_combine.argtypes = [f64p, f64p, i64, i32, i32, f64p, f64p]
        lib.smla_ref_weights.argtypes = [u16p, u16p, i64, i32p, i32, f32, f64p, f64p]
        lib.smla_ref_threads.argtypes = []
        for fn in ("smla_ref_decode", "smla_ref_partial", "smla_ref_combine",
                   "smla_ref_weights", "smla_ref_threads"):
            getattr(lib, fn).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def threads(self) -> int:
        """Threads the oracle uses by default (the process's CPU affinity mask)."""
        return int(self.lib.smla_ref_threads())

    def decode(self, q, kv, idx, scale: float, nthreads: int = 0):
        """Unsplit attention over each token's selected rows.

        q: [..., H, 576] uint16 (bf16 bits); the leading dims are the tokens.
        kv: [N, 576] uint16.  idx: [..., K] int32 with the same leading dims.
        Returns (out [..., H, 512] fp64, lse [..., H] fp64).
        """
        q, kv, idx = _u16(q), _u16(kv), _i32(idx)
        lead = q.shape[:-2]
        heads = q.shape[-2]
        assert q.shape[-1] == D and kv.ndim == 2 and kv.shape[1] == D
        assert idx.shape[:-1] == lead, (idx.shape, q.shape)
        tokens = int(np.prod(lead)) if lead else 1
        topk = idx.shape[-1]
        out = np.empty(lead + (heads, DV), np.float64)
        lse = np.empty(lead + (heads,), np.float64)
        rc = self.lib.smla_ref_decode(_ptr(q, ctypes.c_uint16), _ptr(kv, ctypes.c_uint16),
                                      kv.shape[0], _ptr(idx, ctypes.c_int32), tokens, heads, topk,
                                      ctypes.c_float(scale), _ptr(out, ctypes.c_double),
                                      _ptr(lse, ctypes.c_double), nthreads)
        _check(rc, "smla_ref_decode")
        return out, lse

    def partial(self, q, kv, idx, scale: float, nsplit: int, nthreads: int = 0):
        """Per-split attention over contiguous slices of ceil(K/nsplit) entries.

        Returns (part_o [T, nsplit, H, 512], part_lse [T, nsplit, H]) with T the
        flattened token count.
        """
        q, kv, idx = _u16(q), _u16(kv), _i32(idx)
        heads = q.shape[-2]
        tokens = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
        topk = idx.shape[-1]
        part_o = np.empty((tokens, nsplit, heads, DV), np.float64)
        part_lse = np.empty((tokens, nsplit, heads), np.float64)
        rc = self.lib.smla_ref_partial(_ptr(q, ctypes.c_uint16), _ptr(kv, ctypes.c_uint16),
                                       kv.shape[0], _ptr(idx, ctypes.c_int32), tokens, heads,
                                       topk, ctypes.c_float(scale), nsplit,
                                       _ptr(part_o, ctypes.c_double),
                                       _ptr(part_lse, ctypes.c_double), nthreads)
        _check(rc, "smla_ref_partial")
        return part_o, part_lse

    def combine(self, part_o, part_lse):
        """LSE combine of partials [T, S, H, 512] / [T, S, H] -> ([T, H, 512], [T, H])."""
        part_o = np.ascontiguousarray(part_o, dtype=np.float64)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
        tokens, nsplit, heads = part_lse.shape
        assert part_o.shape == (tokens, nsplit, heads, DV)
        out = np.empty((tokens, heads, DV), np.float64)
        lse = np.empty((tokens, heads), np.float64)
        rc = self.lib.smla_ref_combine(_ptr(part_o, ctypes.c_double),
                                       _ptr(part_lse, ctypes.c_double), tokens, heads, nsplit,
                                       _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
        _check(rc, "smla_ref_combine")
        return out, lse

    def weights(self, q_row, kv, idx_row, scale: float):
        """Softmax weights of one (token, head): (w [K] fp64, lse, n_valid)."""
        q_row, kv, idx_row = _u16(q_row), _u16(kv), _i32(idx_row)
        assert q_row.shape == (D,)
        topk = idx_row.shape[0]
        w = np.empty(max(topk, 1), np.float64)
        lse = np.empty(1, np.float64)
        n = self.lib.smla_ref_weights(_ptr(q_row, ctypes.c_uint16), _ptr(kv, ctypes.c_uint16),
                                      kv.shape[0], _ptr(idx_row, ctypes.c_int32), topk,
                                      ctypes.c_float(scale), _ptr(w, ctypes.c_double),
                                      _ptr(lse, ctypes.c_double))
        if n < 0:
            raise RuntimeError(f"smla_ref_weights failed with status {n}")
        return w[:topk], float(lse[0]), int(n)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


_default = None


def default() -> RefLib:
    """The oracle as built from smla_ref.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = RefLib()
    return _default


def threads() -> int:
    return default().threads()


def decode(q, kv, idx, scale: float, nthreads: int = 0):
    return default().decode(q, kv, idx, scale, nthreads)


def partial(q, kv, idx, scale: float, nsplit: int, nthreads: int = 0):
    return default().partial(q, kv, idx, scale, nsplit, nthreads)


def combine(part_o, part_lse):
    return default().combine(part_o, part_lse)


def weights(q_row, kv, idx_row, scale: float):
    return default().weights(q_row, kv, idx_row, scale)


def rows_of_positions(block_table, page_size: int, pos, kv_rows: int) -> np.ndarray:
    """Cache rows of positions in paged sequences ([NSPLIT] "The Road to This
    Experiment": the cache is reached through per-sequence page tables).

    block_table [B, P] int: page ids of sequence b's pages in order (< 0: no
    page), or None for a flat cache (position = row).  pos [B, Lq, K] int.
    Position x of sequence b is row block_table[b, x // page_size] *
    page_size + x % page_size.  Returns int32 rows of pos's shape, -1 for a
    position < 0 or beyond the table, a missing page, or a row outside
    [0, kv_rows).
    """
    pos = np.asarray(pos, np.int64)
    out = np.full(pos.shape, -1, np.int64)
    for b in range(pos.shape[0]):
        for i in range(pos.shape[1]):
            for k in range(pos.shape[2]):
                x = int(pos[b, i, k])
                if x < 0:
                    continue
                if block_table is None:
                    row = x
                else:
                    page_i, offset = divmod(x, page_size)
                    if page_i >= block_table.shape[1] or block_table[b, page_i] < 0:
                        continue
                    row = int(block_table[b, page_i]) * page_size + offset
                if row < kv_rows:
                    out[b, i, k] = row
    return out.astype(np.int32)


def dense_positions(ctx_len, max_ctx: int, q_len: int) -> np.ndarray:
    """The implicit list of a dense call ([NSPLIT] "The Occupancy Insight",
    "The Broader Context": the verify kernel splits the whole context): every
    token of sequence b takes positions 0 .. ctx_len[b]-1, then -1 up to
    max_ctx entries.  Returns int32 [B, q_len, max_ctx]."""
    ctx_len = np.asarray(ctx_len, np.int64)
    out = np.full((len(ctx_len), q_len, max_ctx), -1, np.int64)
    for b, c in enumerate(ctx_len):
        n = min(int(c), max_ctx)
        out[b, :, :n] = np.arange(n)
    return out.astype(np.int32)


def score_keys(scores) -> np.ndarray:
    """Rank keys of fp32 scores: the IEEE total order of their bit patterns
    as unsigned 32-bit integers (a negative value's bits all flipped, any
    other value's sign bit set), so -NaN < -inf < ... < -0 < +0 < ... <
    +inf < +NaN.  Returns uint64 (no wrap in later arithmetic)."""
    u = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    neg = (u >> np.uint32(31)) == 1
    return np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint64)


def topk_positions(scores, ctx_len, topk: int) -> np.ndarray:
    """The top-k producer ([BISECT] "The Context": an indexer picks the
    candidate positions; [SPLITK] "The Split-K Imperative": the top-k set is
    the candidate tokens retrieved from the cache).  The pages give no
    indexer math, so the scores are an input.

    scores [B, Lq, M] fp32; ctx_len [B] int or None (M).  For row (b, t) with
    n = min(max(ctx_len[b], 0), M): sort positions 0..n-1 by rank key
    descending, ties by position ascending; take the first topk; return them
    in ascending position order, -1 after the last when n < topk.
    Returns int32 [B, Lq, topk]."""
    scores = np.asarray(scores, dtype=np.float32)
    B, Lq, M = scores.shape
    keys = score_keys(scores)
    out = np.full((B, Lq, topk), -1, np.int64)
    for b in range(B):
        n = M if ctx_len is None else min(max(int(ctx_len[b]), 0), M)
        for t in range(Lq):
            k = keys[b, t, :n].astype(np.int64)
            order = np.lexsort((np.arange(n), -k))  # key descending, then position
            chosen = np.sort(order[:topk])
            out[b, t, :len(chosen)] = chosen
    return out.astype(np.int32)
