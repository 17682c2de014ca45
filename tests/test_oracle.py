"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` takes an oracle build and raises AssertionError when the build
disagrees with the mathematics or with a number the pages print:

* brute-force dense softmax attention (numpy fp64) when the list is a
  permutation of the whole cache (gather, QK over all 576 columns, softmax,
  PV over the first 512 columns, order invariance);
* closed forms: one-entry lists, two-entry lists, q = 0 / scale = 0,
  duplicate entries;
* invariants: weights sum to 1, masked entries change nothing (bit for bit),
  the LSE combine of ANY partition equals the unsplit result;
* the pages' tokens-per-split figures (2875 and 719 at 46K context).

``test_mutants_are_caught`` rebuilds the oracle with one plausible mistake at
a time (a dropped term, a wrong index or sign, a transposed operand) and
checks that at least one pin fails for every mutant.
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from workloads import SCALE, bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "pages_numbers.json")))


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def dense_attention(q_bits, kv_bits, scale):
    """Textbook softmax(scale * q k^T) v over every cache row (numpy fp64).
    q [H, 576], kv [N, 576]; v = kv[:, :512]."""
    q, kv = f64(q_bits), f64(kv_bits)
    s = float(np.float32(scale)) * (q @ kv.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ kv[:, :512], (m + np.log(z))[:, 0]


def rel_close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    return float(np.max(np.abs(a - b))) <= tol * scale if b.size else True


# --------------------------------------------------------------------- pins

def pin_dense(ref):
    rng = np.random.default_rng(11)
    T, H, N = 3, 5, 96
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (T, H, 576))
    idx = np.stack([rng.permutation(N) for _ in range(T)]).astype(np.int32)
    for scale in (SCALE, 1.0):
        out, lse = ref.decode(q, kv, idx, scale)
        for t in range(T):
            od, ld = dense_attention(q[t], kv, scale)
            assert rel_close(out[t], od, 1e-12), f"dense O mismatch t={t} scale={scale}"
            assert rel_close(lse[t], ld, 1e-12), f"dense LSE mismatch t={t} scale={scale}"


def pin_topk1(ref):
    rng = np.random.default_rng(12)
    T, H, N = 4, 3, 50
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (T, H, 576))
    idx = rng.integers(0, N, size=(T, 1)).astype(np.int32)
    out, lse = ref.decode(q, kv, idx, SCALE)
    for t in range(T):
        r = idx[t, 0]
        assert np.array_equal(out[t], np.broadcast_to(f64(kv[r, :512]), (H, 512))), "K=1: O != V row"
        s = float(np.float32(SCALE)) * (f64(q[t]) @ f64(kv[r]))
        assert rel_close(lse[t], s, 1e-13), "K=1: LSE != score"


def pin_weights(ref):
    rng = np.random.default_rng(13)
    N, K = 300, 257
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (576,), std=2.0)
    idx = rng.choice(N, K, replace=False).astype(np.int32)
    masked = rng.choice(K, 40, replace=False)
    idx[masked[:20]] = -1
    idx[masked[20:]] = N + rng.integers(0, 1000, 20)
    w, lse, n = ref.weights(q, kv, idx, SCALE)
    assert n == K - 40
    assert np.all(w[masked] == 0.0), "masked entries must carry zero weight"
    assert np.all(w >= 0.0)
    assert abs(w.sum() - 1.0) <= 1e-14 * K, f"weights sum {w.sum()}"


def pin_partitions(ref):
    rng = np.random.default_rng(14)
    T, H, N, K = 2, 3, 200, 150
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (T, H, 576))
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[0, rng.choice(K, 30, replace=False)] = -1
    out, lse = ref.decode(q, kv, idx, SCALE)
    # contiguous slices of ceil(K/S) entries, including splits that are empty
    for nsplit in (1, 2, 3, 7, 149, 150, 151, 200):
        po, pl = ref.partial(q, kv, idx, SCALE, nsplit)
        co, cl = ref.combine(po, pl)
        assert rel_close(co, out, 1e-12) and rel_close(cl, lse, 1e-12), f"contiguous nsplit={nsplit}"
    # arbitrary partitions: strided and random (some parts empty)
    parts_list = [np.arange(K) % 4, rng.integers(0, 6, K), np.where(np.arange(K) < 5, 0, 2)]
    for parts in parts_list:
        P = int(parts.max()) + 1
        po = np.empty((T, P, H, 512))
        pl = np.empty((T, P, H))
        for p in range(P):
            sub = np.where(parts[None, :] == p, idx, -1).astype(np.int32)
            o_p, l_p = ref.decode(q, kv, sub, SCALE)
            po[:, p], pl[:, p] = o_p, l_p
        co, cl = ref.combine(po, pl)
        assert rel_close(co, out, 1e-12) and rel_close(cl, lse, 1e-12), "random partition"
    # a partition whose parts are all empty
    po = np.zeros((1, 3, 2, 512))
    pl = np.full((1, 3, 2), -np.inf)
    co, cl = ref.combine(po, pl)
    assert np.all(co == 0.0) and np.all(cl == -np.inf)


def pin_zero_q(ref):
    rng = np.random.default_rng(15)
    N, K = 80, 33
    kv = normal_bf16(rng, (N, 576))
    idx = rng.choice(N, K, replace=False).astype(np.int32)
    idx[[3, 9, 20]] = -1
    valid = idx[idx >= 0]
    mean_v = f64(kv[valid, :512]).mean(axis=0)
    qz = np.zeros((1, 2, 576), np.uint16)
    out, lse = ref.decode(qz, kv, idx[None], SCALE)
    assert rel_close(out[0], np.broadcast_to(mean_v, (2, 512)), 1e-13), "q=0: O != mean V"
    assert rel_close(lse[0], np.full(2, np.log(len(valid))), 1e-14), "q=0: LSE != ln|J|"
    qr = normal_bf16(rng, (1, 2, 576))
    out, lse = ref.decode(qr, kv, idx[None], 0.0)
    assert rel_close(out[0], np.broadcast_to(mean_v, (2, 512)), 1e-13), "scale=0: O != mean V"
    assert rel_close(lse[0], np.full(2, np.log(len(valid))), 1e-14), "scale=0: LSE != ln|J|"


def pin_k2(ref):
    rng = np.random.default_rng(16)
    N = 40
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (1, 4, 576), std=1.5)
    idx = np.array([[7, 31]], np.int32)
    out, lse = ref.decode(q, kv, idx, SCALE)
    sc = float(np.float32(SCALE))
    v1, v2 = f64(kv[7, :512]), f64(kv[31, :512])
    for h in range(4):
        s1 = sc * (f64(q[0, h]) @ f64(kv[7]))
        s2 = sc * (f64(q[0, h]) @ f64(kv[31]))
        sig = 1.0 / (1.0 + np.exp(s2 - s1))
        assert rel_close(out[0, h], sig * v1 + (1.0 - sig) * v2, 1e-13), "K=2: O closed form"
        assert rel_close(lse[0, h], np.logaddexp(s1, s2), 1e-13), "K=2: LSE closed form"


def pin_masking(ref):
    rng = np.random.default_rng(17)
    N = 120
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (1, 3, 576))
    base = rng.choice(N, 60, replace=False).astype(np.int32)
    junk = np.array([-1, -1, N, N + 7, -5, 2**31 - 1, -(2**31), -1], np.int32)
    ins = np.sort(rng.choice(len(base) + len(junk), len(junk), replace=False))
    full = np.empty(len(base) + len(junk), np.int32)
    mask = np.zeros(len(full), bool)
    mask[ins] = True
    full[mask] = junk
    full[~mask] = base
    o1, l1 = ref.decode(q, kv, base[None], SCALE)
    o2, l2 = ref.decode(q, kv, full[None], SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "masked entries changed the result"
    allm = np.full((1, 9), -1, np.int32)
    o3, l3 = ref.decode(q, kv, allm, SCALE)
    assert np.all(o3 == 0.0) and np.all(l3 == -np.inf), "empty set: O=0, LSE=-inf"
    o4, l4 = ref.decode(q, kv, np.zeros((1, 0), np.int32), SCALE)
    assert np.all(o4 == 0.0) and np.all(l4 == -np.inf), "topk=0: O=0, LSE=-inf"


def pin_duplicates(ref):
    rng = np.random.default_rng(18)
    N = 30
    kv = normal_bf16(rng, (N, 576))
    q = normal_bf16(rng, (1, 2, 576), std=1.5)
    a, b = 4, 22
    out, lse = ref.decode(q, kv, np.array([[a, b, a]], np.int32), SCALE)
    sc = float(np.float32(SCALE))
    for h in range(2):
        sa = sc * (f64(q[0, h]) @ f64(kv[a]))
        sb = sc * (f64(q[0, h]) @ f64(kv[b]))
        ea, eb = 2.0 * np.exp(sa), np.exp(sb)
        o = (ea * f64(kv[a, :512]) + eb * f64(kv[b, :512])) / (ea + eb)
        assert rel_close(out[0, h], o, 1e-13), "duplicate entries are separate terms"
        assert rel_close(lse[0, h], np.log(ea + eb), 1e-13)


def pin_pages_split_rule(ref):
    g = GOLDEN["tokens_per_split"]
    K = g["context"]
    kv = np.zeros((1, 576), np.uint16)
    q = np.zeros((1, 1, 576), np.uint16)
    idx = np.zeros((1, K), np.int32)
    for case in g["cases"]:
        S, per = case["nsplit"], case["per_split"]
        _, pl = ref.partial(q, kv, idx, SCALE, S)
        counts = np.rint(np.exp(pl[0, :, 0])).astype(np.int64)
        assert counts[0] == per, f"{K} entries / {S} splits: {counts[0]} per split, pages say {per}"
        assert counts.sum() == K and np.all(counts[:-1] == per), "slices must tile the list"


PINS = [pin_dense, pin_topk1, pin_weights, pin_partitions, pin_zero_q, pin_k2, pin_masking,
        pin_duplicates, pin_pages_split_rule]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(ref, pin):
    pin(ref)


def test_threads_and_empty(ref):
    assert ref.threads() >= 1
    q = np.zeros((0, 4, 576), np.uint16)
    out, lse = ref.decode(q, np.zeros((1, 576), np.uint16), np.zeros((0, 5), np.int32), SCALE)
    assert out.shape == (0, 4, 512) and lse.shape == (0, 4)


def test_bf16_rounding_generator():
    """The input generator's bf16 rounding is round-to-nearest-even."""
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5, 0.0], np.float32)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert np.array_equal(got, want), got


# ------------------------------------------------------------------ mutants

SRC = os.path.join(os.path.dirname(HERE), "oracle", "smla_ref.c")

MUTANTS = {
    "value_from_rope_side": ("const uint16_t *v = kv + (int64_t)idx_row[j] * REF_D;",
                             "const uint16_t *v = kv + (int64_t)idx_row[j] * REF_D + 64;"),
    "qk_over_512_only": ("for (int d = 0; d < REF_D; ++d) dot +=",
                         "for (int d = 0; d < REF_DV; ++d) dot +="),
    "scale_dropped": ("s[j - lo] = scale * dot;", "s[j - lo] = dot;"),
    "lse_without_max": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "lse_base2": ("*lse_out = m + log(z);", "*lse_out = m + log2(z);"),
    "masked_weight_counted": ("? exp(s[j - lo] - m) : 0.0;", "? exp(s[j - lo] - m) : 1.0;"),
    "split_floor": ("int per = (topk + nsplit - 1) / nsplit;", "int per = topk / nsplit;"),
    "combine_sign": ("double w = exp(l - mx);", "double w = exp(mx - l);"),
    "combine_no_normalise": ("for (int c = 0; c < REF_DV; ++c) o[c] /= wsum;", ""),
    "q_rows_transposed": ("jb->q + ((int64_t)t * jb->heads + h) * REF_D",
                          "jb->q + ((int64_t)h * jb->tokens + t) * REF_D"),
    "list_of_token0": ("const int32_t *idx_row = jb->idx + (int64_t)t * jb->topk;",
                       "const int32_t *idx_row = jb->idx;"),
    "partial_layout_split_major": ("int64_t slot = ((int64_t)t * ns + sp) * jb->heads + h;",
                                   "int64_t slot = ((int64_t)sp * jb->tokens + t) * jb->heads + h;"),
    "softmax_not_normalised": ("for (int j = lo; j < hi; ++j) w[j - lo] /= z;", ""),
}


def _build_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = os.path.join(tmp, f"{name}.c")
    open(path, "w").write(src.replace(old, new))
    so = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-pthread", "-o", so, path, "-lm"],
                   check=True)
    return so


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.RefLib(_build_mutant(tmp, name, old, new))
        caught = []
        for pin in PINS:
            try:
                pin(lib)
            except (AssertionError, RuntimeError, FloatingPointError, ValueError):
                caught.append(pin.__name__)
        assert caught, f"no pin catches mutant {name}"


# ------------------------------------------------------ paged and dense maps

def test_pin_rows_of_positions_worked_example():
    # sequence 0 owns pages 3, 0, 2 (in that order), 4 tokens per page; page
    # slot 3 of sequence 1 is missing.  Position 5 is page 1 (id 0), offset 1
    # -> row 1; position 9 is page 2 (id 2), offset 1 -> row 9; position 12 is
    # page 3, beyond sequence 0's three pages -> masked; position 3 of
    # sequence 1 is its page 0 (id 1), offset 3 -> row 7; its position 13 is
    # page 3, id -1 -> masked.  With a 12-row cache, position 0 of sequence 0
    # (page id 3, offset 0 = row 12) and position 8 of sequence 1 (page id 3,
    # offset 0 = row 12) fall outside the cache -> masked.
    table = np.array([[3, 0, 2, -1], [1, 2, 3, -1]], np.int32)
    pos = np.array([[[0, 5, 9, 12, -1]], [[3, 13, 8, -7, 4]]], np.int32)
    got = oracle.rows_of_positions(table, 4, pos, kv_rows=12)
    assert got[0, 0].tolist() == [-1, 1, 9, -1, -1]
    assert got[1, 0].tolist() == [7, -1, -1, -1, 8]
    got16 = oracle.rows_of_positions(table, 4, pos, kv_rows=16)
    assert got16[0, 0].tolist() == [12, 1, 9, -1, -1]
    assert got16[1, 0].tolist() == [7, -1, 12, -1, 8]


def test_pin_rows_of_positions_identity_and_bijection():
    rng = np.random.default_rng(7)
    P, page = 6, 8
    ident = np.tile(np.arange(P, dtype=np.int32), (2, 1))
    pos = rng.integers(-3, P * page + 5, size=(2, 3, 40)).astype(np.int32)
    rows = oracle.rows_of_positions(ident, page, pos, kv_rows=P * page)
    inside = (pos >= 0) & (pos < P * page)
    assert (rows[inside] == pos[inside]).all() and (rows[~inside] == -1).all()
    # a permuted table maps the sequence's positions one-to-one onto its pages' rows
    perm = rng.permutation(P).astype(np.int32)[None, :]
    allpos = np.arange(P * page, dtype=np.int32)[None, None, :]
    r = oracle.rows_of_positions(perm, page, allpos, kv_rows=P * page)
    assert sorted(r.ravel().tolist()) == list(range(P * page))
    # flat cache: positions are rows, clipped at kv_rows
    flat = oracle.rows_of_positions(None, page, pos, kv_rows=20)
    assert ((flat == pos) | (flat == -1)).all() and (flat[(pos >= 0) & (pos < 20)] >= 0).all()


def test_pin_dense_positions():
    d = oracle.dense_positions([3, 0, 7], max_ctx=5, q_len=2)
    assert d.shape == (3, 2, 5)
    assert d[0, 1].tolist() == [0, 1, 2, -1, -1]
    assert d[1, 0].tolist() == [-1] * 5
    assert d[2, 0].tolist() == [0, 1, 2, 3, 4]


# ------------------------------------------------------------ top-k producer

def _beats(a: float, b: float) -> bool:
    """Whether score a ranks above score b, from float comparisons (not from
    bit patterns): any +NaN above everything else, any -NaN below; among the
    rest the larger value, and between equal values +0 above -0."""
    import math
    an, bn = math.isnan(a), math.isnan(b)
    sa, sb = math.copysign(1.0, a) > 0, math.copysign(1.0, b) > 0
    if an or bn:
        ra = 2 if an and sa else -2 if an else 0
        rb = 2 if bn and sb else -2 if bn else 0
        return ra > rb
    if a != b:
        return a > b
    return sa and not sb  # +0 above -0; identical values tie


def _brute_topk(row, n, k):
    """Position i is chosen iff fewer than k positions beat it, where j beats
    i if its score ranks above i's, or ties with it at a lower position."""
    vals = [float(v) for v in row[:n]]
    chosen = []
    for i in range(n):
        beaten_by = sum(1 for j in range(n) if j != i and
                        (_beats(vals[j], vals[i]) or (not _beats(vals[i], vals[j]) and j < i)))
        if beaten_by < k:
            chosen.append(i)
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_pin_topk_brute_force(kind):
    rng = np.random.default_rng({"normal": 11, "ties": 12, "special": 13}[kind])
    B, Lq, M = 3, 2, 70
    if kind == "normal":
        s = rng.standard_normal((B, Lq, M)).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(-3, 4, size=(B, Lq, M)).astype(np.float32) * np.float32(0.25)
    else:
        pool = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -np.inf, np.nan, -np.nan, 1e-40, -1e-40],
                        np.float32)
        s = pool[rng.integers(0, len(pool), size=(B, Lq, M))]
    ctx = [70, 33, 5]
    for k in (1, 4, 17, 40, 70, 80):
        got = oracle.topk_positions(s, ctx, k)
        for b in range(B):
            for t in range(Lq):
                assert got[b, t].tolist() == _brute_topk(s[b, t], min(ctx[b], M), k), (kind, k, b, t)


def test_pin_topk_special_cases():
    s = np.zeros((2, 1, 50), np.float32)  # all equal: the lowest positions win
    assert oracle.topk_positions(s, None, 7)[0, 0].tolist() == list(range(7))
    got = oracle.topk_positions(s, [3, -4], 5)  # short and negative contexts: -1 padding
    assert got[0, 0].tolist() == [0, 1, 2, -1, -1] and got[1, 0].tolist() == [-1] * 5
    assert oracle.topk_positions(s, [500, 50], 50)[0, 0].tolist() == list(range(50))  # clipped at M
    r = np.arange(50, dtype=np.float32)[None, None, :].repeat(2, axis=0)  # increasing: the last k
    assert oracle.topk_positions(r, None, 6)[1, 0].tolist() == list(range(44, 50))
    # the same set as a partition of distinct values by a different library routine
    rng = np.random.default_rng(5)
    d = rng.permutation(4000).astype(np.float32)[None, None, :] - 1999.5
    want = np.sort(np.argpartition(-d[0, 0], 300)[:300])
    assert oracle.topk_positions(d, None, 300)[0, 0].tolist() == want.tolist()
