// Top-k producer for gfx950: per query token, the topk positions of the
// largest index scores, ascending ("The Negative Result That Refined the
// Hunt", section "The Context": the indexer produces the candidate positions
// the sparse decode then attends to; "The Moment of Truth", section "The
// Split-K Imperative": the top-k set is the set of candidate tokens the
// kernel retrieves from the cache).  The pages give no indexer math, so the
// scores are an input.
//
// Order.  A score's rank is its fp32 bit pattern mapped to a 32-bit key that
// preserves IEEE total order (negative values: all bits flipped; others: the
// sign bit set), so -NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN, and
// equal keys rank the lower position first.  The selected set is then
// unique, and it is written in ascending position order.
//
// Algorithm: one workgroup per row.  A radix select over the key finds the
// topk-th largest key T digit by digit (11, 11 and 10 bits), each digit from
// an LDS histogram of the keys whose higher bits match the digits found so
// far.  The first digit's histogram covers the whole row.  When every key
// at or above its digit fits in LDS (and the row spans more than one tile),
// a second pass copies them there with their positions, in position order,
// and the rest runs on that copy: the last two digits, then the ordered
// selection below over the copy.
// Otherwise (heavy ties) the keys of the digit's own bin are copied into LDS
// when they fit (one reservation per wave; else the last two digits re-read
// the row), and a last pass walks the row in position order.  The ordered
// selection: each thread over 16 consecutive positions per tile, an element
// is taken if its key exceeds T, or equals T and fewer than (topk - count
// above T) equal keys precede it; its output slot is the count of taken
// elements before it: one block scan per tile of per-thread counts, then bit
// counts inside the thread.  Rows with no more valid positions than topk
// take them all and pad with -1.  The counting passes read coalesced tiles, the next tile's loads
// issued before the current one is counted; 16-byte loads when rows are
// 16-byte aligned.  After the first pass the row is served by the L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;   // 11-bit digits (the last digit has 10 bits)
constexpr int kPerScan = 16;  // elements per thread per tile in the counting passes
constexpr int kPer = 16;      // ... in the ordered pass (two ballots per element)
constexpr int kCandCap = 8192;  // keys of the first digit's bin kept in LDS

__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (lane i
// gets v_0 + ... + v_i): within each row of 16 lanes by shifts of 1, 2, 4
// and 8, then the last lane of row 0 added to row 1 and of row 2 to row 3,
// then lane 31 added to rows 2 and 3.  Lanes whose source lies outside the
// row add 0.  (A shuffle loop goes through the LDS crossbar: six dependent
// round trips.)
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sum of one value per thread over a workgroup of NT
// threads; *total receives the sum.  sw: NT / 64 + 1 words of LDS.
template <int NT = kTopkThreads>
__device__ __forceinline__ uint32_t scan_excl(uint32_t v, uint32_t* sw, uint32_t* total) {
  constexpr int kW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_scan_incl(v);
  if (lane == 63) sw[w] = inc;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = lane < kW ? sw[lane] : 0u;
    const uint32_t ti = wave_scan_incl(t);
    if (lane < kW) sw[lane] = ti - t;
    if (lane == kW - 1) sw[kW] = ti;
  }
  __syncthreads();
  const uint32_t r = sw[w] + inc - v;
  *total = sw[kW];
  __syncthreads();  // sw is reused by the next call
  return r;
}

// Position of element e of thread t in a tile of P * kTopkThreads positions
// starting at base.  With 16-byte loads (V4) a thread reads 4 consecutive
// positions per load: base + ((e / 4) * kTopkThreads + t) * 4 + e % 4;
// otherwise base + e * kTopkThreads + t.  Either way a load instruction of
// a wave reads one contiguous span (coalesced).
template <bool V4>
__device__ __forceinline__ int tile_pos(int base, int e) {
  return V4 ? base + ((e >> 2) * kTopkThreads + (int)threadIdx.x) * 4 + (e & 3)
            : base + e * kTopkThreads + (int)threadIdx.x;
}

// Raw scores of P elements, element e at position pos(e): the loads only,
// so a caller keeps them in flight while it works on earlier data and takes
// the keys (raw_keys) where it uses them.  Every element is loaded, without
// branches: a position at or past the row's end reads a clamped address in
// the row (mc = the row length of the score array) and has its valid bit
// clear, so the wait counts the compiler derives for these loads are exact.
// With V4, elements 4g .. 4g+3 are 4 consecutive positions from a multiple
// of 4 (one 16-byte load; mc is then a multiple of 4).
template <int P, bool V4, class Pos>
__device__ __forceinline__ void load_raw(const float* sc, int n, int mc, Pos pos, float (&v)[P],
                                         uint32_t& valid) {
  static_assert(P <= 32 && P % 4 == 0, "element count");
  if constexpr (V4) {
#pragma unroll
    for (int g = 0; g < P / 4; ++g) {
      const float4 x = *(const float4*)(sc + min(pos(4 * g), mc - 4));
      v[4 * g] = x.x;
      v[4 * g + 1] = x.y;
      v[4 * g + 2] = x.z;
      v[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) v[e] = sc[min(pos(e), mc - 1)];
  }
  valid = 0;
#pragma unroll
  for (int e = 0; e < P; ++e) valid |= (uint32_t)(pos(e) < n) << e;
}
template <int P>
__device__ __forceinline__ void raw_keys(const float (&v)[P], uint32_t (&k)[P]) {
#pragma unroll
  for (int e = 0; e < P; ++e) k[e] = score_key(v[e]);
}

// f(base, keys, valid) over the tiles of a row, in order, with the next
// tile's loads in flight while f works on the current one (the loads of one
// tile are a memory round trip).  f returns false to stop early.
template <int P, bool V4, class F>
__device__ __forceinline__ void for_tiles(const float* sc, int n, int mc, F&& f) {
  float v[P], vn[P];
  uint32_t valid, vv;
  load_raw<P, V4>(sc, n, mc, [](int e) { return tile_pos<V4>(0, e); }, v, valid);
  for (int base = 0; base < n; base += P * kTopkThreads) {
    // the next tile, or this one again at the end (cached; never used): a
    // load issued on every path keeps the wait counts exact
    const int nb = base + P * kTopkThreads < n ? base + P * kTopkThreads : base;
    load_raw<P, V4>(sc, n, mc, [nb](int e) { return tile_pos<V4>(nb, e); }, vn, vv);
    uint32_t k[P];
    raw_keys(v, k);
    if (!f(base, k, valid)) break;
#pragma unroll
    for (int e = 0; e < P; ++e) v[e] = vn[e];
    valid = vv;
  }
}

// The digit (bits [sh, sh + width)) at which the count of counted keys,
// from the top, reaches `need`: returns it in sel[0] and the count of keys
// in higher bins in sel[1] (one thread finds the crossing).
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* sw,
                                           uint32_t* sel) {
  const int tid = threadIdx.x;
  const int hi = kBins - 1 - 2 * tid, lo = hi - 1;  // bins past the digit's width are empty
  const uint32_t ch = hist[hi], cl = hist[lo];
  uint32_t tot;
  const uint32_t ex = scan_excl(ch + cl, sw, &tot);
  if (ex < need && ex + ch >= need) {
    sel[0] = (uint32_t)hi;
    sel[1] = ex;
  } else if (ex + ch < need && ex + ch + cl >= need) {
    sel[0] = (uint32_t)lo;
    sel[1] = ex + ch;
  }
  __syncthreads();
}

// find_digit for a workgroup of NT threads (kBins / NT bins per thread, from
// the top).  The caller knows that at least `need` keys were counted.
template <int NT>
__device__ __forceinline__ void find_digit_nt(const uint32_t* hist, uint32_t need, uint32_t* sw,
                                              uint32_t* sel) {
  constexpr int B = kBins / NT;
  const int top = kBins - 1 - B * (int)threadIdx.x;
  uint32_t c[B], sum = 0;
#pragma unroll
  for (int i = 0; i < B; ++i) {
    c[i] = hist[top - i];
    sum += c[i];
  }
  uint32_t tot;
  const uint32_t ex = scan_excl<NT>(sum, sw, &tot);
  if (ex < need && ex + sum >= need) {
    uint32_t run = ex;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (run < need && run + c[i] >= need) {
        sel[0] = (uint32_t)(top - i);
        sel[1] = run;
      }
      run += c[i];
    }
  }
  __syncthreads();
}

// LDS of a row's selection (one workgroup of kTopkThreads).
struct TopkSmem {
  uint32_t hist[kBins];
  uint32_t sw[kTopkWaves + 1];
  uint32_t sel[2];  // the digit found, the count of keys above it
  uint32_t ncand;
  uint32_t cand[kCandCap];  // keys (of the first digit's bin, or the row's candidates)
  int32_t cpos[kCandCap];   // positions of the row's candidates (select kernel)
};

__device__ __forceinline__ int row_len(const TopkParams& p, int64_t row) {
  int n = p.max_ctx;
  if (p.ctx) n = min(max(p.ctx[(int)(row / p.q_len)], 0), p.max_ctx);
  return n;
}

// every valid position of a row with n <= topk, then -1
__device__ __forceinline__ void take_all(const TopkParams& p, int64_t row, int n) {
  int32_t* out = p.out + row * p.topk;
  for (int i = threadIdx.x; i < p.topk; i += blockDim.x) out[i] = i < n ? i : -1;
}

// kPer consecutive raw scores from position p0 (load_raw)
template <bool V4>
__device__ __forceinline__ void load_chunk(const float* sc, int p0, int n, int mc, float (&v)[kPer],
                                           uint32_t& valid) {
  load_raw<kPer, V4>(sc, n, mc, [p0](int e) { return p0 + e; }, v, valid);
}

// A row's keys with first digit >= b1, with their positions, into LDS
// (sm.cand, sm.cpos) in ascending position order: thread t takes positions
// base + 16 t .. + 15 of each tile, one block scan of the per-thread counts
// gives its slots; the next tile's loads are issued before the current one is
// counted.  The caller knows the count fits kCandCap.
template <bool V4>
__device__ __forceinline__ void ordered_candidates(const float* sc, int n, int mc, uint32_t b1,
                                                   TopkSmem& sm) {
  const int tid = threadIdx.x;
  uint32_t run = 0;  // candidates stored so far
  float v[kPer], vn[kPer];
  uint32_t valid, vv;
  load_chunk<V4>(sc, kPer * tid, n, mc, v, valid);
  for (int base = 0; base < n; base += kPer * kTopkThreads) {
    // the next span, or this one again at the end (cached; never used)
    const int nb = base + kPer * kTopkThreads < n ? base + kPer * kTopkThreads : base;
    load_chunk<V4>(sc, nb + kPer * tid, n, mc, vn, vv);
    uint32_t k[kPer];
    raw_keys(v, k);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)((valid >> e & 1) && (k[e] >> 21) >= b1) << e;
    uint32_t tot;
    uint32_t o = run + scan_excl((uint32_t)__builtin_popcount(m), sm.sw, &tot);
    if (m) {
      const int p0 = base + kPer * tid;
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (m >> e & 1) {
          sm.cand[o] = k[e];
          sm.cpos[o] = p0 + e;
          ++o;
        }
    }
    run += tot;
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = vn[e];
    valid = vv;
  }
}

// The last two digits among a row's candidates in LDS (sm.cand keys and
// sm.cpos positions, `total` of them in ascending position order: every key
// with first digit >= b1), then the ordered selection over them: the keys
// above the topk-th largest key T, and the first `need` keys equal to T
// (need: topk minus the count of keys with first digit above b1).
__device__ __forceinline__ void select_candidates(const TopkParams& p, int64_t row, TopkSmem& sm,
                                                  uint32_t b1, uint32_t need, uint32_t total) {
  const int tid = threadIdx.x;
  // the last two digits among the candidates with first digit b1
  uint32_t prefix = b1;
#pragma unroll 1
  for (int level = 1; level < 3; ++level) {
    const int sh = level == 1 ? 10 : 0;
    const int width = level == 1 ? 11 : 10;
    const int hsh = sh + width;
    const uint32_t mask = (1u << width) - 1;
    for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < total; i += kTopkThreads) {
      const uint32_t k = sm.cand[i];
      if ((k >> hsh) == prefix) atomicAdd(&sm.hist[(k >> sh) & mask], 1u);
    }
    __syncthreads();
    find_digit(sm.hist, need, sm.sw, sm.sel);
    prefix = (prefix << width) | sm.sel[0];
    need -= sm.sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // ordered selection over the candidates (ascending positions): thread t
  // holds candidates 16 t .. 16 t + 15 (total <= kCandCap <= 16 * threads)
  static_assert(kCandCap <= kPer * kTopkThreads, "one tile of candidates");
  const int i0 = kPer * tid;
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const bool ok = (uint32_t)(i0 + e) < total;
    const uint32_t k = ok ? sm.cand[i0 + e] : 0u;
    gtm |= (uint32_t)(ok && k > T) << e;
    eqm |= (uint32_t)(ok && k == T) << e;
  }
  uint32_t tot;
  const uint32_t ex = scan_excl((uint32_t)__builtin_popcount(gtm) | ((uint32_t)__builtin_popcount(eqm) << 16),
                                sm.sw, &tot);
  int32_t* out = p.out + row * p.topk;
  if (gtm | eqm) {
    const uint32_t gt_ex = ex & 0xffffu, eq_ex = ex >> 16;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t below = (1u << e) - 1;
      const uint32_t gt_before = gt_ex + (uint32_t)__builtin_popcount(gtm & below);
      const uint32_t eq_before = eq_ex + (uint32_t)__builtin_popcount(eqm & below);
      if ((gtm >> e & 1) || ((eqm >> e & 1) && eq_before < need)) {
        const uint32_t slot = gt_before + min(eq_before, need);
        if (slot < (uint32_t)p.topk) out[slot] = sm.cpos[i0 + e];
      }
    }
  }
}

// The whole selection of one row (n > topk) by one workgroup.  V4: the row
// starts 16-byte aligned (16-byte loads).
template <bool V4>
__device__ void topk_row(const TopkParams& p, int64_t row, int n, TopkSmem& sm) {
  uint32_t* hist = sm.hist;
  uint32_t* sw = sm.sw;
  uint32_t* sel = sm.sel;
  uint32_t& ncand = sm.ncand;
  uint32_t* cand = sm.cand;
  const int tid = threadIdx.x;
  const float* sc = p.scores + row * p.max_ctx;
  int32_t* out = p.out + row * p.topk;

  // ---- first digit (bits 21..31) over the whole row.  Rows of more than
  // one tile count into four copies of the histogram (lane % 4 picks one;
  // bin i of copy c at word 2048 c + (i ^ 16 c), so the copies of a bin sit
  // in four different banks) held in the candidate area, which is free until
  // the counts are summed: the keys crowd into few bins, and with one copy
  // the lanes' atomics to a bin wait on each other (64 x 32768: 23.0 ->
  // 22.4 us; on a one-tile row the extra clearing and summing cost more)
  const bool copies = n > kPerScan * kTopkThreads;
  uint32_t* sub = cand;
  static_assert(4 * kBins <= kCandCap, "four histogram copies in the candidate area");
  if (copies) {
    for (int i = tid; i < 4 * kBins; i += kTopkThreads) sub[i] = 0;
  } else {
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  }
  if (tid == 0) ncand = 0;
  __syncthreads();
  if (copies) {
    const int c = tid & 3;
    uint32_t* const dst = sub + c * kBins;
    const uint32_t sw16 = 16u * (uint32_t)c;
    for_tiles<kPerScan, V4>(sc, n, p.max_ctx, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
#pragma unroll
      for (int j = 0; j < kPerScan; ++j)
        if (valid >> j & 1) atomicAdd(&dst[(k[j] >> 21) ^ sw16], 1u);
      return true;
    });
  } else {
    for_tiles<kPerScan, V4>(sc, n, p.max_ctx, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
#pragma unroll
      for (int j = 0; j < kPerScan; ++j)
        if (valid >> j & 1) atomicAdd(&hist[k[j] >> 21], 1u);
      return true;
    });
  }
  __syncthreads();
  if (copies) {
    for (int i = tid; i < kBins; i += kTopkThreads)
      hist[i] = sub[i] + sub[kBins + (i ^ 16)] + sub[2 * kBins + (i ^ 32)] + sub[3 * kBins + (i ^ 48)];
    __syncthreads();
  }
  uint32_t need = (uint32_t)p.topk;
  find_digit(hist, need, sw, sel);
  uint32_t prefix = sel[0];
  need -= sel[1];
  const uint32_t in_bin = hist[prefix];
  const uint32_t total = sel[1] + in_bin;  // keys with first digit >= prefix
  const bool cached = in_bin <= (uint32_t)kCandCap;
  __syncthreads();
  if (total <= (uint32_t)kCandCap && n > kPer * kTopkThreads) {
    // all of them, with positions, into LDS in position order: the last two
    // digits and the ordered selection then never read the row again (for
    // rows of more than one tile: on a one-tile row the extra block scan of
    // this pass costs more than the pass over the row it saves, 12.3 against
    // 11.7 us on 1024 positions; 64 rows of 32768: 22.8 against 25.4 us)
    ordered_candidates<V4>(sc, n, p.max_ctx, prefix, sm);
    __syncthreads();
    select_candidates(p, row, sm, prefix, need, total);
    return;
  }

  // ---- keys of that bin into LDS (order irrelevant: only counted below)
  const int lane = tid & 63;
  if (cached) {
    for_tiles<kPerScan, V4>(sc, n, p.max_ctx, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
      uint32_t mm = 0;  // bit j: element j is in the bin
#pragma unroll
      for (int j = 0; j < kPerScan; ++j) mm |= (uint32_t)((valid >> j & 1) && (k[j] >> 21) == prefix) << j;
      // one LDS reservation per wave: its lanes' counts, scanned
      const uint32_t c = (uint32_t)__builtin_popcount(mm);
      const uint32_t inc = wave_scan_incl(c);
      uint32_t wbase = 0;
      if (lane == 63 && inc) wbase = atomicAdd(&ncand, inc);
      uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63) + inc - c;
      if (mm) {
#pragma unroll
        for (int j = 0; j < kPerScan; ++j)
          if (mm >> j & 1) cand[o++] = k[j];
      }
      return true;
    });
    __syncthreads();
  }

  // ---- second and third digits (bits 10..20, then 0..9) among the keys
  // whose higher digits match: from the LDS copy, else from the row
#pragma unroll 1
  for (int level = 1; level < 3; ++level) {
    const int sh = level == 1 ? 10 : 0;
    const int width = level == 1 ? 11 : 10;
    const int hsh = sh + width;
    const uint32_t mask = (1u << width) - 1;
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    if (cached) {
      for (uint32_t i = tid; i < in_bin; i += kTopkThreads) {
        const uint32_t k = cand[i];
        if ((k >> hsh) == prefix) atomicAdd(&hist[(k >> sh) & mask], 1u);
      }
    } else {
      for_tiles<kPerScan, V4>(sc, n, p.max_ctx, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
#pragma unroll
        for (int j = 0; j < kPerScan; ++j)
          if ((valid >> j & 1) && (k[j] >> hsh) == prefix) atomicAdd(&hist[(k[j] >> sh) & mask], 1u);
        return true;
      });
    }
    __syncthreads();
    find_digit(hist, need, sw, sel);
    prefix = (prefix << width) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // the topk-th largest key; `need` keys equal to it are taken

  // ---- ordered selection: keys above T, and the first `need` keys equal to
  // T.  Thread t walks positions base + 16 t .. + 15 of each tile (so the
  // order of positions is the order of threads); one block scan of the
  // packed counts (above | equal << 16, at most 16384 each per tile) gives
  // each thread the number of taken elements before its own, and only
  // threads holding such elements do more.
  uint32_t written = 0, ties_seen = 0;
  for (int base = 0; base < n && written < (uint32_t)p.topk; base += kPer * kTopkThreads) {
    const int p0 = base + kPer * tid;
    float v[kPer];
    if (V4 && p0 + kPer <= n) {
#pragma unroll
      for (int g = 0; g < kPer / 4; ++g) {
        const float4 x = *(const float4*)(sc + p0 + 4 * g);
        v[4 * g] = x.x;
        v[4 * g + 1] = x.y;
        v[4 * g + 2] = x.z;
        v[4 * g + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[e] = p0 + e < n ? sc[p0 + e] : 0.f;
    }
    uint32_t gtm = 0, eqm = 0;  // bit e: element e above / equal to T
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t k = score_key(v[e]);
      const bool ok = p0 + e < n;
      gtm |= (uint32_t)(ok && k > T) << e;
      eqm |= (uint32_t)(ok && k == T) << e;
    }
    uint32_t tot;
    const uint32_t ex = scan_excl((uint32_t)__builtin_popcount(gtm) | ((uint32_t)__builtin_popcount(eqm) << 16),
                                  sw, &tot);
    const uint32_t rem = need > ties_seen ? need - ties_seen : 0u;  // ties still to take
    if (gtm | eqm) {
      const uint32_t gt_ex = ex & 0xffffu, eq_ex = ex >> 16;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const uint32_t below = (1u << e) - 1;
        const uint32_t gt_before = gt_ex + (uint32_t)__builtin_popcount(gtm & below);
        const uint32_t eq_before = eq_ex + (uint32_t)__builtin_popcount(eqm & below);
        if ((gtm >> e & 1) || ((eqm >> e & 1) && eq_before < rem)) {
          const uint32_t slot = written + gt_before + min(eq_before, rem);
          if (slot < (uint32_t)p.topk) out[slot] = p0 + e;
        }
      }
    }
    written += (tot & 0xffffu) + min(tot >> 16, rem);
    ties_seen += tot >> 16;
  }
}

// Kernel arguments: the fields of TopkParams as separate scalars, in its
// order.  The library is built with kernel-argument preloading, so the first
// 13 dwords (the score, length and output addresses, rows, q_len, max_ctx,
// topk and the workspace) reach SGPRs before the waves start, and a
// workgroup's first score loads wait on no read of the argument segment.
#define SMLA_TOPK_ARGS                                                                       \
  const float *a_scores, const int32_t *a_ctx, int32_t *a_out, int64_t a_rows, int a_q_len, \
      int a_max_ctx, int a_topk, void *a_ws, size_t a_ws_row_bytes, int a_chunks, int a_sub
#define SMLA_TOPK_PARAMS \
  { a_scores, a_ctx, a_out, a_rows, a_q_len, a_max_ctx, a_topk, a_ws, a_ws_row_bytes, a_chunks, a_sub }

template <bool V4>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ TopkSmem sm;
  if (p.topk <= 0) return;
  const int64_t row = blockIdx.x;
  const int n = row_len(p, row);
  if (n <= p.topk)
    take_all(p, row, n);
  else
    topk_row<V4>(p, row, n, sm);
}

// ---------------------------------------------------------------------------
// Multi-workgroup form for few long rows (one workgroup per row would leave
// most CUs idle).  Four launches, each row cut into chunks of sub x kSub
// positions; no atomics in device memory, no waits between workgroups:
// A chunk is `sub` sub-chunks of kSub positions, one workgroup looping over
// them (the next sub-chunk's loads issued before the current one is
// counted): the host takes sub > 1 when many rows would otherwise give
// several chunk workgroups per CU, which cuts the histograms written and
// summed.
//   1. topk_hist_kernel (row x chunk): the chunk's first-digit histogram,
//      all 2048 bins written to the workspace;
//   2. topk_scan_kernel (row): the row's histogram (sum over its chunks), the
//      first digit b1 and the count above it; for every chunk, its count of
//      keys with digit >= b1 and the exclusive prefix of those counts (its
//      offset in the row's candidate list); the total;
//   3. topk_cand_kernel (row x chunk): the chunk's keys with digit >= b1,
//      with their positions, written in position order from its offset, so
//      the row's candidate list is in ascending position order;
//   4. topk_select_kernel (row): the candidates into LDS, the last two digits
//      among those with digit b1, then the ordered selection over the
//      candidates (no sort needed).  A row with more candidates than LDS
//      holds takes the one-workgroup path (topk_row) instead.
// ---------------------------------------------------------------------------
constexpr int kChunkThreads = 256;
constexpr int kSub = kChunkThreads * kPer;  // 4096 positions per sub-chunk

enum : uint32_t { kMetaTrivial = 1u, kMetaFallback = 2u };

struct TopkWs {  // a row's slice of the workspace
  uint32_t* hist;  // [chunks][kBins]
  uint32_t* off;   // [chunks + 1] candidate offsets, then the total
  uint32_t* meta;  // [4]: flags, b1, need after the first digit, total
  uint2* cand;     // [kCandCap] (key, position)
};
__device__ __forceinline__ TopkWs row_ws(const TopkParams& p, int64_t row) {
  uint8_t* base = (uint8_t*)p.ws + row * p.ws_row_bytes;
  TopkWs w;
  w.cand = (uint2*)base;
  w.hist = (uint32_t*)(base + kCandCap * sizeof(uint2));
  w.off = w.hist + (size_t)p.chunks * kBins;
  w.meta = w.off + p.chunks + 1;
  return w;
}

template <bool V4>
__global__ __launch_bounds__(kChunkThreads) void topk_hist_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ uint32_t hist[kBins];
  const int64_t row = blockIdx.x / p.chunks;
  const int c = blockIdx.x % p.chunks;
  const int n = row_len(p, row);
  const int base = c * p.sub * kSub;
  if (n <= p.topk || base >= n) return;  // trivial row, or past its end
  const TopkWs w = row_ws(p, row);
  for (int i = threadIdx.x; i < kBins; i += kChunkThreads) hist[i] = 0;
  const float* sc = p.scores + row * p.max_ctx;
  float v[kPer], vn[kPer];
  uint32_t valid, vv;
  load_chunk<V4>(sc, base + kPer * threadIdx.x, n, p.max_ctx, v, valid);
  __syncthreads();
  for (int g = 0; g < p.sub; ++g) {
    const bool more = g + 1 < p.sub && base + (g + 1) * kSub < n;
    // the next sub-chunk, or this one again (cached; never used)
    const int nb = base + (more ? g + 1 : g) * kSub;
    load_chunk<V4>(sc, nb + kPer * threadIdx.x, n, p.max_ctx, vn, vv);
    uint32_t k[kPer];
    raw_keys(v, k);
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (valid >> e & 1) atomicAdd(&hist[k[e] >> 21], 1u);
    if (!more) break;
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = vn[e];
    valid = vv;
  }
  __syncthreads();
  uint32_t* dst = w.hist + (size_t)c * kBins;
  for (int i = threadIdx.x; i < kBins; i += kChunkThreads) dst[i] = hist[i];
}

__global__ __launch_bounds__(kTopkThreads) void topk_scan_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sw[kTopkWaves + 1];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t cnt[kTopkThreads];  // per chunk (a loop covers more chunks)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = row_len(p, row);
  const TopkWs w = row_ws(p, row);
  if (n <= p.topk) {
    if (tid == 0) w.meta[0] = kMetaTrivial;
    return;
  }
  const int nch = (n + p.sub * kSub - 1) / (p.sub * kSub);
  // (loads are issued 16 at a time: a loop of dependent sums would cost one
  // memory round trip per chunk)
  for (int i = tid; i < kBins; i += kTopkThreads) {
    uint32_t t = 0;
    for (int c0 = 0; c0 < nch; c0 += 16) {
      uint32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = c0 + u < nch ? w.hist[(size_t)(c0 + u) * kBins + i] : 0u;
#pragma unroll
      for (int u = 0; u < 16; ++u) t += v[u];
    }
    hist[i] = t;
  }
  __syncthreads();
  find_digit(hist, (uint32_t)p.topk, sw, sel);
  const uint32_t b1 = sel[0], need = (uint32_t)p.topk - sel[1];
  // chunk c's keys with digit >= b1: wave (c % 16) sums bins b1 .. 2047
  uint32_t run = 0;  // offsets so far (thread 0 only)
  for (int c0 = 0; c0 < nch; c0 += kTopkThreads) {
    for (int c = c0 + wave; c < min(nch, c0 + kTopkThreads); c += kTopkWaves) {
      uint32_t t = 0;
      const uint32_t* hc = w.hist + (size_t)c * kBins;
      for (int i0 = (int)b1 + lane; i0 < kBins; i0 += 64 * 8) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + 64 * u < kBins ? hc[i0 + 64 * u] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) t += v[u];
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
      if (lane == 0) cnt[c - c0] = t;
    }
    __syncthreads();
    if (tid == 0) {
      for (int c = c0; c < min(nch, c0 + kTopkThreads); ++c) {
        w.off[c] = run;
        run += cnt[c - c0];
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    w.off[nch] = run;
    w.meta[0] = run > (uint32_t)kCandCap ? kMetaFallback : 0u;
    w.meta[1] = b1;
    w.meta[2] = need;
    w.meta[3] = run;
  }
}

template <bool V4>
__global__ __launch_bounds__(kChunkThreads) void topk_cand_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ uint32_t sw[kChunkThreads / 64 + 1];
  const int64_t row = blockIdx.x / p.chunks;
  const int c = blockIdx.x % p.chunks;
  const int n = row_len(p, row);
  const int base = c * p.sub * kSub;
  if (n <= p.topk || base >= n) return;
  const TopkWs w = row_ws(p, row);
  const float* sc = p.scores + row * p.max_ctx;
  float v[kPer], vn[kPer];
  uint32_t valid, vv;
  load_chunk<V4>(sc, base + kPer * threadIdx.x, n, p.max_ctx, v, valid);  // in flight with the reads below
  const uint32_t flags = w.meta[0], b1 = w.meta[1];
  uint32_t off = w.off[c];
  if (flags != 0u) return;  // trivial or fallback row
  for (int g = 0; g < p.sub; ++g) {
    const int p0 = base + g * kSub + kPer * threadIdx.x;
    const bool more = g + 1 < p.sub && base + (g + 1) * kSub < n;
    // the next sub-chunk, or this one again (cached; never used)
    const int nb = base + (more ? g + 1 : g) * kSub;
    load_chunk<V4>(sc, nb + kPer * threadIdx.x, n, p.max_ctx, vn, vv);
    uint32_t k[kPer];
    raw_keys(v, k);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)((valid >> e & 1) && (k[e] >> 21) >= b1) << e;
    uint32_t tot;
    uint32_t o = off + scan_excl<kChunkThreads>((uint32_t)__builtin_popcount(m), sw, &tot);
    if (m) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (m >> e & 1) w.cand[o++] = make_uint2(k[e], (uint32_t)(p0 + e));
    }
    off += tot;
    if (!more) break;
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = vn[e];
    valid = vv;
  }
}

template <bool V4>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ TopkSmem sm;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = row_len(p, row);
  if (n <= p.topk) {
    take_all(p, row, n);
    return;
  }
  const TopkWs w = row_ws(p, row);
  if (w.meta[0] == kMetaFallback) {
    topk_row<V4>(p, row, n, sm);
    return;
  }
  const uint32_t b1 = w.meta[1], total = w.meta[3];
  uint32_t need = w.meta[2];
  {
    constexpr int kL = kCandCap / kTopkThreads;  // all loads in flight at once
    uint2 e[kL];
#pragma unroll
    for (int u = 0; u < kL; ++u) {
      const uint32_t i = tid + u * kTopkThreads;
      e[u] = i < total ? w.cand[i] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kL; ++u) {
      const uint32_t i = tid + u * kTopkThreads;
      if (i < total) {
        sm.cand[i] = e[u].x;
        sm.cpos[i] = (int32_t)e[u].y;
      }
    }
  }
  select_candidates(p, row, sm, b1, need, total);
}

// ---------------------------------------------------------------------------
// Sampled form for few long rows: two launches, and the scores are read once.
//   1. topk_scand_kernel (chunk x row, chunks of sub <= 4 sub-chunks of kSub
//      positions, the next one's loads issued before the current one is
//      counted).  Every chunk
//      workgroup of a row takes the same sample of the row: 256
//      blocks of 16 consecutive positions at even strides, or the whole row
//      when it holds at most 4096 positions.  From the sample's keys (two
//      LDS histogram passes, 11 + 11 bits) it finds tau, the key at which R
//      sample keys lie at or above (tau rounded down to 22 bits), with R
//      about 1.5 x topk x (sample / row) + 32, so that about 1.5 x topk of
//      the row's keys are expected at or above tau.  It then writes its own
//      keys >= tau with their positions, in position order, to its region
//      of the row's candidate area (kCandCap / chunks-of-the-row entries),
//      and their count (more than the region holds: overflow).
//   2. topk_sel2_kernel (row): the regions concatenated in chunk order (so
//      in position order) into LDS, the three digits of the topk-th largest
//      key T among them, then the ordered selection (select_candidates).
// Exactness: if at least topk keys are >= tau then T >= tau, so every key
// >= T is a candidate.  A row with fewer than topk candidates, or a region
// that overflowed, takes the one-workgroup path in launch 2.  No atomics in
// device memory; the workspace needs no clearing (every region a row reads
// is written by the same call).
// ---------------------------------------------------------------------------
constexpr int kSampleBlocks = 256;  // one 16-position block per chunk thread
constexpr int kSample = kSampleBlocks * 16;
static_assert(kSampleBlocks == kChunkThreads, "one sample block per thread");
constexpr int kSampledMaxChunks = 64;  // regions of at least 128 entries
constexpr int kSampledMaxSub = 4;      // sub-chunks per chunk (longer rows: four launches)
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
constexpr int kStageLoads = kCandCap * 8 / 16 / kTopkThreads;  // 16-byte loads per thread
static_assert(kStageLoads * kTopkThreads * 16 == kCandCap * 8, "staging covers the area");

struct TopkWs2 {
  uint2* cand;    // [kCandCap] (key, position), region c at c * (kCandCap / nch)
  uint32_t* cnt;  // [chunks] candidates found per chunk
};
__device__ __forceinline__ TopkWs2 row_ws2(const TopkParams& p, int64_t row) {
  uint8_t* base = (uint8_t*)p.ws + row * p.ws_row_bytes;
  return TopkWs2{(uint2*)base, (uint32_t*)(base + kCandCap * sizeof(uint2))};
}

template <bool V4>
__global__ __launch_bounds__(kChunkThreads) void topk_scand_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sw[kChunkThreads / 64 + 1];
  __shared__ uint32_t sel[2];
  const int tid = threadIdx.x;
  // chunk-major numbering: every row's chunk 0 first, then every row's chunk
  // 1, ..., so the chunks that exist (shorter rows have fewer; the others'
  // workgroups exit at once) spread evenly over the CUs (ragged rows: 35.3 ->
  // 33.9 us per call against row-major); with rows a multiple of 8, all of a
  // row's chunks sit on XCD row % 8 (the dispatcher's round robin), so its
  // sample is fetched from HBM once
  const int c = (int)(blockIdx.x / p.rows);
  const int64_t row = blockIdx.x % p.rows;
  const int n = row_len(p, row);
  const int span = p.sub * kSub;  // p.sub <= kSampledMaxSub (host)
  const int base = c * span;
  if (n <= p.topk || base >= n) return;  // trivial row, or past its end
  const TopkWs2 w = row_ws2(p, row);
  const float* sc = p.scores + row * p.max_ctx;
  // the sample's loads, then this chunk's first sub-chunk's: the sample is
  // waited for first, the sub-chunk stays in flight through tau
  const bool whole = n <= kSample;
  const int s0 = whole ? 16 * tid : (int)(((int64_t)tid * n / kSampleBlocks) & ~3LL);
  float sr[16];
  uint32_t sv;
  load_chunk<V4>(sc, s0, n, p.max_ctx, sr, sv);
  float v[kPer], vn[kPer];
  uint32_t valid, vv;
  load_chunk<V4>(sc, base + kPer * tid, n, p.max_ctx, v, valid);
  uint32_t sk[16];
  raw_keys(sr, sk);
  for (int i = tid; i < kBins; i += kChunkThreads) hist[i] = 0;
  const int S = whole ? n : kSample;
  const int64_t r_est = (3LL * p.topk * S) / (2LL * n) + 32;
  const uint32_t R = (uint32_t)(whole ? p.topk : (r_est < S ? r_est : S));
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (sv >> e & 1) atomicAdd(&hist[sk[e] >> 21], 1u);
  __syncthreads();
  find_digit_nt<kChunkThreads>(hist, R, sw, sel);
  const uint32_t d1 = sel[0], need2 = R - sel[1];
  for (int i = tid; i < kBins; i += kChunkThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if ((sv >> e & 1) && (sk[e] >> 21) == d1) atomicAdd(&hist[(sk[e] >> 10) & (kBins - 1)], 1u);
  __syncthreads();
  find_digit_nt<kChunkThreads>(hist, need2, sw, sel);
  const uint32_t tau = (d1 << 21) | (sel[0] << 10);
  const int nch = (n + span - 1) / span;
  const uint32_t cap = (uint32_t)(kCandCap / nch);
  uint2* const region = w.cand + (size_t)c * cap;
  uint32_t off = 0;
  for (int g = 0; g < p.sub; ++g) {
    const int p0 = base + g * kSub + kPer * tid;
    const bool more = g + 1 < p.sub && base + (g + 1) * kSub < n;
    // the next sub-chunk, or this one again (cached; never used)
    const int nb = base + (more ? g + 1 : g) * kSub;
    load_chunk<V4>(sc, nb + kPer * tid, n, p.max_ctx, vn, vv);
    uint32_t k[kPer];
    raw_keys(v, k);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)((valid >> e & 1) && k[e] >= tau) << e;
    uint32_t tot;
    uint32_t o = off + scan_excl<kChunkThreads>((uint32_t)__builtin_popcount(m), sw, &tot);
    if (m) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (m >> e & 1) {
          if (o < cap) region[o] = make_uint2(k[e], (uint32_t)(p0 + e));
          ++o;
        }
    }
    off += tot;
    if (!more) break;
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = vn[e];
    valid = vv;
  }
  if (tid == 0) w.cnt[c] = off;
}

template <bool V4>
__global__ __launch_bounds__(kTopkThreads) void topk_sel2_kernel(SMLA_TOPK_ARGS) {
  const TopkParams p = SMLA_TOPK_PARAMS;
  __shared__ TopkSmem sm;
  __shared__ __attribute__((aligned(16))) uint2 stage[kCandCap];  // the row's candidate area
  __shared__ uint32_t off_s[kSampledMaxChunks + 1];
  __shared__ uint32_t bad_s;
  const int tid = threadIdx.x;
  // row r on XCD r % 8, where the chunk launch put its chunks (rows a
  // multiple of 8), so its candidates are in that XCD's L2
  const int64_t row = blockIdx.x;
  const int n = row_len(p, row);
  if (n <= p.topk) {
    take_all(p, row, n);
    return;
  }
  const TopkWs2 w = row_ws2(p, row);
  const int span = p.sub * kSub;
  const int nch = (n + span - 1) / span;  // <= kSampledMaxChunks (host)
  if (nch > kSampledMaxChunks) {  // never taken: the host sizes the chunks
    topk_row<V4>(p, row, n, sm);
    return;
  }
  const uint32_t cap = (uint32_t)(kCandCap / nch);
  // the row's whole candidate area (64 KB, whatever the counts) into LDS by
  // LDS-DMA, in flight together with the chunks' counts: one round trip
  // (reads past a region's count stay in the area and are dropped)
  {
    const u32x4v* src = (const u32x4v*)w.cand + tid;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);  // the LDS base is wave-uniform
    uint8_t* const st = (uint8_t*)stage + wave_u * 64 * 16;
#pragma unroll
    for (int u = 0; u < kStageLoads; ++u) {
      auto* dst = (__attribute__((address_space(3))) uint8_t*)(st + u * kTopkThreads * 16);
      asm volatile("" : "+s"(dst));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + u * kTopkThreads),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  }
  if (tid < 64) {  // the counts and their prefix in the first wave
    const uint32_t v = tid < nch ? w.cnt[tid] : 0u;
    const uint32_t vc = v > cap ? cap : v;
    const uint32_t inc = wave_scan_incl(vc);
    if (tid < nch) off_s[tid] = inc - vc;
    const bool over = __any(v > cap);
    if (tid == nch - 1) {
      off_s[nch] = inc;
      bad_s = (uint32_t)over | (uint32_t)(inc < (uint32_t)p.topk);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();
  if (bad_s) {  // tau too high, or a region overflowed: the one-workgroup path
    topk_row<V4>(p, row, n, sm);
    return;
  }
  const uint32_t total = off_s[nch];  // <= kCandCap
  // the regions, in chunk order, from the staged area (wave v: chunks v, v + 16, ...)
  {
    const int lane = tid & 63, wave = tid >> 6;
    for (int c = wave; c < nch; c += kTopkWaves) {
      const uint32_t o0 = off_s[c], cn = off_s[c + 1] - o0;
      const uint2* rs = stage + (size_t)c * cap;
      for (uint32_t j = lane; j < cn; j += 64) {
        const uint2 e = rs[j];
        sm.cand[o0 + j] = e.x;
        sm.cpos[o0 + j] = (int32_t)e.y;
      }
    }
  }
  __syncthreads();
  // first digit of T among the candidates (every key above tau's is here)
  for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < total; i += kTopkThreads) atomicAdd(&sm.hist[sm.cand[i] >> 21], 1u);
  __syncthreads();
  find_digit(sm.hist, (uint32_t)p.topk, sm.sw, sm.sel);
  const uint32_t b1 = sm.sel[0], need = (uint32_t)p.topk - sm.sel[1];
  __syncthreads();
  select_candidates(p, row, sm, b1, need, total);
}

}  // namespace

// sized for one sub-chunk per chunk, the most chunks any call uses
size_t topk_ws_row_bytes(int max_ctx) {
  const size_t chunks = ((size_t)max_ctx + kSub - 1) / kSub;
  const size_t b = kCandCap * sizeof(uint2) + (chunks * kBins + chunks + 1 + 4) * sizeof(uint32_t);
  return (b + 255) / 256 * 256;
}

int topk_chunks(int max_ctx, int sub) { return (max_ctx + sub * kSub - 1) / (sub * kSub); }

int topk_sampled_max_chunks() { return kSampledMaxChunks; }
int topk_sampled_max_sub() { return kSampledMaxSub; }

#define SMLA_TOPK_PASS(p) \
  (p).scores, (p).ctx, (p).out, (p).rows, (p).q_len, (p).max_ctx, (p).topk, (p).ws, (p).ws_row_bytes, (p).chunks, \
      (p).sub

template <bool V4>
static hipError_t launch_topk_t(const TopkParams& p, hipStream_t st) {
  if (!p.ws) {
    hipLaunchKernelGGL(topk_kernel<V4>, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st,
                       SMLA_TOPK_PASS(p));
    return hipGetLastError();
  }
  const unsigned rc = (unsigned)(p.rows * p.chunks);
  if (p.sampled) {
    if (p.sub > kSampledMaxSub) return hipErrorInvalidValue;  // the host never asks for it
    hipLaunchKernelGGL(topk_scand_kernel<V4>, dim3(rc), dim3(kChunkThreads), 0, st, SMLA_TOPK_PASS(p));
    hipLaunchKernelGGL(topk_sel2_kernel<V4>, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st,
                       SMLA_TOPK_PASS(p));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_hist_kernel<V4>, dim3(rc), dim3(kChunkThreads), 0, st, SMLA_TOPK_PASS(p));
  hipLaunchKernelGGL(topk_scan_kernel, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st,
                     SMLA_TOPK_PASS(p));
  hipLaunchKernelGGL(topk_cand_kernel<V4>, dim3(rc), dim3(kChunkThreads), 0, st, SMLA_TOPK_PASS(p));
  hipLaunchKernelGGL(topk_select_kernel<V4>, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st,
                     SMLA_TOPK_PASS(p));
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const bool v4 = ((uintptr_t)p.scores & 15) == 0 && p.max_ctx % 4 == 0;
  return v4 ? launch_topk_t<true>(p, st) : launch_topk_t<false>(p, st);
}

}  // namespace smla
