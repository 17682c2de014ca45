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
// far.  The first digit's histogram covers the whole row; the keys in its
// bin are then copied, with their positions, into LDS (when they fit), so
// the last two digits never touch memory again; otherwise (heavy ties) those
// digits re-read the row.  A last pass walks the row in position order: an
// element is taken if its key exceeds T, or equals T and fewer than
// (topk - count above T) equal keys precede it.  Its output slot is the count
// of taken elements before it: inside a wave from ballots (a masked
// popcount), across the (element, wave) blocks of a tile from one 256-entry
// scan.  Rows with no more valid positions than topk take them all and pad
// with -1.  Every pass reads coalesced tiles (element j of thread t is
// position base + j * 1024 + t) with 16 loads in flight per thread; after the
// first pass the row is served by the L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;   // 11-bit digits (the last digit has 10 bits)
constexpr int kPer = 16;      // elements per thread per tile (loads in flight)
constexpr int kTile = kTopkThreads * kPer;
constexpr int kCandCap = 8192;  // keys of the first digit's bin kept in LDS

__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one value per thread over the workgroup; *total
// receives the sum.  sw: kTopkWaves + 1 words of LDS.
__device__ __forceinline__ uint32_t scan_excl(uint32_t v, uint32_t* sw, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) sw[w] = inc;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = lane < kTopkWaves ? sw[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(ti, d, 64);
      if (lane >= d) ti += y;
    }
    if (lane < kTopkWaves) sw[lane] = ti - t;
    if (lane == kTopkWaves - 1) sw[kTopkWaves] = ti;
  }
  __syncthreads();
  const uint32_t r = sw[w] + inc - v;
  *total = sw[kTopkWaves];
  __syncthreads();  // sw is reused by the next call
  return r;
}

// Keys of one coalesced tile: element j of thread t is position
// base + j * kTopkThreads + t; positions at or past n read as key 0 with
// valid = false.  All kPer loads are issued before any is used.
__device__ __forceinline__ void load_tile(const float* sc, int base, int n, uint32_t (&k)[kPer],
                                          uint32_t& valid) {
  float v[kPer];
  valid = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int pos = base + j * kTopkThreads + (int)threadIdx.x;
    v[j] = pos < n ? sc[pos] : 0.f;
    valid |= (uint32_t)(pos < n) << j;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) k[j] = score_key(v[j]);
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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sw[kTopkWaves + 1];
  __shared__ uint32_t sel[2];  // the digit found, the count of keys above it
  __shared__ uint32_t ncand;
  __shared__ uint32_t cand[kCandCap];  // keys of the first digit's bin
  __shared__ uint32_t blk[kPer * kTopkWaves + 1];  // per (element, wave) counts, then prefixes

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / p.q_len);
  const float* sc = p.scores + row * p.max_ctx;
  int32_t* out = p.out + row * p.topk;
  int n = p.max_ctx;
  if (p.ctx) n = min(max(p.ctx[b], 0), p.max_ctx);
  if (p.topk <= 0) return;

  if (n <= p.topk) {  // every valid position, then -1
    for (int i = tid; i < p.topk; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }

  // ---- first digit (bits 21..31) over the whole row
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  if (tid == 0) ncand = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kTile) {
    uint32_t k[kPer], valid;
    load_tile(sc, base, n, k, valid);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (valid >> j & 1) atomicAdd(&hist[k[j] >> 21], 1u);
  }
  __syncthreads();
  uint32_t need = (uint32_t)p.topk;
  find_digit(hist, need, sw, sel);
  uint32_t prefix = sel[0];
  need -= sel[1];
  const uint32_t in_bin = hist[prefix];
  const bool cached = in_bin <= (uint32_t)kCandCap;
  __syncthreads();

  // ---- keys of that bin into LDS (order irrelevant: only counted below)
  if (cached) {
    for (int base = 0; base < n; base += kTile) {
      uint32_t k[kPer], valid;
      load_tile(sc, base, n, k, valid);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if ((valid >> j & 1) && (k[j] >> 21) == prefix) cand[atomicAdd(&ncand, 1u)] = k[j];
    }
    __syncthreads();
  }

  // ---- second and third digits (bits 10..20, then 0..9) among the keys
  // whose higher digits match
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
      for (int base = 0; base < n; base += kTile) {
        uint32_t k[kPer], valid;
        load_tile(sc, base, n, k, valid);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if ((valid >> j & 1) && (k[j] >> hsh) == prefix) atomicAdd(&hist[(k[j] >> sh) & mask], 1u);
      }
    }
    __syncthreads();
    find_digit(hist, need, sw, sel);
    prefix = (prefix << width) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // the topk-th largest key; `need` keys equal to it are taken

  // ---- ordered selection: keys above T, and the first `need` keys equal to
  // T.  Position order inside a tile is (element j, wave, lane); counts are
  // packed as (above | equal << 16), at most 16384 each per tile.
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t written = 0, ties_seen = 0;
  for (int base = 0; base < n && written < (uint32_t)p.topk; base += kTile) {
    uint32_t k[kPer], valid;
    load_tile(sc, base, n, k, valid);
    uint64_t gtb[kPer], eqb[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool ok = valid >> j & 1;
      gtb[j] = __ballot(ok && k[j] > T);
      eqb[j] = __ballot(ok && k[j] == T);
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        blk[j * kTopkWaves + wave] =
            (uint32_t)__builtin_popcountll(gtb[j]) | ((uint32_t)__builtin_popcountll(eqb[j]) << 16);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the 256 block counts, 4 per lane
      constexpr int kB = kPer * kTopkWaves / 64;
      uint32_t c[kB], sum = 0;
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        c[i] = blk[lane * kB + i];
        sum += c[i];
      }
      uint32_t inc = sum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
      }
      uint32_t run = inc - sum;
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        blk[lane * kB + i] = run;
        run += c[i];
      }
      if (lane == 63) blk[kPer * kTopkWaves] = inc;
    }
    __syncthreads();
    const uint32_t rem = need > ties_seen ? need - ties_seen : 0u;  // ties still to take
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t pre = blk[j * kTopkWaves + wave];
      const bool gt = gtb[j] >> lane & 1, eq = eqb[j] >> lane & 1;
      const uint32_t gt_before =
          (pre & 0xffffu) + __builtin_amdgcn_mbcnt_hi((uint32_t)(gtb[j] >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)gtb[j], 0u));
      const uint32_t eq_before =
          (pre >> 16) + __builtin_amdgcn_mbcnt_hi((uint32_t)(eqb[j] >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)eqb[j], 0u));
      if (gt || (eq && eq_before < rem)) {
        const uint32_t slot = written + gt_before + min(eq_before, rem);
        if (slot < (uint32_t)p.topk) out[slot] = base + j * kTopkThreads + tid;
      }
    }
    const uint32_t tot = blk[kPer * kTopkWaves];
    written += (tot & 0xffffu) + min(tot >> 16, rem);
    ties_seen += tot >> 16;
    __syncthreads();  // blk is rewritten by the next tile
  }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace smla
