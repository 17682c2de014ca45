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
// bin are then copied into LDS (when they fit; one reservation per wave), so
// the last two digits never touch memory again; otherwise (heavy ties) those
// digits re-read the row.  A last pass walks the row in position order, each
// thread over 16 consecutive positions per tile: an element is taken if its
// key exceeds T, or equals T and fewer than (topk - count above T) equal keys
// precede it.  Its output slot is the count of taken elements before it:
// one block scan per tile of per-thread counts, then bit counts inside the
// thread.  Rows with no more valid positions than topk take them all and pad
// with -1.  The counting passes read coalesced tiles, the next tile's loads
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

// Keys of one tile; positions at or past n read as key 0 with their valid
// bit clear.  All loads are issued before any is used.
template <int P, bool V4>
__device__ __forceinline__ void load_tile(const float* sc, int base, int n, uint32_t (&k)[P],
                                          uint32_t& valid) {
  static_assert(P <= 32 && P % 4 == 0, "tile shape");
  float v[P];
  valid = 0;
  if constexpr (V4) {
#pragma unroll
    for (int g = 0; g < P / 4; ++g) {
      const int p0 = tile_pos<true>(base, 4 * g);
      if (p0 + 3 < n) {
        const float4 x = *(const float4*)(sc + p0);
        v[4 * g] = x.x;
        v[4 * g + 1] = x.y;
        v[4 * g + 2] = x.z;
        v[4 * g + 3] = x.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * g + c] = p0 + c < n ? sc[p0 + c] : 0.f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int pos = tile_pos<false>(base, e);
      v[e] = pos < n ? sc[pos] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < P; ++e) {
    valid |= (uint32_t)(tile_pos<V4>(base, e) < n) << e;
    k[e] = score_key(v[e]);
  }
}

// f(base, keys, valid) over the tiles of a row, in order, with the next
// tile's loads issued before f works on the current one (the loads of one
// tile are a memory round trip; this overlaps it with the previous tile's
// work).  f returns false to stop early.
template <int P, bool V4, class F>
__device__ __forceinline__ void for_tiles(const float* sc, int n, F&& f) {
  uint32_t k[P], kn[P], valid, vn = 0;
  load_tile<P, V4>(sc, 0, n, k, valid);
  for (int base = 0; base < n; base += P * kTopkThreads) {
    const int nb = base + P * kTopkThreads;
    if (nb < n) load_tile<P, V4>(sc, nb, n, kn, vn);
    if (!f(base, k, valid)) break;
#pragma unroll
    for (int e = 0; e < P; ++e) k[e] = kn[e];
    valid = vn;
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

// V4: every row starts 16-byte aligned (16-byte loads).
template <bool V4>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sw[kTopkWaves + 1];
  __shared__ uint32_t sel[2];  // the digit found, the count of keys above it
  __shared__ uint32_t ncand;
  __shared__ uint32_t cand[kCandCap];  // keys of the first digit's bin

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
  for_tiles<kPerScan, V4>(sc, n, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
#pragma unroll
    for (int j = 0; j < kPerScan; ++j)
      if (valid >> j & 1) atomicAdd(&hist[k[j] >> 21], 1u);
    return true;
  });
  __syncthreads();
  uint32_t need = (uint32_t)p.topk;
  find_digit(hist, need, sw, sel);
  uint32_t prefix = sel[0];
  need -= sel[1];
  const uint32_t in_bin = hist[prefix];
  const bool cached = in_bin <= (uint32_t)kCandCap;
  __syncthreads();

  // ---- keys of that bin into LDS (order irrelevant: only counted below)
  const int lane = tid & 63;
  if (cached) {
    for_tiles<kPerScan, V4>(sc, n, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
      uint32_t mm = 0;  // bit j: element j is in the bin
#pragma unroll
      for (int j = 0; j < kPerScan; ++j) mm |= (uint32_t)((valid >> j & 1) && (k[j] >> 21) == prefix) << j;
      // one LDS reservation per wave: its lanes' counts, scanned
      const uint32_t c = (uint32_t)__builtin_popcount(mm);
      uint32_t inc = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
      }
      uint32_t wbase = 0;
      if (lane == 63 && inc) wbase = atomicAdd(&ncand, inc);
      uint32_t o = __shfl(wbase, 63, 64) + inc - c;
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
      for_tiles<kPerScan, V4>(sc, n, [&](int, const uint32_t(&k)[kPerScan], uint32_t valid) {
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

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const bool v4 = ((uintptr_t)p.scores & 15) == 0 && p.max_ctx % 4 == 0;
  if (v4)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st, p);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace smla
