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
// topk-th largest key T in three histogram passes (11, 11 and 10 bits, each
// over the elements whose higher bits match the bins found so far; LDS
// histograms).  A last pass walks the row in position order, one element per
// thread per tile: an element is taken if its key exceeds T, or equals T and
// fewer than (topk - count above T) equal keys precede it; one block-wide scan
// per tile gives each taken element its output slot.  Rows with no more valid
// positions than topk take them all and pad with -1.  Loads are coalesced
// (thread t reads position base + t); after the first pass the row is served
// by the L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;  // 11-bit digits (the last digit has 10 bits)

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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sw[kTopkWaves + 1];
  __shared__ uint32_t sel[2];  // the bin found, the count of keys above it

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

  // ---- radix select of the topk-th largest key: digit d of the key is
  // bits [sh, sh + width) with (sh, width) = (21, 11), (10, 11), (0, 10);
  // prefix = the key bits above the digit found so far
  uint32_t prefix = 0, need = (uint32_t)p.topk;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int sh = level == 0 ? 21 : level == 1 ? 10 : 0;
    const int width = level == 2 ? 10 : 11;
    const int hsh = sh + width;  // bits of the prefix start here (32: none)
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kTopkThreads) {
      const int pos = base + tid;
      if (pos < n) {
        const uint32_t k = score_key(sc[pos]);
        if (hsh >= 32 || (k >> hsh) == prefix)
          atomicAdd(&hist[(k >> sh) & ((1u << width) - 1)], 1u);
      }
    }
    __syncthreads();
    // scan the bins from the top: thread t holds bins hi = kBins-1-2t and
    // lo = hi - 1 (bins past the digit's width are empty)
    const int hi = kBins - 1 - 2 * tid, lo = hi - 1;
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
    prefix = (prefix << width) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // the topk-th largest key; `need` equal keys are taken

  // ---- ordered selection: keys above T, and the first `need` keys equal to T
  uint32_t written = 0, ties_seen = 0;
  for (int base = 0; base < n && written < (uint32_t)p.topk; base += kTopkThreads) {
    const int pos = base + tid;
    uint32_t gt = 0, eq = 0;
    if (pos < n) {
      const uint32_t k = score_key(sc[pos]);
      gt = k > T;
      eq = k == T;
    }
    uint32_t tot;
    const uint32_t ex = scan_excl(gt | (eq << 16), sw, &tot);
    const uint32_t gt_ex = ex & 0xffffu, eq_ex = ex >> 16;
    const uint32_t gt_tot = tot & 0xffffu, eq_tot = tot >> 16;
    const uint32_t rem = need > ties_seen ? need - ties_seen : 0u;  // ties still to take
    const bool take = gt || (eq && eq_ex < rem);
    const uint32_t slot = written + gt_ex + min(eq_ex, rem);
    if (take && slot < (uint32_t)p.topk) out[slot] = pos;
    written += gt_tot + min(eq_tot, rem);
    ties_seen += eq_tot;
  }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.rows), dim3(kTopkThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace smla
