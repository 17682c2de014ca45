// smla_kernels.hip -- gfx950 kernels for sparse MLA decode with split-K over
// the top-k list: the split kernel (gather -> QK^T -> online softmax -> PV ->
// partial or final output) and the log-sum-exp combine kernel.
//
// Pages (cited by title and section):
//   [SPLITK] "The Moment of Truth: Validating Split-K Parallelization for
//            Blackwell MLA Decode" -- "The Split-K Imperative": the top-k
//            list is partitioned across blocks, each block writes a partial
//            attention output, a log-sum-exp combine kernel merges them; the
//            heads of a group are processed together with matrix
//            multiply-accumulate instead of one head per thread.
//   [NSPLIT] "The Occupancy Hypothesis: How One Kernel Parameter Unlocked
//            1.8x Decode Speedup on Blackwell" -- "The Broader Context":
//            flash-decode style partial + reduce.
//
// Design for CDNA4 (gfx950, wave64):
//   * workgroup = (token, head block, split); a head block is 16, 32 or 64
//     heads (by head count) in groups of 16, the N width of one MFMA.
//   * the split's rows are gathered in 32-row tiles (x 1152 B) by LDS-DMA
//     (global_load_lds, 16 bytes per lane), straight into LDS tile buffers
//     laid out for the measured bank rules (two: tile n+1 loads while tile n
//     is computed; four in split64_kernel: two tiles in flight).  Every wave of the workgroup reads the same tile,
//     so a row is fetched from HBM once per workgroup.
//   * S^T = KV_tile * Q^T on v_mfma_f32_16x16x32_bf16 (rows on M, heads on N)
//     so that each lane owns one head: the online-softmax max needs two
//     cross-lane exchanges per tile and the running sum none until the end.
//     In 16-head blocks the waves of the group pair up along K (even / odd
//     K-steps) and add their halves through LDS.  64-head blocks over long
//     slices specialise their waves (split64_kernel): four compute scores,
//     each holding Q of two head groups for one half of the tile rows (one
//     operand read feeds two MFMAs), and four hold O and accumulate the PV
//     of the previous tile beside them, one of each kind per SIMD; over
//     short slices every wave does both ("row halves").  The two halves of
//     a head agree on the running max through LDS, and the bf16 weights go
//     to LDS for the PV.
//   * O^T += V^T * P^T on the same MFMA; the softmax output is already laid
//     out as the B operand (no shuffles; in 64-head blocks it is written to
//     LDS in that layout), V^T comes from LDS transpose reads; the waves
//     split the 512 value columns.
//   * masked entries (-1, out of range, past the slice end) load a static
//     all-zero row, so their V contribution is exactly zero, and get a score
//     of -inf.
//   * the partials are merged by a second launch (combine kernels), or, for
//     smla_decode_fused, inside the split launch (fused_combine).
//     split64_kernel stages what it writes at the end (the final bf16 output
//     with NSPLIT 1, else the fp32 partials) in its free tile buffers and
//     stores it 1 KB of a head row per wave instruction.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "smla_internal.h"

namespace smla {

// Native clang vectors throughout: arrays of them stay in registers (HIP's
// uint4/float4 are class types that keep loop-carried arrays on the stack).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowGran = kRow * 2 / 16;          // 72 16-byte granules per row
constexpr int kKSteps = kRow / 32;               // 18 MFMA K-steps over 576 columns

// Row read for masked list entries: all zeros, so masked rows add exactly
// nothing to P*V (and never carry non-finite stale data).
__device__ __attribute__((aligned(16))) u32x4 g_zero_row[kRowGran];

// Reductions over the four lanes l, l^16, l^32, l^48 (one MFMA column: the
// same head in the four lane groups) with the gfx950 permlane swaps: a swap
// of a value with itself leaves each lane holding its own value and the
// partner's, so no LDS round trip is needed.
__device__ __forceinline__ float max4_lanes(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4_lanes(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The value of lane l ^ 8 (DPP row rotate by 8 within each row of 16 lanes).
__device__ __forceinline__ float ror8_lanes(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Row indices are int32, so a row is valid iff 0 <= r < min(kv_rows, 2^31-1);
// one unsigned compare covers both bounds.
__device__ __forceinline__ uint32_t rows32(int64_t kv_rows) {
  return (uint32_t)(kv_rows < 0x7fffffffLL ? kv_rows : 0x7fffffffLL);
}

// Round two values to bf16 (nearest even) and pack them, a in the low half
// (one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Tile layout in LDS: the row is cut into 9 blocks of 8 granules (16 bytes
// each, 128 bytes per block); block kb of all TR rows is stored together,
// 128 bytes per row, and inside a row's 128 bytes granule c sits at
// c ^ h(j), h(j) = j & 6:
//     slot(j, k) = (k / 8) * TR * 8 + j * 8 + ((k % 8) ^ h(j))
// The gfx950 LDS has 64 four-byte banks.  Measured bank behaviour (conflict
// counters on access-pattern probes): an 8-byte read serves 32 consecutive
// lanes per cycle; a 16-byte read serves lanes 0-7 of one 16-lane group
// together with lanes 8-15 of its partner group (g ^ 1).  Hence:
//   * an LDS-DMA wave instruction fills 64 consecutive slots = 8 rows x one
//     full 128-byte line each (coalesced, and a contiguous 1 KiB in LDS), and
//     every lane keeps one fixed tile row for all loads of a tile;
//   * the QK^T operand read (group g: granule x ^ g of rows j = 0..15): the
//     even (odd) rows of each half-group take distinct slots j & 6, and the
//     partner group's rows 8..15 read granule x ^ g ^ 1, the other slot of
//     each pair, so each cycle's 16 reads hit 16 distinct 16-byte slots;
//   * the V^T transpose read (32 lanes: rows 8a..8a+7, two granules, two
//     8-byte halves): among rows of one parity h/2 takes 4 distinct values,
//     so the granule pairs {2c, 2c+1} ^ h land on distinct bank groups.
// All operand addresses are a few per-lane bases plus constants.
__device__ __forceinline__ int hsw(int j) { return j & 6; }

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barriers without the vmcnt(0) a __syncthreads() fence implies.
// The signal fences stop the compiler from moving memory accesses across the
// barrier (they emit no instructions).
__device__ __forceinline__ void barrier_raw() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// LDS writes of this wave complete, then barrier.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
  barrier_raw();
}

typedef short shortx4 __attribute__((ext_vector_type(4)));

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, output
// lane i, element e receives element i % 4 of the 8 bytes addressed by lane
// 4 * e + i / 4 of the same group.
__device__ __forceinline__ shortx4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(__attribute__((address_space(3))) uint8_t*)p);
}


// ---------------------------------------------------------------------------
// Single-launch combine ([SPLITK] "The Split-K Imperative": the partials of
// the NSPLIT slices are merged by log-sum-exp; here the split workgroups do
// it themselves instead of a second launch).  The NSPLIT workgroups of a
// unit (token, head block) share four words in the caller's sync buffer,
// zero between calls: arrive, depart and a 64-bit claim mask.
//   1. Each workgroup writes its partial with device-coherent stores, waits
//      until they have completed, passes a workgroup barrier, and takes an
//      arrival ticket with an agent-scope release (acquire too: the last
//      arriver reads the others' partials).
//   2. A workgroup waits, with a bounded number of polls, until all NSPLIT
//      tickets are out (the last arriver does not wait), takes an
//      agent-scope acquire fence, then claims its own slice of the unit's
//      output (claim bit = its split index) and merges it from the NSPLIT
//      partials.
//   3. The last arriver then claims every slice still unclaimed and merges
//      those too: slices of workgroups that gave up waiting (which happens
//      only if the unit's workgroups are not resident together), so every
//      slice is merged exactly once and no wait is unbounded.
//   4. Each workgroup departs with an agent-scope release; the last to
//      depart takes an acquire fence and clears the four words for the next
//      call.
// A slice is a contiguous range of the unit's (head, 4-column) quads; its
// merge is the combine kernel's arithmetic: a running maximum over the
// splits' LSE, weights exp(LSE_s - max), empty splits (LSE = -inf) weight 0.
// The partials travel between XCDs, whose L2 caches are not coherent with
// each other for ordinary accesses: they are written and read with
// agent-scope atomic accesses (8 bytes each), which the L2 keeps coherent.
// (Ordinary 16-byte stores and loads, ordered only by the ticket's release
// and acquire, measured mixed: batched 69.3 -> 64.9 us per step and tiny
// 8.65 -> 8.07, but long 13.9 -> 15.3 and spec 27.0 -> 30.0; every form
// stays slower than two launches.)
// The ticket's agent-scope release and acquire still cost an L2 writeback
// and invalidate on this target (the compiler's implementation of those
// orderings), part of why the single launch is slower than two.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(float* p, floatx4 v) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  uint64_t* q = (uint64_t*)p;
  __hip_atomic_store(q, (uint64_t)u[0] | ((uint64_t)u[1] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (uint64_t)u[2] | ((uint64_t)u[3] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ floatx4 ld_agent(const float* p) {
  uint64_t* q = (uint64_t*)const_cast<float*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return floatx4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                 __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}
__device__ __forceinline__ float ld_agent1(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge slice c of unit (tok, heads h0 .. h0+hv-1) into out / lse; NT
// threads, LDS scratch of NT * 24 bytes at `lds`.
template <int NT>
__device__ __forceinline__ void merge_slice(const SplitParams& p, int tok, int h0, int hv, int c,
                                            uint8_t* lds) {
  const int tid = threadIdx.x, S = p.nsplit;
  const int Q = hv * (kDV / 4);
  const int qlo = (int)((int64_t)c * Q / S), qhi = (int)((int64_t)(c + 1) * Q / S);
  const int P = qhi - qlo;
  if (P <= 0) return;  // uniform
  // G thread groups share the splits of a quad when the slice is small
  int G = 1;
  while (2 * G * P <= NT && 2 * G <= S) G *= 2;
  const int TPG = NT / G, grp = tid / TPG, lt = tid % TPG;
  const int64_t stride = (int64_t)p.heads * kDV;
  floatx4* acc_s = (floatx4*)lds;
  float* m_s = (float*)(lds + NT * 16);
  float* w_s = m_s + NT;
  for (int base = 0; base < P; base += TPG) {
    const int qi = base + lt;
    const bool act = qi < P;
    const int q = qlo + (act ? qi : P - 1);
    const int h = h0 + q / (kDV / 4), col = (q % (kDV / 4)) * 4;
    const float* lse_in = p.part_lse + (int64_t)tok * S * p.heads + h;
    const float* o_in = p.part_o + ((int64_t)tok * S * p.heads + h) * kDV + col;
    float m = -__builtin_inff(), w = 0.f;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    constexpr int PER = 4;
    for (int s0 = grp; s0 < S; s0 += G * PER) {
      floatx4 v[PER];
      float l[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int sp = s0 + u * G;
        v[u] = sp < S ? ld_agent(o_in + sp * stride) : floatx4{0.f, 0.f, 0.f, 0.f};
        l[u] = sp < S ? ld_agent1(lse_in + (int64_t)sp * p.heads) : -__builtin_inff();
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        if (l[u] == -__builtin_inff()) continue;
        if (l[u] > m) {
          const float r = __builtin_amdgcn_exp2f((m - l[u]) * kLog2e);  // 0 while m = -inf
          acc *= r;
          w *= r;
          m = l[u];
        }
        const float e = __builtin_amdgcn_exp2f((l[u] - m) * kLog2e);
        acc += e * v[u];
        w += e;
      }
    }
    if (G > 1) {  // merge the groups: M = max m_g, weights exp(m_g - M)
      acc_s[tid] = acc;
      m_s[tid] = m;
      w_s[tid] = w;
      __syncthreads();
      if (grp == 0) {
        float M = -__builtin_inff();
        for (int g2 = 0; g2 < G; ++g2) M = fmaxf(M, m_s[lt + g2 * TPG]);
        acc = floatx4{0.f, 0.f, 0.f, 0.f};
        w = 0.f;
        if (M != -__builtin_inff()) {
          for (int g2 = 0; g2 < G; ++g2) {
            const float mg = m_s[lt + g2 * TPG];
            if (mg == -__builtin_inff()) continue;
            const float f = __builtin_amdgcn_exp2f((mg - M) * kLog2e);
            acc += f * acc_s[lt + g2 * TPG];
            w += f * w_s[lt + g2 * TPG];
          }
        }
        m = M;
      }
      __syncthreads();
    }
    if (grp == 0 && act) {
      const bool any = w > 0.f;
      const float inv = any ? 1.f / w : 0.f;
      const int64_t th = (int64_t)tok * p.heads + h;
      *(u32x2*)(p.out + th * kDV + col) =
          u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
      if (col == 0) p.lse[th] = any ? m + __logf(w) : -__builtin_inff();
    }
  }
}

// Steps 1-4 above for split `split` of unit `unit`; lds: NT * 24 bytes of
// merge scratch, bc: 16 bytes for broadcasts (both free LDS).
template <int NT>
__device__ __forceinline__ void fused_combine(const SplitParams& p, int unit, int tok, int h0, int hv,
                                              int split, uint8_t* lds, uint32_t* bc) {
  const int tid = threadIdx.x;
  const uint32_t S = (uint32_t)p.nsplit;
  uint32_t* sy = p.sync + 4 * (int64_t)unit;  // arrive, depart, claim (2 words)
  // 1. every wave's partial stores have completed before the ticket is taken
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0) {
    // release: this workgroup's partial stores (every wave's, ordered before
    // this by the barrier) happen before the ticket; acquire: the last
    // arriver's loads of the others' partials happen after their tickets
    const uint32_t t = __hip_atomic_fetch_add(sy, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    bool ready = t == S - 1;
    for (int i = 0; !ready && i < p.merge_polls; ++i) {
      __builtin_amdgcn_s_sleep(4);
      ready = __hip_atomic_load(sy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= S;
    }
    // the poll saw every ticket: the partials' stores happen before the
    // merge's loads (the workgroup barrier below extends this to every wave)
    if (ready && t != S - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t own = 0;
    if (ready) {
      const uint32_t bit = 1u << (split & 31);
      own = (__hip_atomic_fetch_or(sy + 2 + (split >> 5), bit, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) & bit) == 0;
    }
    bc[0] = own;
    bc[1] = t == S - 1;
  }
  __syncthreads();
  const bool own = bc[0] != 0, last = bc[1] != 0;
  // 2. this workgroup's own slice
  if (own) merge_slice<NT>(p, tok, h0, hv, split, lds);
  // 3. the last arriver takes every slice nobody has claimed yet
  if (last) {
    if (tid == 0) {
      const uint32_t all0 = S >= 32 ? 0xffffffffu : (1u << S) - 1;
      const uint32_t all1 = S >= 64 ? 0xffffffffu : S > 32 ? (1u << (S - 32)) - 1 : 0u;
      const uint32_t o0 =
          __hip_atomic_fetch_or(sy + 2, all0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t o1 = all1 ? __hip_atomic_fetch_or(sy + 3, all1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)
                               : 0u;
      bc[2] = all0 & ~o0;
      bc[3] = all1 & ~o1;
    }
    __syncthreads();
    uint64_t todo = (uint64_t)bc[2] | ((uint64_t)bc[3] << 32);
    while (todo) {  // uniform
      merge_slice<NT>(p, tok, h0, hv, __builtin_ctzll(todo), lds);
      todo &= todo - 1;
    }
  }
  // 4. depart; the last one out clears the words (every other workgroup's
  // accesses to them happen before its release, so none reads them after
  // the clear; the next call is ordered after this one)
  if (tid == 0 &&
      __hip_atomic_fetch_add(sy + 1, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == S - 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) __hip_atomic_store(sy + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Split kernel.  HG head groups of 16 per workgroup; each wave owns GPW
// head groups and one of NCS column slices of the 512 value columns; the PV
// work and the O accumulators are divided among the NCS waves that share
// head groups.  KS is the number of waves that share a head group's QK^T
// along K:
//   KS = 1: every wave computes all of QK^T for its head groups;
//   KS = 2: the K-steps of one parity, the two parities adding their halves
//           through LDS, after which both waves hold all of S;
//   KS = 1 with GPW = 4 (HG = 4, NCS = 8: "row halves", eight waves, two
//           per SIMD): wave w = (kq, rh) holds Q of head group kq for all 18
//           K-steps and computes the scores of tile rows 16 rh .. 16 rh + 15
//           for those 16 heads, with no exchange of partial scores; a head's
//           rows are split over the two row halves, whose waves agree on the
//           running max through LDS.  Each wave holds O of all 64 heads for
//           one eighth of the value columns, so each V^T read feeds four
//           MFMAs.  Per tile: two workgroup barriers in the usual case (tile
//           landed, weights written) and no exchange of partial scores.
//           Used over slices of fewer than kDeepTiles tiles; longer slices
//           take split64_kernel (role-specialised waves, below).
// TR rows per tile, two tile buffers: tile n+1 loads while tile n is
// computed.
// ---------------------------------------------------------------------------
// The dispatcher hands workgroup i to XCD i % kXcds (round robin over the
// eight XCDs, each with its own L2).  This renumbering gives every XCD a
// contiguous range of logical ids, so that neighbouring logical workgroups,
// which share input rows, also share an L2.  It is a bijection for any grid
// size, so correctness does not depend on the dispatch order.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  const int xcd = bid % kXcds, k = bid / kXcds;
  const int per = n / kXcds, rem = n % kXcds;
  return xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
}

// The L LDS-DMA loads of one lane for one tile: load `it` copies the 16 bytes
// at src + 128*STEP*it to lds + 16*NT*it + 16*lane.  The builtin's immediate
// offset moves the global and the LDS address alike, so every load takes its
// global offset as that immediate and the LDS pointer is moved back by the
// same amount: all loads of the tile then read one address register, rather
// than one temporary each (a register that a load in flight reads must not be
// reused until the load completes, which would force waits on every load).
//
// The LDS destination (wave-uniform) is passed through an empty asm
// statement in a scalar register, so the compiler no longer knows which
// buffer a load writes, and M0 is set from it directly (held in vector
// registers it took one register per load and buffer, and a readfirstlane
// before every load).  Its own wait
// insertion would otherwise guard reads of one buffer against loads in flight
// into another, and at some control-flow joins it loses track of which is
// which and waits for every outstanding load, draining the pipeline.  The
// order of loads and reads is kept by hand instead: a tile is read only after
// the loading waves have waited for its loads (vmcnt) and the workgroup has
// passed a barrier, and the opaque store still keeps the compiler from moving
// LDS accesses across the load.
template <int NT, int STEP, int IT>
__device__ __forceinline__ void dma_one(const u32x4* src, uint8_t* lds) {
  constexpr int off = 128 * STEP * IT;
  static_assert(off < 4096, "immediate offset range");
  auto* dst = (__attribute__((address_space(3))) uint8_t*)(lds + 16 * NT * IT - off);
  asm volatile("" : "+s"(dst));
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, off, 0);
}
template <int NT, int STEP, int... IT>
__device__ __forceinline__ void dma_tile(const u32x4* src, uint8_t* lds,
                                         std::integer_sequence<int, IT...>) {
  (dma_one<NT, STEP, IT>(src, lds), ...);
}

// Keeps a value in its registers up to this point.
__device__ __forceinline__ void keep_live(uint64_t v) { asm volatile("" ::"v"(v)); }

// Kernel arguments.  What a workgroup needs before its first memory access
// (the list, q and cache addresses and the sizes that locate its slice)
// comes first, as separate scalar arguments: the library is built with
// kernel-argument preloading, so the dispatcher places those 14 dwords in
// SGPRs before the waves start and the first list load waits on no read of
// the argument segment (0.3 us, a cold scalar load, at the head of every
// workgroup's chain of dependent accesses).  The rest of SplitParams travels
// in a struct, which is never preloaded.
struct SplitTail {
  const int32_t* table;
  const int32_t* ctx;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  uint32_t* sync;
  int src, max_pages, page_size, merge_polls;
  float scale_log2;
};

template <int HG, int NCS, int GPW, int TR, int KS, int SRC>
__global__ __launch_bounds__(64 * (HG / GPW) * NCS)
__attribute__((amdgpu_waves_per_eu(2)))  // every class: two waves per SIMD, at most 256 registers
void split_kernel(const int32_t* a_idx, const uint16_t* a_q, const uint16_t* a_kv, int64_t a_kv_rows,
                  int a_topk, int a_per_split, int a_nsplit, int a_heads, int a_tokens, int a_q_len,
                  SplitTail tl) {
  SplitParams p;
  p.idx = a_idx;
  p.q = a_q;
  p.kv = a_kv;
  p.kv_rows = a_kv_rows;
  p.topk = a_topk;
  p.per_split = a_per_split;
  p.nsplit = a_nsplit;
  p.heads = a_heads;
  p.tokens = a_tokens;
  p.q_len = a_q_len;
  p.table = tl.table;
  p.ctx = tl.ctx;
  p.out = tl.out;
  p.lse = tl.lse;
  p.part_o = tl.part_o;
  p.part_lse = tl.part_lse;
  p.sync = tl.sync;
  p.src = tl.src;
  p.max_pages = tl.max_pages;
  p.page_size = tl.page_size;
  p.merge_polls = tl.merge_polls;
  p.scale_log2 = tl.scale_log2;
  static_assert(HG % GPW == 0, "whole head groups per wave");
  constexpr bool KSPLIT = KS == 2;          // K-split pairs
  constexpr bool KRH = KS == 1 && GPW == 4;  // row halves: one head group's scores a wave
  static_assert(KS == 1 || KS == 2, "K-split factor");
  static_assert(!KSPLIT || NCS % 2 == 0, "K-split pairs waves of opposite parity");
  static_assert(!KRH || (HG == 4 && NCS == 8 && TR == 32), "row-half shape: 8 waves x 2 row blocks");
  constexpr int NT = 64 * (HG / GPW) * NCS;
  // waves that issue the tile loads: all of them, or half of them when the
  // tile's wave loads do not split evenly (36 per 32-row tile: not over 8)
  constexpr int DW = (TR * kRowGran) % NT == 0 ? NT / 64 : NT / 128;
  constexpr int NTD = 64 * DW;
  constexpr int RB = TR / 16;                 // 16-row blocks per tile (QK^T M blocks)
  constexpr int KP = TR / 32;                 // 32-row K-steps of PV per tile
  constexpr int L = TR * kRowGran / NTD;      // DMA instructions per loading thread per tile
  constexpr int kTileBytes = TR * kRow * 2;
  constexpr int CB = (kDV / 16) / NCS;        // 16-column blocks of O per wave
  // QK^T K-steps per wave: all 18, with K-split pairs the 9 of one parity
  constexpr int KSW = KSPLIT ? kKSteps / 2 : kKSteps;
  static_assert(TR * kRowGran % NTD == 0, "tile must split evenly over the loading threads");
  static_assert(TR % 32 == 0, "tile shape");
  // list entries staged at a time (the K-split 16-head workgroup stages
  // 1024 so that two of them fit a CU's LDS)
  constexpr int LCAP = split_list_cap(NCS, KS);
  // K-split: one slot of partial scores per (head group, K parity); the
  // waves of a head group with cs < 2 write them, every wave reads the other
  // parity's slot
  constexpr int kXsSlots = KSPLIT ? (NT / 64 / NCS) * 2 : 1;

  // One __shared__ object per buffer: each access below names its buffer at
  // compile time, which lets the compiler see that a read of one buffer does
  // not alias the LDS-DMA writes in flight into another (otherwise it waits
  // for every outstanding load before each LDS read).
  __shared__ __attribute__((aligned(16))) uint8_t tb0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[kTileBytes];
  __shared__ __attribute__((aligned(16))) int list_s[LCAP];
  // K-split pairs: partial S^T per (head group, parity) slot: [slot][gi][rb][lane]
  __shared__ __attribute__((aligned(16))) floatx4 xs[KSPLIT ? kXsSlots * GPW * RB * 64 : 1];
  // row halves: the bf16 weights P^T as PV B operands, [head group][g][head][8]
  // (each row half writing its 4 slots), and the rescale factors per head
  __shared__ __attribute__((aligned(16))) u32x4 ps[KRH ? HG * 64 : 1];
  __shared__ float alpha_s[KRH ? HG * 16 : 1];
  // row halves: each wave's per-head maximum over its row half and its
  // share of the final sums, [wave][head]; whether a wave's heads need
  // their running max moved in this tile, [wave]
  __shared__ float rmax_s[KRH ? (NT / 64) * 16 : 1];
  __shared__ float rsum_s[KRH ? (NT / 64) * 16 : 1];
  __shared__ __attribute__((aligned(16))) int rflag_s[KRH ? NT / 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;    // lane group: selects the K slots of MFMA operands
  const int l16 = lane & 15;  // MFMA row / column within a 16-wide block
  const int hg0 = (wave / NCS) * GPW;  // first head group of this wave
  const int cs = wave % NCS;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // row halves: wave = (kq, rh) -- scores of head group kq, tile rows
  // 16 rh .. +15; wave (kq, 1 - rh) holds the group's other rows
  const int kq = wave_u & 3, rh = wave_u >> 2;

  // workgroup -> (token, split, head block) in the XCD-contiguous numbering.
  // Over slices of at least 8 tiles the head blocks of a (token, split) are
  // numbered fastest: they gather the same rows and, as neighbours on one
  // XCD, the second block's gathers hit that L2 (72 heads over 65536
  // positions: 36.2 -> 35.2 us); over shorter slices the splits are fastest
  // (the same at 16384 positions: 21.5 against 22.9 us).  Either way a
  // token's workgroups are contiguous, so its q rows meet in one L2.
  const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
  constexpr int kHeadsPerBlock = HG * 16;
  const int hblocks = (p.heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const bool hb_fast = p.per_split >= 8 * TR;  // uniform
  const int hblk = hb_fast ? wg % hblocks : (wg / p.nsplit) % hblocks;
  const int split = hb_fast ? (wg / hblocks) % p.nsplit : wg % p.nsplit;
  const int tok = wg / hblocks / p.nsplit;
  const int unit = tok * hblocks + hblk;  // (token, head block): the splits merged together

  // this lane's head in each of the wave's head groups
  int h[GPW];
  bool h_ok[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    h[gi] = hblk * kHeadsPerBlock + (hg0 + gi) * 16 + l16;
    h_ok[gi] = h[gi] < p.heads;
  }

  // this split's slice of the list; the first chunk's entries are loaded
  // before q, so that the tile loads can start as soon as the list is in
  const int lo = min(split * p.per_split, p.topk);
  const int hi = min(lo + p.per_split, p.topk);
  const int32_t* idx_row = p.idx ? p.idx + (int64_t)tok * p.topk : nullptr;
  // the row of list entry e, or -1: straight from the list, or a position of
  // the token's sequence mapped through its page table (row = page id *
  // page_size + offset in the page); a position outside the table, a missing
  // page or a row outside the cache is masked like -1
  // (SRC, the row source, is a template argument: a plain list of rows
  // compiles to nothing but the list load)
  const int seq = SRC == kSrcRows ? 0 : tok / p.q_len;
  int ctx_seq = 0;
  if (SRC == kSrcDense) ctx_seq = p.ctx[seq];
  const int32_t* tab = SRC != kSrcRows && p.table ? p.table + (int64_t)seq * p.max_pages : nullptr;
  auto entry = [&](int e) __attribute__((always_inline)) -> int32_t {
    if constexpr (SRC == kSrcRows) return idx_row[e];
    const int32_t pos = SRC == kSrcDense ? (e < ctx_seq ? e : -1) : idx_row[e];
    if (!tab || pos < 0) return pos;
    const int pg_i = pos / p.page_size;
    if (pg_i >= p.max_pages) return -1;
    const int32_t pg = tab[pg_i];
    if (pg < 0) return -1;
    const int64_t row = (int64_t)pg * p.page_size + (pos - pg_i * p.page_size);
    return row < p.kv_rows && row <= 0x7fffffff ? (int32_t)row : -1;
  };
  // 64-head blocks with positions: the sequence's page-table slice (up to
  // kTabStage pages) is loaded with the positions, not after them, and staged
  // in LDS (in the score-exchange buffer, idle whenever the list is staged),
  // so that mapping a position is an LDS read instead of a second HBM round
  // trip behind the position's load.  (The 16- and 32-head workgroups fill
  // exactly half a CU's LDS each, so they keep the direct lookup.)
  constexpr int kTabStage = 512;
  constexpr int TI = (kTabStage + NT - 1) / NT;
  const bool tab_lds =
      SRC == kSrcPositions && KRH && tab != nullptr && p.max_pages <= kTabStage;
  // the table's LDS stage: the weights' buffer, idle whenever the list is staged
  int32_t* const tab_stage = (int32_t*)ps;
  int tv[TI];
  if (tab_lds) {
#pragma unroll
    for (int u = 0; u < TI; ++u) {
      const int i = u * NT + tid;
      tv[u] = i < p.max_pages ? tab[i] : -1;
    }
  }
  constexpr int LI = LCAP / NT;
  int lv[LI];
  auto load_list = [&](int clo, int n_ent) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int e = clo + min(u * NT + tid, n_ent - 1);
      // a staged table: the raw position now, its row once the table is in LDS
      lv[u] = tab_lds ? idx_row[e] : entry(e);
    }
  };
  if (lo < hi) load_list(lo, min(hi - lo, LCAP));

  // Q^T as the B operand of S^T = KV * Q^T: lane (g, l16) holds
  // q[h][32*ks + 8*g .. +7] for each of the wave's K-steps ks (zeros for
  // padding heads, read from the zero row: 72 granules cover 18 K-steps x 4
  // groups): all 18, with K-split pairs 2k + (cs & 1)
  // row halves: Q of head group kq, all 18 K-steps
  bf16x8 qf[KRH ? kKSteps : 1];
  if constexpr (KRH) {
    const int hq_ = hblk * kHeadsPerBlock + kq * 16 + l16;
    const u32x4* qrow = hq_ < p.heads ? (const u32x4*)(p.q + ((int64_t)tok * p.heads + hq_) * kRow) + g
                                      : g_zero_row + g;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) qf[k] = __builtin_bit_cast(bf16x8, qrow[4 * k]);
  }
  bf16x8 qb[KRH ? 1 : GPW][KRH ? 1 : KSW];
#pragma unroll
  for (int gi = 0; gi < (KRH ? 0 : GPW); ++gi) {
    const u32x4* qrow = h_ok[gi]
                            ? (const u32x4*)(p.q + ((int64_t)tok * p.heads + h[gi]) * kRow) + g
                            : g_zero_row + g;
    if (KSPLIT) qrow += 4 * (cs & 1);
#pragma unroll
    for (int k = 0; k < KSW; ++k) {
      qb[gi][k] = __builtin_bit_cast(bf16x8, qrow[k * 4 * (KSPLIT ? 2 : 1)]);
    }
  }

  // QK^T operand: row 16*rb + l16, granule 4*ks + g, i.e. block ks/2 and
  // in-block granule (4*(ks&1) + g) ^ h(l16) = (g ^ h) ^ 4*(ks&1).
  const int hq = hsw(l16);
  const int qk_even = l16 * 128 + (g ^ hq) * 16;
  const int qk_odd = l16 * 128 + ((g ^ hq) ^ 4) * 16;
  // K-split: K-step 2k + par is block k, in-block half par (par = cs & 1)
  const int qk_half = (cs & 1) ? qk_odd : qk_even;
  // row halves: rows 16 rh + l16, K-steps of either parity
  const int qk_rh_e = qk_even + rh * 16 * 128, qk_rh_o = qk_odd + rh * 16 * 128;
  // V^T transpose read: source lane (e, s') of group g reads row 4g + e
  // (+16 for slots 4-7, +32 per PV K-step), columns 16*cb + 4s' .. +3 =
  // granule 2cb + b0 (b0 = s' >> 1) at byte 8*b1 (b1 = s' & 1); in-block
  // granule (2*(cb%4) + b0) ^ h(4g + e) (rows +16 and +32 share h).
  const int tr_e = l16 >> 2, tr_b0 = (l16 >> 1) & 1, tr_b1 = l16 & 1;
  const int tr_h = hsw(4 * g + tr_e);
  int pv_base[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)  // (this wave's columns start at block 4*CB*cs / 4)
    pv_base[c] = (4 * g + tr_e) * 128 + ((2 * c + tr_b0) ^ tr_h) * 16 + 8 * tr_b1 +
                 cs * (CB / 4) * TR * 128;

  // DMA: wave instruction it fills slots 64*m .. 64*m + 63, m = it*WPB + wave
  // (WPB = DW, the loading waves): block kb = m / RG, rows 8*(m % RG) + lane/8
  // (RG = TR/8 row groups per block), in-block slot lane % 8, which holds
  // granule (lane % 8) ^ h(row).  If RG >= WPB a lane cycles through
  // DP = RG / WPB rows (d = it % DP, kb = it / DP); otherwise it keeps one
  // row and kb = it * (WPB / RG) + wave / RG.
  constexpr int WPB = DW;
  constexpr int RG = TR / 8;
  static_assert(RG % WPB == 0 || WPB % RG == 0, "row period");
  constexpr int DP = RG > WPB ? RG / WPB : 1;
  int dma_row[DP], dma_gran[DP];
#pragma unroll
  for (int d = 0; d < DP; ++d) {
    const int m = d * WPB + wave;
    dma_row[d] = 8 * (m % RG) + (lane >> 3);
    dma_gran[d] = (lane & 7) ^ hsw(dma_row[d]);
    if (DP == 1) dma_gran[d] += 8 * (wave / RG);
  }

  float m_run[GPW], l_run[GPW];  // running max (log2 units) and this lane's share of the sum
  floatx4 oacc[GPW][CB];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    m_run[gi] = -__builtin_inff();
    l_run[gi] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[gi][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // LDS-DMA loads of tile t (list entries t*TR.. of the staged chunk); a
  // masked entry or one past the chunk loads the zero row.  The L loads of a
  // lane share one 64-bit address (see dma_tile), returned so that the caller
  // keeps it live until the loads are known to be complete.
  static_assert(DP == 1, "one row per lane per tile");
  auto issue = [&](uint8_t* buf, int t, int ntiles) __attribute__((always_inline)) -> uint64_t {
    // a masked entry loads the zero row (every call has t < ntiles)
    const int32_t r = t < ntiles ? list_s[min(t * TR + dma_row[0], LCAP - 1)] : -1;
    const uintptr_t hit = (uintptr_t)(p.kv + (int64_t)r * kRow);
    const u32x4* src = (const u32x4*)(r >= 0 ? hit : (uintptr_t)g_zero_row) + dma_gran[0];
    if (wave < DW)
      dma_tile<NTD, WPB / RG>(src, buf + wave_u * 64 * 16, std::make_integer_sequence<int, L>{});
    return (uint64_t)(uintptr_t)src;
  };

  // Consume tile t held in T, row halves.
  auto compute_rh = [&](const uint8_t* T, int t) __attribute__((always_inline)) {
    if constexpr (KRH) {
      // validity of this lane's rows, read ahead of the QK^T
      const i32x4 r4 = *(const i32x4*)(list_s + t * TR + 16 * rh + 4 * g);
      // ---- S^T of rows 16 rh .. +15, head group kq, all 18 K-steps (two
      // accumulation chains).  The operand reads run D ahead of their MFMAs,
      // in this order (scheduling barriers): left to itself the compiler kept
      // two to four in flight, and the phase waited on LDS latency (8 ahead:
      // 64 x 128 heads 102.5 -> 100 us per launch)
      floatx4 a2[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
      constexpr int D = 8;
      bf16x8 op[D];
#pragma unroll
      for (int k = 0; k < D; ++k)
        op[k] = *(const bf16x8*)(T + ((k & 1) ? qk_rh_o : qk_rh_e) + (k >> 1) * TR * 128);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) {
        a2[k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[k % D], qf[k], a2[k & 1], 0, 0, 0);
        if (k + D < kKSteps)
          op[k % D] = *(const bf16x8*)(T + (((k + D) & 1) ? qk_rh_o : qk_rh_e) + ((k + D) >> 1) * TR * 128);
        __builtin_amdgcn_sched_barrier(0);
      }
      const floatx4 sv = a2[0] + a2[1];

      // ---- online softmax over this row half; a head's two row halves
      // must use the same running max, so the weights are computed against
      // the current one and redone, in every wave, in the rare tile where
      // some head's maximum grows by more than 2^8 (the first tile always)
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = r4[i] >= 0 ? sv[i] * p.scale_log2 : -__builtin_inff();
      const float mxh = max4_lanes(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      float pw[4];
      // weights against the running max, written as the rows 16 rh + 4 g + i
      // = K slots 4 rh + i of the PV B operand of lane group g, head l16
      auto weights = [&]() __attribute__((always_inline)) {
        const float m_use = m_run[0] == -__builtin_inff() ? 0.f : m_run[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
        *(u32x2*)((uint8_t*)ps + (kq * 64 + lane) * 16 + 8 * rh) =
            u32x2{pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3])};
      };
      weights();
      const int need_w = __any(mxh > m_run[0] + kRescaleLog2);
      if (lane == 0) rflag_s[wave_u] = need_w;
      if (g == 0) rmax_s[wave_u * 16 + l16] = mxh;
      barrier_lds();
      // the flags, the weights of all four head groups and this wave's V^T
      // operands in one LDS round trip (the weights are read again if the
      // rare path below rewrites them)
      const i32x4 fa = *(const i32x4*)rflag_s;
      const i32x4 fb = *(const i32x4*)(rflag_s + 4);
      bf16x8 pq[HG];
#pragma unroll
      for (int gi = 0; gi < HG; ++gi) pq[gi] = __builtin_bit_cast(bf16x8, ps[gi * 64 + lane]);
      bf16x8 vt[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int off = pv_base[cb & 3] + (cb >> 2) * TR * 128;
        const shortx4 v2[2] = {lds_tr16(T + off), lds_tr16(T + off + 16 * 128)};
        vt[cb] = __builtin_bit_cast(bf16x8, v2);
      }
      if ((fa[0] | fa[1] | fa[2] | fa[3]) | (fb[0] | fb[1] | fb[2] | fb[3])) {  // the same in every wave
        // both row halves of a head take the same decision from the same
        // two maxima: move the running max when the tile's exceeds it by
        // more than 2^8 (alpha exactly 1 otherwise)
        const float mt = fmaxf(mxh, rmax_s[(wave_u ^ 4) * 16 + l16]);
        float alpha = 1.f;
        if (mt > m_run[0] + kRescaleLog2) {
          const float m_new = fmaxf(m_run[0], mt);
          alpha = __builtin_amdgcn_exp2f(m_run[0] - m_new);  // 0 while m_run = -inf
          l_run[0] *= alpha;
          m_run[0] = m_new;
        }
        if (rh == 0 && g == 0) alpha_s[kq * 16 + l16] = alpha;
        weights();
        barrier_lds();
        float al[HG];
        bool scale = false;
#pragma unroll
        for (int gi = 0; gi < HG; ++gi) {
          al[gi] = alpha_s[gi * 16 + l16];
          scale |= al[gi] != 1.f;
          pq[gi] = __builtin_bit_cast(bf16x8, ps[gi * 64 + lane]);
        }
        if (__any(scale)) {
#pragma unroll
          for (int gi = 0; gi < HG; ++gi)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) oacc[gi][cb] *= al[gi];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[0] += pw[i];

      // ---- O^T += V^T * P^T over this wave's eighth of the columns, all
      // four head groups (each V^T operand feeds four MFMAs)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int gi = 0; gi < HG; ++gi)
          oacc[gi][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[cb], pq[gi], oacc[gi][cb], 0, 0, 0);
    }
  };

  // Consume tile t held in T.
  auto compute = [&](const uint8_t* T, int t) __attribute__((always_inline)) {
   if constexpr (!KRH) {
    // ---- S^T = KV_tile * Q^T: RB 16-row blocks, 18 K-steps of 32 columns
    floatx4 sacc[GPW][RB];
    if constexpr (KSPLIT) {
      // this wave's 9 K-steps (parity cs): all operand reads first, then the
      // MFMAs (each read feeds the wave's GPW head groups) in two chains per
      // row block and head group
      bf16x8 av[KSW][RB];
#pragma unroll
      for (int k = 0; k < KSW; ++k)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          av[k][rb] = *(const bf16x8*)(T + qk_half + k * TR * 128 + rb * 16 * 128);
      floatx4 acc2[2][GPW][RB];
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc2[0][gi][rb] = acc2[1][gi][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSW; ++k)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi)
            acc2[k & 1][gi][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                av[k][rb], qb[gi][k], acc2[k & 1][gi][rb], 0, 0, 0);
      // exchange the half sums with the partner wave (same heads, other
      // parity); own + partner is the same sum in both waves (addition
      // commutes), so both hold bitwise the same scores
      const int par = cs & 1;
      const int my_slot = (wave / NCS) * 2 + par, other_slot = my_slot ^ 1;
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          sacc[gi][rb] = acc2[0][gi][rb] + acc2[1][gi][rb];
          if (cs < 2) xs[((my_slot * GPW + gi) * RB + rb) * 64 + lane] = sacc[gi][rb];
        }
      barrier_lds();
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[gi][rb] += xs[((other_slot * GPW + gi) * RB + rb) * 64 + lane];
    } else {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[gi][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int off = ((ks & 1) ? qk_odd : qk_even) + (ks >> 1) * TR * 128 + rb * 16 * 128;
          const bf16x8 a = *(const bf16x8*)(T + off);
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi)
            sacc[gi][rb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[gi][ks], sacc[gi][rb], 0, 0, 0);
        }
      }
    }

    // ---- online softmax; lane holds rows j = 16*rb + 4*g + i of head h
    // validity of the rows this lane holds (shared by the wave's head groups)
    bool ok[4 * RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int e0 = t * TR + rb * 16 + 4 * g;
      const i32x4 r4 = *(const i32x4*)(list_s + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) ok[rb * 4 + i] = r4[i] >= 0;
    }
    float s[GPW][4 * RB];
    float tmax[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[gi][rb * 4 + i] = ok[rb * 4 + i] ? sacc[gi][rb][i] * p.scale_log2 : -__builtin_inff();
      float mx = s[gi][0];
#pragma unroll
      for (int i = 1; i < 4 * RB; ++i) mx = fmaxf(mx, s[gi][i]);
      tmax[gi] = max4_lanes(mx);
    }
    // Lazy rescaling: the running max only moves when a head's tile max
    // exceeds it by more than 2^8 (in base 2), so O and l are rescaled
    // rarely; meanwhile the weights exp2(s - m) stay below 2^8.
    bool grow = false;
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) grow |= tmax[gi] > m_run[gi] + kRescaleLog2;
    if (__any(grow)) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const float m_new = fmaxf(m_run[gi], tmax[gi]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[gi] - m_new);  // 0 while m_run = -inf
        l_run[gi] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[gi][cb] *= alpha;
        m_run[gi] = m_new;
      }
    }

    // P^T as the B operand of K-step kp: K slot s <-> tile row
    // 32*kp + 16*(s/4) + 4*g + s%4, i.e. the rows this lane already holds.
    bf16x8 pb[GPW][KP];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const float m_use = m_run[gi] == -__builtin_inff() ? 0.f : m_run[gi];
      float pv[4 * RB];
#pragma unroll
      for (int i = 0; i < 4 * RB; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(s[gi][i] - m_use);
        l_run[gi] += pv[i];
      }
#pragma unroll
      for (int kp = 0; kp < KP; ++kp) {
        const float* v = pv + 8 * kp;
        const u32x4 pw = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        pb[gi][kp] = __builtin_bit_cast(bf16x8, pw);
      }
    }

    // ---- O^T += V^T * P^T; the A operand (V^T, tile rows on K) comes from
    // two transpose reads: slots 0-3 = rows 4g..4g+3, slots 4-7 = rows
    // 16+4g..16+4g+3 of the K-step, column l16 of the 16-column block.
    if constexpr (KSPLIT) {
      // all transpose reads of the wave's column blocks first, then the MFMAs
      shortx4 vt[CB][KP][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
          const int off = pv_base[cb & 3] + (cb >> 2) * TR * 128 + 32 * kp * 128;
          vt[cb][kp][0] = lds_tr16(T + off);
          vt[cb][kp][1] = lds_tr16(T + off + 16 * 128);
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, vt[cb][kp]);
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi)
            oacc[gi][cb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[gi][kp], oacc[gi][cb], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
          const int off = pv_base[cb & 3] + (cb >> 2) * TR * 128 + 32 * kp * 128;
          const shortx4 v_lo = lds_tr16(T + off);
          const shortx4 v_hi = lds_tr16(T + off + 16 * 128);
          const shortx4 a8[2] = {v_lo, v_hi};
          const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi)
            oacc[gi][cb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[gi][kp], oacc[gi][cb], 0, 0, 0);
        }
      }
    }
   }
  };

  // Software pipeline over the tiles of each staged chunk of the list.
  // stage a chunk of the list in one memory round trip: all loads (issued
  // earlier), then all stores; the first chunk's loads went out before q.
  // Every slot is written, and any entry that is masked (-1, out of range,
  // past the chunk) is stored as -1, so later reads test only r >= 0.
  const uint32_t kv32 = rows32(p.kv_rows);
  auto store_list = [&](int n_ent) __attribute__((always_inline)) {
    if (tab_lds) {  // uniform: stage the table, then map the positions through it
      int32_t* ts = tab_stage;
#pragma unroll
      for (int u = 0; u < TI; ++u) {
        const int i = u * NT + tid;
        if (i < kTabStage) ts[i] = tv[u];
      }
      barrier_lds();
#pragma unroll
      for (int u = 0; u < LI; ++u) {
        const int32_t pos = lv[u];
        const int pg_i = pos / p.page_size;
        const bool in_tab = pos >= 0 && pg_i < p.max_pages;
        const int32_t pg_s = ts[in_tab ? pg_i : 0];  // every read in bounds
        const int32_t pg = in_tab ? pg_s : -1;
        const int64_t row = (int64_t)pg * p.page_size + (pos - pg_i * p.page_size);
        lv[u] = pg >= 0 && row < p.kv_rows && row <= 0x7fffffff ? (int32_t)row : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int e = u * NT + tid;
      list_s[e] = (e < n_ent && (uint32_t)lv[u] < kv32) ? lv[u] : -1;
    }
    barrier_lds();
  };
  if (lo < hi) store_list(min(hi - lo, LCAP));
  auto buf = [&](auto bconst) __attribute__((always_inline)) -> uint8_t* {
    constexpr int b = decltype(bconst)::value;
    return b == 0 ? tb0 : tb1;
  };
  for (int clo = lo; clo < hi; clo += LCAP) {
    const int n_ent = min(hi - clo, LCAP);
    const int ntiles = (n_ent + TR - 1) / TR;
    // two buffers: tile n+1 loads while tile n is computed (the refill past
    // the last tile is skipped)
    uint64_t addr[2] = {};  // per buffer: the address its last loads read
    addr[0] = issue(tb0, 0, ntiles);
    // one pipeline step on buffer b (a compile-time constant)
    auto step = [&](auto bconst, int n) __attribute__((always_inline)) {
      constexpr int b = decltype(bconst)::value, bn = b ^ 1;
      wait_vmcnt<0>();  // tile n landed
      keep_live(addr[b]);  // its loads are done: their address may go
      barrier_raw();
      // refill the buffer every wave finished with in the previous step
      if (n + 1 < ntiles) addr[bn] = issue(buf(std::integral_constant<int, bn>{}), n + 1, ntiles);
      if constexpr (KRH)
        compute_rh(buf(bconst), n);
      else
        compute(buf(bconst), n);
    };
    for (int n0 = 0; n0 < ntiles; n0 += 2) {
      step(std::integral_constant<int, 0>{}, n0);
      if (n0 + 1 < ntiles) step(std::integral_constant<int, 1>{}, n0 + 1);
    }
    keep_live(addr[0]);
    keep_live(addr[1]);
    barrier_raw();  // list_s and the buffers are reused by the next chunk
    const int nxt = clo + LCAP;
    if (nxt < hi) {
      load_list(nxt, min(hi - nxt, LCAP));
      store_list(min(hi - nxt, LCAP));
    }
  }

  // ---- epilogue: O / l and LSE = (m * ln 2) + ln l.  Per head group: 1 / l
  // for this lane's head, and the LSE of head lse_h if this lane writes it
  float inv[GPW], lse_v[GPW];
  int lse_h[GPW];
  bool lse_w[GPW];
  if constexpr (KRH) {
    // a row half's share of its owned head's sum (its four lane groups),
    // then the two halves added in the same order by every wave, which
    // needs all four groups' sums for its eighth of O's columns
    const float lh = sum4_lanes(l_run[0]);
    if (g == 0) rsum_s[wave_u * 16 + l16] = lh;
    barrier_lds();
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      // owners of group gi: waves gi (rows 0-15) and gi + 4 (rows 16-31)
      const float l = rsum_s[gi * 16 + l16] + rsum_s[(gi + 4) * 16 + l16];
      inv[gi] = l > 0.f ? 1.f / l : 0.f;
      lse_v[gi] = l > 0.f ? m_run[0] * kLn2 + __logf(l) : -__builtin_inff();
      lse_h[gi] = h[gi];
      lse_w[gi] = gi == kq && rh == 0 && g == 0;
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const float l_tot = sum4_lanes(l_run[gi]);
      const bool any = l_tot > 0.f;
      inv[gi] = any ? 1.f / l_tot : 0.f;
      lse_v[gi] = any ? m_run[gi] * kLn2 + __logf(l_tot) : -__builtin_inff();
      lse_h[gi] = h[gi];
      lse_w[gi] = g == 0 && cs == 0;
    }
  }
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    if (lse_w[gi] && lse_h[gi] < p.heads) {
      const int64_t th = (int64_t)tok * p.heads + lse_h[gi];
      const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + lse_h[gi];
      if (p.nsplit == 1)
        p.lse[th] = lse_v[gi];
      else if (p.sync)  // read by other workgroups in this launch: coherent store
        __hip_atomic_store(p.part_lse + slot, lse_v[gi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        p.part_lse[slot] = lse_v[gi];
    }
    if (!h_ok[gi]) continue;
    const int64_t th = (int64_t)tok * p.heads + h[gi];
    if (p.nsplit == 1) {
      uint16_t* orow = p.out + th * kDV;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c0 = (cs * CB + cb) * 16 + 4 * g;
        const floatx4 o = oacc[gi][cb] * inv[gi];
        *(u32x2*)(orow + c0) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    } else {
      const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + h[gi];
      float* orow = p.part_o + slot * kDV;
      if (p.sync) {  // read by other workgroups in this launch: coherent stores
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          st_agent(orow + (cs * CB + cb) * 16 + 4 * g, oacc[gi][cb] * inv[gi]);
      } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int c0 = (cs * CB + cb) * 16 + 4 * g;
          *(floatx4*)(orow + c0) = oacc[gi][cb] * inv[gi];
        }
      }
    }
  }
  if (p.sync && p.nsplit > 1)  // single launch: merge the unit's partials here
    fused_combine<NT>(p, unit, tok, hblk * kHeadsPerBlock,
                      min(kHeadsPerBlock, p.heads - hblk * kHeadsPerBlock), split, tb0,
                      (uint32_t*)tb1);
}

// ---------------------------------------------------------------------------
// 64-head blocks with role-specialised waves.  Of the eight waves, four
// (waves 0-3) compute scores: wave (hp, rh) holds Q of head groups 2hp and
// 2hp+1 over all 576 columns and computes their scores for tile rows
// 16 rh .. +15, each operand read feeding two MFMAs; the other four (waves
// 4-7) hold O of all 64 heads over 128 of the 512 value columns, accumulate
// the PV and issue the tile loads.  A SIMD carries one wave of each kind, so
// tile n+1's scores and tile n's PV run side by side.  Per tile step n (one
// barrier): the score waves settle tile n's weights (the rare rescale when a
// head's maximum grows by more than 2^8, agreed between the two row halves)
// and compute tile n+1's; the PV waves apply tile n's rescale factors and
// accumulate its PV, and refill the buffer tile n-1 left with tile n+3.
// Weights, flags and half maxima are double-buffered by tile parity; four
// tile buffers keep two tiles in flight.  The two kinds run separate loops
// with the same sequence of barriers, so neither holds the other's registers.
// ---------------------------------------------------------------------------
template <int SRC>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(2)))
void split64_kernel(const int32_t* a_idx, const uint16_t* a_q, const uint16_t* a_kv, int64_t a_kv_rows,
                    int a_topk, int a_per_split, int a_nsplit, int a_heads, int a_tokens, int a_q_len,
                    SplitTail tl) {
  SplitParams p;
  p.idx = a_idx;
  p.q = a_q;
  p.kv = a_kv;
  p.kv_rows = a_kv_rows;
  p.topk = a_topk;
  p.per_split = a_per_split;
  p.nsplit = a_nsplit;
  p.heads = a_heads;
  p.tokens = a_tokens;
  p.q_len = a_q_len;
  p.table = tl.table;
  p.ctx = tl.ctx;
  p.out = tl.out;
  p.lse = tl.lse;
  p.part_o = tl.part_o;
  p.part_lse = tl.part_lse;
  p.sync = tl.sync;
  p.src = tl.src;
  p.max_pages = tl.max_pages;
  p.page_size = tl.page_size;
  p.merge_polls = tl.merge_polls;
  p.scale_log2 = tl.scale_log2;
  constexpr int NT = 512, TR = kTileRows, HG = 4;
  constexpr int kTileBytes = TR * kRow * 2;
  // the list stage is a ring of LCAP entries (32 tiles) beside four tile
  // buffers: the score waves load the entries of tiles n+16 .. n+31 at step
  // n (n a multiple of 16) and store them one step later (two for positions,
  // whose page-table lookup is a second load) into the slots of tiles
  // n-16 .. n-1, which every wave is done with; so a slice of any length
  // streams through without draining the tile pipeline
  constexpr int LCAP = 1024;
  constexpr int LI = LCAP / NT;
  constexpr int NTD = 256;                      // loading threads: the four PV waves
  constexpr int L = TR * kRowGran / NTD;        // 9 loads per loading lane per tile
  constexpr int CBP = 8;                        // 16-column blocks of O per PV wave
  constexpr int kStageRow = 1056;               // staged output row: 1 KB + 32 B (banks)
  constexpr int kStageRowF = 2080;              // staged fp32 partial row: 2 KB + 32 B
  static_assert(16 * kStageRowF <= TR * kRow * 2, "16 staged partial rows fit a tile buffer");
  static_assert(32 * kStageRow <= TR * kRow * 2, "32 staged rows fit a tile buffer");
  static_assert(TR == 32 && L == 9, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t tb0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tb2[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tb3[kTileBytes];
  __shared__ __attribute__((aligned(16))) int list_s[LCAP];
  // bf16 weights as PV B operands [parity][head group][g][head][8]
  __shared__ __attribute__((aligned(16))) u32x4 ps[2 * HG * 64];
  // half maxima [parity][group][row half][head], flags [parity][score wave]
  __shared__ float rmax_s[2 * HG * 2 * 16];
  __shared__ __attribute__((aligned(16))) int rflag_s[2 * 4];
  __shared__ float alpha_s[HG * 16];
  __shared__ float rsum_s[HG * 2 * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
  constexpr int kHeadsPerBlock = 64;
  const int hblocks = (p.heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const bool hb_fast = p.per_split >= 8 * TR;
  const int hblk = hb_fast ? wg % hblocks : (wg / p.nsplit) % hblocks;
  const int split = hb_fast ? (wg / hblocks) % p.nsplit : wg % p.nsplit;
  const int tok = wg / hblocks / p.nsplit;
  const int unit = tok * hblocks + hblk;

  const int lo = min(split * p.per_split, p.topk);
  const int hi = min(lo + p.per_split, p.topk);
  const int32_t* idx_row = p.idx ? p.idx + (int64_t)tok * p.topk : nullptr;
  const int seq = SRC == kSrcRows ? 0 : tok / p.q_len;
  int ctx_seq = 0;
  if (SRC == kSrcDense) ctx_seq = p.ctx[seq];
  const int32_t* tab = SRC != kSrcRows && p.table ? p.table + (int64_t)seq * p.max_pages : nullptr;
  auto entry = [&](int e) __attribute__((always_inline)) -> int32_t {
    if constexpr (SRC == kSrcRows) return idx_row[e];
    const int32_t pos = SRC == kSrcDense ? (e < ctx_seq ? e : -1) : idx_row[e];
    if (!tab || pos < 0) return pos;
    const int pg_i = pos / p.page_size;
    if (pg_i >= p.max_pages) return -1;
    const int32_t pg = tab[pg_i];
    if (pg < 0) return -1;
    const int64_t row = (int64_t)pg * p.page_size + (pos - pg_i * p.page_size);
    return row < p.kv_rows && row <= 0x7fffffff ? (int32_t)row : -1;
  };
  // the sequence's page-table slice staged in LDS (in the weights area, idle
  // whenever the list is staged) when it fits
  constexpr int kTabStage = 512;
  constexpr int TI = (kTabStage + NT - 1) / NT;
  const bool tab_lds = SRC == kSrcPositions && tab != nullptr && p.max_pages <= kTabStage;
  int32_t* const tab_stage = (int32_t*)ps;
  int tv[TI];
  if (tab_lds) {
#pragma unroll
    for (int u = 0; u < TI; ++u) {
      const int i = u * NT + tid;
      tv[u] = i < p.max_pages ? tab[i] : -1;
    }
  }
  int lv[LI];
  auto load_list = [&](int clo, int n_ent) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int e = clo + min(u * NT + tid, n_ent - 1);
      lv[u] = tab_lds ? idx_row[e] : entry(e);
    }
  };
  if (lo < hi) load_list(lo, min(hi - lo, LCAP));
  const uint32_t kv32 = rows32(p.kv_rows);
  auto store_list = [&](int n_ent) __attribute__((always_inline)) {
    if (tab_lds) {
      int32_t* ts = tab_stage;
#pragma unroll
      for (int u = 0; u < TI; ++u) {
        const int i = u * NT + tid;
        if (i < kTabStage) ts[i] = tv[u];
      }
      barrier_lds();
#pragma unroll
      for (int u = 0; u < LI; ++u) {
        const int32_t pos = lv[u];
        const int pg_i = pos / p.page_size;
        const bool in_tab = pos >= 0 && pg_i < p.max_pages;
        const int32_t pg_s = ts[in_tab ? pg_i : 0];
        const int32_t pg = in_tab ? pg_s : -1;
        const int64_t row = (int64_t)pg * p.page_size + (pos - pg_i * p.page_size);
        lv[u] = pg >= 0 && row < p.kv_rows && row <= 0x7fffffff ? (int32_t)row : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int e = u * NT + tid;
      list_s[e] = (e < n_ent && (uint32_t)lv[u] < kv32) ? lv[u] : -1;
    }
    barrier_lds();
  };
  auto buf = [&](auto bconst) __attribute__((always_inline)) -> uint8_t* {
    constexpr int b = decltype(bconst)::value;
    return b == 0 ? tb0 : b == 1 ? tb1 : b == 2 ? tb2 : tb3;
  };
  const int n_all = hi - lo;                  // entries of the slice
  const int ntiles = (n_all + TR - 1) / TR;   // its tiles
  // the ring slot of entry e (tile-aligned: a tile never wraps)
  auto ring = [&](int e) __attribute__((always_inline)) -> int { return e & (LCAP - 1); };

  float lse_out = -__builtin_inff();  // score waves: the LSE of this lane's head (rows 0-15 waves)
  bool lse_w = false;
  int lse_h = 0;

  if (wave_u < 4) {
    // ============================ score waves ============================
    const int hp = wave_u & 1, rh = wave_u >> 1;
    // the list is staged before q is loaded: q's 36 loads a lane would
    // otherwise hold the staging barrier, and with it the first tiles' loads,
    // behind their issue (batched 46.6 -> 46.0 us per step)
    if (lo < hi) store_list(min(n_all, LCAP));
    bf16x8 qf[2][kKSteps];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int hq = hblk * kHeadsPerBlock + (2 * hp + gi) * 16 + l16;
      const u32x4* qrow = hq < p.heads ? (const u32x4*)(p.q + ((int64_t)tok * p.heads + hq) * kRow) + g
                                       : g_zero_row + g;
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) qf[gi][k] = __builtin_bit_cast(bf16x8, qrow[4 * k]);
    }
    // ring refill: two entries per score lane (256 lanes, 16 tiles)
    int rv[2] = {-1, -1}, rt[2] = {-1, -1};
    auto ring_load = [&](int n) __attribute__((always_inline)) {  // tiles n+16 .. n+31
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = (n + 16) * TR + u * 256 + tid;
        if constexpr (SRC == kSrcDense)
          rv[u] = e < n_all && lo + e < ctx_seq ? lo + e : -1;
        else
          rv[u] = e < n_all ? idx_row[lo + e] : -1;
      }
    };
    auto ring_table = [&]() __attribute__((always_inline)) {  // positions: their page ids
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pos = rv[u];
        const int pg_i = pos >= 0 ? pos / p.page_size : 0;
        rt[u] = tab && pos >= 0 && pg_i < p.max_pages ? tab[pg_i] : -1;
      }
    };
    auto ring_store = [&](int n) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = (n + 16) * TR + u * 256 + tid;
        int32_t v = rv[u];
        if constexpr (SRC != kSrcRows) {  // a position: mapped through the page table, if any
          const int pos = rv[u];
          const int pg_i = pos >= 0 ? pos / p.page_size : 0;
          const int64_t row = (int64_t)rt[u] * p.page_size + (pos - pg_i * p.page_size);
          v = !tab ? pos : (rt[u] >= 0 && pos >= 0 && row < p.kv_rows && row <= 0x7fffffff ? (int32_t)row : -1);
        }
        list_s[ring(e)] = (e < n_all && (uint32_t)v < kv32) ? v : -1;
      }
    };
    const int hq = hsw(l16);
    const int qk_e = l16 * 128 + (g ^ hq) * 16 + rh * 16 * 128;
    const int qk_o = l16 * 128 + ((g ^ hq) ^ 4) * 16 + rh * 16 * 128;
    float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};
    float sc[2][4], pw[2][4], mxh[2] = {0.f, 0.f};
    auto weights = [&](u32x4* wb) __attribute__((always_inline)) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float m_use = m_run[gi] == -__builtin_inff() ? 0.f : m_run[gi];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[gi][i] = __builtin_amdgcn_exp2f(sc[gi][i] - m_use);
        *(u32x2*)((uint8_t*)wb + ((2 * hp + gi) * 64 + lane) * 16 + 8 * rh) =
            u32x2{pack_bf16x2(pw[gi][0], pw[gi][1]), pack_bf16x2(pw[gi][2], pw[gi][3])};
      }
    };
    // scores of tile t into weights wb, flag fb, half maxima mb
    auto qk = [&](const uint8_t* T, int t, u32x4* wb, float* mb, int* fb) __attribute__((always_inline)) {
      floatx4 acc[2][2] = {{floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}},
                           {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}}};
      constexpr int D = 6;
      bf16x8 op[D];
#pragma unroll
      for (int k = 0; k < D; ++k)
        op[k] = *(const bf16x8*)(T + ((k & 1) ? qk_o : qk_e) + (k >> 1) * TR * 128);
      // validity of this lane's rows, read with the first operands (after the
      // MFMAs its LDS round trip would wait in front of the softmax)
      const i32x4 r4 = *(const i32x4*)(list_s + ring(t * TR) + 16 * rh + 4 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
          acc[gi][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[k % D], qf[gi][k], acc[gi][k & 1], 0, 0, 0);
        if (k + D < kKSteps)
          op[k % D] = *(const bf16x8*)(T + (((k + D) & 1) ? qk_o : qk_e) + ((k + D) >> 1) * TR * 128);
        __builtin_amdgcn_sched_barrier(0);
      }
      bool grow = false;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const floatx4 sv = acc[gi][0] + acc[gi][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[gi][i] = r4[i] >= 0 ? sv[i] * p.scale_log2 : -__builtin_inff();
        mxh[gi] = max4_lanes(fmaxf(fmaxf(sc[gi][0], sc[gi][1]), fmaxf(sc[gi][2], sc[gi][3])));
        grow |= mxh[gi] > m_run[gi] + kRescaleLog2;
      }
      weights(wb);
      const int need_w = __any(grow);
      if (lane == 0) fb[wave_u] = need_w;
      if (g == 0) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) mb[((2 * hp + gi) * 2 + rh) * 16 + l16] = mxh[gi];
      }
    };
    // tile n's weights settled (rare path with its barrier), its share of
    // the sums taken
    auto settle = [&](u32x4* wb, const float* mb, const int* fb) __attribute__((always_inline)) {
      const i32x4 fa = *(const i32x4*)fb;
      if (fa[0] | fa[1] | fa[2] | fa[3]) {  // the same in every wave
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const float mt = fmaxf(mxh[gi], mb[((2 * hp + gi) * 2 + (rh ^ 1)) * 16 + l16]);
          float alpha = 1.f;
          if (mt > m_run[gi] + kRescaleLog2) {
            const float m_new = fmaxf(m_run[gi], mt);
            alpha = __builtin_amdgcn_exp2f(m_run[gi] - m_new);
            l_run[gi] *= alpha;
            m_run[gi] = m_new;
          }
          if (rh == 0 && g == 0) alpha_s[(2 * hp + gi) * 16 + l16] = alpha;
        }
        weights(wb);
        barrier_lds();
      }
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int i = 0; i < 4; ++i) l_run[gi] += pw[gi][i];
    };
    if (lo < hi) {
      barrier_raw();  // tile 0 landed
      qk(tb0, 0, ps, rmax_s, rflag_s);
      auto step = [&](auto jc, int n) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value, b1 = (j + 1) % 4, pb = j & 1;
        barrier_lds();
        // ring refill (uniform conditions)
        const int nr = n & ~15;
        if (nr >= 16 && (nr + 16) * TR < n_all) {
          if (n == nr) ring_load(nr);
          if constexpr (SRC != kSrcRows) {
            if (n == nr + 1) ring_table();
            if (n == nr + 2) ring_store(nr);
          } else {
            if (n == nr + 1) ring_store(nr);
          }
        }
        if (n < ntiles) settle(ps + pb * HG * 64, rmax_s + pb * HG * 32, rflag_s + pb * 4);
        if (n + 1 < ntiles)
          qk(buf(std::integral_constant<int, b1>{}), n + 1, ps + (pb ^ 1) * HG * 64,
             rmax_s + (pb ^ 1) * HG * 32, rflag_s + (pb ^ 1) * 4);
      };
      for (int n0 = 0; n0 < ntiles; n0 += 4) {
        step(std::integral_constant<int, 0>{}, n0);
        step(std::integral_constant<int, 1>{}, n0 + 1);
        step(std::integral_constant<int, 2>{}, n0 + 2);
        step(std::integral_constant<int, 3>{}, n0 + 3);
      }
      barrier_lds();
    }
    // this row half's share of each head's sum, then the LSE (rows 0-15 waves)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const float lh = sum4_lanes(l_run[gi]);
      if (g == 0) rsum_s[((2 * hp + gi) * 2 + rh) * 16 + l16] = lh;
    }
    barrier_lds();
    if (rh == 0 && g == 0) {
      // two heads per lane: groups 2hp and 2hp+1; the second is written below
      const float l0 = rsum_s[((2 * hp) * 2) * 16 + l16] + rsum_s[((2 * hp) * 2 + 1) * 16 + l16];
      const float l1 = rsum_s[((2 * hp + 1) * 2) * 16 + l16] + rsum_s[((2 * hp + 1) * 2 + 1) * 16 + l16];
      const int h0 = hblk * kHeadsPerBlock + (2 * hp) * 16 + l16;
      const float lse0 = l0 > 0.f ? m_run[0] * kLn2 + __logf(l0) : -__builtin_inff();
      lse_out = l1 > 0.f ? m_run[1] * kLn2 + __logf(l1) : -__builtin_inff();
      lse_h = h0 + 16;
      lse_w = true;
      if (h0 < p.heads) {
        const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + h0;
        if (p.nsplit == 1)
          p.lse[(int64_t)tok * p.heads + h0] = lse0;
        else if (p.sync)
          __hip_atomic_store(p.part_lse + slot, lse0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          p.part_lse[slot] = lse0;
      }
    }
  } else {
    // ============================== PV waves ==============================
    const int c = wave_u - 4;  // value columns 128 c .. +127
    floatx4 oacc[HG][CBP];
#pragma unroll
    for (int gi = 0; gi < HG; ++gi)
#pragma unroll
      for (int cb = 0; cb < CBP; ++cb) oacc[gi][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (lo < hi) store_list(min(n_all, LCAP));
    const int tr_e = l16 >> 2, tr_b0 = (l16 >> 1) & 1, tr_b1 = l16 & 1;
    const int tr_h = hsw(4 * g + tr_e);
    int pv_base[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      pv_base[q4] = (4 * g + tr_e) * 128 + ((2 * q4 + tr_b0) ^ tr_h) * 16 + 8 * tr_b1 + 2 * c * TR * 128;
    // tile loads: this wave's rows 8c .. 8c+7 of the tile, granule lane%8
    const int dma_row = 8 * c + (lane >> 3);
    const int dma_gran = (lane & 7) ^ hsw(dma_row);
    auto issue = [&](uint8_t* bp, int t) __attribute__((always_inline)) -> uint64_t {
      const int32_t r = t < ntiles ? list_s[ring(t * TR) + dma_row] : -1;
      const uintptr_t hit = (uintptr_t)(p.kv + (int64_t)r * kRow);
      const u32x4* src = (const u32x4*)(r >= 0 ? hit : (uintptr_t)g_zero_row) + dma_gran;
      dma_tile<NTD, 1>(src, bp + c * 64 * 16, std::make_integer_sequence<int, L>{});
      return (uint64_t)(uintptr_t)src;
    };
    auto pv = [&](const uint8_t* T, const u32x4* wb) __attribute__((always_inline)) {
      bf16x8 pq[HG];
#pragma unroll
      for (int gi = 0; gi < HG; ++gi) pq[gi] = __builtin_bit_cast(bf16x8, wb[gi * 64 + lane]);
#pragma unroll
      for (int cb = 0; cb < CBP; ++cb) {
        const int off = pv_base[cb & 3] + (cb >> 2) * TR * 128;
        const shortx4 v2[2] = {lds_tr16(T + off), lds_tr16(T + off + 16 * 128)};
        const bf16x8 vt = __builtin_bit_cast(bf16x8, v2);
#pragma unroll
        for (int gi = 0; gi < HG; ++gi)
          oacc[gi][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pq[gi], oacc[gi][cb], 0, 0, 0);
      }
    };
    // the rescale factors of tile n when the score waves moved a maximum
    auto settle = [&](const int* fb) __attribute__((always_inline)) {
      const i32x4 fa = *(const i32x4*)fb;
      if (fa[0] | fa[1] | fa[2] | fa[3]) {  // the same in every wave
        barrier_lds();
        float al[HG];
        bool scale = false;
#pragma unroll
        for (int gi = 0; gi < HG; ++gi) {
          al[gi] = alpha_s[gi * 16 + l16];
          scale |= al[gi] != 1.f;
        }
        if (__any(scale)) {
#pragma unroll
          for (int gi = 0; gi < HG; ++gi)
#pragma unroll
            for (int cb = 0; cb < CBP; ++cb) oacc[gi][cb] *= al[gi];
        }
      }
    };
    if (lo < hi) {
      uint64_t addr[4] = {};
      addr[0] = issue(tb0, 0);
      addr[1] = issue(tb1, 1);
      addr[2] = issue(tb2, 2);
      wait_vmcnt<2 * L>();  // tile 0 landed
      keep_live(addr[0]);
      barrier_raw();
      auto step = [&](auto jc, int n) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value, b1 = (j + 1) % 4, bf = (j + 3) % 4, pb = j & 1;
        wait_vmcnt<L>();  // tile n+1 landed (tile n+2's loads may be out)
        keep_live(addr[b1]);
        barrier_lds();
        addr[bf] = issue(buf(std::integral_constant<int, bf>{}), n + 3);
        if (n < ntiles) {
          settle(rflag_s + pb * 4);
          pv(buf(jc), ps + pb * HG * 64);
        }
      };
      for (int n0 = 0; n0 < ntiles; n0 += 4) {
        step(std::integral_constant<int, 0>{}, n0);
        step(std::integral_constant<int, 1>{}, n0 + 1);
        step(std::integral_constant<int, 2>{}, n0 + 2);
        step(std::integral_constant<int, 3>{}, n0 + 3);
      }
      wait_vmcnt<0>();  // the refills past the last tile
#pragma unroll
      for (int b = 0; b < 4; ++b) keep_live(addr[b]);
      barrier_lds();
    }
    barrier_lds();  // the score waves' sums are in
#pragma unroll
    for (int gi = 0; gi < HG; ++gi) {
      const float l = rsum_s[(gi * 2) * 16 + l16] + rsum_s[(gi * 2 + 1) * 16 + l16];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int h = hblk * kHeadsPerBlock + gi * 16 + l16;
      if (h >= p.heads) continue;
      if (p.nsplit == 1) {
        // into LDS (the free tile buffers, head rows of kStageRow bytes);
        // copied out below with 16-byte stores, 1 KB per wave instruction
        const int r = gi * 16 + l16;
        uint8_t* srow = (r < 32 ? tb0 : tb1) + (r & 31) * kStageRow;
#pragma unroll
        for (int cb = 0; cb < CBP; ++cb) {
          const int c0 = (c * CBP + cb) * 16 + 4 * g;
          const floatx4 o = oacc[gi][cb] * inv;
          *(u32x2*)(srow + c0 * 2) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
      } else {
        const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + h;
        float* orow = p.part_o + slot * kDV;
        if (p.sync) {
#pragma unroll
          for (int cb = 0; cb < CBP; ++cb) st_agent(orow + (c * CBP + cb) * 16 + 4 * g, oacc[gi][cb] * inv);
        } else {
          // into LDS (16 head rows of kStageRowF bytes per tile buffer),
          // copied out below with 16-byte stores, 1 KB per wave instruction
          const int r = gi * 16 + l16;
          uint8_t* const sb = r < 16 ? tb0 : r < 32 ? tb1 : r < 48 ? tb2 : tb3;
          uint8_t* const srow = sb + (r & 15) * kStageRowF;
#pragma unroll
          for (int cb = 0; cb < CBP; ++cb) {
            const int c0 = (c * CBP + cb) * 16 + 4 * g;
            *(floatx4*)(srow + c0 * 4) = oacc[gi][cb] * inv;
          }
        }
      }
    }
  }
  if (p.nsplit > 1 && !p.sync) {  // the staged partials of the block's heads, row by row
    barrier_lds();
    const int hv = min(kHeadsPerBlock, p.heads - hblk * kHeadsPerBlock);
    const int64_t slot0 = ((int64_t)tok * p.nsplit + split) * p.heads + hblk * kHeadsPerBlock;
#pragma unroll
    for (int u = 0; u < kHeadsPerBlock * 128 / NT; ++u) {
      const int q = u * NT + tid, r = q >> 7, c16 = q & 127;
      if (r < hv) {
        const uint8_t* const sb = r < 16 ? tb0 : r < 32 ? tb1 : r < 48 ? tb2 : tb3;
        const floatx4 v = *(const floatx4*)(sb + (r & 15) * kStageRowF + c16 * 16);
        *(floatx4*)(p.part_o + (slot0 + r) * kDV + c16 * 4) = v;
      }
    }
  }
  // the staged outputs of the block's heads, row by row; non-temporal stores
  // (nothing in the launch reads them back), which leave every workgroup
  // together at the end: ragged 90.2 -> 88.3 us per launch
  if (p.nsplit == 1) {
    barrier_lds();
    const int hv = min(kHeadsPerBlock, p.heads - hblk * kHeadsPerBlock);
#pragma unroll
    for (int u = 0; u < kHeadsPerBlock * 64 / NT; ++u) {
      const int q = u * NT + tid, r = q >> 6, c16 = q & 63;
      if (r < hv) {
        const uint8_t* srow = (r < 32 ? tb0 : tb1) + (r & 31) * kStageRow;
        const u32x4 v = *(const u32x4*)(srow + c16 * 16);
        __builtin_nontemporal_store(v, (u32x4*)(p.out + ((int64_t)tok * p.heads + hblk * kHeadsPerBlock + r) * kDV + c16 * 8));
      }
    }
  }
  // the second head of each score lane (group 2hp+1)
  if (lse_w && lse_h < p.heads) {
    const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + lse_h;
    if (p.nsplit == 1)
      p.lse[(int64_t)tok * p.heads + lse_h] = lse_out;
    else if (p.sync)
      __hip_atomic_store(p.part_lse + slot, lse_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      p.part_lse[slot] = lse_out;
  }
  if (p.sync && p.nsplit > 1)  // single launch: merge the unit's partials here
    fused_combine<NT>(p, unit, tok, hblk * kHeadsPerBlock, min(kHeadsPerBlock, p.heads - hblk * kHeadsPerBlock),
                      split, tb0, (uint32_t*)tb1);
}

// The workgroup's index in the combine grid.  With at least as many tokens as
// XCDs the split kernel's XCD-contiguous numbering puts each token's splits
// on one XCD; taking the combine's workgroups in the same numbering then
// merges a token's partials on that XCD (spec, 9 tokens: 13.1 -> 12.7 us per
// call; batched: 46.3 -> 46.0 us).  With fewer tokens a token's splits span
// every XCD, and the plain order measured faster (long: 9.56 against 10.05).
__device__ __forceinline__ int combine_order(const CombineParams& p) {
  return p.tokens >= kXcds ? xcd_contiguous(blockIdx.x, gridDim.x) : (int)blockIdx.x;
}

// ---------------------------------------------------------------------------
// Combine kernel ([SPLITK] "The Split-K Imperative").  Workgroup = (token,
// head, quarter of the 512 columns): 32 threads cover the quarter in 4-float
// and SG groups of them take interleaved splits; each thread issues all of
// its partial-O loads before any arithmetic (a chain of dependent loads would
// cost one cache round trip per split), then an LDS reduction over the groups.
// ---------------------------------------------------------------------------
constexpr int kCombCols = 128;               // columns per workgroup
constexpr int kCombC4 = kCombCols / 4;       // 4-float lanes per split group

template <int SG, int PER>
__global__ __launch_bounds__(kCombC4 * SG)
void combine_kernel(const float* a_part_o, const float* a_part_lse, uint16_t* a_out, float* a_lse,
                    int a_tokens, int a_heads, int a_nsplit) {
  const CombineParams p{a_part_o, a_part_lse, a_out, a_lse, a_tokens, a_heads, a_nsplit};
  __shared__ floatx4 acc_s[SG][kCombC4];
  __shared__ float m_s[SG], w_s[SG];

  const int tid = threadIdx.x;
  const int wg = combine_order(p);
  const int quarter = wg & 3;
  const int th_id = wg >> 2;                  // token * heads + head
  const int tok = th_id / p.heads;
  const int h = th_id % p.heads;
  const int S = p.nsplit;
  const float* lse_in = p.part_lse + (int64_t)tok * S * p.heads + h;
  const int c4 = tid % kCombC4;
  const int sg = tid / kCombC4;
  const int col = quarter * kCombCols + c4 * 4;
  const float* o_in = p.part_o + ((int64_t)tok * S * p.heads + h) * kDV + col;
  const int64_t stride = (int64_t)p.heads * kDV;

  // Each thread merges its own splits (sg, sg + SG, ...) with a running
  // maximum, its O slices and LSE values of a round loaded together:
  // (m, w, acc) = (max LSE, sum exp(LSE - m), sum exp(LSE - m) O).
  float m = -__builtin_inff(), w = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < S; s0 += SG * PER) {
    floatx4 v[PER];
    float l[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int s = s0 + u * SG;
      v[u] = s < S ? *(const floatx4*)(o_in + s * stride) : floatx4{0.f, 0.f, 0.f, 0.f};
      l[u] = s < S ? lse_in[(int64_t)s * p.heads] : -__builtin_inff();
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      // an empty split (LSE = -inf) contributes nothing, whatever its slot holds
      if (l[u] == -__builtin_inff()) continue;
      if (l[u] > m) {
        const float r = __builtin_amdgcn_exp2f((m - l[u]) * kLog2e);  // 0 while m = -inf
        acc *= r;
        w *= r;
        m = l[u];
      }
      const float e = __builtin_amdgcn_exp2f((l[u] - m) * kLog2e);
      acc += e * v[u];
      w += e;
    }
  }
  // merge the SG groups: M = max m_g, O = sum f_g acc_g / sum f_g w_g with
  // f_g = exp(m_g - M), LSE = M + ln sum f_g w_g
  acc_s[sg][c4] = acc;
  if (c4 == 0) {
    m_s[sg] = m;
    w_s[sg] = w;
  }
  __syncthreads();
  if (sg != 0) return;
  float M = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < SG; ++i) M = fmaxf(M, m_s[i]);
  floatx4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int i = 0; i < SG; ++i) {
      if (m_s[i] == -__builtin_inff()) continue;
      const float f = __builtin_amdgcn_exp2f((m_s[i] - M) * kLog2e);
      num += f * acc_s[i][c4];
      den += f * w_s[i];
    }
  }
  const bool any = den > 0.f;
  const float inv = any ? 1.f / den : 0.f;
  const int64_t th = (int64_t)tok * p.heads + h;
  *(u32x2*)(p.out + th * kDV + col) =
      u32x2{pack_bf16x2(num[0] * inv, num[1] * inv), pack_bf16x2(num[2] * inv, num[3] * inv)};
  if (tid == 0 && quarter == 0) p.lse[th] = any ? M + __logf(den) : -__builtin_inff();
}

// Combine for many (token, head) pairs: one thread per 4 output columns of
// one pair, 128 threads per pair, two pairs per workgroup.  Every thread
// walks all splits itself (the pair's LSE values are the same addresses for
// its 128 threads), so there is no LDS, no barrier and no cross-wave
// reduction; the grid alone supplies the parallelism.
constexpr int kWidePairs = 2;
// from this many (token, head) pairs on, the wide combine has >= 512
// workgroups, enough to cover the device
constexpr int64_t kWideMinPairs = 1024;

template <int CH>
__global__ __launch_bounds__(128 * kWidePairs)
void combine_wide_kernel(const float* a_part_o, const float* a_part_lse, uint16_t* a_out,
                         float* a_lse, int a_tokens, int a_heads, int a_nsplit) {
  const CombineParams p{a_part_o, a_part_lse, a_out, a_lse, a_tokens, a_heads, a_nsplit};
  const int64_t th = (int64_t)combine_order(p) * kWidePairs + (threadIdx.x >> 7);
  if (th >= (int64_t)p.tokens * p.heads) return;
  const int c4 = threadIdx.x & 127;
  const int64_t tok = th / p.heads;
  const int h = (int)(th - tok * p.heads);
  const int S = p.nsplit;
  const float* lse_in = p.part_lse + tok * S * p.heads + h;
  const float* o_in = p.part_o + (tok * S * p.heads + h) * kDV + c4 * 4;
  const int64_t stride = (int64_t)p.heads * kDV;

  // a round: CH splits' O slices and LSE values, all loads in flight together
  floatx4 v[CH];
  float l[CH];
  auto load_round = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int s = s0 + u;
      v[u] = s < S ? *(const floatx4*)(o_in + s * stride) : floatx4{0.f, 0.f, 0.f, 0.f};
      l[u] = s < S ? lse_in[(int64_t)s * p.heads] : -__builtin_inff();
    }
  };
  load_round(0);
  float mx = -__builtin_inff();
  if (S <= CH) {  // one round holds every split: a single memory round trip
#pragma unroll
    for (int u = 0; u < CH; ++u) mx = fmaxf(mx, l[u]);
  } else {
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, lse_in[(int64_t)s * p.heads]);
  }
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = 0;;) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float w = (mx == -__builtin_inff() || l[u] == -__builtin_inff())
                          ? 0.f
                          : __builtin_amdgcn_exp2f((l[u] - mx) * kLog2e);
      wsum += w;
      // a zero weight (empty split) contributes nothing, whatever its slot holds
      if (w != 0.f) acc += w * v[u];
    }
    s0 += CH;
    if (s0 >= S) break;
    load_round(s0);
  }
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  *(u32x2*)(p.out + th * kDV + c4 * 4) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (c4 == 0) p.lse[th] = any ? mx + __logf(wsum) : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// LDS of one split workgroup: the tile buffers (two, or three for 64-head
// blocks over long slices), the staged index list, with K-split pairs the
// exchange slots of partial scores (one 16-row block of 16 heads = 1 KiB per
// slot, head group and row block), with row halves the bf16 weights, the
// rescale factors and two floats and a flag per (wave, owned head)
constexpr int split_lds_bytes(int waves, int ncs, int gpw, int ks) {
  return 2 * kTileRows * kRow * 2 + split_list_cap(ncs, ks) * 4 +
         (ks == 2 ? (waves / ncs) * 2 * gpw * (kTileRows / 16) * 64 * 16 : 0) +
         (ks == 1 && gpw == 4 ? gpw * 64 * 16 + gpw * 16 * 4 + 2 * waves * 16 * 4 + waves * 4 : 0);
}
constexpr int kCuLdsBytes = 160 * 1024;

static SplitTail split_tail(const SplitParams& p) {
  SplitTail t;
  t.table = p.table;
  t.ctx = p.ctx;
  t.out = p.out;
  t.lse = p.lse;
  t.part_o = p.part_o;
  t.part_lse = p.part_lse;
  t.sync = p.sync;
  t.src = p.src;
  t.max_pages = p.max_pages;
  t.page_size = p.page_size;
  t.merge_polls = p.merge_polls;
  t.scale_log2 = p.scale_log2;
  return t;
}

template <int HG, int NCS, int GPW, int TR, int KS>
static hipError_t launch_split_t(const SplitParams& p, int hblocks, hipStream_t st) {
  static_assert(TR == kTileRows, "the planner's tile");
  const int64_t nwg = (int64_t)p.nsplit * p.tokens * hblocks;
  const dim3 grid((unsigned)nwg), block(64 * (HG / GPW) * NCS);
  const SplitTail t = split_tail(p);
  switch (p.src) {
    case kSrcPositions:
      hipLaunchKernelGGL((split_kernel<HG, NCS, GPW, TR, KS, kSrcPositions>), grid, block, 0,
                         st, p.idx, p.q, p.kv, p.kv_rows, p.topk, p.per_split, p.nsplit, p.heads,
                         p.tokens, p.q_len, t);
      break;
    case kSrcDense:
      hipLaunchKernelGGL((split_kernel<HG, NCS, GPW, TR, KS, kSrcDense>), grid, block, 0, st,
                         p.idx, p.q, p.kv, p.kv_rows, p.topk, p.per_split, p.nsplit, p.heads,
                         p.tokens, p.q_len, t);
      break;
    default:
      hipLaunchKernelGGL((split_kernel<HG, NCS, GPW, TR, KS, kSrcRows>), grid, block, 0, st,
                         p.idx, p.q, p.kv, p.kv_rows, p.topk, p.per_split, p.nsplit, p.heads,
                         p.tokens, p.q_len, t);
  }
  return hipGetLastError();
}

// Per head class:
//  * up to 16 heads: 4 waves sharing one 16-head group, each with a quarter
//    of the 512 V columns, in K-split pairs (even / odd K-steps of QK^T);
//    two workgroups per CU;
//  * up to 32 heads: 4 waves = 2 head groups x 2 column halves, each wave
//    all of QK^T; two workgroups per CU;
//  * more (64-head blocks): over slices of at least kDeepTiles tiles,
//    split64_kernel (four score waves holding Q of two head groups each and
//    four PV waves holding O, four tile buffers); over shorter slices 8
//    waves in row halves (each wave the scores of one head group over half
//    the tile rows and all of K, and O of all 64 heads over an eighth of the
//    value columns).  Either is one workgroup per CU (two waves per SIMD).
static_assert(kCuLdsBytes / split_lds_bytes(4, 4, 1, 2) == 2, "two 16-head workgroups per CU");
static_assert(kCuLdsBytes / split_lds_bytes(4, 2, 1, 1) == 2, "two 32-head workgroups per CU");
static_assert(split_lds_bytes(8, 8, 4, 1) <= kCuLdsBytes, "one 64-head workgroup per CU");

// 64-head blocks over slices of at least this many tiles take split64_kernel
// (its rounds of four steps pad a short slice's tail with refills past the
// end).  Measured against the row halves: 128 x 128 heads with 64-tile
// slices 103 -> 90 us per launch; 72 folded heads over 16384 positions
// (4-tile slices) 21.6 -> 20.7 us; over 4096 (1-tile slices) equal; 64 x 64
// heads with 2-tile slices 139 -> 159 us.
constexpr int kDeepTiles = 4;

static hipError_t launch_split64(const SplitParams& p, int hblocks, hipStream_t st) {
  const int64_t nwg = (int64_t)p.nsplit * p.tokens * hblocks;
  const dim3 grid((unsigned)nwg), block(512);
  const SplitTail t = split_tail(p);
  switch (p.src) {
    case kSrcPositions:
      hipLaunchKernelGGL((split64_kernel<kSrcPositions>), grid, block, 0, st, p.idx, p.q, p.kv, p.kv_rows,
                         p.topk, p.per_split, p.nsplit, p.heads, p.tokens, p.q_len, t);
      break;
    case kSrcDense:
      hipLaunchKernelGGL((split64_kernel<kSrcDense>), grid, block, 0, st, p.idx, p.q, p.kv, p.kv_rows,
                         p.topk, p.per_split, p.nsplit, p.heads, p.tokens, p.q_len, t);
      break;
    default:
      hipLaunchKernelGGL((split64_kernel<kSrcRows>), grid, block, 0, st, p.idx, p.q, p.kv, p.kv_rows,
                         p.topk, p.per_split, p.nsplit, p.heads, p.tokens, p.q_len, t);
  }
  return hipGetLastError();
}

hipError_t launch_split(const SplitParams& p, hipStream_t st) {
  if (p.heads <= 16) return launch_split_t<1, 4, 1, 32, 2>(p, 1, st);
  if (p.heads <= 32) return launch_split_t<2, 2, 1, 32, 1>(p, 1, st);
  const int hblocks = (p.heads + 63) / 64;
  if ((p.per_split + kTileRows - 1) / kTileRows >= kDeepTiles) return launch_split64(p, hblocks, st);
  return launch_split_t<4, 8, 4, 32, 1>(p, hblocks, st);
}

int split_heads_per_block(int heads) { return heads <= 16 ? 16 : heads <= 32 ? 32 : 64; }

// workgroups of the head class resident per CU: LDS bounds the 4-wave
// classes at two; the 8-wave class at 2 waves per SIMD is one per CU
int split_blocks_per_cu(int heads) {
  if (heads <= 16) return kCuLdsBytes / split_lds_bytes(4, 4, 1, 2);
  if (heads <= 32) return kCuLdsBytes / split_lds_bytes(4, 2, 1, 1);
  return 1;
}

template <int SG, int PER>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t st) {
  const int64_t nwg = (int64_t)p.tokens * p.heads * (kDV / kCombCols);
  hipLaunchKernelGGL((combine_kernel<SG, PER>), dim3((unsigned)nwg), dim3(kCombC4 * SG), 0, st,
                     p.part_o, p.part_lse, p.out, p.lse, p.tokens, p.heads, p.nsplit);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t st) {
  const int64_t pairs = (int64_t)p.tokens * p.heads;
  if (pairs >= kWideMinPairs) {
    const int64_t nwg = (pairs + kWidePairs - 1) / kWidePairs;
    // rounds of 4 splits when that covers them all (fewer registers, so every
    // workgroup of a large grid is resident at once), else of 8
    if (p.nsplit <= 4)
      hipLaunchKernelGGL((combine_wide_kernel<4>), dim3((unsigned)nwg), dim3(128 * kWidePairs), 0,
                         st, p.part_o, p.part_lse, p.out, p.lse, p.tokens, p.heads, p.nsplit);
    else
      hipLaunchKernelGGL((combine_wide_kernel<8>), dim3((unsigned)nwg), dim3(128 * kWidePairs), 0,
                         st, p.part_o, p.part_lse, p.out, p.lse, p.tokens, p.heads, p.nsplit);
    return hipGetLastError();
  }
  // few pairs: the splits of one pair are spread over the waves of a
  // workgroup (split groups x loads in flight per thread, sized so one round
  // covers up to 128 splits; at 33-64 splits 8 groups of 8 loads measured
  // 0.1 us per call faster than 16 groups of 4 on one token x 8 heads, the
  // LDS merge of the groups being shorter)
  if (p.nsplit > 64) return launch_combine_t<16, 8>(p, st);
  if (p.nsplit > 32) return launch_combine_t<8, 8>(p, st);
  if (p.nsplit > 8) return launch_combine_t<8, 4>(p, st);
  return launch_combine_t<4, 2>(p, st);
}

}  // namespace smla
