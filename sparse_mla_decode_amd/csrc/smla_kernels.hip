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
//   * workgroup = (token, split, head block); a head block is up to 64 heads
//     = 4 groups of 16 (the M/N width of one MFMA), one or two waves each.
//   * the split's rows are gathered in tiles of 32 or 64 rows (x 1152 B)
//     with 16-byte loads by all threads, staged through registers into a
//     padded LDS tile (double buffered): the loads of tile n+1 are in flight
//     while tile n is computed.  Every wave of the workgroup reads the
//     same LDS tile, so a row is fetched from HBM once per workgroup.
//   * S^T = KV_tile * Q^T on v_mfma_f32_16x16x32_bf16 (rows on M, heads on N)
//     so that each lane owns one head: the online-softmax max needs only two
//     cross-lane exchanges per tile and the running sum none until the end.
//   * O^T += V^T * P^T on the same MFMA; the softmax output is already laid
//     out as the B operand (no shuffles), V^T is read from the LDS tile.
//   * masked entries (-1, out of range, past the slice end) load a static
//     all-zero row, so their V contribution is exactly zero, and get a score
//     of -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowGran = kRow * 2 / 16;          // 72 16-byte granules per row
constexpr int kKSteps = kRow / 32;               // 18 MFMA K-steps over 576 columns

// Row read for masked list entries: all zeros, so masked rows add exactly
// nothing to P*V (and never carry non-finite stale data).
__device__ __attribute__((aligned(16))) uint4 g_zero_row[kRowGran];

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// LDS row pitch: 1152 bytes of row + 16 of padding.  The pad shifts each row
// by one 16-byte bank group, so the 16 rows one MFMA operand read touches
// land in distinct banks (a bare 1152-byte pitch is a multiple of the bank
// span), and every operand address is a per-lane base plus a constant.
constexpr int kPitch = kRow * 2 + 16;
__device__ __forceinline__ int tile_off(int j, int k) { return j * kPitch + k * 16; }

__device__ __forceinline__ bool row_ok(int32_t r, int64_t kv_rows) {
  return r >= 0 && (int64_t)r < kv_rows;
}

// Round to bf16 (nearest even) and pack two values.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  uint16_t ux, uy;
  __builtin_memcpy(&ux, &x, 2);
  __builtin_memcpy(&uy, &y, 2);
  return (uint32_t)ux | ((uint32_t)uy << 16);
}

// ---------------------------------------------------------------------------
// Split kernel.  HG head groups of 16 per workgroup, NCS column slices of the
// 512 value columns per head group, one wave per (head group, column slice).
// Every wave computes S for its head group; the PV work and the O
// accumulators are divided among the NCS waves that share a head group.
// TR rows per LDS tile; each thread moves TR*72/threads granules per tile.
// ---------------------------------------------------------------------------
template <int HG, int NCS, int TR>
__global__ __launch_bounds__(64 * HG * NCS) __attribute__((amdgpu_waves_per_eu(2)))
void split_kernel(SplitParams p) {
  constexpr int kThreads = 64 * HG * NCS;
  constexpr int kTileRows = TR;
  constexpr int RB = TR / 16;                      // 16-row blocks per tile
  constexpr int KP = TR / 32;                      // 32-row K-steps of PV per tile
  constexpr int kTileGran = kTileRows * kRowGran;
  constexpr int kLoadsPerThread = kTileGran / kThreads;
  constexpr int kTileBytes = kTileRows * kPitch;
  constexpr int CB = (kDV / 16) / NCS;  // 16-column blocks of O per wave
  static_assert(kTileGran % kThreads == 0, "tile must split evenly over the threads");
  static_assert(TR % 32 == 0, "tile rows must be a multiple of the PV K-step");

  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTileBytes];
  __shared__ int tile_valid[2][kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;    // lane group: selects the K slots of MFMA operands
  const int l16 = lane & 15;  // MFMA row / column within a 16-wide block
  const int hg = wave / NCS;
  const int cs = wave % NCS;

  // workgroup -> (split, token, head block); splits vary fastest
  const int wg = blockIdx.x;
  const int split = wg % p.nsplit;
  const int rest = wg / p.nsplit;
  const int tok = rest % p.tokens;
  const int hblk = rest / p.tokens;

  const int h = hblk * (HG * 16) + hg * 16 + l16;  // this lane's head
  const bool h_ok = h < p.heads;

  // Q^T as the B operand of S^T = KV * Q^T: lane (g, l16) holds
  // q[h][32*ks + 8*g .. +7] for every K-step ks (zeros for padding heads).
  bf16x8 qb[kKSteps];
  {
    const uint16_t* qrow = p.q + ((int64_t)tok * p.heads + (h_ok ? h : 0)) * kRow + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      uint4 v = h_ok ? *(const uint4*)(qrow + ks * 32) : make_uint4(0, 0, 0, 0);
      qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // this split's slice of the list
  const int lo = min(split * p.per_split, p.topk);
  const int hi = min(lo + p.per_split, p.topk);
  const int ntiles = (hi - lo + kTileRows - 1) / kTileRows;
  const int32_t* idx_row = p.idx + (int64_t)tok * p.topk;

  // Gather slots: thread tid moves granules q = it*256 + tid of a tile,
  // i.e. row j = q / 72, granule k = q % 72.
  int rows_cur[kLoadsPerThread];
  int rows_next[kLoadsPerThread];
  uint4 stage[kLoadsPerThread];

  auto load_rows = [&](int t, int (&rows)[kLoadsPerThread]) {
#pragma unroll
    for (int it = 0; it < kLoadsPerThread; ++it) {
      const int j = (it * kThreads + tid) / kRowGran;
      const int e = lo + t * kTileRows + j;
      rows[it] = e < hi ? idx_row[e] : -1;
    }
  };
  auto issue = [&](const int (&rows)[kLoadsPerThread]) {
#pragma unroll
    for (int it = 0; it < kLoadsPerThread; ++it) {
      const int k = (it * kThreads + tid) % kRowGran;
      const int32_t r = rows[it];
      const uint4* src = row_ok(r, p.kv_rows)
                             ? (const uint4*)(p.kv + (int64_t)r * kRow) + k
                             : g_zero_row + k;
      stage[it] = *src;
    }
  };
  auto commit = [&](int buf, const int (&rows)[kLoadsPerThread]) {
#pragma unroll
    for (int it = 0; it < kLoadsPerThread; ++it) {
      const int q = it * kThreads + tid;
      const int j = q / kRowGran, k = q % kRowGran;
      *(uint4*)(&tile[buf][tile_off(j, k)]) = stage[it];
      if (k == 0) tile_valid[buf][j] = row_ok(rows[it], p.kv_rows);
    }
  };

  float m_run = -__builtin_inff();  // running max of log2-scaled scores (per head)
  float l_run = 0.f;                // this lane's share of the running sum
  floatx4 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    load_rows(0, rows_cur);
    issue(rows_cur);
    if (ntiles > 1) load_rows(1, rows_next);
  }

  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    commit(buf, rows_cur);
    __syncthreads();
    if (n + 1 < ntiles) {
#pragma unroll
      for (int it = 0; it < kLoadsPerThread; ++it) rows_cur[it] = rows_next[it];
      issue(rows_cur);
      if (n + 2 < ntiles) load_rows(n + 2, rows_next);
    }

    const uint8_t* T = tile[buf];

    // ---- S^T = KV_tile * Q^T: RB 16-row blocks, 18 K-steps of 32 columns
    floatx4 sacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int j = rb * 16 + l16;
        const bf16x8 a = *(const bf16x8*)(T + tile_off(j, ks * 4 + g));
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], sacc[rb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax; lane holds rows j = 16*rb + 4*g + i of head h
    float s[4 * RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = rb * 16 + 4 * g + i;
        s[rb * 4 + i] = tile_valid[buf][j] ? sacc[rb][i] * p.scale_log2 : -__builtin_inff();
      }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 4 * RB; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    float pv[4 * RB];
#pragma unroll
    for (int i = 0; i < 4 * RB; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] *= alpha;

    // P^T as the B operand of K-step kp: K slot s <-> tile row
    // 32*kp + 16*(s/4) + 4*g + s%4, i.e. the rows this lane already holds.
    bf16x8 pb[KP];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      const float* v = pv + 8 * kp;
      const uint4 pw = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      pb[kp] = __builtin_bit_cast(bf16x8, pw);
    }

    // ---- O^T += V^T * P^T; A operand: V[row(s)][c], c = column of this lane
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = (cs * CB + cb) * 16 + l16;
#pragma unroll
      for (int kp = 0; kp < KP; ++kp) {
        uint16_t av[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int j = 32 * kp + 16 * (sl >> 2) + 4 * g + (sl & 3);
          av[sl] = *(const uint16_t*)(T + j * kPitch + c * 2);
        }
        const uint4 aw = make_uint4((uint32_t)av[0] | ((uint32_t)av[1] << 16),
                                    (uint32_t)av[2] | ((uint32_t)av[3] << 16),
                                    (uint32_t)av[4] | ((uint32_t)av[5] << 16),
                                    (uint32_t)av[6] | ((uint32_t)av[7] << 16));
        oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw),
                                                           pb[kp], oacc[cb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: O / l and LSE = (m * ln 2) + ln l
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? m_run * kLn2 + __logf(l_tot) : -__builtin_inff();

  if (!h_ok) return;
  const int64_t th = (int64_t)tok * p.heads + h;
  if (p.nsplit == 1) {
    uint16_t* orow = p.out + th * kDV;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = (cs * CB + cb) * 16 + 4 * g;
      const floatx4 o = oacc[cb] * inv;
      *(uint2*)(orow + c0) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
    if (g == 0 && cs == 0) p.lse[th] = lse_v;
  } else {
    const int64_t slot = ((int64_t)tok * p.nsplit + split) * p.heads + h;
    float* orow = p.part_o + slot * kDV;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c0 = (cs * CB + cb) * 16 + 4 * g;
      const floatx4 o = oacc[cb] * inv;
      *(float4*)(orow + c0) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (g == 0 && cs == 0) p.part_lse[slot] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// Combine kernel ([SPLITK] "The Split-K Imperative").  One workgroup per
// (token, head); 128 threads cover the 512 columns as float4, and SG such
// groups take interleaved splits before an LDS reduction.
// ---------------------------------------------------------------------------
template <int SG>
__global__ __launch_bounds__(128 * SG) void combine_kernel(CombineParams p) {
  constexpr int NT = 128 * SG;
  __shared__ float w_s[kMaxNsplit];
  __shared__ float red[NT / 64];
  __shared__ float4 acc_s[SG > 1 ? SG - 1 : 1][128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tok = blockIdx.x / p.heads;
  const int h = blockIdx.x % p.heads;
  const int S = p.nsplit;
  const float* lse_in = p.part_lse + (int64_t)tok * S * p.heads + h;

  // M = max_s LSE_s
  float mx = -__builtin_inff();
  for (int s = tid; s < S; s += NT) mx = fmaxf(mx, lse_in[(int64_t)s * p.heads]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();

  // w_s = exp(LSE_s - M); W = sum_s w_s
  float ws = 0.f;
  for (int s = tid; s < S; s += NT) {
    const float l = lse_in[(int64_t)s * p.heads];
    const float w = (mx == -__builtin_inff() || l == -__builtin_inff())
                        ? 0.f
                        : __builtin_amdgcn_exp2f((l - mx) * kLog2e);
    w_s[s] = w;
    ws += w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ws += __shfl_xor(ws, o, 64);
  if (lane == 0) red[wave] = ws;
  __syncthreads();
  float wsum = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) wsum += red[w];

  // sum_s w_s O_s over this thread's splits
  const int c4 = tid % 128;
  const int sg = tid / 128;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* o_in = p.part_o + ((int64_t)tok * S * p.heads + h) * kDV + c4 * 4;
  for (int s = sg; s < S; s += SG) {
    const float w = w_s[s];
    if (w != 0.f) {
      const float4 v = *(const float4*)(o_in + (int64_t)s * p.heads * kDV);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  if (SG > 1) {
    if (sg > 0) acc_s[sg - 1][c4] = acc;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
      for (int i = 0; i < SG - 1; ++i) {
        const float4 v = acc_s[i][c4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
  }
  if (sg != 0) return;
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  const int64_t th = (int64_t)tok * p.heads + h;
  *(uint2*)(p.out + th * kDV + c4 * 4) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  if (tid == 0) p.lse[th] = any ? mx + __logf(wsum) : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int HG, int NCS, int TR>
static hipError_t launch_split_t(const SplitParams& p, int hblocks, hipStream_t st) {
  const int64_t nwg = (int64_t)p.nsplit * p.tokens * hblocks;
  hipLaunchKernelGGL((split_kernel<HG, NCS, TR>), dim3((unsigned)nwg), dim3(64 * HG * NCS), 0,
                     st, p);
  return hipGetLastError();
}

hipError_t launch_split(const SplitParams& p, hipStream_t st) {
  if (p.heads <= 16) return launch_split_t<1, 4, 32>(p, 1, st);
  if (p.heads <= 32) return launch_split_t<2, 2, 32>(p, 1, st);
  return launch_split_t<4, 2, 64>(p, (p.heads + 63) / 64, st);
}

int split_heads_per_block(int heads) { return heads <= 16 ? 16 : heads <= 32 ? 32 : 64; }

template <int SG>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t st) {
  const int64_t nwg = (int64_t)p.tokens * p.heads;
  hipLaunchKernelGGL((combine_kernel<SG>), dim3((unsigned)nwg), dim3(128 * SG), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t st) {
  // more split groups when there are many splits per (token, head)
  if (p.nsplit >= 32) return launch_combine_t<8>(p, st);
  if (p.nsplit >= 8) return launch_combine_t<4>(p, st);
  if (p.nsplit >= 2) return launch_combine_t<2>(p, st);
  return launch_combine_t<1>(p, st);
}

}  // namespace smla
