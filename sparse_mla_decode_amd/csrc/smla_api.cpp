// smla_api.cpp -- the C ABI declared in include/smla.h: argument validation,
// the NSPLIT planner, workspace sizing and kernel launches.  Host code only;
// the kernels live in smla_kernels.hip.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/smla.h"
#include "smla_internal.h"

#define SMLA_API extern "C" __attribute__((visibility("default")))

namespace {

static_assert(SMLA_MAX_NSPLIT == smla::kMaxNsplit, "limits out of sync");
static_assert(SMLA_ROW == smla::kRow && SMLA_DV == smla::kDV, "widths out of sync");

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// CU count of the current device, queried once per device.
int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SMLA_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return SMLA_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      c <= 0) {
    (void)hipGetLastError();
    return SMLA_ERR_DEVICE;
  }
  if (dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return SMLA_OK;
}

bool dims_ok(int batch, int q_len, int heads, int topk) {
  if (batch < 0 || q_len < 0 || topk < 0 || topk > SMLA_MAX_TOPK) return false;
  if (heads < 1 || heads > SMLA_MAX_HEADS) return false;
  const int64_t tokens = (int64_t)batch * q_len;
  return tokens <= (int64_t)1 << 30;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// workspace: part_o at offset 0, then part_lse at a 256-byte boundary
size_t lse_offset(int64_t tokens, int heads, int nsplit) {
  return round_up((size_t)tokens * nsplit * heads * SMLA_DV * sizeof(float), 256);
}

size_t ws_bytes(int64_t tokens, int heads, int nsplit) {
  if (nsplit <= 1) return 0;
  return lse_offset(tokens, heads, nsplit) + (size_t)tokens * nsplit * heads * sizeof(float);
}

// Where a call's rows come from (smla::RowSource and its tables).
struct Source {
  int src = smla::kSrcRows;
  const int32_t* idx = nullptr;    // rows or positions [T, topk]
  const int32_t* table = nullptr;  // [batch, max_pages] or null
  const int32_t* ctx = nullptr;    // [batch] (dense)
  int max_pages = 0, page_size = 1;
};

// A dense call's q_len tokens attend to the same positions, so they can be
// folded into the head dimension: q [B, q_len, H, 576] is q [B, 1, q_len*H,
// 576] byte for byte (out and lse likewise), and each context row is then
// gathered once per head block rather than once per token.  Folding moves the
// call to the larger head-block kernel, whose start-up costs more, so it pays
// only for long contexts (measured for 9 tokens x 8 heads: 18.9 vs 22.0 us at
// 4096 positions unfolded vs folded, 33.8 vs 29.1 at 16384, 93 vs 48 at 65536).
constexpr int kDenseFoldMinCtx = 8192;
bool dense_folds(int q_len, int heads, int max_ctx) {
  return q_len > 1 && (int64_t)q_len * heads <= SMLA_MAX_HEADS && max_ctx >= kDenseFoldMinCtx;
}

// Whether a decode call with NSPLIT > 1 merges inside the split launch: its
// (token, head block) units fit the sync words (16 bytes each), NSPLIT fits
// the 64-bit claim mask, and the grid fits the device's resident workgroups.
int single_launch(int64_t tokens, int heads, int nsplit, int* single) {
  *single = 0;
  if (nsplit < 2 || nsplit > SMLA_FUSED_MAX_NSPLIT) return SMLA_OK;
  int cus = 0;
  const int rc = device_cus(&cus);
  if (rc != SMLA_OK) return rc;
  const int hpb = smla::split_heads_per_block(heads);
  const int64_t units = tokens * ((heads + hpb - 1) / hpb);
  *single = units <= SMLA_FUSED_SYNC_BYTES / 16 &&
            nsplit * units <= (int64_t)cus * smla::split_blocks_per_cu(heads);
  return SMLA_OK;
}

// The single-launch merge's arguments (smla_decode_fused).
struct Fused {
  uint32_t* sync = nullptr;
  size_t sync_bytes = 0;
  int merge_polls = 0;
};

// Shared by every decode entry point (combine = true) and smla_split
// (combine = false); fused (non-null): merge inside the split launch when
// single_launch allows it.  topk is the list length (the longest context
// when dense).
int run(const void* q, const void* kv, const Source& so, void* out, float* lse, float scale,
        int nsplit, int batch, int q_len, int heads, int topk, int64_t kv_rows, void* ws,
        size_t ws_size, void* stream, bool combine, const Fused* fused = nullptr) {
  if (!dims_ok(batch, q_len, heads, topk) || kv_rows < 0) return SMLA_ERR_DIM;
  if (so.table && (so.page_size < 1 || so.max_pages < 0)) return SMLA_ERR_DIM;
  if (nsplit < 0 || nsplit > SMLA_MAX_NSPLIT) return SMLA_ERR_NSPLIT;
  if (fused && fused->merge_polls < 0) return SMLA_ERR_DIM;
  const int64_t tokens = (int64_t)batch * q_len;
  if (tokens == 0) return SMLA_OK;  // nothing to compute, nothing written

  if (nsplit == 0) {
    int cus = 0;
    const int rc = device_cus(&cus);
    if (rc != SMLA_OK) return rc;
    nsplit = smla_plan_nsplit_cus(cus, batch, q_len, heads, topk);
    if (nsplit < 1) return nsplit;
  }
  const bool partials = nsplit > 1;
  const bool writes_out = !partials || combine;

  const bool lists = so.src != smla::kSrcDense;
  if (!q || (lists && topk > 0 && !so.idx) || (kv_rows > 0 && !kv)) return SMLA_ERR_NULL;
  if (so.src == smla::kSrcPositions && !so.table) return SMLA_ERR_NULL;
  if (so.src == smla::kSrcDense && !so.ctx) return SMLA_ERR_NULL;
  if (writes_out && (!out || !lse)) return SMLA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(so.idx, 4) || !aligned(so.table, 4) ||
      !aligned(so.ctx, 4))
    return SMLA_ERR_ALIGN;
  if (writes_out && (!aligned(out, 16) || !aligned(lse, 4))) return SMLA_ERR_ALIGN;
  if (partials) {
    if (!ws || ws_size < ws_bytes(tokens, heads, nsplit)) return SMLA_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return SMLA_ERR_ALIGN;
  }
  const int64_t hblocks = (heads + smla::split_heads_per_block(heads) - 1) /
                          smla::split_heads_per_block(heads);
  if ((int64_t)nsplit * tokens * hblocks > 0x7fffffffLL) return SMLA_ERR_DIM;

  hipStream_t st = (hipStream_t)stream;
  smla::SplitParams sp;
  sp.q = (const uint16_t*)q;
  sp.kv = (const uint16_t*)kv;
  sp.idx = so.idx;
  sp.src = so.src;
  sp.table = so.src == smla::kSrcRows ? nullptr : so.table;
  sp.ctx = so.ctx;
  sp.max_pages = so.max_pages;
  sp.page_size = so.page_size;
  sp.q_len = q_len;
  sp.out = (uint16_t*)out;
  sp.lse = lse;
  sp.part_o = partials ? (float*)ws : nullptr;
  sp.part_lse = partials ? (float*)((char*)ws + lse_offset(tokens, heads, nsplit)) : nullptr;
  sp.kv_rows = kv_rows;
  sp.tokens = (int)tokens;
  sp.heads = heads;
  sp.topk = topk;
  sp.nsplit = nsplit;
  sp.per_split = topk == 0 ? 0 : (topk + nsplit - 1) / nsplit;
  sp.scale_log2 = scale * smla::kLog2e;
  // the merge runs inside the split launch when the unit's workgroups can all
  // be resident at once (so none waits on one that has not started) and the
  // unit count and NSPLIT fit the workspace's sync words; else a second launch
  sp.sync = nullptr;
  sp.merge_polls = 0;
  if (partials && combine && fused) {
    int single = 0;
    const int rc = single_launch(tokens, heads, nsplit, &single);
    if (rc != SMLA_OK) return rc;
    if (single) {
      if (!fused->sync) return SMLA_ERR_NULL;
      if (!aligned(fused->sync, 4)) return SMLA_ERR_ALIGN;
      if (fused->sync_bytes < SMLA_FUSED_SYNC_BYTES) return SMLA_ERR_WORKSPACE;
      sp.sync = fused->sync;
      sp.merge_polls = fused->merge_polls;
    }
  }
  if (smla::launch_split(sp, st) != hipSuccess) {
    (void)hipGetLastError();
    return SMLA_ERR_LAUNCH;
  }
  if (partials && combine && !sp.sync) {
    smla::CombineParams cp;
    cp.part_o = sp.part_o;
    cp.part_lse = sp.part_lse;
    cp.out = (uint16_t*)out;
    cp.lse = lse;
    cp.tokens = (int)tokens;
    cp.heads = heads;
    cp.nsplit = nsplit;
    if (smla::launch_combine(cp, st) != hipSuccess) {
      (void)hipGetLastError();
      return SMLA_ERR_LAUNCH;
    }
  }
  return SMLA_OK;
}

}  // namespace

SMLA_API int smla_plan_nsplit_cus(int cus, int batch, int q_len, int heads, int topk) {
  if (cus < 1 || !dims_ok(batch, q_len, heads, topk)) return SMLA_ERR_DIM;
  const int64_t tokens = (int64_t)batch * q_len;
  if (tokens == 0 || topk == 0) return 1;
  const int hpb = smla::split_heads_per_block(heads);
  const int64_t units = tokens * ((heads + hpb - 1) / hpb);  // workgroups per split
  // A split workgroup costs a fixed start-up (list, q, first gather) plus one
  // step per 32-row tile, and at small batch the whole call is one such
  // latency chain.  So: the most splits whose workgroups get a CU each (one
  // workgroup per CU: where LDS would fit two, the second on a CU ran no
  // faster than one more tile per workgroup, and more splits cost the combine
  // more; measured on 9 tokens x 8 heads: 22 splits of 3 tiles 13.3 us per
  // step, 32 of 2 tiles 14.5 us), each split at least one whole tile ...
  constexpr int kTile = smla::kTileRows;
  const int64_t slots = cus;
  int64_t ns = slots / units;
  const int64_t max_ns = topk / kTile;
  if (ns > max_ns) ns = max_ns;
  if (ns > SMLA_MAX_NSPLIT) ns = SMLA_MAX_NSPLIT;
  if (ns < 1) ns = 1;
  // ... then the fewest splits with that many tiles each: same latency, fewer
  // workgroups and less partial (O, LSE) traffic for the combine
  const int64_t tiles = ((topk + ns - 1) / ns + kTile - 1) / kTile;
  ns = (topk + tiles * kTile - 1) / (tiles * kTile);
  return (int)ns;
}

SMLA_API int smla_plan_nsplit(int batch, int q_len, int heads, int topk) {
  if (!dims_ok(batch, q_len, heads, topk)) return SMLA_ERR_DIM;
  int cus = 0;
  const int rc = device_cus(&cus);
  if (rc != SMLA_OK) return rc;
  return smla_plan_nsplit_cus(cus, batch, q_len, heads, topk);
}

SMLA_API size_t smla_workspace_bytes(int batch, int q_len, int heads, int nsplit) {
  if (batch < 0 || q_len < 0 || heads < 1 || nsplit < 0) return 0;
  return ws_bytes((int64_t)batch * q_len, heads, nsplit);
}

SMLA_API int smla_fused_in_launch(int batch, int q_len, int heads, int nsplit) {
  if (batch < 0 || q_len < 0 || heads < 1 || heads > SMLA_MAX_HEADS) return SMLA_ERR_DIM;
  if (nsplit < 1 || nsplit > SMLA_MAX_NSPLIT) return SMLA_ERR_NSPLIT;
  int single = 0;
  const int rc = single_launch((int64_t)batch * q_len, heads, nsplit, &single);
  return rc != SMLA_OK ? rc : single;
}

SMLA_API size_t smla_workspace_lse_offset(int batch, int q_len, int heads, int nsplit) {
  if (batch < 0 || q_len < 0 || heads < 1 || nsplit < 1) return 0;
  return lse_offset((int64_t)batch * q_len, heads, nsplit);
}

SMLA_API int smla_decode(const void* q, const void* kv_cache, const int32_t* topk_idx, void* out,
                         float* lse, float scale, int nsplit, int batch, int q_len, int heads,
                         int topk, int64_t kv_rows, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  Source so;
  so.idx = topk_idx;
  return run(q, kv_cache, so, out, lse, scale, nsplit, batch, q_len, heads, topk, kv_rows,
             workspace, workspace_bytes, hip_stream, true);
}

SMLA_API int smla_decode_fused(const void* q, const void* kv_cache, const int32_t* topk_idx,
                               void* out, float* lse, float scale, int nsplit, int batch,
                               int q_len, int heads, int topk, int64_t kv_rows, void* workspace,
                               size_t workspace_bytes, uint32_t* sync, size_t sync_bytes,
                               int merge_polls, void* hip_stream) {
  Source so;
  so.idx = topk_idx;
  Fused fu;
  fu.sync = sync;
  fu.sync_bytes = sync_bytes;
  fu.merge_polls = merge_polls;
  return run(q, kv_cache, so, out, lse, scale, nsplit, batch, q_len, heads, topk, kv_rows,
             workspace, workspace_bytes, hip_stream, true, &fu);
}

SMLA_API int smla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_table,
                               int max_pages, int page_size, const int32_t* topk_pos, void* out,
                               float* lse, float scale, int nsplit, int batch, int q_len,
                               int heads, int topk, int64_t kv_rows, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  Source so;
  so.src = smla::kSrcPositions;
  so.idx = topk_pos;
  so.table = block_table;
  so.max_pages = max_pages;
  so.page_size = page_size;
  return run(q, kv_cache, so, out, lse, scale, nsplit, batch, q_len, heads, topk, kv_rows,
             workspace, workspace_bytes, hip_stream, true);
}

SMLA_API int smla_decode_dense(const void* q, const void* kv_cache, const int32_t* block_table,
                               int max_pages, int page_size, const int32_t* ctx_len, int max_ctx,
                               void* out, float* lse, float scale, int nsplit, int batch,
                               int q_len, int heads, int64_t kv_rows, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  Source so;
  so.src = smla::kSrcDense;
  so.table = block_table;
  so.ctx = ctx_len;
  so.max_pages = block_table ? max_pages : 0;
  so.page_size = page_size;
  if (dense_folds(q_len, heads, max_ctx))
    return run(q, kv_cache, so, out, lse, scale, nsplit, batch, 1, q_len * heads, max_ctx,
               kv_rows, workspace, workspace_bytes, hip_stream, true);
  return run(q, kv_cache, so, out, lse, scale, nsplit, batch, q_len, heads, max_ctx, kv_rows,
             workspace, workspace_bytes, hip_stream, true);
}

SMLA_API int smla_plan_nsplit_dense(int batch, int q_len, int heads, int max_ctx) {
  if (!dims_ok(batch, q_len, heads, max_ctx)) return SMLA_ERR_DIM;
  if (dense_folds(q_len, heads, max_ctx)) return smla_plan_nsplit(batch, 1, q_len * heads, max_ctx);
  return smla_plan_nsplit(batch, q_len, heads, max_ctx);
}

SMLA_API int smla_split(const void* q, const void* kv_cache, const int32_t* topk_idx, void* out,
                        float* lse, float scale, int nsplit, int batch, int q_len, int heads,
                        int topk, int64_t kv_rows, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  Source so;
  so.idx = topk_idx;
  return run(q, kv_cache, so, out, lse, scale, nsplit, batch, q_len, heads, topk, kv_rows,
             workspace, workspace_bytes, hip_stream, false);
}

SMLA_API int smla_combine(const float* part_o, const float* part_lse, void* out, float* lse,
                          int tokens, int heads, int nsplit, void* hip_stream) {
  if (tokens < 0 || heads < 1 || heads > SMLA_MAX_HEADS) return SMLA_ERR_DIM;
  if (nsplit < 1 || nsplit > SMLA_MAX_NSPLIT) return SMLA_ERR_NSPLIT;
  if (tokens == 0) return SMLA_OK;
  if (!part_o || !part_lse || !out || !lse) return SMLA_ERR_NULL;
  if (!aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(out, 16) || !aligned(lse, 4))
    return SMLA_ERR_ALIGN;
  if ((int64_t)tokens * heads > 0x7fffffffLL) return SMLA_ERR_DIM;
  smla::CombineParams cp;
  cp.part_o = part_o;
  cp.part_lse = part_lse;
  cp.out = (uint16_t*)out;
  cp.lse = lse;
  cp.tokens = tokens;
  cp.heads = heads;
  cp.nsplit = nsplit;
  if (smla::launch_combine(cp, (hipStream_t)hip_stream) != hipSuccess) {
    (void)hipGetLastError();
    return SMLA_ERR_LAUNCH;
  }
  return SMLA_OK;
}

// the multi-workgroup top-k forms pay for their extra launch(es) when the
// rows alone leave CUs idle and rows are long (measured: 1 x 65536 and 128
// rows up to 131072 gain, 64 x 32768 loses)
constexpr int kTopkMultiMinChunks = 12;  // 45057 positions and more
bool topk_multi_auto(int64_t rows, int max_ctx, int cus) {
  return rows < 2 * (int64_t)cus && smla::topk_chunks(max_ctx, 1) >= kTopkMultiMinChunks;
}
// sub-chunks per chunk workgroup: as many as keep about kTopkChunkWgPerCu
// chunk workgroups per CU (one when a few rows need every chunk to fill the
// device; measured on 128 rows up to 131072 with four launches: 4 per CU
// 44.7 us, 2 per CU 50.0, 8 per CU 46.8)
constexpr int kTopkChunkWgPerCu = 4;
int topk_sub(int64_t rows, int max_ctx, int cus) {
  const int64_t subs = rows * smla::topk_chunks(max_ctx, 1);
  const int64_t s = subs / ((int64_t)kTopkChunkWgPerCu * cus);
  return (int)(s < 1 ? 1 : s > 8 ? 8 : s);
}

SMLA_API size_t smla_topk_workspace_bytes(int batch, int q_len, int max_ctx) {
  if (batch < 0 || q_len < 0 || max_ctx < 0) return 0;
  return (size_t)batch * q_len * smla::topk_ws_row_bytes(max_ctx);
}

SMLA_API int smla_topk(const float* scores, const int32_t* ctx_len, int batch, int q_len,
                       int max_ctx, int topk, int32_t* out_pos, void* workspace,
                       size_t workspace_bytes, int form, void* hip_stream) {
  if (batch < 0 || q_len < 0 || max_ctx < 0 || topk < 0 || topk > SMLA_MAX_TOPK)
    return SMLA_ERR_DIM;
  if (form != SMLA_TOPK_AUTO && form != SMLA_TOPK_ROWS && form != SMLA_TOPK_CHUNKS &&
      form != SMLA_TOPK_SAMPLED)
    return SMLA_ERR_DIM;
  const int64_t rows = (int64_t)batch * q_len;
  if (rows == 0 || topk == 0) return SMLA_OK;
  if (rows > 0x7fffffffLL) return SMLA_ERR_DIM;
  if (!out_pos || (max_ctx > 0 && !scores)) return SMLA_ERR_NULL;
  if (!aligned(scores, 4) || !aligned(ctx_len, 4) || !aligned(out_pos, 4) || !aligned(workspace, 256))
    return SMLA_ERR_ALIGN;
  smla::TopkParams tp;
  tp.scores = scores;
  tp.ctx = ctx_len;
  tp.out = out_pos;
  tp.rows = rows;
  tp.q_len = q_len;
  tp.max_ctx = max_ctx;
  tp.topk = topk;
  tp.ws = nullptr;
  tp.ws_row_bytes = smla::topk_ws_row_bytes(max_ctx);
  tp.sub = 1;
  tp.chunks = smla::topk_chunks(max_ctx, 1);
  tp.sampled = 0;
  // the sampled form takes at most maxc chunks per row and maxs sub-chunks
  // per chunk (rows up to maxc x maxs x 4096 positions): the sub-chunks per
  // chunk it uses for a wish of `sub`, or 0 when max_ctx is too long for it
  const int maxc = smla::topk_sampled_max_chunks(), maxs = smla::topk_sampled_max_sub();
  auto sampled_sub = [&](int sub) {
    const int c1 = smla::topk_chunks(max_ctx, 1);
    const int need = (c1 + maxc - 1) / maxc;
    const int s2 = sub > need ? (sub < maxs ? sub : maxs) : need;
    return s2 <= maxs && s2 >= need ? s2 : 0;
  };
  if (form != SMLA_TOPK_ROWS && workspace && workspace_bytes >= (size_t)rows * tp.ws_row_bytes &&
      rows * tp.chunks <= 0x7fffffffLL && tp.chunks >= 2) {
    if (form == SMLA_TOPK_CHUNKS) {
      int cus = 0;  // sub-chunks per chunk as the automatic choice takes them
      const int rc = device_cus(&cus);
      if (rc != SMLA_OK) return rc;
      tp.ws = workspace;
      tp.sub = topk_sub(rows, max_ctx, cus);
      tp.chunks = smla::topk_chunks(max_ctx, tp.sub);
    } else if (form == SMLA_TOPK_SAMPLED) {
      tp.ws = workspace;  // rows too long for the sampled form: four launches
      const int ss = sampled_sub(1);
      if (ss > 0) {
        tp.sampled = 1;
        tp.sub = ss;
        tp.chunks = smla::topk_chunks(max_ctx, tp.sub);
      }
    } else {
      int cus = 0;
      const int rc = device_cus(&cus);
      if (rc != SMLA_OK) return rc;
      if (topk_multi_auto(rows, max_ctx, cus)) {
        tp.ws = workspace;
        tp.sub = topk_sub(rows, max_ctx, cus);
        const int ss = sampled_sub(tp.sub);  // 0: rows too long for the sampled form
        if (ss > 0) {
          tp.sampled = 1;
          tp.sub = ss;
        }
        tp.chunks = smla::topk_chunks(max_ctx, tp.sub);
      }
    }
  }
  if (smla::launch_topk(tp, (hipStream_t)hip_stream) != hipSuccess) {
    (void)hipGetLastError();
    return SMLA_ERR_LAUNCH;
  }
  return SMLA_OK;
}

SMLA_API const char* smla_status_str(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_NULL: return "a required pointer is NULL";
    case SMLA_ERR_DIM: return "invalid size (negative, zero heads, or above a limit)";
    case SMLA_ERR_NSPLIT: return "nsplit out of range";
    case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SMLA_ERR_ALIGN: return "pointer misaligned";
    case SMLA_ERR_DEVICE: return "no usable device";
    case SMLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
