/*
 * smla.h -- sparse MLA decode attention with split-K over the top-k list,
 * for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes.
 *
 * What is computed.  Every query token t attends only to the cache rows its
 * top-k list selects.  A cache row holds 576 bf16 values: 512 latent columns
 * followed by 64 rope columns; the value vector of a row is its first 512
 * columns, the key is the whole row.  For head h, with J the list entries
 * whose row r satisfies 0 <= r < kv_rows:
 *     s_j = scale * <q[t,h,0:576], kv[r_j,0:576]>
 *     out[t,h,0:512] = sum_j softmax(s)_j kv[r_j,0:512]   (bf16, RNE)
 *     lse[t,h]       = ln sum_j exp(s_j)                   (fp32)
 * An empty J gives out = 0 and lse = -inf.  List entries equal to -1, or any
 * other value outside [0, kv_rows), carry zero weight; they are data, not
 * errors.  Duplicate entries are separate softmax terms.
 *
 * Split-K ("The Moment of Truth: Validating Split-K Parallelization for
 * Blackwell MLA Decode", section "The Split-K Imperative"): the list of each
 * token is cut into NSPLIT contiguous slices of ceil(topk / NSPLIT) entries
 * (the last one short or empty); each slice yields a partial (O, LSE) and a
 * log-sum-exp combine merges the partials in fp32.  NSPLIT multiplies the
 * number of workgroups so that small batches still fill the GPU ("The
 * Occupancy Hypothesis: How One Kernel Parameter Unlocked 1.8x Decode Speedup
 * on Blackwell", sections "The Occupancy Insight" and "The Broader Context").
 *
 * Layouts (contiguous, row-major, device memory):
 *   q          [batch, q_len, heads, 576]   bf16
 *   kv_cache   [kv_rows, 576]               bf16  (a paged pool is passed flat:
 *                                                  physical row = page*64 + slot)
 *   topk_idx   [batch, q_len, topk]         int32 physical row indices
 *   out        [batch, q_len, heads, 512]   bf16
 *   lse        [batch, q_len, heads]        fp32
 *   workspace  part_o [T, NSPLIT, heads, 512] fp32 at byte offset 0, then
 *              part_lse [T, NSPLIT, heads] fp32 at byte offset
 *              smla_workspace_lse_offset (256-byte aligned); T = batch * q_len.
 *              Scratch: any content on entry; after a call with NSPLIT > 1
 *              it holds that call's partials.
 * q, kv_cache, out and workspace must be 16-byte aligned; topk_idx and lse
 * 4-byte aligned.
 *
 * Ownership and execution.  The caller owns every buffer, including the
 * workspace; the library allocates no device memory and keeps no per-call
 * state (its only global is a per-device cache of the CU count).  Work is
 * enqueued on `hip_stream` (a hipStream_t; NULL = the legacy default stream)
 * and the call returns without waiting for it: buffers must stay alive and
 * unmodified until the stream has passed the call.  The calls never
 * synchronise the host, so they can be captured into a HIP graph.  Calls on
 * different streams that share a workspace race.
 *
 * Errors.  Every entry point returns SMLA_OK (0) or a negative smla_status.
 * Arguments are validated before anything is enqueued; on an error nothing is
 * launched and nothing is written.  A failed launch returns SMLA_ERR_LAUNCH
 * (the HIP error state is cleared).  Faults inside a kernel surface at the
 * caller's next synchronisation.  NaN or Inf inside q or the selected rows
 * propagate; they are not checked.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum smla_status {
  SMLA_OK = 0,
  SMLA_ERR_NULL = -1,      /* a required pointer is NULL */
  SMLA_ERR_DIM = -2,       /* a size is negative, zero where it must not be, or above a limit */
  SMLA_ERR_NSPLIT = -3,    /* nsplit < 0 or > SMLA_MAX_NSPLIT */
  SMLA_ERR_WORKSPACE = -4, /* nsplit > 1 and the workspace is NULL or too small */
  SMLA_ERR_ALIGN = -5,     /* a pointer breaks the alignment rules above */
  SMLA_ERR_DEVICE = -6,    /* no usable gfx950 device / device query failed */
  SMLA_ERR_LAUNCH = -7     /* a kernel launch failed */
};

#define SMLA_ROW 576          /* q and cache row width (bf16 elements) */
#define SMLA_DV 512           /* value / output width (bf16 elements) */
#define SMLA_MAX_NSPLIT 1024  /* largest NSPLIT accepted */
#define SMLA_MAX_HEADS 4096   /* largest head count accepted */
#define SMLA_MAX_TOPK (1 << 24)
#define SMLA_FUSED_SYNC_BYTES 16384  /* synchronisation words of smla_decode_fused */
#define SMLA_FUSED_MAX_NSPLIT 64     /* largest NSPLIT merged inside the split launch */
#define SMLA_NOALLOC_SCRATCH_BYTES (64 << 20) /* partials area of smla_decode_noalloc */

/*
 * NSPLIT the planner picks for a call of this shape on the current device
 * (its CU count is queried once per device).  Returns >= 1, or a negative
 * status (SMLA_ERR_DIM for bad sizes, SMLA_ERR_DEVICE if no device).
 */
int smla_plan_nsplit(int batch, int q_len, int heads, int topk);

/*
 * The same planner as a pure function of the CU count: no device access, so
 * it runs (and is tested) on hosts without a GPU.  The rule: the largest
 * NSPLIT whose workgroups (batch * q_len * head blocks * NSPLIT) get one CU
 * each, with at least one 32-row tile per split; then the fewest splits
 * that keep the same number of tiles per split.  It
 * fills every CU at batch 1 and drops to NSPLIT 1 once the batch alone
 * fills the device ("The Occupancy Hypothesis", "The Occupancy Insight":
 * blocks in flight, not per-block work, hide memory latency; "The Split-K
 * Imperative": split the list only as far as the grid needs).
 */
int smla_plan_nsplit_cus(int cus, int batch, int q_len, int heads, int topk);

/* Bytes of workspace smla_decode / smla_split need (0 when nsplit <= 1). */
size_t smla_workspace_bytes(int batch, int q_len, int heads, int nsplit);

/* Byte offset of part_lse inside the workspace (256-byte aligned). */
size_t smla_workspace_lse_offset(int batch, int q_len, int heads, int nsplit);

/*
 * 1 if smla_decode_fused with this shape and an explicit nsplit merges the
 * partials inside the split launch (the conditions stated there), 0 if it
 * launches the combine kernel too (or nsplit == 1: no merge at all), or a
 * negative smla_status.  Uses the current device's CU count.
 */
int smla_fused_in_launch(int batch, int q_len, int heads, int nsplit);

/*
 * Full decode: the split kernel over every (token, split) and, when
 * NSPLIT > 1, the combine kernel (smla_combine).  nsplit == 0 asks the planner
 * (smla_plan_nsplit); size the workspace with smla_workspace_bytes for the
 * NSPLIT actually used.  nsplit > topk is allowed (surplus splits are empty).
 * batch == 0, q_len == 0 or topk == 0 are valid: the first two launch
 * nothing; topk == 0 writes out = 0, lse = -inf.
 */
int smla_decode(const void *q, const void *kv_cache, const int32_t *topk_idx, void *out,
                float *lse, float scale, int nsplit, int batch, int q_len, int heads, int topk,
                int64_t kv_rows, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * smla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument.  The partials of a call with NSPLIT > 1 go to a static
 * device array of SMLA_NOALLOC_SCRATCH_BYTES per device, which the library
 * holds until the process ends; a call whose partials need more
 * (smla_workspace_bytes above that) returns SMLA_ERR_WORKSPACE and launches
 * nothing.  Every call on a device shares that device's array, which keeps
 * the last call's partials: calls that overlap on one device (on different
 * streams, or from host threads with no order between them) race.  The first
 * call on a device looks up the array's device address (SMLA_ERR_DEVICE if
 * that fails).  Allocates and frees nothing.  Other arguments, results and
 * errors as smla_decode.
 */
int smla_decode_noalloc(const void *q, const void *kv_cache, const int32_t *topk_idx, void *out,
                        float *lse, float scale, int nsplit, int batch, int q_len, int heads,
                        int topk, int64_t kv_rows, void *hip_stream);

/*
 * smla_decode with the log-sum-exp merge inside the split launch (one kernel
 * instead of two; "The Split-K Imperative": the partials of the slices are
 * merged by log-sum-exp), when 2 <= NSPLIT <= SMLA_FUSED_MAX_NSPLIT,
 * tokens * head blocks <= SMLA_FUSED_SYNC_BYTES / 16 (head blocks of 16, 32
 * or 64 heads, by head count) and the grid fits the device's resident
 * workgroups (smla_fused_in_launch); otherwise exactly smla_decode (the
 * sync words are then not touched).
 *   sync [SMLA_FUSED_SYNC_BYTES] (4-byte aligned): synchronisation words of
 *     the in-launch merge, owned by the caller.  They must be zero before
 *     their first use and every call leaves them zero, whatever its shape,
 *     so one zeroed buffer serves any sequence of calls on one stream.  May
 *     be NULL when the call does not merge in the launch.
 *   merge_polls (>= 0): bound on the polls (each a short sleep and one
 *     device-scope load) of a workgroup waiting for the other partials of
 *     its unit; 0 = never wait, the last workgroup to arrive merges the
 *     whole unit (same results, bit for bit).  2048 is a good default.
 * The NSPLIT workgroups of a (token, head block) write their partials with
 * device-coherent stores, then take a ticket with an agent-scope release;
 * a workgroup that sees every ticket out (an agent-scope acquire) merges
 * one slice of the output, and the last to arrive merges the slices of any
 * that stopped waiting, so no wait is unbounded even on a shared device.
 * Same arithmetic as smla_combine; the merge order within a slice is fixed,
 * so results repeat bit for bit.  On MI355X this form is slower than the two
 * launches of smla_decode (its cross-XCD handoffs cost more than a kernel
 * boundary); it serves callers that need a single launch.  Other arguments,
 * the workspace and the errors as smla_decode; SMLA_ERR_NULL if the call
 * merges in the launch and sync is NULL, SMLA_ERR_WORKSPACE if sync_bytes <
 * SMLA_FUSED_SYNC_BYTES, SMLA_ERR_DIM if merge_polls < 0.
 */
int smla_decode_fused(const void *q, const void *kv_cache, const int32_t *topk_idx, void *out,
                      float *lse, float scale, int nsplit, int batch, int q_len, int heads,
                      int topk, int64_t kv_rows, void *workspace, size_t workspace_bytes,
                      uint32_t *sync, size_t sync_bytes, int merge_polls, void *hip_stream);

/*
 * smla_decode over a paged cache, with the page-table lookup done in the
 * kernel ("The Occupancy Hypothesis", "The Road to This Experiment": the
 * serving cache is reached through per-sequence page tables).
 *   block_table [batch, max_pages] int32: page ids of each sequence's pages
 *     in order; a page id < 0 marks no page.  Required (non-NULL).
 *   page_size: tokens per page (>= 1); the cache holds page id p's token t at
 *     row p * page_size + t.
 *   topk_pos [batch, q_len, topk] int32: positions within the token's own
 *     sequence (not rows).  Position x maps to row
 *     block_table[b][x / page_size] * page_size + x % page_size.
 * A position that is < 0 or beyond the table (x / page_size >= max_pages), a
 * missing page, or a row outside [0, kv_rows) carries zero weight, like -1 in
 * smla_decode.  Results equal smla_decode's on the translated rows, bit for
 * bit.  Rows must fit in int32.  Other arguments, the workspace and the
 * errors as smla_decode.
 */
int smla_decode_paged(const void *q, const void *kv_cache, const int32_t *block_table,
                      int max_pages, int page_size, const int32_t *topk_pos, void *out,
                      float *lse, float scale, int nsplit, int batch, int q_len, int heads,
                      int topk, int64_t kv_rows, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/*
 * Dense KV-split decode: every query token of sequence b attends to all
 * positions 0 .. ctx_len[b]-1 of its sequence, split into NSPLIT contiguous
 * slices ("The Occupancy Hypothesis", "The Occupancy Insight" and "The
 * Broader Context": the verify kernel splits the whole context, flash-decode
 * style, partial + reduce).  There is no list: the implicit list of a token
 * is 0 .. max_ctx-1, and entries at or beyond ctx_len[b] are masked.
 *   ctx_len [batch] int32 (>= 0; values above max_ctx are attended only up to
 *     max_ctx);  max_ctx: the longest context, the implicit list length
 *     (plays topk's part for the planner and the workspace).
 *   block_table / max_pages / page_size: as smla_decode_paged, or block_table
 *     NULL for a flat cache in which position x is row x.
 * Results equal smla_decode with topk_idx[b, i, :] = the rows of positions
 * 0 .. ctx_len[b]-1 (then -1).  Since the q_len tokens of a sequence share
 * those positions, for long contexts (max_ctx >= 8192, q_len > 1, q_len*heads
 * <= SMLA_MAX_HEADS) the call treats them as q_len*heads heads of one token
 * (q, out and lse are laid out alike either way): each context row is then
 * gathered once per head block, not once per token.  NSPLIT 0 asks
 * smla_plan_nsplit_dense; the workspace size is the same for either view.
 * Errors as smla_decode (SMLA_ERR_NULL if ctx_len is NULL).
 */
/*
 * NSPLIT the planner picks for smla_decode_dense of this shape: the
 * smla_plan_nsplit rule applied to the shape the call runs as (folded or
 * not, see smla_decode_dense).  Same returns as smla_plan_nsplit.
 */
int smla_plan_nsplit_dense(int batch, int q_len, int heads, int max_ctx);

int smla_decode_dense(const void *q, const void *kv_cache, const int32_t *block_table,
                      int max_pages, int page_size, const int32_t *ctx_len, int max_ctx,
                      void *out, float *lse, float scale, int nsplit, int batch, int q_len,
                      int heads, int64_t kv_rows, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/*
 * The split kernel alone ("The Split-K Imperative": each block computes a
 * partial attention output over its slice of the list).  With NSPLIT > 1 it
 * writes part_o / part_lse into the workspace (layout above; an empty slice
 * gives O = 0, LSE = -inf) and leaves out / lse untouched (they may be NULL);
 * with NSPLIT == 1 it writes out / lse directly.  Arguments as smla_decode.
 */
int smla_split(const void *q, const void *kv_cache, const int32_t *topk_idx, void *out,
               float *lse, float scale, int nsplit, int batch, int q_len, int heads, int topk,
               int64_t kv_rows, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * The combine kernel alone ("The Split-K Imperative": the log-sum-exp
 * combine merges the partials).  For every (token, head): M = max_s LSE_s;
 * M = -inf gives out = 0, lse = -inf; else w_s = exp(LSE_s - M),
 * out = sum_s w_s O_s / sum_s w_s (fp32, then bf16 RNE), lse = M + ln sum_s w_s.
 * A split with LSE_s = -inf has weight 0 and its O_s slot is not used, so it
 * may hold anything (NaN included).
 * part_o [tokens, nsplit, heads, 512] fp32 (16-byte aligned),
 * part_lse [tokens, nsplit, heads] fp32; 1 <= nsplit <= SMLA_MAX_NSPLIT.
 */
int smla_combine(const float *part_o, const float *part_lse, void *out, float *lse, int tokens,
                 int heads, int nsplit, void *hip_stream);

/*
 * Top-k producer, the step before the path ("The Negative Result That
 * Refined the Hunt", section "The Context": an indexer selects the candidate
 * positions; "The Moment of Truth", section "The Split-K Imperative": the
 * top-k set is the set of candidate tokens retrieved from the cache).  The
 * pages give no indexer math: the scores are an input.  For every row (b, t)
 * of scores [batch, q_len, max_ctx] fp32 (row stride max_ctx), with
 * n = min(max(ctx_len[b], 0), max_ctx) (ctx_len NULL: n = max_ctx), writes to
 * out_pos [batch, q_len, topk] int32 the positions of the topk largest
 * scores among positions 0 .. n-1, in ascending position order; when
 * n <= topk, positions 0 .. n-1 followed by -1.  Ranking: the IEEE total
 * order of the fp32 bit patterns (-NaN < -inf < ... < -0 < +0 < ... < +inf <
 * +NaN), equal values ranking the lower position first, so the selected set
 * is unique.  The output is the topk_pos of smla_decode_paged (or, for a flat
 * cache where positions are rows, the topk_idx of smla_decode).  scores,
 * ctx_len and out_pos 4-byte aligned; scores may be NULL when max_ctx == 0.
 * batch, q_len or topk 0 launch nothing.
 *
 * Work split (`form`).  SMLA_TOPK_ROWS: one workgroup selects each row.
 * SMLA_TOPK_CHUNKS: when a workspace of smla_topk_workspace_bytes is given
 * and a row spans at least two chunks of 4096 positions, each row is cut
 * into chunks over several workgroups (four launches: chunk histograms, a
 * row scan, candidate lists in position order, the selection), else as
 * SMLA_TOPK_ROWS.  A chunk is one or more sub-chunks of 4096 positions,
 * about four chunk workgroups per CU.  SMLA_TOPK_SAMPLED: as SMLA_TOPK_CHUNKS, but in two
 * launches that read the scores once: each chunk workgroup takes a
 * threshold from a fixed sample of its row and writes its keys at or above
 * it, and one workgroup per row selects among them (rows where the
 * threshold proves too high or a chunk's share of the candidate list
 * overflows are selected by one workgroup from the whole row, so the output
 * is exact); rows longer than 1048576 positions take the four launches.
 * SMLA_TOPK_AUTO: the sampled form when the chunked forms were measured
 * faster (a workspace is given, there are fewer rows than twice the CUs and
 * a row spans at least 12 chunks), else one workgroup per row.  Every form
 * gives the same output.  The workspace (256-byte aligned) is scratch: any
 * content on entry, nothing kept after the call.
 * Errors as smla_decode (SMLA_ERR_DEVICE only when SMLA_TOPK_AUTO or
 * SMLA_TOPK_CHUNKS with a workspace needs the CU count and it cannot be
 * read; SMLA_ERR_DIM for an unknown form).
 */
int smla_topk(const float *scores, const int32_t *ctx_len, int batch, int q_len, int max_ctx,
              int topk, int32_t *out_pos, void *workspace, size_t workspace_bytes, int form,
              void *hip_stream);

enum smla_topk_form { SMLA_TOPK_AUTO = 0, SMLA_TOPK_ROWS = 1, SMLA_TOPK_CHUNKS = 2, SMLA_TOPK_SAMPLED = 3 };

/* Bytes of workspace for smla_topk's multi-workgroup form. */
size_t smla_topk_workspace_bytes(int batch, int q_len, int max_ctx);

/* Static description of a status code (never NULL). */
const char *smla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
