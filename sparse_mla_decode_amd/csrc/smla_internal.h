// smla_internal.h -- parameter blocks shared by the C-ABI layer and the
// gfx950 kernels.  Not part of the public interface (include/smla.h is).
#ifndef SMLA_INTERNAL_H
#define SMLA_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kRow = 576;          // q / cache row width (bf16)
constexpr int kDV = 512;           // value width (bf16)
constexpr int kMaxNsplit = 1024;   // must equal SMLA_MAX_NSPLIT
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
// the running max of a head moves only when a tile max exceeds it by this
// much (base-2 exponent), bounding the unnormalised weights by 2^8
constexpr float kRescaleLog2 = 8.0f;
// rows of the list a split workgroup gathers and contracts per step
constexpr int kTileRows = 32;
// list entries a split workgroup stages in LDS at a time
constexpr int kListCap = 2048;
// ... per configuration: the K-split workgroup whose 4 waves share one head
// group (column quarters) stages half as many, so that two fit a CU's LDS
constexpr int split_list_cap(int ncs, int ks) { return ks == 2 && ncs == 4 ? 1024 : kListCap; }

// Where the rows of a token's list come from.
enum RowSource : int {
  kSrcRows = 0,       // idx holds cache rows
  kSrcPositions = 1,  // idx holds positions in the token's sequence, mapped to
                      // rows through the sequence's page table
  kSrcDense = 2,      // no list: entry e is position e of the sequence (e <
                      // ctx[b]), mapped through the page table if there is one
};

struct SplitParams {
  const uint16_t* q;    // [T, H, 576] bf16 bits
  const uint16_t* kv;   // [kv_rows, 576]
  const int32_t* idx;   // [T, topk] (rows or positions; unused when dense)
  int src;              // RowSource
  const int32_t* table; // [batch, max_pages] page ids (-1 = none), or null:
                        // positions are rows
  const int32_t* ctx;   // [batch] context lengths (dense)
  int max_pages, page_size, q_len;
  uint16_t* out;        // [T, H, 512] bf16 (nsplit == 1)
  float* lse;           // [T, H]            (nsplit == 1)
  float* part_o;        // [T, S, H, 512]    (nsplit > 1)
  float* part_lse;      // [T, S, H]         (nsplit > 1)
  uint32_t* sync;       // [units][4] single-launch combine words (zero between
                        // calls), or null: partials only
  int merge_polls;      // bound on a waiting workgroup's polls (single launch)
  int64_t kv_rows;
  int tokens, heads, topk, nsplit, per_split;
  float scale_log2;     // scale * log2(e): scores are kept in base 2
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int tokens, heads, nsplit;
};

struct TopkParams {
  const float* scores;  // [rows, max_ctx] fp32 index scores
  const int32_t* ctx;   // [batch] valid positions per sequence, or null: max_ctx
  int32_t* out;         // [rows, topk] selected positions, ascending, -1 padded
  int64_t rows;         // batch * q_len
  int q_len, max_ctx, topk;
  void* ws;             // multi-workgroup form: rows x ws_row_bytes, or null
  size_t ws_row_bytes;
  int chunks;           // chunks of a max_ctx row (multi-workgroup form)
  int sub;              // sub-chunks of 4096 positions per chunk
  int sampled;          // multi-workgroup form: 1 sampled (two launches), 0 four launches
};

hipError_t launch_topk(const TopkParams& p, hipStream_t st);
size_t topk_ws_row_bytes(int max_ctx);  // workspace of one row (multi-workgroup form)
int topk_chunks(int max_ctx, int sub);
int topk_sampled_max_chunks();  // most chunks per row of the sampled form
int topk_sampled_max_sub();     // most sub-chunks per chunk of the sampled form
hipError_t launch_split(const SplitParams& p, hipStream_t st);
hipError_t launch_combine(const CombineParams& p, hipStream_t st);
int split_heads_per_block(int heads);
// split workgroups of a call with this many heads that one CU holds at once
int split_blocks_per_cu(int heads);

}  // namespace smla

#endif
