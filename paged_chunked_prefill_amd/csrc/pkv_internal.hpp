// Internal definitions shared by the host planner and the HIP kernels of
// libpkv. Not part of the public ABI (include/pkv.h is).
#pragma once

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Query-head rows per attention work item: waves of 32 rows each. Rows are
// (token, head-in-group) pairs of one KV head, token-major, so a tile holds
// rows / G consecutive chunk tokens. The bf16 kernel runs 8 waves (256 rows)
// per workgroup, one workgroup per CU (2 waves per SIMD): every K/V tile staged
// in LDS then serves 256 rows. The fp32 kernel runs 4 waves (128 rows), two
// workgroups per CU.
constexpr int kWavesBf16 = 8;
constexpr int kWavesF32 = 4;
constexpr int kMaxGroup = 128;  // largest GQA group size (query heads per KV head)
inline int waves_per_item(int dtype) { return dtype == PKV_DTYPE_BF16 ? kWavesBf16 : kWavesF32; }
inline int rows_per_item(int dtype) { return 32 * waves_per_item(dtype); }
inline int slots_per_cu(int dtype) { return dtype == PKV_DTYPE_BF16 ? 1 : 2; }
// Keys per KV tile staged in LDS (bf16 / fp32 instantiations).
constexpr int kTileKeysBf16 = 64;
constexpr int kTileKeysF32 = 32;
// Every split of a one-token row covers whole 64-key blocks, so the tile
// boundaries of both instantiations stay aligned to absolute positions.
constexpr int kSplitGranule = 64;
// paged_extend_attn_append fuses the append into the bf16 attention launch
// while the plan's busiest workgroup slot streams at most this many 64-key
// blocks: the fused gather's per-lane addresses cost a little per block, the
// separate append launch a fixed few microseconds.
constexpr int kFuseMaxSlotBlocks = 128;
// Cap on the KV splits of one prefill tile.
constexpr int kMaxPrefillSplits = 16;
// Compute units of an MI355X: the planner's count when no device can be queried.
constexpr int kNominalCUs = 256;
// XCDs (each with its own L2); workgroups are dispatched to them round-robin.
constexpr int kXcds = 8;

// One unit of attention work = one workgroup: a tile of consecutive chunk
// tokens of one request, all G query heads of one KV head, over the key
// positions [kv_begin, kv_end) (the whole visible range, or one split of it).
// The planner resolves the request's offsets into the item, so a workgroup
// starts from this one 32-byte record.
struct alignas(16) WorkItem {
  int32_t req;         // request index b (page-table row, or index into req_pool_indices)
  int32_t head_split;  // KV head hk << 16 | the tile's split count S << 8 | split index k (S = 1, k = 0 unsplit)
  int32_t tok0;        // global token index of the tile's first token: qo_indptr[b] + first chunk token
  int32_t pos0;        // its absolute position: P_b + first chunk token
  int32_t q_count;     // tokens in the tile (all inside the chunk); 0: a padding item, skipped
  int32_t kv_begin;    // first key position this item covers
  int32_t kv_end;      // one past the last key position (<= N_b)
  int32_t part_row;    // -1: write `out`; else partial slot of the tile's first token
};
static_assert(sizeof(WorkItem) == 32, "work item layout");
// Widths of head_split's split index and split count fields; the KV head takes
// the bits above them, 15 of them below the sign bit (validate_shape bounds
// num_kv_heads by kMaxKvHeads accordingly).
constexpr int kSplitBits = 8;
static_assert(PKV_MAX_SPLITS < (1 << kSplitBits), "split index and count fit their fields");
constexpr int kMaxKvHeads = 1 << (31 - 2 * kSplitBits);
// Non-causal plans put an item's pos0 (the position its causal bound is taken
// from) past every key, so the kernels' causal test passes for all of them.
constexpr int32_t kNonCausalPos = 1 << 30;

// Byte offsets of the sections of the metadata buffer (host staging and its
// device copy share the layout). Each section starts on a 256-byte boundary.
struct MetaLayout {
  size_t qo_indptr, kv_indptr, prefix_lens, items, split_rows, status, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline MetaLayout meta_layout(int32_t batch, int32_t n_items, int32_t n_split_rows) {
  MetaLayout m;
  size_t off = 0;
  m.qo_indptr = off;   off = align256(off + sizeof(int32_t) * (size_t(batch) + 1));
  m.kv_indptr = off;   off = align256(off + sizeof(int32_t) * (size_t(batch) + 1));
  m.prefix_lens = off; off = align256(off + sizeof(int32_t) * size_t(batch));
  m.items = off;       off = align256(off + sizeof(WorkItem) * size_t(n_items));
  m.split_rows = off;  off = align256(off + 2 * sizeof(int32_t) * size_t(n_split_rows));
  m.status = off;      off = align256(off + sizeof(int32_t));
  m.total = off;
  return m;
}

// Split partials in the workspace: for partial slot s, query head h, split k
//   o_part [s][h][k][D] unnormalised output: bf16 for bf16 inputs (the output
//                       precision; half the bytes the combine has to move),
//                       fp32 for fp32 inputs
//   ml_part[s][h][k][2] fp32 (running max in log2 units, running sum)
inline size_t part_elem_bytes(int32_t dtype) { return dtype == PKV_DTYPE_BF16 ? 2 : 4; }
inline size_t workspace_o_bytes(int32_t n_split_rows, int32_t hq, int32_t max_splits, int32_t d, int32_t dtype) {
  return align256(part_elem_bytes(dtype) * size_t(n_split_rows) * hq * max_splits * d);
}
inline size_t workspace_bytes(int32_t n_split_rows, int32_t hq, int32_t max_splits, int32_t d, int32_t dtype) {
  if (n_split_rows == 0) return 0;
  return workspace_o_bytes(n_split_rows, hq, max_splits, d, dtype) +
         align256(sizeof(float) * size_t(n_split_rows) * hq * max_splits * 2);
}

// Host planner (planner.cpp). Fills `meta_host` (may be NULL for a size query)
// and the host fields of `plan`. Returns a PKV status; sets the error text.
int plan_extend(int32_t batch, const int32_t* prefix_lens, const int32_t* chunk_lens, const pkv_shape* shape,
                int32_t window, int32_t flags, int32_t decode_splits, int32_t num_cus, void* meta_host,
                size_t meta_host_bytes, pkv_plan* plan, size_t* meta_bytes_out);

int validate_shape(const pkv_shape* shape);

// Thread-local error text (api.hip).
int set_error(int status, const char* fmt, ...);

// Kernel launchers (append.hip, extend_attn.hip). Arguments are validated by
// the callers in api.hip.
struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* req_pool_indices;
  const int32_t* qo_indptr;
  const int32_t* prefix_lens;
  const WorkItem* items;
  const int32_t* split_rows;
  int32_t* status;
  void* out;
  void* o_part;   // bf16 or fp32 by dtype, see workspace_o_bytes
  float* ml_part;
  int32_t n_items;
  int32_t n_split_rows;
  int32_t max_splits;
  int32_t total_q;
  int32_t window;
  float scale_log2;   // softmax scale * log2(e)
  pkv_shape shape;
  // explicit keep-mask, or nullptr: bytes [B][mask_heads][mask_rows][mask_kv_stride]
  const uint8_t* mask = nullptr;
  int32_t mask_heads = 1, mask_rows = 1, mask_kv_stride = 0;
  // fused append (bf16 only): the chunk's K/V rows, also written into the pools
  // by the attention launch itself; nullptr for the plain attention
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  void* k_pool_w = nullptr;
  void* v_pool_w = nullptr;
};

int launch_extend_attn(const AttnArgs& a, void* stream);

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* req_pool_indices;
  const int32_t* qo_indptr;
  const int32_t* prefix_lens;
  int32_t* status;
  int32_t batch;
  int32_t total_q;
  pkv_shape shape;
  // rotary embedding fused with the append (rope_table == nullptr: plain append)
  const void* q = nullptr;
  void* q_out = nullptr;
  const float* rope_table = nullptr;   // [rope_table_len][D/2][2] (cos, sin)
  int32_t rope_table_len = 0;
};

int launch_append(const AppendArgs& a, void* stream);

// Copies `bytes` (a multiple of 256) from a device-readable address of pinned
// host memory to device memory with a kernel (append.hip).
int launch_meta_copy(const void* src_dev, void* dst, size_t bytes, void* stream);

}  // namespace pkv
