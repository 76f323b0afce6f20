// Host-side step metadata for paged extend attention: indptrs, prefix lengths
// and the attention work list. Pure C++; no HIP call is made here.
//
// AReno PR #642 ("What does this PR do?") carries per-request prefix and
// total-KV lengths in the step metadata so that one attention call serves a
// batch of mixed prefix/chunk lengths. AstrAI compare v1.3.12..925cbed
// (astrai/inference/core/cache.py, KVCache and PagePool.bind_tasks) builds
// kv_indptr once per step as the prefix sum of per-request total lengths so
// that no layer rebuilds it; csrc/kernels/attn_dispatchers.cuh
// (compute_num_splits) sizes the KV splits of one-token rows from the
// compute-unit count. This planner keeps those roles and adds what a
// work-list launch needs: tiles of GQA-packed query rows, their visible key
// ranges (causal and window bounds), and split slots for the combine step.
#include <algorithm>
#include <cstring>
#include <tuple>
#include <vector>

#include "pkv_internal.hpp"

namespace pkv {

int validate_shape(const pkv_shape* s) {
  if (!s) return set_error(PKV_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hkv=%d)", s->num_q_heads,
                     s->num_kv_heads);
  if (s->num_kv_heads >= kMaxKvHeads)
    return set_error(PKV_ERR_UNSUPPORTED, "num_kv_heads %d is not supported (at most %d)", s->num_kv_heads,
                     kMaxKvHeads - 1);
  if (s->num_q_heads % s->num_kv_heads)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                     s->num_q_heads, s->num_kv_heads);
  if (s->page_size < 1) return set_error(PKV_ERR_INVALID_ARGUMENT, "page_size must be >= 1 (got %d)", s->page_size);
  if (s->num_pages < 1) return set_error(PKV_ERR_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", s->num_pages);
  if (s->dtype != PKV_DTYPE_BF16 && s->dtype != PKV_DTYPE_FP32)
    return set_error(PKV_ERR_UNSUPPORTED, "dtype %d is not supported (0 = bf16, 1 = fp32)", s->dtype);
  if (s->head_dim != 64 && s->head_dim != 128)
    return set_error(PKV_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", s->head_dim);
  const int64_t page_bytes = int64_t(s->page_size) * s->num_kv_heads * s->head_dim * (s->dtype == PKV_DTYPE_BF16 ? 2 : 4);
  const int64_t row_bytes = page_bytes / s->page_size;
  if (row_bytes >= (int64_t(1) << 24))
    return set_error(PKV_ERR_UNSUPPORTED, "one token row of one pool spans %lld bytes (at most 2^24-1 supported)",
                     (long long)row_bytes);
  if (page_bytes > INT32_MAX)
    return set_error(PKV_ERR_UNSUPPORTED, "one page of one pool spans %lld bytes (at most 2^31-1 supported)",
                     (long long)page_bytes);
  if (s->num_q_heads / s->num_kv_heads > kMaxGroup)
    return set_error(PKV_ERR_UNSUPPORTED, "GQA group size %d exceeds %d", s->num_q_heads / s->num_kv_heads, kMaxGroup);
  return PKV_OK;
}

namespace {

struct Tile {
  int32_t req, q_begin, q_count, kv_lo, kv_hi;
  bool one_token;  // the request's whole chunk is a single token
};

int32_t ceil_div(int64_t a, int64_t b) { return int32_t((a + b - 1) / b); }

// The planner's buffers, kept per thread and reused from call to call: after a
// thread's first few plans no call allocates.
struct Scratch {
  std::vector<Tile> tiles;
  std::vector<int32_t> qo_start, tile_splits, req_splits, group_base, gid, split_rows, xcd_count, xcd_start;
  std::vector<WorkItem> items, ordered;
  std::vector<int64_t> cost, group_cost;
  std::vector<uint64_t> packed, gpacked;
  std::vector<uint8_t> xcd_of;
  std::vector<uint32_t> by_xcd;
};

Scratch& scratch() {
  static thread_local Scratch s;
  return s;
}

// Reorder items so that position i (dispatched to XCD i % kXcds) holds work of
// the locality group assigned to that XCD; see the dispatch-order comment in
// plan_extend. gid[i] is item i's group, numbered 0..ng-1 in (request, KV head,
// split) order. Falls back to plain longest-first when there are fewer items
// than twice the XCDs.
void xcd_order(Scratch& sc, int32_t ng) {
  const std::vector<WorkItem>& in = sc.items;
  const std::vector<int64_t>& c = sc.cost;
  std::vector<WorkItem>& out = sc.ordered;
  const size_t n = in.size();
  out.clear();
  // Longest first, ties in the planner's order: one integer sort of
  // (max cost - cost, index) packed into 64 bits (costs < 2^31 per item).
  const int64_t cmax = n ? *std::max_element(c.begin(), c.end()) : 0;
  sc.packed.resize(n);
  for (size_t i = 0; i < n; ++i) sc.packed[i] = (uint64_t(cmax - c[i]) << 32) | uint64_t(i);
  std::sort(sc.packed.begin(), sc.packed.end());
  if (n < size_t(kXcds) * 2) {
    for (uint64_t pk : sc.packed) out.push_back(in[pk & 0xffffffffu]);
    return;
  }
  // groups to XCDs: largest first (ties in group order), each to the least-loaded XCD
  sc.group_cost.assign(size_t(ng), 0);
  for (size_t i = 0; i < n; ++i) sc.group_cost[size_t(sc.gid[i])] += c[i];
  const int64_t gmax = *std::max_element(sc.group_cost.begin(), sc.group_cost.end());
  sc.gpacked.resize(size_t(ng));
  for (int32_t g = 0; g < ng; ++g) sc.gpacked[size_t(g)] = (uint64_t(gmax - sc.group_cost[size_t(g)]) << 32) | uint64_t(g);
  std::sort(sc.gpacked.begin(), sc.gpacked.end());
  int64_t load[kXcds] = {};
  sc.xcd_of.resize(size_t(ng));
  for (uint64_t gp : sc.gpacked) {
    const uint32_t g = uint32_t(gp & 0xffffffffu);
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += sc.group_cost[g];
    sc.xcd_of[g] = uint8_t(best);
  }
  // per-XCD lists in longest-first order (one flat array, counted first), then
  // dealt out round-robin
  int32_t cnt[kXcds] = {}, at[kXcds];
  for (size_t i = 0; i < n; ++i) ++cnt[sc.xcd_of[size_t(sc.gid[i])]];
  at[0] = 0;
  for (int x = 1; x < kXcds; ++x) at[x] = at[x - 1] + cnt[x - 1];
  int32_t start[kXcds];
  std::copy(at, at + kXcds, start);
  sc.by_xcd.resize(n);
  for (uint64_t pk : sc.packed) {
    const uint32_t i = uint32_t(pk & 0xffffffffu);
    sc.by_xcd[size_t(at[sc.xcd_of[size_t(sc.gid[i])]]++)] = i;
  }
  int32_t next[kXcds] = {};
  out.reserve(n);
  for (size_t i = 0; out.size() < n; ++i) {
    int x = int(i % kXcds);
    if (next[x] >= cnt[x]) {
      // this XCD's list is used up: hand its slot the next item of the fullest list
      int best = -1;
      for (int y = 0; y < kXcds; ++y)
        if (next[y] < cnt[y] && (best < 0 || cnt[y] - next[y] > cnt[best] - next[best])) best = y;
      x = best;
    }
    out.push_back(in[sc.by_xcd[size_t(start[x] + next[x]++)]]);
  }
}

}  // namespace

int plan_extend(int32_t batch, const int32_t* prefix_lens, const int32_t* chunk_lens, const pkv_shape* shape,
                int32_t window, int32_t flags, int32_t decode_splits, int32_t num_cus, void* meta_host,
                size_t meta_host_bytes, pkv_plan* plan, size_t* meta_bytes_out) {
  if (int st = validate_shape(shape)) return st;
  if (batch < 1) return set_error(PKV_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (!prefix_lens || !chunk_lens) return set_error(PKV_ERR_INVALID_ARGUMENT, "length arrays must not be NULL");
  if (decode_splits < 0 || decode_splits > PKV_MAX_SPLITS)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "decode_splits must be in 0..%d (got %d)", PKV_MAX_SPLITS,
                     decode_splits);
  if (flags & ~PKV_FLAG_NON_CAUSAL)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", unsigned(flags));
  const bool causal = !(flags & PKV_FLAG_NON_CAUSAL);
  if (!causal && window > 0)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "a sliding window (%d) needs the causal mask", window);
  if (num_cus < 1) num_cus = kNominalCUs;

  const int32_t hq = shape->num_q_heads, hkv = shape->num_kv_heads;
  const int32_t group = hq / hkv;
  const int32_t tile_tokens = std::max(1, rows_per_item(shape->dtype) / group);

  // ---- per-request sums (int32 range checked in 64-bit)
  int64_t total_q = 0, total_kv = 0;
  int32_t max_q = 0, max_kv = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t P = prefix_lens[b], L = chunk_lens[b];
    if (P < 0 || L < 0)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "request %d: negative length (prefix %lld, chunk %lld)", b,
                       (long long)P, (long long)L);
    const int64_t N = P + L;
    if (N > INT32_MAX) return set_error(PKV_ERR_INVALID_ARGUMENT, "request %d: prefix + chunk overflows int32", b);
    total_q += L;
    total_kv += N;
    if (total_q > INT32_MAX || total_kv > INT32_MAX)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "batch token counts overflow int32");
    max_q = std::max<int32_t>(max_q, int32_t(L));
    max_kv = std::max<int32_t>(max_kv, int32_t(N));
  }

  Scratch& sc = scratch();
  std::vector<int32_t>& qo_start = sc.qo_start;
  qo_start.assign(size_t(batch), 0);
  for (int32_t b = 1; b < batch; ++b) qo_start[b] = qo_start[b - 1] + chunk_lens[b - 1];

  // ---- tiles of GQA-packed query rows and their visible key ranges
  std::vector<Tile>& tiles = sc.tiles;
  tiles.clear();
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t P = prefix_lens[b], L = chunk_lens[b];
    for (int32_t q0 = 0; q0 < L; q0 += tile_tokens) {
      Tile t;
      t.req = b;
      t.q_begin = q0;
      t.q_count = std::min(tile_tokens, L - q0);
      // the tile's first row sees keys from max(0, P+q0-W+1); its last row up to P+q0+count-1
      t.kv_lo = window > 0 ? int32_t(std::max<int64_t>(0, int64_t(P) + q0 - window + 1)) : 0;
      t.kv_hi = causal ? P + q0 + t.q_count : P + L;   // non-causal: every row sees the whole request
      t.one_token = (L == 1);
      tiles.push_back(t);
    }
  }

  // ---- KV splits.
  // One-token rows: the explicit count, or enough splits to give the GPU about
  // two items per compute unit. Prefill tiles: when the launch has fewer items
  // than resident workgroup slots, tiles are cut into key ranges so that the
  // launch has at most one item per slot (a second round of items would double
  // the time of the slots that run it) with the largest item as small as that
  // allows; a tile's cost is its 64-key blocks times its live 32-row waves.
  auto granules_of = [](const Tile& t) {
    return std::max(1, ceil_div(t.kv_hi, kSplitGranule) - t.kv_lo / kSplitGranule);
  };
  auto waves_of = [group](const Tile& t) { return ceil_div(int64_t(t.q_count) * group, 32); };
  int32_t base_items = 0, n_one = 0;
  int64_t total_cost = 0;
  for (const Tile& t : tiles) {
    base_items += hkv;
    n_one += t.one_token;
    total_cost += int64_t(hkv) * granules_of(t) * waves_of(t);
  }
  int32_t auto_splits = 1;
  if (decode_splits == 0 && n_one > 0 && base_items > 0)
    auto_splits = std::min<int32_t>(PKV_MAX_SPLITS, std::max<int32_t>(1, ceil_div(2LL * num_cus, base_items)));
  const int64_t slots = int64_t(num_cus) * slots_per_cu(shape->dtype);
  auto prefill_cap = [&](const Tile& t) {
    return std::min<int64_t>(kMaxPrefillSplits, std::max(1, granules_of(t) / 2));
  };
  auto one_token_splits = [&](const Tile& t) {
    return decode_splits > 0 ? std::min(decode_splits, granules_of(t))
                             : std::min(auto_splits, std::max(1, granules_of(t) / 2));
  };
  // items of the launch when every prefill tile is cut into pieces of cost <= u
  auto items_at = [&](int64_t u) {
    int64_t n = 0;
    for (const Tile& t : tiles) {
      const int64_t c = int64_t(granules_of(t)) * waves_of(t);
      n += int64_t(hkv) * (t.one_token ? one_token_splits(t) : std::min(prefill_cap(t), (c + u - 1) / u));
    }
    return n;
  };
  int64_t unit = 0;  // 0: prefill tiles stay whole
  if (base_items < slots) {
    int64_t lo = 1, hi = 1;
    for (const Tile& t : tiles) hi = std::max<int64_t>(hi, int64_t(granules_of(t)) * waves_of(t));
    // smallest piece cost whose item count fits the slots (counts fall as u grows)
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (items_at(mid) <= slots) hi = mid; else lo = mid + 1;
    }
    unit = lo;
  }

  // splits of every tile; a request's locality groups are (KV head, split) pairs
  // up to its largest split count, numbered in (request, KV head, split) order
  std::vector<int32_t>& tile_splits = sc.tile_splits;
  tile_splits.resize(tiles.size());
  std::vector<int32_t>& req_splits = sc.req_splits;
  req_splits.assign(size_t(batch), 0);
  int64_t n_alloc = 0;
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    const Tile& t = tiles[ti];
    int32_t splits = 1;
    if (t.one_token) {
      splits = one_token_splits(t);
    } else if (unit > 0) {
      const int64_t want = (int64_t(granules_of(t)) * waves_of(t) + unit - 1) / unit;
      splits = int32_t(std::max<int64_t>(1, std::min(want, prefill_cap(t))));
    }
    tile_splits[ti] = splits;
    req_splits[size_t(t.req)] = std::max(req_splits[size_t(t.req)], splits);
    n_alloc += int64_t(hkv) * splits;
  }
  std::vector<int32_t>& group_base = sc.group_base;
  group_base.resize(size_t(batch));
  int32_t n_groups = 0;
  for (int32_t b = 0; b < batch; ++b) {
    group_base[size_t(b)] = n_groups;
    n_groups += hkv * req_splits[size_t(b)];
  }

  std::vector<WorkItem>& items = sc.items;
  items.clear();
  items.reserve(size_t(n_alloc));
  std::vector<int32_t>& gid = sc.gid;
  gid.clear();
  gid.reserve(size_t(n_alloc));
  std::vector<int32_t>& split_rows = sc.split_rows;  // pairs (token, splits)
  split_rows.clear();
  int32_t n_split_rows = 0, max_splits = 1;
  for (size_t ti = 0; ti < tiles.size(); ++ti) {
    const Tile& t = tiles[ti];
    const int32_t g0 = t.kv_lo / kSplitGranule;
    const int32_t granules = granules_of(t);
    const int32_t splits = tile_splits[ti];
    int32_t part_row = -1;
    if (splits > 1) {
      part_row = n_split_rows;
      n_split_rows += t.q_count;
      max_splits = std::max(max_splits, splits);
    }
    const int32_t rs = req_splits[size_t(t.req)], gb = group_base[size_t(t.req)];
    for (int32_t h = 0; h < hkv; ++h) {
      for (int32_t k = 0; k < splits; ++k) {
        WorkItem it;
        it.req = t.req;
        it.head_split = (h << (2 * kSplitBits)) | (splits << kSplitBits) | k;
        it.tok0 = qo_start[t.req] + t.q_begin;
        it.pos0 = causal ? prefix_lens[t.req] + t.q_begin : kNonCausalPos;
        it.q_count = t.q_count;
        if (splits == 1) {
          it.kv_begin = t.kv_lo;
          it.kv_end = t.kv_hi;
        } else {
          const int32_t ga = g0 + int32_t(int64_t(k) * granules / splits);
          const int32_t gbk = g0 + int32_t(int64_t(k + 1) * granules / splits);
          it.kv_begin = std::max(t.kv_lo, ga * kSplitGranule);
          it.kv_end = std::min(t.kv_hi, gbk * kSplitGranule);
        }
        it.part_row = part_row;
        items.push_back(it);
        gid.push_back(gb + h * rs + k);
      }
    }
    if (splits > 1) {
      // token indices are global: qo_indptr[req] + q_begin + i
      for (int32_t i = 0; i < t.q_count; ++i) {
        split_rows.push_back(qo_start[t.req] + t.q_begin + i);
        split_rows.push_back(splits);
      }
    }
  }

  // Dispatch order. Workgroups go to the 8 XCDs round-robin (workgroup i runs on
  // XCD i mod 8), and each XCD has its own L2. Items that read the same keys --
  // same request, KV head and split -- are grouped and each group is placed on
  // one XCD (groups assigned greedily to the least-loaded XCD, largest first),
  // so the tiles that stream one KV head stay together in one L2. Within an XCD
  // the longest items go first; an item's time grows with its key range times
  // its live 32-row waves. A size query (no meta_host) needs no order.
  std::vector<int64_t>& cost = sc.cost;
  cost.resize(items.size());
  for (size_t i = 0; i < items.size(); ++i) {
    const WorkItem& a = items[i];
    cost[i] = int64_t(a.kv_end - a.kv_begin) * ((int64_t(a.q_count) * group + 31) / 32);
  }
  if (meta_host) xcd_order(sc, n_groups);
  const std::vector<WorkItem>& ordered = meta_host ? sc.ordered : items;
  const int32_t n_items = int32_t(ordered.size());
  const MetaLayout lay = meta_layout(batch, n_items, n_split_rows);
  if (meta_bytes_out) *meta_bytes_out = lay.total;
  // key blocks the busiest workgroup slot streams: the longest item, or the
  // average per slot when there are more items than slots
  int64_t max_blocks = 0, sum_blocks = 0;
  for (const WorkItem& it : ordered) {
    const int64_t nb = it.kv_end > it.kv_begin ? ceil_div(it.kv_end, kSplitGranule) - it.kv_begin / kSplitGranule : 0;
    max_blocks = std::max(max_blocks, nb);
    sum_blocks += nb;
  }
  const int64_t slot_blocks = std::max(max_blocks, (sum_blocks + slots - 1) / slots);

  if (plan) {
    std::memset(plan, 0, sizeof(*plan));
    plan->batch = batch;
    plan->total_q = int32_t(total_q);
    plan->max_q_len = max_q;
    plan->max_kv_len = max_kv;
    plan->n_items = n_items;
    plan->n_split_rows = n_split_rows;
    plan->max_splits = max_splits;
    plan->window = window;
    plan->flags = flags;
    plan->slot_blocks = int32_t(std::min<int64_t>(slot_blocks, INT32_MAX));
    plan->num_cus = num_cus;
    plan->shape = *shape;
    plan->workspace_bytes = workspace_bytes(n_split_rows, hq, max_splits, shape->head_dim, shape->dtype);
  }

  if (meta_host) {
    if (meta_host_bytes < lay.total)
      return set_error(PKV_ERR_WORKSPACE, "meta_host holds %zu bytes, %zu needed", meta_host_bytes, lay.total);
    char* base = static_cast<char*>(meta_host);
    std::memset(base, 0, lay.total);
    int32_t* qo = reinterpret_cast<int32_t*>(base + lay.qo_indptr);
    int32_t* kv = reinterpret_cast<int32_t*>(base + lay.kv_indptr);
    int32_t* pre = reinterpret_cast<int32_t*>(base + lay.prefix_lens);
    qo[0] = 0;
    kv[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
      qo[b + 1] = qo[b] + chunk_lens[b];
      kv[b + 1] = kv[b] + prefix_lens[b] + chunk_lens[b];
      pre[b] = prefix_lens[b];
    }
    if (n_items) std::memcpy(base + lay.items, ordered.data(), sizeof(WorkItem) * ordered.size());
    if (n_split_rows) std::memcpy(base + lay.split_rows, split_rows.data(), sizeof(int32_t) * split_rows.size());
  }
  return PKV_OK;
}

}  // namespace pkv
