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

// Predicted time of one bf16 work item on MI355X, in ns (per-workgroup
// timestamps of the attention kernel): about 5.6 us of its own (the Q rows and
// the first K/V tiles into LDS, the first scores, the output stores; more for
// the first workgroup on each compute unit, the same for every plan), then
// 1390 + 67 w ns per 64-key block for w live 32-row waves. A split item also costs about 26 ns of
// HBM time for its partial rows (256 rows of D values and (max, sum), written
// and read back by the combine).
constexpr int64_t kItemNs = 5600;
constexpr int64_t kBlockNs = 1390;
constexpr int64_t kBlockWaveNs = 67;
constexpr int64_t kPartialNs = 26;
// Cap on the pieces of one tile in a stream plan (its split count).
constexpr int32_t kMaxStreamSplits = 32;
// Most splits a tile takes in the equal cuts: the prefill cap, or a one-token
// row's count (at most PKV_MAX_SPLITS).
constexpr int32_t kMaxSplitsAny = kMaxPrefillSplits > PKV_MAX_SPLITS ? kMaxPrefillSplits : PKV_MAX_SPLITS;
// Within an XCD, workgroups go to its 4 shader engines in turn -- the XCD's
// j-th workgroup to engine class j mod 4 -- strictly in order: a workgroup
// waits for a free compute unit of its engine and holds back every later one
// of its XCD (per-workgroup hardware ids and timestamps on MI355X).
constexpr int kSeClasses = 4;

// One piece of a stream plan: 64-key blocks [g0, g1) of a tile, in run `run`,
// starting `start` ns after the run's first piece.
struct Piece {
  int32_t tile, g0, g1, run;
  int64_t start;
};
// A stream-plan item placed for dispatch: XCD, shader-engine class, whether it
// is its run's first piece (0) or a later one (1), its predicted start within
// its run (later pieces), its duration, and its index in the item list.
struct Placed {
  int32_t xcd, cls, later;
  int64_t key, dur;
  int32_t seq;
};

// The planner's buffers, kept per thread and reused from call to call: after a
// thread's first few plans no call allocates.
struct Scratch {
  std::vector<Tile> tiles;
  std::vector<int32_t> qo_start, tile_splits, tile_part, req_splits, group_base, gid, xcd_count, xcd_start;
  std::vector<WorkItem> items, ordered;
  std::vector<int64_t> cost, group_cost;
  std::vector<uint64_t> packed, gpacked;
  std::vector<uint8_t> xcd_of;
  std::vector<uint32_t> by_xcd;
  // stream plan
  std::vector<int64_t> block_ns, run_load, run_blocks;
  std::vector<int32_t> piece_count, piece_next, bucket;
  std::vector<Piece> pieces;
  std::vector<Placed> placed;
  std::vector<int32_t> run_first, run_cls, run_xcd;
  std::vector<WorkItem> piece_item;
  std::vector<int64_t> piece_dur;
};

Scratch& scratch() {
  static thread_local Scratch s;
  return s;
}

// Order keys ascending, ties by index: (key << 32 | index) for keys[0..n),
// by a counting sort when the keys span fewer than kCountingRange values (the
// usual case: a launch's items come from a few tile shapes), else by a
// comparison sort. Keys are >= 0 and < 2^31.
constexpr int64_t kCountingRange = 4096;
void sort_by_key(const int64_t* keys, size_t n, std::vector<int32_t>& bucket, std::vector<uint64_t>& packed) {
  packed.resize(n);
  int64_t kmin = INT64_MAX, kmax = 0;
  for (size_t i = 0; i < n; ++i) {
    kmin = std::min(kmin, keys[i]);
    kmax = std::max(kmax, keys[i]);
  }
  if (n > 0 && kmax - kmin < kCountingRange) {
    const size_t range = size_t(kmax - kmin) + 1;
    bucket.assign(range + 1, 0);
    for (size_t i = 0; i < n; ++i) ++bucket[size_t(keys[i] - kmin) + 1];
    for (size_t b = 0; b < range; ++b) bucket[b + 1] += bucket[b];
    for (size_t i = 0; i < n; ++i)
      packed[size_t(bucket[size_t(keys[i] - kmin)]++)] = (uint64_t(keys[i]) << 32) | uint64_t(i);
  } else {
    for (size_t i = 0; i < n; ++i) packed[i] = (uint64_t(keys[i]) << 32) | uint64_t(i);
    std::sort(packed.begin(), packed.end());
  }
}

// Reorder items so that position i (dispatched to XCD i % kXcds) holds work of
// the locality group assigned to that XCD; see the dispatch-order comment in
// plan_extend. gid[i] is item i's group, numbered 0..ng-1 in (request, KV head,
// split) order; cost[i] its cost (largest cmax; overwritten here) and
// group_cost[g] the sum over group g. Falls back to plain longest-first when
// there are fewer items than twice the XCDs.
void xcd_order(Scratch& sc, int32_t ng, int64_t cmax) {
  const std::vector<WorkItem>& in = sc.items;
  std::vector<int64_t>& c = sc.cost;
  std::vector<WorkItem>& out = sc.ordered;
  const size_t n = in.size();
  // Longest first, ties in the planner's order: ascending (max cost - cost, index).
  for (size_t i = 0; i < n; ++i) c[i] = cmax - c[i];
  sort_by_key(c.data(), n, sc.bucket, sc.packed);
  out.resize(n);
  WorkItem* o = out.data();
  if (n < size_t(kXcds) * 2) {
    for (uint64_t pk : sc.packed) *o++ = in[pk & 0xffffffffu];
    return;
  }
  // groups to XCDs: largest first (ties in group order), each to the least-loaded XCD
  int64_t gmax = 0;
  for (int32_t g = 0; g < ng; ++g) gmax = std::max(gmax, sc.group_cost[size_t(g)]);
  for (int32_t g = 0; g < ng; ++g) sc.group_cost[size_t(g)] = gmax - sc.group_cost[size_t(g)];
  sort_by_key(sc.group_cost.data(), size_t(ng), sc.bucket, sc.gpacked);
  int64_t load[kXcds] = {};
  sc.xcd_of.resize(size_t(ng));
  for (uint64_t gp : sc.gpacked) {
    const uint32_t g = uint32_t(gp & 0xffffffffu);
    int best = 0;
    int64_t least = load[0];
    for (int x = 1; x < kXcds; ++x) {   // (selects, not branches: the loads are near-equal)
      const bool lt = load[x] < least;
      best = lt ? x : best;
      least = lt ? load[x] : least;
    }
    load[best] += gmax - int64_t(gp >> 32);
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
  for (size_t i = 0; i < n; ++i) {
    int x = int(i % kXcds);
    if (next[x] >= cnt[x]) {
      // this XCD's list is used up: hand its slot the next item of the fullest list
      int best = -1;
      for (int y = 0; y < kXcds; ++y)
        if (next[y] < cnt[y] && (best < 0 || cnt[y] - next[y] > cnt[best] - next[best])) best = y;
      x = best;
    }
    *o++ = in[sc.by_xcd[size_t(start[x] + next[x]++)]];
  }
}

// Stream cut: one KV head's work -- each tile's 64-key blocks [g0(t), g1(t)),
// tiles in order -- laid end to end and cut into runs of predicted time <= T
// (ns), each piece (the blocks of one tile inside one run) charged a
// prologue. Returns the runs used, or limit + 1 as soon as more are needed or
// a tile would get more than kMaxStreamSplits pieces. T must fit a prologue
// and one block of every tile.
int32_t stream_cut(const std::vector<Tile>& tiles, Scratch& sc, int64_t T, int32_t limit, bool keep) {
  sc.piece_count.assign(tiles.size(), 0);
  if (keep) sc.pieces.clear();
  int32_t runs = 0;
  int64_t room = -1;
  for (size_t t = 0; t < tiles.size(); ++t) {
    const int64_t bns = sc.block_ns[t];
    int32_t g = tiles[t].kv_lo / kSplitGranule;
    const int32_t ge = g + std::max(1, ceil_div(tiles[t].kv_hi, kSplitGranule) - g);
    while (g < ge) {
      if (room < kItemNs + bns) {
        if (++runs > limit) return limit + 1;
        room = T;
      }
      const int32_t take = int32_t(std::min<int64_t>(ge - g, (room - kItemNs) / bns));
      if (++sc.piece_count[t] > kMaxStreamSplits) return limit + 1;
      if (keep) sc.pieces.push_back(Piece{int32_t(t), g, g + take, runs - 1, T - room});
      room -= kItemNs + take * bns;
      g += take;
    }
  }
  return runs;
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
  for (const Tile& t : tiles) {
    base_items += hkv;
    n_one += t.one_token;
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

  // each split tile's partial rows (tile_part; -1 when unsplit): one per token
  std::vector<int32_t>& tile_part = sc.tile_part;
  tile_part.resize(tiles.size());
  int32_t n_split_rows = 0, max_splits = 1;
  auto number_split_rows = [&]() {
    n_split_rows = 0;
    max_splits = 1;
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      tile_part[ti] = -1;
      if (tile_splits[ti] > 1) {
        tile_part[ti] = n_split_rows;
        n_split_rows += tiles[ti].q_count;
        max_splits = std::max(max_splits, tile_splits[ti]);
      }
    }
  };
  number_split_rows();

  // The items, with what the plan needs of each: its dispatch cost (64-key
  // blocks x live 32-row waves) and its locality group's total, its predicted
  // time for the stream-plan test (longest, sum, split items), and the key
  // blocks per slot. A tile's splits have the same key ranges and costs for
  // every KV head.
  std::vector<WorkItem>& items = sc.items;
  items.resize(size_t(n_alloc));
  std::vector<int32_t>& gid = sc.gid;
  gid.resize(size_t(n_alloc));
  std::vector<int64_t>& cost = sc.cost;
  cost.resize(size_t(n_alloc));
  sc.group_cost.assign(size_t(n_groups), 0);
  int64_t cost_max = 0, cur_max = 0, cur_sum = 0, cur_split = 0, max_blocks = 0, sum_blocks = 0;
  {
    WorkItem* out = items.data();
    int32_t* out_gid = gid.data();
    int64_t* out_cost = cost.data();
    int32_t kv_begin[kMaxSplitsAny], kv_end[kMaxSplitsAny];
    int64_t kcost[kMaxSplitsAny];
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      const Tile& t = tiles[ti];
      const int32_t g0 = t.kv_lo / kSplitGranule;
      const uint32_t granules = uint32_t(granules_of(t));   // < 2^25: k * granules fits 32 bits
      const int32_t splits = tile_splits[ti];
      if (splits == 1) {
        kv_begin[0] = t.kv_lo;
        kv_end[0] = t.kv_hi;
      } else {
        int32_t ga = g0;
        for (int32_t k = 0; k < splits; ++k) {
          const int32_t gbk = g0 + int32_t(uint32_t(k + 1) * granules / uint32_t(splits));
          kv_begin[k] = std::max(t.kv_lo, ga * kSplitGranule);
          kv_end[k] = std::min(t.kv_hi, gbk * kSplitGranule);
          ga = gbk;
        }
      }
      const int64_t waves = waves_of(t);
      const int64_t block_ns = kBlockNs + kBlockWaveNs * std::min<int64_t>(8, waves);
      for (int32_t k = 0; k < splits; ++k) {
        const int64_t nb =
            kv_end[k] > kv_begin[k] ? ceil_div(kv_end[k], kSplitGranule) - kv_begin[k] / kSplitGranule : 0;
        kcost[k] = nb * waves;
        cost_max = std::max(cost_max, kcost[k]);
        cur_max = std::max(cur_max, kItemNs + nb * block_ns);
        cur_sum += hkv * (kItemNs + nb * block_ns);
        max_blocks = std::max(max_blocks, nb);
        sum_blocks += hkv * nb;
      }
      if (tile_part[ti] >= 0) cur_split += int64_t(hkv) * splits;
      const int32_t rs = req_splits[size_t(t.req)], gb = group_base[size_t(t.req)];
      WorkItem it;
      it.req = t.req;
      it.tok0 = qo_start[size_t(t.req)] + t.q_begin;
      it.pos0 = causal ? prefix_lens[t.req] + t.q_begin : kNonCausalPos;
      it.q_count = t.q_count;
      it.part_row = tile_part[ti];
      for (int32_t h = 0; h < hkv; ++h) {
        for (int32_t k = 0; k < splits; ++k) {
          it.head_split = (h << (2 * kSplitBits)) | (splits << kSplitBits) | k;
          it.kv_begin = kv_begin[k];
          it.kv_end = kv_end[k];
          *out++ = it;
          *out_gid++ = gb + h * rs + k;
          *out_cost++ = kcost[k];
          sc.group_cost[size_t(gb + h * rs + k)] += kcost[k];
        }
      }
    }
  }

  // ---- Stream plan. Equal cuts of each tile, one item per slot, leave the
  // slots as uneven as the tiles (a causal chunk's later tiles see more keys).
  // The alternative: one KV head's tiles cut end to end into runs of nearly
  // equal predicted time (stream_cut), one run per slot, every KV head cut
  // alike on its own share of the slots (the combine takes one split count per
  // token), the runs spread evenly over the XCDs with each head's runs on
  // neighbouring ones. A run of several pieces relies on how the hardware
  // hands out workgroups (kSeClasses): each shader engine's next workgroup
  // goes to the first of its compute units that frees up, so each engine
  // class gets runs of similar first pieces and its later pieces in the order
  // of their predicted start, and shorter class lists are padded with empty
  // items. Taken when its predicted time, partials included, is at least 1/32
  // below the plan above; only for bf16 lists with prefill tiles, automatic
  // splits and at most one item per slot.
  bool streamed = false;
  int64_t stream_blocks = 0;
  const int64_t runs_per_head = slots / hkv;
  std::vector<WorkItem>& ordered_out = sc.ordered;
  if (shape->dtype == PKV_DTYPE_BF16 && decode_splits == 0 && n_one < int32_t(tiles.size()) && runs_per_head >= 1 &&
      int64_t(items.size()) <= slots) {
    // the plan above: its longest item (one per slot), its mean load per slot and its partials
    const int64_t cur_cost = cur_max + kPartialNs * cur_split;
    // the equal cuts already load every slot within 1/16 of the mean: no cut does better by 1/32
    const bool even = cur_max * 16 <= (cur_sum + slots - 1) / slots * 17;
    // Run time bounds: at least a piece of one block, and at least the block
    // work over the runs plus a prologue (every run has one); a greedy cut at
    // the work over the runs plus one prologue per tile over the runs, two more
    // prologues and a block always fits (a run leaves less than a prologue and
    // a block unused, and a cut adds one prologue).
    sc.block_ns.resize(tiles.size());
    int64_t piece_min = 0, work = 0, block_max = 0;
    for (size_t t = 0; t < tiles.size(); ++t) {
      sc.block_ns[t] = kBlockNs + kBlockWaveNs * std::min<int64_t>(8, waves_of(tiles[t]));
      piece_min = std::max(piece_min, kItemNs + sc.block_ns[t]);
      block_max = std::max(block_max, sc.block_ns[t]);
      work += int64_t(granules_of(tiles[t])) * sc.block_ns[t];
    }
    const int64_t total = work + int64_t(tiles.size()) * kItemNs;   // everything in one run
    const int32_t limit = int32_t(std::min<int64_t>(runs_per_head, INT32_MAX - 1));
    int64_t lo = std::max(piece_min, (work + limit - 1) / limit + kItemNs);
    int64_t hi = std::min(total, (total + limit - 1) / limit + 2 * kItemNs + block_max);
    lo = std::min(lo, hi);
    // No cut can beat the plan above by 1/32 when even the bound cannot (a
    // near-even plan): no search. Otherwise the shortest run time (to within
    // 1/256) whose cut fits; at `total` everything fits one run, one piece a
    // tile, so only the split cap can make `hi` fail.
    int32_t runs = 0;
    if (!even && lo + lo / 32 < cur_cost) {
      if (stream_cut(tiles, sc, hi, limit, false) > limit) hi = total;
      while (hi - lo > std::max<int64_t>(64, hi / 256)) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (stream_cut(tiles, sc, mid, limit, false) <= limit) hi = mid; else lo = mid + 1;
      }
      runs = stream_cut(tiles, sc, hi, limit, true);
    }
    // the cut's predicted time: its busiest run plus the partials of split tiles
    int64_t stream_cost = 0;
    std::vector<int64_t>& run_blocks = sc.run_blocks;
    if (runs > 0) {
      sc.run_load.assign(size_t(runs), 0);
      run_blocks.assign(size_t(runs), 0);
      for (const Piece& pc : sc.pieces) {
        sc.run_load[size_t(pc.run)] += kItemNs + int64_t(pc.g1 - pc.g0) * sc.block_ns[size_t(pc.tile)];
        run_blocks[size_t(pc.run)] += pc.g1 - pc.g0;
      }
      int64_t split_pieces = 0;
      for (int32_t c : sc.piece_count) split_pieces += c > 1 ? c : 0;
      stream_cost = *std::max_element(sc.run_load.begin(), sc.run_load.end()) + kPartialNs * hkv * split_pieces;
    }
    if (runs > 0 && stream_cost + stream_cost / 32 < cur_cost) {
      streamed = true;
      stream_blocks = *std::max_element(run_blocks.begin(), run_blocks.end());
      // split counts: the tiles' pieces
      for (size_t t = 0; t < tiles.size(); ++t) tile_splits[t] = sc.piece_count[t];
      number_split_rows();
      // split index of each piece (a tile's pieces come in key order) and each
      // run's first piece (a run's pieces are consecutive)
      const size_t np = sc.pieces.size();
      sc.piece_next.assign(tiles.size(), 0);
      gid.resize(np);
      sc.run_first.assign(size_t(runs) + 1, 0);
      for (size_t i = 0; i < np; ++i) {
        gid[i] = sc.piece_next[size_t(sc.pieces[i].tile)]++;
        ++sc.run_first[size_t(sc.pieces[i].run) + 1];
      }
      for (int32_t r = 0; r < runs; ++r) sc.run_first[size_t(r) + 1] += sc.run_first[size_t(r)];
      // runs by the length of their first piece (the same for every KV head)
      sc.packed.resize(size_t(runs));
      for (int32_t r = 0; r < runs; ++r) {
        const Piece& f = sc.pieces[size_t(sc.run_first[size_t(r)])];
        sc.packed[size_t(r)] = (uint64_t(f.g1 - f.g0) * uint64_t(sc.block_ns[size_t(f.tile)]) << 20) | uint64_t(r);
      }
      std::sort(sc.packed.begin(), sc.packed.end());
      // (head, run) -> XCD; per XCD the runs in that order are dealt to the
      // engine classes in turn (rank mod kSeClasses), heads one after another
      const int64_t total_runs = int64_t(runs) * hkv;   // <= slots: at most slots / 8 runs per XCD
      // run j = h * runs + r goes to XCD floor(8 j / total_runs) (a table, no division per run)
      sc.run_xcd.resize(size_t(total_runs));
      for (int64_t j = 0, x = 0; j < total_runs; ++j) {
        while ((x + 1) * total_runs <= j * kXcds) ++x;
        sc.run_xcd[size_t(j)] = int32_t(x);
      }
      auto xcd_of_run = [&](int32_t h, int32_t r) { return sc.run_xcd[size_t(h) * size_t(runs) + size_t(r)]; };
      sc.run_cls.assign(size_t(total_runs), 0);
      int32_t rank[kXcds] = {};
      for (int32_t h = 0; h < hkv; ++h)
        for (uint64_t pk : sc.packed) {
          const int32_t r = int32_t(pk & 0xfffff);
          sc.run_cls[size_t(h) * size_t(runs) + size_t(r)] = rank[xcd_of_run(h, r)]++ % kSeClasses;
        }
      // items, then (XCD, class) buckets: the first pieces in the dealing
      // order above, then the later pieces by predicted start. Each piece's
      // item (KV head 0) and predicted duration, once for every head.
      sc.piece_item.resize(np);
      sc.piece_dur.resize(np);
      for (size_t i = 0; i < np; ++i) {
        const Piece& pc = sc.pieces[i];
        const Tile& tl = tiles[size_t(pc.tile)];
        const int32_t S = sc.piece_count[size_t(pc.tile)];
        WorkItem& it = sc.piece_item[i];
        it.req = tl.req;
        it.head_split = (S << kSplitBits) | gid[i];
        it.tok0 = qo_start[size_t(tl.req)] + tl.q_begin;
        it.pos0 = causal ? prefix_lens[tl.req] + tl.q_begin : kNonCausalPos;
        it.q_count = tl.q_count;
        it.kv_begin = std::max(tl.kv_lo, pc.g0 * kSplitGranule);
        it.kv_end = std::min(tl.kv_hi, pc.g1 * kSplitGranule);
        it.part_row = tile_part[size_t(pc.tile)];
        sc.piece_dur[i] = kItemNs + int64_t(pc.g1 - pc.g0) * sc.block_ns[size_t(pc.tile)];
      }
      int32_t cnt[kXcds][kSeClasses] = {};
      items.resize(np * size_t(hkv));
      sc.placed.resize(np * size_t(hkv));
      {
        int32_t k = 0;
        for (int32_t h = 0; h < hkv; ++h)
          for (uint64_t pk : sc.packed) {
            const int32_t r = int32_t(pk & 0xfffff);
            const int32_t x = xcd_of_run(h, r), c = sc.run_cls[size_t(h) * size_t(runs) + size_t(r)];
            const int32_t f0 = sc.run_first[size_t(r)], f1 = sc.run_first[size_t(r) + 1];
            for (int32_t i = f0; i < f1; ++i, ++k) {
              sc.placed[size_t(k)] =
                  Placed{x, c, i > f0 ? 1 : 0, i > f0 ? sc.pieces[size_t(i)].start : 0, sc.piece_dur[size_t(i)], k};
              WorkItem& it = items[size_t(k)];
              it = sc.piece_item[size_t(i)];
              it.head_split |= h << (2 * kSplitBits);
            }
            cnt[x][c] += f1 - f0;
          }
      }
      // bucket offsets; first pieces keep their order, later ones are sorted per bucket
      int32_t off[kXcds][kSeClasses + 1], nfirst[kXcds][kSeClasses] = {};
      {
        int32_t at = 0;
        for (int x = 0; x < kXcds; ++x)
          for (int c = 0; c < kSeClasses; ++c) {
            off[x][c] = at;
            at += cnt[x][c];
          }
      }
      {
        int32_t fill[kXcds][kSeClasses];
        for (int x = 0; x < kXcds; ++x)
          for (int c = 0; c < kSeClasses; ++c) fill[x][c] = off[x][c];
        for (const Placed& pl : sc.placed) nfirst[pl.xcd][pl.cls] += pl.later == 0;
        // first pieces in dealing order, then later pieces
        int32_t lat[kXcds][kSeClasses];
        for (int x = 0; x < kXcds; ++x)
          for (int c = 0; c < kSeClasses; ++c) lat[x][c] = off[x][c] + nfirst[x][c];
        sc.by_xcd.resize(sc.placed.size());
        for (uint32_t k = 0; k < sc.placed.size(); ++k) {
          const Placed& pl = sc.placed[k];
          sc.by_xcd[size_t(pl.later ? lat[pl.xcd][pl.cls]++ : fill[pl.xcd][pl.cls]++)] = k;
        }
        for (int x = 0; x < kXcds; ++x)
          for (int c = 0; c < kSeClasses; ++c) {
            auto b = sc.by_xcd.begin() + off[x][c] + nfirst[x][c], e = sc.by_xcd.begin() + off[x][c] + cnt[x][c];
            std::sort(b, e, [&](uint32_t u, uint32_t v) {
              const Placed &a = sc.placed[u], &q = sc.placed[v];
              return a.key != q.key ? a.key < q.key : a.dur != q.dur ? a.dur > q.dur : u < v;
            });
          }
      }
      // workgroup (kSeClasses r + c) * kXcds + x: XCD x's (kSeClasses r + c)-th,
      // on engine class c -- the r-th item of that class; a class with fewer
      // items than the XCD's longest is padded with empty ones
      size_t n_pos = 0;
      for (int x = 0; x < kXcds; ++x) {
        int32_t depth = 0;
        for (int c = 0; c < kSeClasses; ++c) depth = std::max(depth, cnt[x][c]);
        n_pos = std::max(n_pos, size_t(depth) * kSeClasses * kXcds);
      }
      WorkItem pad;
      std::memset(&pad, 0, sizeof(pad));   // q_count 0: skipped by the kernels
      pad.part_row = -1;
      ordered_out.assign(n_pos, pad);
      for (int x = 0; x < kXcds; ++x)
        for (int c = 0; c < kSeClasses; ++c)
          for (int32_t r = 0; r < cnt[x][c]; ++r)
            ordered_out[(size_t(r) * kSeClasses + size_t(c)) * kXcds + size_t(x)] =
                items[size_t(sc.placed[sc.by_xcd[size_t(off[x][c] + r)]].seq)];
      while (!ordered_out.empty() && ordered_out.back().q_count == 0) ordered_out.pop_back();
    }
  }

  // Dispatch order. Workgroups go to the 8 XCDs round-robin (workgroup i runs on
  // XCD i mod 8), and each XCD has its own L2. Items that read the same keys --
  // same request, KV head and split -- are grouped and each group is placed on
  // one XCD (groups assigned greedily to the least-loaded XCD, largest first),
  // so the tiles that stream one KV head stay together in one L2. Within an XCD
  // the longest items go first; an item's time grows with its key range times
  // its live 32-row waves. A size query (no meta_host) needs no order.
  if (!streamed && meta_host) xcd_order(sc, n_groups, cost_max);
  const std::vector<WorkItem>& ordered = streamed || meta_host ? sc.ordered : items;
  const int32_t n_items = int32_t(ordered.size());
  const MetaLayout lay = meta_layout(batch, n_items, n_split_rows);
  if (meta_bytes_out) *meta_bytes_out = lay.total;
  // key blocks the busiest workgroup slot streams: the longest item, or the
  // average per slot when there are more items than slots
  const int64_t slot_blocks = streamed ? stream_blocks : std::max(max_blocks, (sum_blocks + slots - 1) / slots);

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
    // every section is written in full below: zero only the padding between
    // sections and the status word
    auto zero = [base](size_t from, size_t to) { std::memset(base + from, 0, to - from); };
    zero(lay.qo_indptr + sizeof(int32_t) * (size_t(batch) + 1), lay.kv_indptr);
    zero(lay.kv_indptr + sizeof(int32_t) * (size_t(batch) + 1), lay.prefix_lens);
    zero(lay.prefix_lens + sizeof(int32_t) * size_t(batch), lay.items);
    zero(lay.items + sizeof(WorkItem) * ordered.size(), lay.split_rows);
    zero(lay.split_rows + 2 * sizeof(int32_t) * size_t(n_split_rows), lay.total);
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
    // split rows: (global token, split count) for every token of a split tile, in partial-row order
    int32_t* sr = reinterpret_cast<int32_t*>(base + lay.split_rows);
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      if (tile_part[ti] < 0) continue;
      const Tile& t = tiles[ti];
      int32_t* row = sr + 2 * size_t(tile_part[ti]);
      const int32_t tok = qo_start[size_t(t.req)] + t.q_begin;
      for (int32_t i = 0; i < t.q_count; ++i) {
        row[2 * i] = tok + i;
        row[2 * i + 1] = tile_splits[ti];
      }
    }
  }
  return PKV_OK;
}

}  // namespace pkv
