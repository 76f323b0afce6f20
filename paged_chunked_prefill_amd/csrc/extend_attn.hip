// Paged extend attention for chunked prefill on CDNA4 (gfx950).
//
// What is computed (AReno PR #642, "What does this PR do?"): every query row of
// the current chunk attends to its request's cached prefix plus its own chunk,
// with the causal mask aligned bottom-right -- row i of a chunk that follows P
// cached tokens sees key positions 0..P+i -- optionally limited to a sliding
// window of W positions ending at its own. Query head h reads KV head
// h / (Hq/Hkv) (AstrAI compare v1.3.12..925cbed, attn_paged_test.cu CPU
// reference for paged prefill).
//
// How (one workgroup per planner work item = GQA-packed query tile x key range):
//  * The tile's rows are (token, query head) pairs of one KV head; eight waves
//    own 32 rows each (256 rows), so every K/V tile staged in LDS serves all
//    G heads of 256/G tokens.
//  * Keys are walked in 64-key tiles aligned to absolute positions, through a
//    4-stage LDS ring. A tile is gathered from the paged pool straight into
//    LDS (global_load_lds, 16 bytes per lane, no register staging): the page
//    id of each group of rows is a scalar load, and positions outside the
//    item's key range read the nearest key inside it, which the mask removes.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K rows come from LDS, the wave's
//    Q rows stay in registers. Each lane then holds 16 scores of one query row
//    per 32-key block, so the row max needs one cross-half permlane swap and
//    the exponentials are plain per-lane VALU work (exp2 with the softmax
//    scale folded with log2 e).
//  * O^T += V^T P^T on the same MFMA: P^T is the score accumulator converted
//    to bf16 in place (its register layout is already the B-operand layout);
//    V^T fragments come from LDS through ds_read_b64_tr_b16, which transposes
//    4x16-element blocks on the fly, so V needs no transposed copy.
//  * Two groups of four waves (one wave of each on every SIMD) run the tile
//    program one segment apart: one group's MFMA segment (PV of tile t, S of
//    tile t+1) overlaps the other group's softmax segment.
//  * Online softmax (running max and sum per row); split items store the
//    unnormalised output with (max, sum) and a combine kernel merges splits.
// fp32 inputs take a separate, simpler kernel (4 waves, 128 rows, 32-key tiles
// staged through registers into a double-buffered LDS tile, v_mfma_f32_32x32x2f32).
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <utility>

#include "pkv_internal.hpp"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* req_pool_indices;
  const WorkItem* items;
  int32_t* status;
  void* out;
  void* o_part;     // bf16 partials for the bf16 kernel, fp32 for the fp32 kernel
  float* ml_part;
  int32_t page_table_stride;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t page_size;
  int32_t page_shift;  // log2(page_size) when a power of two, else -1
  int32_t num_pages;
  int32_t window;
  int32_t total_q;
  int32_t max_splits;
  float scale_log2;
  // explicit keep-mask (only the MASK kernels read these): byte (b, h, i, j) at
  // mask[((b * mask_heads + h) * mask_rows + i) * mask_kv_stride + j], a size-1
  // head or row axis shared; i is the chunk row, j the absolute key position
  const uint8_t* mask;
  int32_t mask_heads;
  int32_t mask_rows;
  int32_t mask_kv_stride;
  const int32_t* qo_indptr;
  // fused append (FUSED kernels only): the chunk's own K/V rows [total_q][Hkv][D],
  // read by the gather for positions >= P_b and copied into their pool slots
  const void* k_new;
  const void* v_new;
  void* k_pool_w;
  void* v_pool_w;
  const int32_t* prefix_lens;
};

// Byte offset of the mask row of (request, query head, chunk row).
__device__ inline int64_t mask_row_offset(const Params& p, int req, int head, int chunk_row) {
  const int h = p.mask_heads > 1 ? head : 0;
  const int i = p.mask_rows > 1 ? chunk_row : 0;
  return (int64_t(req * p.mask_heads + h) * p.mask_rows + i) * p.mask_kv_stride;
}

// Value of the same query row held by the other half of the wave (lanes l and
// l^32 hold the two halves of one row's scores).
__device__ inline float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-item geometry shared by both instantiations.
struct ItemView {
  int req, kv_head, split, nsplit, q_count, kv_begin, kv_end, part_row;
  int tok0, pos0, pt_row;
};

__device__ inline ItemView load_item(const Params& p) {
  const WorkItem it = p.items[blockIdx.x];
  ItemView v;
  v.req = it.req;
  v.kv_head = it.head_split >> (2 * kSplitBits);
  v.split = it.head_split & ((1 << kSplitBits) - 1);
  v.nsplit = max(1, (it.head_split >> kSplitBits) & ((1 << kSplitBits) - 1));
  v.part_row = it.part_row;
  v.tok0 = it.tok0;
  v.pos0 = it.pos0;
  v.q_count = it.q_count;
  v.kv_begin = max(it.kv_begin, 0);
  // never read past the page table's row, whatever the item says
  const int64_t addressable = int64_t(p.page_table_stride) * p.page_size;
  v.kv_end = int(min(int64_t(it.kv_end), addressable));
  v.pt_row = p.req_pool_indices ? p.req_pool_indices[it.req] : it.req;
  return v;
}

// Is key position j visible from the query at absolute position qpos?
__device__ inline bool key_visible(int j, int qpos, int kv_begin, int kv_end, int window) {
  return j >= kv_begin && j < kv_end && j <= qpos && (window <= 0 || j > qpos - window);
}

// ---------------------------------------------------------------------------
// bf16: 64-key tiles, 32x32x16 MFMA, K/V gathered straight into LDS
// ---------------------------------------------------------------------------

// Sixteen zero bytes per lane: the source of every key slot that must read as
// zeros (a page id outside the pool).
__device__ __attribute__((aligned(16))) const uint32_t g_zero_rows[64 * 4] = {};

// Scores are kept relative to a per-row reference m_ref (log2 units), set by
// the row's first tile with a visible key to that tile's max. Later tiles are
// weighted against the reference without taking their max (which costs 24
// VALU instructions per wave and tile); only when some lane's sum of its 32
// weights exceeds kLazyLimit does the tile get its scores again (recomputed:
// the weights overwrote them) and its max, and every row of the wave whose
// max beat its reference is raised to it (O and the running sum rescaled).
// Every weight therefore stays at most 2^7, a reference trails its row's
// running max by at most 7 (a larger gap makes a weight above 2^7: caught),
// and it never exceeds that max, so no weight underflows because of it.
constexpr float kLazyLimit = 128.f;

// s_waitcnt immediate: vmcnt(N), lgkmcnt(0), expcnt unchanged (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
constexpr int kWaitVm = (N & 15) | ((N >> 4) << 14) | (7 << 4);
// s_waitcnt lgkmcnt(0) alone (vmcnt 63 and expcnt 7 do not wait)
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS address `lds` + 16 l. Issued as inline asm so that the
// compiler does not track these LDS writes (it would otherwise make every LDS
// read wait for them); the kernel orders them itself with s_waitcnt vmcnt and
// barriers. m0 is reserved by the compiler and set here for each copy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "m0");
}
__device__ __forceinline__ void lds_copy16(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(vaddr), "s"(lds)
               : "m0");
}
#pragma clang diagnostic pop

template <int D>
struct Bf16Tile {
  static constexpr int BC = kTileKeysBf16;       // keys per tile
  static constexpr int ROWB = D * 2;             // LDS bytes per key row (no padding; XOR swizzle instead)
  static constexpr int TILEB = BC * ROWB;        // one K (or V) tile
  static constexpr int STAGE = 2 * TILEB;        // K then V
  static constexpr int NSTAGE = 4;               // LDS ring of tiles
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;            // rows one wave-wide 1 KiB copy covers
  static constexpr int NW = kWavesBf16;          // waves per workgroup
  static constexpr int LOADS = BC / RPI / NW;    // such copies per wave per tensor and tile
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  // The item's Q rows are gathered into LDS once, over the ring's last stage
  // (first written by the gather of tile 3, after the prologue) and the space
  // after the ring, then read into registers.
  static constexpr int QBYTES = 32 * NW * ROWB;             // 32 rows per wave
  static constexpr int QOFF = (NSTAGE - 1) * STAGE;
  static constexpr int LDS_BYTES = QOFF + QBYTES;
  static constexpr int QCOPIES = QBYTES / 1024 / NW;        // wave-wide 1 KiB copies per wave
  static_assert(QBYTES >= STAGE, "the Q region covers the last stage");
  // XOR swizzles of the 16-byte chunks of a row (64 banks of 4 bytes = 256 B
  // per bank row; a D=64 row is half of one). K: the 16 lanes of a b128 read
  // that issue together read 16 rows at one chunk index; chunk c of row r sits
  // at c ^ (r mod 16) for D=128, at c ^ ((r/2) mod 8) for D=64, so they cover
  // all 64 banks. V: a half-wave of transposing reads takes 64 bytes (a group
  // of 4 chunks) from each of 4 consecutive rows; the group index is XORed with
  // r mod 4 (D=128) or (r/2) mod 2 (D=64) so the 4 rows use disjoint banks.
  // K's depends on r modulo 16 and V's on r modulo 4; the row offsets added
  // to a lane's base row (multiples of 32 for K, of 8 for V) keep them.
  static __device__ int kswz(int r) { return CH == 16 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ int vswz(int r) { return CH == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Keep-mask helpers (MASK instantiation). Word K of a lane's tile holds the
// mask bytes of keys 32(K/4) + 8(K%4) + 4half .. +3 after the lane's tile
// base: loads the compiler does not see (see the kernel), with the offsets as
// immediates.
template <int K>
__device__ __forceinline__ void load_mask_word(uint32_t& w, const uint8_t* a) {
  asm volatile("global_load_dword %0, %1, off offset:%2" : "=v"(w) : "v"(a), "n"(32 * (K >> 2) + 8 * (K & 3)));
}
template <int... K>
__device__ __forceinline__ void load_mask_words(uint32_t* w, const uint8_t* a, std::integer_sequence<int, K...>) {
  (load_mask_word<K>(w[K], a), ...);
}
// Issue order of the MFMA segment (see seg_M below): PV and S steps
// alternate (even steps PV, odd steps S), each one MFMA whose A fragment was
// read from LDS AHEAD steps earlier (two transposing reads for PV, one b128 read
// for S). Pins that order in the scheduler: the first reads, then per step the
// reads of step+AHEAD and the step's MFMA.
template <int ST, int NSTEP, int AHEAD>
__device__ __forceinline__ void pin_m_schedule() {
  constexpr int kMaskMfma = 0x008, kMaskDsRead = 0x100;
  if constexpr (ST == 0) {
    constexpr int first = AHEAD + (AHEAD + 1) / 2;   // 2 reads per even step, 1 per odd step
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, first, 0);
  }
  if constexpr (ST + AHEAD < NSTEP)
    __builtin_amdgcn_sched_group_barrier(kMaskDsRead, (ST + AHEAD) % 2 == 0 ? 2 : 1, 0);
  __builtin_amdgcn_sched_group_barrier(kMaskMfma, 1, 0);
  if constexpr (ST + 1 < NSTEP) pin_m_schedule<ST + 1, NSTEP, AHEAD>();
}

template <int D, bool POW2_PAGES, bool MASK, bool FUSED>
__global__ __launch_bounds__(64 * kWavesBf16, 2) void extend_attn_bf16(const Params p) {
  using T = Bf16Tile<D>;
  static_assert(!(MASK && FUSED), "the fused append has no masked form");
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
  const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) char*)smem));

  const ItemView it = load_item(p);
  if (it.q_count <= 0) return;   // (uniform) a padding item covers no row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int G = p.group;

  // this lane's query row: tile row r = token * G + head-in-group
  const int r = wave * 32 + l32;
  const int tok = r / G, gh = r - tok * G;
  const int gtok = it.tok0 + tok;                            // global token index
  const bool row_live = tok < it.q_count && gtok < p.total_q;
  const int qpos = it.pos0 + tok;                            // absolute query position
  const int head = it.kv_head * G + gh;
  const bool wave_live = wave * 32 < it.q_count * G;
  const int qpos_first = it.pos0;
  const int qpos_last = it.pos0 + it.q_count - 1;

  f32x16 o[T::DBLK];
#pragma unroll
  for (int db = 0; db < T::DBLK; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max of this row, log2 units (scaled scores)
  float l_run = 0.f;        // running sum of 2^(s - m_ref) over the keys this lane holds
  bool need_ref = true;     // (uniform) some row of the wave still has m_ref = -inf

  const int t0 = (it.kv_begin / T::BC) * T::BC;
  const int ntiles = it.kv_end > it.kv_begin ? (it.kv_end - t0 + T::BC - 1) / T::BC : 0;
  const int32_t* pt = p.page_table + int64_t(it.pt_row) * p.page_table_stride;
  const char* kpool = static_cast<const char*>(p.k_pool);
  const char* vpool = static_cast<const char*>(p.v_pool);
  const int ps = p.page_size, ps_shift = p.page_shift;
  const uint32_t row_bytes = uint32_t(p.num_kv_heads) * D * 2;   // < 2^24, checked on the host
  const uint32_t page_bytes = uint32_t(ps) * row_bytes;          // < 2^31, checked on the host
  const int kv_last = it.kv_end - 1;

  // Fused append (FUSED): key positions >= P_b are the chunk's own rows. The
  // gather reads them from k_new / v_new (position P_b + i is token
  // qo_indptr[b] + i there), never from the pool slots this launch is filling;
  // the owner item of each new row (below) copies it into its slot.
  int fresh0 = INT_MAX;        // P_b: first position read from k_new / v_new
  int tile_pos = 0;            // position of the tile's first token
  const char* knew = nullptr;  // K row of position P_b (all KV heads)
  const char* vnew = nullptr;
  if constexpr (FUSED) {
    fresh0 = ((const __attribute__((address_space(4))) int32_t*)p.prefix_lens)[it.req];
    const int qs = ((const __attribute__((address_space(4))) int32_t*)p.qo_indptr)[it.req];
    tile_pos = fresh0 + (it.tok0 - qs);
    knew = static_cast<const char*>(p.k_new) + int64_t(qs) * row_bytes;
    vnew = static_cast<const char*>(p.v_new) + int64_t(qs) * row_bytes;
  }

  // Gather: wave w's copy i fills LDS rows RPI*(NW*i+w) .. +RPI-1 of a tile; lane l
  // covers row RPI*(NW*i+w) + l/CH at LDS chunk l%CH, i.e. source chunk (l%CH) ^ swz(row).
  // Both swizzles depend on the row only modulo CH, the same for every i. A key
  // outside [kv_begin, kv_end) reads the nearest key inside the range instead:
  // finite data that the mask turns into a -inf score and a zero weight, and no
  // slot past the request's positions is ever touched. With POW2_PAGES (a
  // power-of-two page size of at least RPI rows) the RPI rows of one copy share
  // a page, before and after that clamp: its id is one scalar load (constant
  // address space, so it never waits on copies in flight) and the source is a
  // scalar base plus a 32-bit lane offset.
  const int lrow = lane / T::CH;
  const int srow = T::RPI * wave + lrow;   // row modulo CH decides both swizzles
  const uint32_t src_k = uint32_t(it.kv_head) * D * 2 + 16 * ((lane % T::CH) ^ T::kswz(srow));
  const uint32_t src_v = uint32_t(it.kv_head) * D * 2 + 16 * ((lane % T::CH) ^ T::vswz(srow));
  auto clampk = [&](int j) __attribute__((always_inline)) { return min(max(j, it.kv_begin), kv_last); };
  auto page_col = [&](int j) __attribute__((always_inline)) { return POW2_PAGES ? (j >> ps_shift) : j / ps; };
  const __attribute__((address_space(4))) int32_t* pt_const = (const __attribute__((address_space(4))) int32_t*)pt;
  int pg[T::LOADS];  // page ids for the next tile to gather
  bool bad_page = false;
  auto fetch_pages = [&](int* ids, int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int blk = kv0 + T::RPI * (T::NW * i + wave);
      if (POW2_PAGES)
        ids[i] = pt_const[page_col(clampk(blk))];
      else
        ids[i] = pt[page_col(clampk(blk + lrow))];
    }
  };
  // One wave-wide copy of RPI key rows of K and of V: with POW2_PAGES (unfused) a
  // scalar base and a lane offset each, else a full lane address each (a fused
  // copy may take some rows from the pool and the rest from k_new / v_new).
  struct Copy {
    const char* k;
    const char* v;
    uint32_t koff, voff, dst;
  };
  auto prepare = [&](const int* ids, int kv0, uint32_t stage_lds, Copy* cp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int j = clampk(kv0 + T::RPI * (T::NW * i + wave) + lrow);
      const int page = ids[i];
      const bool ok = uint32_t(page) < uint32_t(p.num_pages);
      bad_page |= !ok;
      cp[i].dst = stage_lds + T::RPI * (T::NW * i + wave) * T::ROWB;  // first row of this copy
      if (POW2_PAGES && !FUSED) {
        const uint32_t off = __umul24(uint32_t(j & (ps - 1)), row_bytes);
        const uint64_t pbase = uint64_t(uint32_t(ok ? page : 0)) * page_bytes;
        cp[i].k = ok ? kpool + pbase : reinterpret_cast<const char*>(g_zero_rows);
        cp[i].v = ok ? vpool + pbase : reinterpret_cast<const char*>(g_zero_rows);
        cp[i].koff = ok ? off + src_k : 16u * lane;
        cp[i].voff = ok ? off + src_v : 16u * lane;
      } else {
        const int slot = POW2_PAGES ? (j & (ps - 1)) : j - (j / ps) * ps;
        const uint64_t pbase = uint64_t(uint32_t(ok ? page : 0)) * page_bytes + uint32_t(slot) * row_bytes;
        const char* zero = reinterpret_cast<const char*>(g_zero_rows) + 16 * lane;
        cp[i].k = ok ? kpool + pbase + src_k : zero;
        cp[i].v = ok ? vpool + pbase + src_v : zero;
        if (FUSED && j >= fresh0) {   // a row of this chunk: straight from k_new / v_new
          const int64_t r = int64_t(j - fresh0) * row_bytes;
          cp[i].k = knew + r + src_k;
          cp[i].v = vnew + r + src_v;
        }
        cp[i].koff = cp[i].voff = 0;
      }
    }
  };
  // copy c of a prepared tile: K rows for even c, V rows for odd c
  auto issue = [&](const Copy* cp, int c) __attribute__((always_inline)) {
    const Copy& x = cp[c >> 1];
    if (POW2_PAGES && !FUSED) {
      if (c & 1) lds_copy16(x.v, x.voff, x.dst + T::TILEB); else lds_copy16(x.k, x.koff, x.dst);
    } else {
      if (c & 1) lds_copy16(x.v, x.dst + T::TILEB); else lds_copy16(x.k, x.dst);
    }
  };

  // per-lane LDS read offsets within a stage (the row-block terms are immediates)
  // K (A operand of S^T): row l32 (+32 for the second key block), chunk (2ks+half) ^ swz
  uint32_t koff[T::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < T::KSTEPS; ++ks) koff[ks] = l32 * T::ROWB + 16 * ((2 * ks + half) ^ T::kswz(l32));
  // V (A operand of O^T += V^T P^T via transposing reads): lane 16g+4e+q reads row
  // 4(g/2)+e (+ 32kb2 + 16m2 + 8hi) at d = 32db + 16(g%2) + 4q
  uint32_t voff[T::DBLK];
  {
    const int g4 = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int vr = 4 * (g4 >> 1) + e4;
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
      voff[db] = T::TILEB + vr * T::ROWB + 16 * ((4 * db + 2 * (g4 & 1) + (q4 >> 1)) ^ T::vswz(vr)) + 8 * (q4 & 1);
  }

  // ---- ping-pong schedule -------------------------------------------------
  // Waves w and w+4 share a SIMD. Group 0 (waves 0-3) and group 1 (waves 4-7)
  // run the same per-tile program one segment apart, so that while one group
  // issues its MFMA segment the other runs its softmax (VALU) segment:
  //   segment S0: S(0) = K(0) Q^T                                     (prologue)
  //   segment V:  mask, row max, rescale, P(t) = exp2(S(t) - m)       (VALU)
  //   segment M:  O += V(t)^T P(t), then S(t+1) = K(t+1) Q^T           (MFMA)
  // Slot j lies between block barriers j-1 and j; group 0 runs its segment j in
  // slot j, group 1 in slot j+1. Tile u sits in LDS stage u % 4; its gather is
  // issued in slot 2u-4 (once both groups have read tile u-4 from that stage)
  // and must land before slot 2u, where group 0 first reads K(u). Every barrier
  // first waits for this wave's gathers older than the newest one, so a gather
  // has about three slots to land. Each wave loads the page ids of tile t+3 at
  // the start of its V(t) segment (it reads no LDS, so no LDS wait there has to
  // wait for the scalar loads too: they share one counter) and issues its copies
  // of tile t+3 spread over its M(t) segment, between the MFMAs.
  const int grp = wave >> 2;
  const float c = p.scale_log2;
  const int window = p.window;
  bool newest_issued = false;   // was the most recent gather real (or a clamped one)?
  Copy cp[T::LOADS];
  auto stage_of = [&](int u) __attribute__((always_inline)) {
    return lds0 + uint32_t(u & (T::NSTAGE - 1)) * T::STAGE;
  };
  // wait for LDS reads and for every gather but the newest, then the block barrier.
  // The LDS/scalar wait comes first on its own so that it stays on every path
  // (the compiler then knows no scalar load is pending after a barrier).
  // EXTRA more loads may stay in flight: the keep-mask loads issued after the
  // newest gather (MASK only, see below).
  auto sync = [&](auto extra_c) __attribute__((always_inline)) {
    constexpr int EXTRA = decltype(extra_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (POW2_PAGES && newest_issued)
      __builtin_amdgcn_s_waitcnt(kWaitVm<2 * T::LOADS + EXTRA>);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Keep-mask (MASK): the 32 mask bytes of this lane's row for a tile, as 8
  // words (key block kb2, group g: keys kv0 + 32kb2 + 8g + 4half .. +3, the
  // order of the score accumulator), loaded one tile ahead with loads the
  // compiler does not see (a compiler-visible load would make its first use
  // wait for every gather in flight). They are issued right after the newest
  // gather's copies and before the next ones, so the barrier waits below cover
  // them; each word array is pinned (an empty asm that "writes" it) after such
  // a wait, before its first use. Group starts outside the item's key range
  // are clamped into it (4-byte aligned): those keys are masked by the range.
  constexpr int kMaskWords = 8;
  uint32_t mw_cur[kMaskWords], mw_next[kMaskWords];
  const uint8_t* mrow = nullptr;
  if constexpr (MASK)
    mrow = p.mask + mask_row_offset(p, it.req, head, it.tok0 + (row_live ? tok : 0) - p.qo_indptr[it.req]);
  auto mask_issue = [&](int u, uint32_t* w) __attribute__((always_inline)) {
    const int kvb4 = it.kv_begin & ~3, kvl4 = (it.kv_end - 1) & ~3;
    const int kv0u = t0 + u * T::BC;
    if (kv0u >= kvb4 && kv0u + T::BC - 4 <= kvl4) {
      // (uniform) every word of the tile lies in the range: one address, immediate offsets
      load_mask_words(w, mrow + kv0u + 4 * half, std::make_integer_sequence<int, kMaskWords>{});
    } else {
#pragma unroll
      for (int k = 0; k < kMaskWords; ++k) {
        const int gs = min(max(kv0u + 32 * (k >> 2) + 8 * (k & 3) + 4 * half, kvb4), kvl4);
        asm volatile("global_load_dword %0, %1, off" : "=v"(w[k]) : "v"(mrow + gs));
      }
    }
  };
  auto mask_pin = [&](uint32_t* w) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) asm volatile("" : "+v"(w[k]));
  };

  // Fused append: the S splits of a tile share the copying of its tokens' new
  // rows (KV head of the item): split k takes tokens t = k, k + S, k + 2S, ...
  // (every row once, whatever the key ranges). The first OWN_VECS vectors are
  // loaded with tile 0 (loads the compiler does not see, so the prologue's
  // wait covers them without waiting for tiles 1-2) and stored after that
  // wait; any rest (more than 64 owned tokens at D = 128) after the tile loop.
  // Lane vector v: owned token v / (2 VPR), K for the first VPR vectors, then V.
  constexpr int VPR = D * 2 / 16;                        // 16-byte vectors of one head's row
  constexpr int NOWN = 4;                                // vectors per lane in the prologue copy
  constexpr int OWN_VECS = 64 * kWavesBf16 * NOWN;
  int own_n = 0;   // tokens this item copies
  if constexpr (FUSED)
    own_n = it.split < it.q_count ? (it.q_count - it.split + it.nsplit - 1) / it.nsplit : 0;
  struct OwnVec {
    const char* src;
    char* dst;    // pool slot, page not yet applied
    int col;      // page-table column of the row
  };
  auto own_vec = [&](int v) __attribute__((always_inline)) {
    const int u = v / (2 * VPR), rem = v - u * (2 * VPR);
    const bool isv = rem >= VPR;
    const int e = isv ? rem - VPR : rem;
    const int pos = tile_pos + it.split + u * it.nsplit;
    const int64_t head_off = int64_t(it.kv_head) * D * 2 + 16 * e;
    OwnVec o;
    o.src = (isv ? vnew : knew) + int64_t(pos - fresh0) * row_bytes + head_off;
    o.col = page_col(pos);
    const int slot = pos - o.col * ps;
    o.dst = static_cast<char*>(isv ? p.v_pool_w : p.k_pool_w) + int64_t(slot) * row_bytes + head_off;
    return o;
  };
  u32x4 own_data[NOWN];
  int own_page[NOWN];
  auto own_issue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < NOWN; ++r) {
      if (64 * kWavesBf16 * r < own_n * 2 * VPR) {   // (uniform)
        const int v = min(tid + 64 * kWavesBf16 * r, own_n * 2 * VPR - 1);
        const OwnVec o = own_vec(v);
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(own_data[r]) : "v"(o.src));
        asm volatile("global_load_dword %0, %1, off" : "=v"(own_page[r]) : "v"(pt + o.col));
      }
    }
  };
  auto own_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < NOWN; ++r) {
      if (64 * kWavesBf16 * r < own_n * 2 * VPR) {
        asm volatile("" : "+v"(own_data[r]), "+v"(own_page[r]));   // landed: waited for above
        const int v = tid + 64 * kWavesBf16 * r;
        const bool ok = uint32_t(own_page[r]) < uint32_t(p.num_pages);
        bad_page |= !ok;
        if (v < own_n * 2 * VPR && ok)
          *reinterpret_cast<u32x4*>(own_vec(v).dst + int64_t(own_page[r]) * page_bytes) = own_data[r];
      }
    }
  };

  // prologue part 1: the item's Q rows gathered into LDS like the K rows (same
  // copy shape and swizzle; rows past the item read the item's first token:
  // finite, never stored), issued first.
#pragma unroll
  for (int c = 0; c < T::QCOPIES; ++c) {
    const int r = T::RPI * (T::NW * c + wave) + lrow;   // tile row = token * G + head-in-group
    int qt = r / G;
    const int qh = r - qt * G;
    if (qt >= it.q_count || it.tok0 + qt >= p.total_q) qt = 0;
    const char* src = static_cast<const char*>(p.q) +
                      ((int64_t(it.tok0 + qt) * p.num_q_heads + it.kv_head * G + qh) * D) * 2 +
                      16 * ((lane % T::CH) ^ T::kswz(r));
    lds_copy16(src, lds0 + T::QOFF + T::RPI * (T::NW * c + wave) * T::ROWB);
  }
  // tiles 0..2 in flight. All three are gathered even when the item has fewer
  // (clamped keys, see below), so that every page id is loaded up front with
  // one wait.
  if (ntiles > 0) {
    int ids[3][T::LOADS];
#pragma unroll
    for (int u = 0; u < 3; ++u) fetch_pages(ids[u], t0 + u * T::BC);
    if constexpr (POW2_PAGES) {
      // every id in hand here: the scalar loads go out together, one wait
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int i = 0; i < T::LOADS; ++i) asm volatile("" ::"s"(ids[u][i]));
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      prepare(ids[u], t0 + u * T::BC, stage_of(u), cp);
#pragma unroll
      for (int c2 = 0; c2 < 2 * T::LOADS; ++c2) issue(cp, c2);
      if (MASK && u == 0) mask_issue(0, mw_cur);   // landed with tile 0 at the wait below
      if (FUSED && u == 0) own_issue();            // likewise
    }
    newest_issued = true;
  }
  // Q and tile 0 landed; tiles 1 and 2 may still be in flight (the loop's
  // waits cover them). Without POW2_PAGES the page ids are vector loads the
  // compiler waits for with everything older: wait for all here.
  if (POW2_PAGES && ntiles > 0)
    __builtin_amdgcn_s_waitcnt(kWaitVm<4 * T::LOADS>);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (MASK && ntiles > 0) mask_pin(mw_cur);
  if (FUSED && ntiles > 0) own_store();
  // Q fragments (B operand of S^T = K Q^T): lane holds q[row][16ks + 8half .. +7]
  bf16x8 qf[T::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < T::KSTEPS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(smem + T::QOFF + wave * 32 * T::ROWB + koff[ks]);

  f32x16 s[2];            // scores S^T of the tile in flight (two 32-key blocks)
  bf16x8 pb[2][2];        // P of the tile being accumulated, as B operands
  auto k_frag = [&](uint32_t kb, int ks, int kb2) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(smem + kb + koff[ks] + 32 * kb2 * T::ROWB);
  };
  auto seg_S0 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < T::KSTEPS; ++ks)
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(0, ks, kb2), qf[ks], s[kb2], 0, 0, 0);
    }
  };
  // scores of tile t once more, from K(t) in its LDS stage (intact until the
  // gather of tile t+4, which comes after both groups' M(t)): the same
  // fragments and MFMA order as the S(t) products, so the same bits
  auto recompute_S = [&](int t) __attribute__((always_inline)) {
    const uint32_t kst = uint32_t(t & (T::NSTAGE - 1)) * T::STAGE;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < T::KSTEPS; ++ks) {
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kst, ks, kb2), qf[ks], s[kb2], 0, 0, 0);
        // (a rare path: one fragment read at a time, none hoisted into
        // registers the rest of the loop needs)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto apply_mask = [&](int t) __attribute__((always_inline)) {
    const int kv0 = t0 + t * T::BC;
    // mask: element (kb2, j) is key kv0 + 32kb2 + 8(j/4) + 4half + j%4 of this lane's row
    const bool full = kv0 >= it.kv_begin && kv0 + T::BC <= it.kv_end && kv0 + T::BC - 1 <= qpos_first &&
                      (window <= 0 || kv0 > qpos_last - window);
    if (MASK && full) {
      // every key of the tile is in range for every row: the keep-mask alone
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (((mw_cur[4 * kb2 + (j >> 2)] >> (8 * (j & 3))) & 0xffu) == 0) s[kb2][j] = -INFINITY;
    } else if (!full) {
      // this row sees keys lo..hi of the item's range (one unsigned test per key)
      int lo = it.kv_begin, hi = min(kv_last, qpos);
      if (window > 0) lo = max(lo, qpos - window + 1);
      if (hi < lo) lo = hi = kv0 + T::BC;   // nothing visible in this tile
      const uint32_t width = uint32_t(hi - lo);
      const int d0 = kv0 + 4 * half - lo;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (uint32_t(d0 + 32 * kb2 + 8 * (j >> 2) + (j & 3)) > width ||
              (MASK && ((mw_cur[4 * kb2 + (j >> 2)] >> (8 * (j & 3))) & 0xffu) == 0))
            s[kb2][j] = -INFINITY;
    }
  };
  // raise the reference of every row whose max over the tile beat it to that
  // max (both halves of a row agree)
  auto raise_ref = [&]() __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb2][j]);
    mx = other_half_max(mx) * c;   // this row's max over the tile, log2 units
    const bool raise = mx > m_ref;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_ref;
      // lanes that keep their reference (possibly still -inf) must not compute -inf - -inf
      const float alpha = raise ? fast_exp2(m_ref - m_new) : 1.f;   // 0 when m_ref was -inf
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) o[db] *= alpha;
      m_ref = m_new;
    }
  };
  // P = exp2(S*c - m_off), in place over the scores (fp32); returns the sum of
  // this lane's 32 weights
  auto exp_in_place = [&](float m_off) __attribute__((always_inline)) {
    float sum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[kb2][j] = fast_exp2(fmaf(s[kb2][j], c, -m_off));
        sum += s[kb2][j];
      }
    return sum;
  };
  // Softmax segment: a tile is weighted against the current references; a
  // caught tile (kLazyLimit) gets its scores again and raises them, as do the
  // tiles of a wave with a row still lacking a reference (one site for the O
  // rescale).
  auto seg_V = [&](int t) __attribute__((always_inline)) {
    apply_mask(t);
    float lsum = 0.f;
    bool with_max = need_ref;   // (uniform)
    if (!with_max) {
      lsum = exp_in_place(m_ref);
      if (__builtin_amdgcn_ballot_w64(lsum > kLazyLimit)) {
        recompute_S(t);
        apply_mask(t);
        with_max = true;
      }
    }
    if (with_max) {
      raise_ref();
      need_ref = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
      lsum = exp_in_place(m_ref == -INFINITY ? 0.f : m_ref);
    }
    l_run += lsum;
    // P in bf16, laid out as the B operand of O^T += V^T P^T
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < 16; ++j) pb[kb2][j >> 3][j & 7] = (__bf16)s[kb2][j];
  };
  // segment M: O += V(t)^T P(t) and S(t+1) = K(t+1) Q^T, as one straight run of
  // MFMAs. Even step 2i is PV product i (d-block i % DBLK, key quarter i / DBLK),
  // odd step 2i+1 is S product i (k-step i / 2, key block i % 2): an MFMA that
  // accumulates into the registers of an earlier one comes 4 or more MFMAs
  // after it, past its latency. Each A fragment is read from LDS AHEAD steps
  // before its MFMA (at most 6 reads in flight; the LDS counter tracks 15).
  // After the last tile the S products read a stale stage and are never used.
  static_assert(4 * T::DBLK == 2 * T::KSTEPS, "PV and S steps pair up");
  constexpr int NSTEP = 8 * T::DBLK, AHEAD = 4;
  // the copies of a gather go out at these steps, spread over the segment
  constexpr int NCOPY = 2 * T::LOADS, COPY_GAP = NSTEP / NCOPY;
  auto seg_M = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);   // MFMA issue first when the SIMD's other wave is in its V segment
    const uint32_t vst = uint32_t(t & (T::NSTAGE - 1)) * T::STAGE;
    const uint32_t kst = uint32_t((t + 1) & (T::NSTAGE - 1)) * T::STAGE;
    auto frag = [&](int st) __attribute__((always_inline)) {
      const int i = st >> 1;
      if ((st & 1) == 0) {
        const int db = i % T::DBLK, km = i / T::DBLK;
        // the transpose hands lane l the keys 16km+8r+4(l/32)+e at d = 32db + l%32
        const char* va = smem + vst + voff[db] + 16 * km * T::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(va));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(va + 8 * T::ROWB));
        const u32x2 lo32 = __builtin_bit_cast(u32x2, lo), hi32 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a32 = {lo32[0], lo32[1], hi32[0], hi32[1]};
        return __builtin_bit_cast(bf16x8, a32);
      }
      return k_frag(kst, i >> 1, i & 1);
    };
    bf16x8 fr[AHEAD];
#pragma unroll
    for (int st = 0; st < AHEAD; ++st) fr[st] = frag(st);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const bf16x8 a = fr[st % AHEAD];
      if (st + AHEAD < NSTEP) fr[st % AHEAD] = frag(st + AHEAD);
      if (st % COPY_GAP == 2) issue(cp, st / COPY_GAP);
      const int i = st >> 1;
      if ((st & 1) == 0) {
        const int db = i % T::DBLK, km = i / T::DBLK;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[km >> 1][km & 1], o[db], 0, 0, 0);
      } else {
        const int ks = i >> 1, kb2 = i & 1;
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16{} : s[kb2], 0, 0, 0);
      }
    }
    pin_m_schedule<0, NSTEP, AHEAD>();
    __builtin_amdgcn_s_setprio(0);
  };

  // prologue part 2: S(0), group 1 one segment behind
  constexpr auto kNoExtra = std::integral_constant<int, 0>{};
  if (ntiles > 0) {
    if (grp == 1) sync(kNoExtra);
    if (wave_live) seg_S0();
    sync(kNoExtra);
  }
  // tile t: segments V(t) and M(t) = PV(t) + S(t+1). The gather of tile t+3 goes
  // with slot 2t+2: group 1 issues it before its V segment, group 0 before its M
  // segment (both just after the barrier that frees the stage). Group 1 skips
  // the barrier after its very last segment, which balances its extra first one.
  // Past the last tile the gathers still run, of keys clamped to the last one
  // (in bounds, mostly one repeated row) into stages that are no longer read,
  // which keeps the segment free of branches; they are waited for below.
  for (int t = 0; t < ntiles; ++t) {
    const bool last = t + 1 >= ntiles;
    if constexpr (MASK) {
      // tile t's words (loaded one iteration ago, waited for by the last barrier), then tile t+1's
      if (t > 0) {
        mask_pin(mw_next);
#pragma unroll
        for (int k = 0; k < kMaskWords; ++k) mw_cur[k] = mw_next[k];
      }
      mask_issue(t + 1, mw_next);
    }
    fetch_pages(pg, t0 + (t + 3) * T::BC);
    if (wave_live) seg_V(t);
    prepare(pg, t0 + (t + 3) * T::BC, stage_of(t + 3), cp);   // addresses only: nothing is written yet
    sync(std::integral_constant<int, MASK ? kMaskWords : 0>{});   // tile t+2's copies and the mask loads may fly
    if (wave_live) {
      seg_M(t);
    } else {
#pragma unroll
      for (int c2 = 0; c2 < NCOPY; ++c2) issue(cp, c2);
    }
    if (!last || grp == 0) sync(kNoExtra);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm<0>);   // no copy into LDS outlives the workgroup
  if constexpr (FUSED) {
    // owned rows past the prologue's share (plain loads and stores)
    for (int v = tid + (ntiles > 0 ? OWN_VECS : 0); v < own_n * 2 * VPR; v += 64 * kWavesBf16) {
      const OwnVec o = own_vec(v);
      const int page = pt[o.col];
      const bool ok = uint32_t(page) < uint32_t(p.num_pages);
      bad_page |= !ok;
      if (ok) *reinterpret_cast<u32x4*>(o.dst + int64_t(page) * page_bytes) = *reinterpret_cast<const u32x4*>(o.src);
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad_page) && lane == 0) atomicOr(p.status, PKV_STATUS_BAD_PAGE);

  if (!wave_live) return;
  const float l_tot = other_half_sum(l_run);
  const bool split_item = it.part_row >= 0;
  if (split_item && row_live && half == 0) {
    // reference max (log2 units) the partial is relative to, and its sum
    const int64_t prow = (int64_t(it.part_row + tok) * p.num_q_heads + head) * p.max_splits + it.split;
    *reinterpret_cast<f32x2*>(p.ml_part + prow * 2) = f32x2{m_ref, l_tot};
  }
  // The wave's 32 x D tile -- the output (O / l, l = 0 giving 0) or the split's
  // unnormalised partial, both bf16 -- goes out through LDS: written in the
  // accumulator's layout (register j of block db is d = 32db + 8(j/4) + 4half +
  // j%4 of the lane's row), read back as whole rows, so that a store instruction
  // writes RPI complete rows instead of 8 bytes of each of 32 rows. It is staged
  // in the wave's own rows of the stages of tiles ntiles+1 and ntiles+2: rows
  // that only this wave's copies write (they have landed, waited for above) and
  // that no wave reads again (they hold no tile of the item), so no other wave is
  // waited for. Piece g (tile rows RPI g .. RPI g + RPI-1) takes the rows of copy
  // g % LOADS, K tile for (g / LOADS) even, V tile for odd, of the first stage for
  // g < 2 LOADS, of the second for the rest; chunks are XOR-swizzled by row like
  // the K tiles.
  const float scale_out = split_item ? 1.f : (l_tot > 0.f ? 1.f / l_tot : 0.f);
  constexpr int PIECES = 32 / T::RPI;
  static_assert(PIECES == 4 * T::LOADS, "a wave's tile fills its rows of two stages");
  auto piece_base = [&](int g) __attribute__((always_inline)) {
    const uint32_t stage = stage_of(ntiles + 1 + (g >= 2 * T::LOADS ? 1 : 0)) - lds0;
    return stage + uint32_t(((g / T::LOADS) & 1) * T::TILEB) +
           uint32_t(T::RPI * (T::NW * (g % T::LOADS) + wave) * T::ROWB);
  };
  {
    const uint32_t wrow = piece_base(l32 / T::RPI) + uint32_t(l32 % T::RPI) * T::ROWB;
    // (a split's partial is stored unscaled: no multiply)
    auto stage = [&](auto scaled) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 v;
#pragma unroll
          for (int x = 0; x < 4; ++x)
            v[x] = (__bf16)(decltype(scaled)::value ? o[db][4 * jj + x] * scale_out : o[db][4 * jj + x]);
          const int chunk = (4 * db + jj) ^ T::kswz(l32);
          *reinterpret_cast<u32x2*>(smem + wrow + 16 * chunk + 8 * half) = __builtin_bit_cast(u32x2, v);
        }
    };
    if (split_item)
      stage(std::false_type{});
    else
      stage(std::true_type{});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own writes, read back by other lanes
  // every piece read back first (their reads overlap), then stored
  const int ec = lane % T::CH;
  u32x4 val[PIECES];
#pragma unroll
  for (int g = 0; g < PIECES; ++g)
    val[g] = *reinterpret_cast<const u32x4*>(smem + piece_base(g) + (lane / T::CH) * T::ROWB +
                                             16 * (ec ^ T::kswz(T::RPI * g + lane / T::CH)));
  // row (token t, query head h) of the output, or of this split's partials:
  // dst0 + (t Hq + h) * row_stride, with t Hq + h < 256 Hq < 2^30 and
  // row_stride = D or max_splits D (< 2^13)
  uint16_t* const dst0 =
      split_item ? static_cast<uint16_t*>(p.o_part) + (int64_t(it.part_row) * p.num_q_heads * p.max_splits + it.split) * D
                 : static_cast<uint16_t*>(p.out) + int64_t(it.tok0) * p.num_q_heads * D;
  const uint32_t row_stride = uint32_t(split_item ? p.max_splits : 1) * D;
  const int tok_end = min(it.q_count, p.total_q - it.tok0);
  // token = row / G for rows < 256 and G <= 128: (row * ceil(2^16 / G)) >> 16 is exact
  const uint32_t inv_g = (65536u + uint32_t(G) - 1) / uint32_t(G);
  // tile row r = t G + j is query head kv_head G + j of token t: t Hq + h = t (Hq - G) + kv_head G + r
  const int hq_minus_g = p.num_q_heads - G, head0 = it.kv_head * G;
#pragma unroll
  for (int g = 0; g < PIECES; ++g) {
    const int rr = wave * 32 + T::RPI * g + lane / T::CH;   // tile row = token * G + head-in-group
    const int etok = int((uint32_t(rr) * inv_g) >> 16);
    const uint32_t row = uint32_t(etok * hq_minus_g + head0 + rr);
    if (etok < tok_end) *reinterpret_cast<u32x4*>(dst0 + uint64_t(row) * row_stride + 8 * ec) = val[g];
  }
}

// ---------------------------------------------------------------------------
// fp32: 4 waves, 32-key tiles staged through registers, 32x32x2 fp32 MFMA
// ---------------------------------------------------------------------------

template <int D>
struct F32Tile {
  static constexpr int BC = kTileKeysF32;
  static constexpr int KPITCH = D + 1;             // floats per K row (odd pitch: column reads conflict-free)
  static constexpr int VPITCH = D;                 // floats per V row (row reads)
  static constexpr int KFLOATS = BC * KPITCH;
  static constexpr int STAGE = KFLOATS + BC * VPITCH;  // floats
  static constexpr int CHUNKS = D / 4;             // 16-byte chunks per key row
  static constexpr int KEYS_PER_PASS = 256 / CHUNKS;
  static constexpr int LOADS = BC / KEYS_PER_PASS;
  static constexpr int KSTEPS = D / 2;
  static constexpr int DBLK = D / 32;
};

template <int D, bool MASK>
__global__ __launch_bounds__(256) void extend_attn_f32(const Params p) {
  using T = F32Tile<D>;
  __shared__ float smem[2 * T::STAGE];

  const ItemView it = load_item(p);
  if (it.q_count <= 0) return;   // (uniform) a padding item covers no row
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int G = p.group;
  const int r = wave * 32 + l32;
  const int tok = r / G, gh = r - tok * G;
  const int gtok = it.tok0 + tok;
  const bool row_live = tok < it.q_count && gtok < p.total_q;
  const int qpos = it.pos0 + tok;
  const int head = it.kv_head * G + gh;
  const bool wave_live = wave * 32 < it.q_count * G;
  // this row's keep-mask bytes (a row past the item reads the item's first row)
  const uint8_t* mrow = nullptr;
  if constexpr (MASK)
    mrow = p.mask + mask_row_offset(p, it.req, head, it.tok0 + (row_live ? tok : 0) - p.qo_indptr[it.req]);

  // Q operand: lane holds q[row][2ks + half]
  float qf[T::KSTEPS];
  {
    const float* qrow = static_cast<const float*>(p.q) + (int64_t(gtok) * p.num_q_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < T::KSTEPS; ++ks) qf[ks] = row_live ? qrow[2 * ks + half] : 0.f;
  }

  f32x16 o[T::DBLK];
#pragma unroll
  for (int db = 0; db < T::DBLK; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int t0 = (it.kv_begin / T::BC) * T::BC;
  const int ntiles = it.kv_end > it.kv_begin ? (it.kv_end - t0 + T::BC - 1) / T::BC : 0;
  const int32_t* pt = p.page_table + int64_t(it.pt_row) * p.page_table_stride;
  const float* kpool = static_cast<const float*>(p.k_pool);
  const float* vpool = static_cast<const float*>(p.v_pool);
  const int chunk = tid % T::CHUNKS, key_in_pass = tid / T::CHUNKS;
  const int64_t row_elems = int64_t(p.num_kv_heads) * D;

  f32x4 kreg[T::LOADS], vreg[T::LOADS];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int j = kv0 + key_in_pass + i * T::KEYS_PER_PASS;
      kreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      vreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j >= it.kv_begin && j < it.kv_end) {
        const int col = j / p.page_size;
        const int page = pt[col];
        if (page >= 0 && page < p.num_pages) {
          const int64_t off = (int64_t(page) * p.page_size + (j - col * p.page_size)) * row_elems +
                              int64_t(it.kv_head) * D + 4 * chunk;
          kreg[i] = *reinterpret_cast<const f32x4*>(kpool + off);
          vreg[i] = *reinterpret_cast<const f32x4*>(vpool + off);
        } else {
          atomicOr(p.status, PKV_STATUS_BAD_PAGE);
        }
      }
    }
  };
  auto store_tile = [&](int stage) {
    float* kb = smem + stage * T::STAGE;
    float* vb = kb + T::KFLOATS;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int kr = key_in_pass + i * T::KEYS_PER_PASS;
#pragma unroll
      for (int x = 0; x < 4; ++x) kb[kr * T::KPITCH + 4 * chunk + x] = kreg[i][x];
      *reinterpret_cast<f32x4*>(vb + kr * T::VPITCH + 4 * chunk) = vreg[i];
    }
  };

  if (ntiles > 0) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();
  const float c = p.scale_log2;

  for (int tile = 0; tile < ntiles; ++tile) {
    const int kv0 = t0 + tile * T::BC;
    const int stage = tile & 1;
    if (tile + 1 < ntiles) load_tile(kv0 + T::BC);
    if (wave_live) {
      const float* kb = smem + stage * T::STAGE;
      const float* vb = kb + T::KFLOATS;
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < T::KSTEPS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kb[l32 * T::KPITCH + 2 * ks + half], qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kv0 + 8 * (j >> 2) + 4 * half + (j & 3);
        if (!key_visible(key, qpos, it.kv_begin, it.kv_end, p.window) || (MASK && !mrow[key])) s[j] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[j]);
      mx = other_half_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_off = m_new == -INFINITY ? 0.f : m_new * c;
      const float alpha = fast_exp2(m_run * c - m_off);
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] = fast_exp2(fmaf(s[j], c, -m_off));
        lsum += s[j];
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) {
        o[db] *= alpha;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = 8 * (j >> 2) + 4 * half + (j & 3);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb[key * T::VPITCH + 32 * db + l32], s[j], o[db], 0, 0, 0);
        }
      }
    }
    if (tile + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const float l_tot = other_half_sum(l_run);
  if (!row_live) return;
  if (it.part_row < 0) {
    const float den = l_tot > 0.f ? l_tot : INFINITY;
    float* orow = static_cast<float*>(p.out) + (int64_t(gtok) * p.num_q_heads + head) * D;
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 v = {o[db][4 * jj] / den, o[db][4 * jj + 1] / den, o[db][4 * jj + 2] / den,
                         o[db][4 * jj + 3] / den};
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * jj + 4 * half) = v;
      }
  } else {
    const int64_t slot = int64_t(it.part_row + tok) * p.num_q_heads + head;
    const int64_t prow = slot * p.max_splits + it.split;
    float* op = static_cast<float*>(p.o_part) + prow * D;
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 v = {o[db][4 * jj], o[db][4 * jj + 1], o[db][4 * jj + 2], o[db][4 * jj + 3]};
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * jj + 4 * half) = v;
      }
    if (half == 0) {
      p.ml_part[prow * 2] = m_run == -INFINITY ? -INFINITY : m_run * c;
      p.ml_part[prow * 2 + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// split combine: O = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k
// ---------------------------------------------------------------------------

struct CombineParams {
  const void* o_part;   // bf16 when BF16, else fp32
  const float* ml_part;
  const int32_t* split_rows;
  void* out;
  int32_t n_rows;       // split rows x query heads
  int32_t num_q_heads;
  int32_t max_splits;
  int32_t total_q;
};

// One row of 32 lanes per (split row, query head), two rows per wave: each
// lane owns VEC = D/32 consecutive output values and loads them with one
// 8- or 16-byte read per split. Every lane of a row also reads every split's
// (max, sum) -- the same addresses across the row, so one request each -- and
// merges on its own: no exchange between lanes, and the first PF splits'
// values go out together with their (max, sum), right after the row's split
// count. PF is 2, 4 or 8 by the launch's largest split count (up to 16
// splits the rows past 8 take two more short rounds), 32 above that.
template <int D>
struct CombineShape {
  static constexpr int LANES = 32;
  static constexpr int ROWS = 2;
  static constexpr int VEC = D / 32;
};

template <int D, bool BF16, int PF>
__global__ __launch_bounds__(256) void combine_splits(const CombineParams p) {
  using C = CombineShape<D>;
  typedef float fvec __attribute__((ext_vector_type(C::VEC)));
  typedef uint16_t hvec __attribute__((ext_vector_type(C::VEC)));
  const int lane = threadIdx.x & 63;
  const int sub = lane / C::LANES, j = lane % C::LANES;      // row within the wave, lane within the row
  const int wid = (blockIdx.x * 4 + (threadIdx.x >> 6)) * C::ROWS + sub;
  const bool live = wid < p.n_rows;
  const int w = live ? wid : p.n_rows - 1;                    // dead rows mirror the last row, store nothing
  const int slot = w / p.num_q_heads, head = w - slot * p.num_q_heads;
  const int token = p.split_rows[2 * slot];
  const int ns = min(p.split_rows[2 * slot + 1], p.max_splits);
  const int64_t base = (int64_t(slot) * p.num_q_heads + head) * p.max_splits;
  const float2* ml = reinterpret_cast<const float2*>(p.ml_part) + base;
  // lane j's VEC elements of split k's partial row
  auto part = [&](int k) __attribute__((always_inline)) {
    if constexpr (BF16) {
      const hvec h = reinterpret_cast<const hvec*>(static_cast<const uint16_t*>(p.o_part) + base * D)[k * C::LANES + j];
      fvec v;
#pragma unroll
      for (int x = 0; x < C::VEC; ++x) v[x] = __uint_as_float(uint32_t(h[x]) << 16);
      return v;
    } else {
      return reinterpret_cast<const fvec*>(static_cast<const float*>(p.o_part) + base * D)[k * C::LANES + j];
    }
  };
  // Loads past the row's split count read its last split again (in bounds,
  // no branch around the loads) and get weight 0.
  const int klast = max(ns - 1, 0);
  fvec v[PF];
  float2 mlk[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    mlk[u] = ml[min(u, klast)];
    v[u] = part(min(u, klast));
  }
  // the row's reference: the largest split max
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < PF; ++u) M = fmaxf(M, mlk[u].x);   // (the repeated last split changes nothing)
  for (int k = PF; k < ns; k += 4) {
    float2 mm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) mm[u] = ml[min(k + u, klast)];
#pragma unroll
    for (int u = 0; u < 4; ++u) M = fmaxf(M, mm[u].x);
  }
  auto weight = [&](float mk, bool in) __attribute__((always_inline)) {
    return in && mk != -INFINITY ? fast_exp2(mk - M) : 0.f;
  };
  fvec acc = {};
  float den = 0.f;
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const float wk = weight(mlk[u].x, u < ns);
    den += wk * mlk[u].y;
    acc += wk * v[u];
  }
  for (int k = PF; k < ns; k += 4) {   // more splits (long one-token rows): four in flight
    fvec vv[4];
    float2 mm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mm[u] = ml[min(k + u, klast)];
      vv[u] = part(min(k + u, klast));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wk = weight(mm[u].x, k + u < ns);
      den += wk * mm[u].y;
      acc += wk * vv[u];
    }
  }
  if (!live || token < 0 || token >= p.total_q) return;
  if (!(den > 0.f)) den = INFINITY;  // no visible key: output 0
  const int64_t orow = (int64_t(token) * p.num_q_heads + head) * D + C::VEC * j;
  if constexpr (BF16) {
    typedef __bf16 bvec __attribute__((ext_vector_type(C::VEC)));
    bvec o;
#pragma unroll
    for (int x = 0; x < C::VEC; ++x) o[x] = (__bf16)(acc[x] / den);
    *reinterpret_cast<bvec*>(static_cast<__bf16*>(p.out) + orow) = o;
  } else {
    fvec o;
#pragma unroll
    for (int x = 0; x < C::VEC; ++x) o[x] = acc[x] / den;
    *reinterpret_cast<fvec*>(static_cast<float*>(p.out) + orow) = o;
  }
}

template <int D, bool BF16>
void launch_typed(const Params& p, const AttnArgs& a, hipStream_t st) {
  if (a.n_items > 0) {
    if (BF16) {
      // the rows of one wave-wide gather share a page when the page size is a
      // power of two of at least that many rows
      const int ps = a.shape.page_size;
      const dim3 grid(a.n_items), block(64 * kWavesBf16);
      const bool fused = a.k_new != nullptr;
      if ((ps & (ps - 1)) == 0 && ps >= Bf16Tile<D>::RPI) {
        if (a.mask)
          hipLaunchKernelGGL((extend_attn_bf16<D, true, true, false>), grid, block, 0, st, p);
        else if (fused)
          hipLaunchKernelGGL((extend_attn_bf16<D, true, false, true>), grid, block, 0, st, p);
        else
          hipLaunchKernelGGL((extend_attn_bf16<D, true, false, false>), grid, block, 0, st, p);
      } else {
        if (a.mask)
          hipLaunchKernelGGL((extend_attn_bf16<D, false, true, false>), grid, block, 0, st, p);
        else if (fused)
          hipLaunchKernelGGL((extend_attn_bf16<D, false, false, true>), grid, block, 0, st, p);
        else
          hipLaunchKernelGGL((extend_attn_bf16<D, false, false, false>), grid, block, 0, st, p);
      }
    } else {
      if (a.mask)
        hipLaunchKernelGGL((extend_attn_f32<D, true>), dim3(a.n_items), dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((extend_attn_f32<D, false>), dim3(a.n_items), dim3(256), 0, st, p);
    }
  }
  if (a.n_split_rows > 0) {
    CombineParams cp;
    cp.o_part = a.o_part;
    cp.ml_part = a.ml_part;
    cp.split_rows = a.split_rows;
    cp.out = a.out;
    cp.num_q_heads = a.shape.num_q_heads;
    cp.n_rows = a.n_split_rows * a.shape.num_q_heads;
    cp.max_splits = a.max_splits;
    cp.total_q = a.total_q;
    const int rows_per_block = 4 * CombineShape<D>::ROWS;
    const dim3 grid((cp.n_rows + rows_per_block - 1) / rows_per_block), block(256);
    if (cp.max_splits <= 2)
      hipLaunchKernelGGL((combine_splits<D, BF16, 2>), grid, block, 0, st, cp);
    else if (cp.max_splits <= 4)
      hipLaunchKernelGGL((combine_splits<D, BF16, 4>), grid, block, 0, st, cp);
    else if (cp.max_splits <= 16)
      hipLaunchKernelGGL((combine_splits<D, BF16, 8>), grid, block, 0, st, cp);
    else
      hipLaunchKernelGGL((combine_splits<D, BF16, PKV_MAX_SPLITS>), grid, block, 0, st, cp);
  }
}

}  // namespace

int launch_extend_attn(const AttnArgs& a, void* stream) {
  Params p;
  p.q = a.q;
  p.k_pool = a.k_pool;
  p.v_pool = a.v_pool;
  p.page_table = a.page_table;
  p.req_pool_indices = a.req_pool_indices;
  p.items = a.items;
  p.status = a.status;
  p.out = a.out;
  p.o_part = a.o_part;
  p.ml_part = a.ml_part;
  p.page_table_stride = a.page_table_stride;
  p.num_q_heads = a.shape.num_q_heads;
  p.num_kv_heads = a.shape.num_kv_heads;
  p.group = a.shape.num_q_heads / a.shape.num_kv_heads;
  p.page_size = a.shape.page_size;
  p.page_shift = (a.shape.page_size & (a.shape.page_size - 1)) ? -1 : __builtin_ctz(a.shape.page_size);
  p.num_pages = a.shape.num_pages;
  p.window = a.window;
  p.total_q = a.total_q;
  p.max_splits = a.max_splits;
  p.scale_log2 = a.scale_log2;
  p.mask = a.mask;
  p.mask_heads = a.mask_heads;
  p.mask_rows = a.mask_rows;
  p.mask_kv_stride = a.mask_kv_stride;
  p.qo_indptr = a.qo_indptr;
  p.k_new = a.k_new;
  p.v_new = a.v_new;
  p.k_pool_w = a.k_pool_w;
  p.v_pool_w = a.v_pool_w;
  p.prefix_lens = a.prefix_lens;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = a.shape.dtype == PKV_DTYPE_BF16;
  if (a.shape.head_dim == 128) {
    if (bf16) launch_typed<128, true>(p, a, st); else launch_typed<128, false>(p, a, st);
  } else {
    if (bf16) launch_typed<64, true>(p, a, st); else launch_typed<64, false>(p, a, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv
