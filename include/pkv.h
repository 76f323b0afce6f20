/*
 * pkv.h -- C ABI of the paged extend-attention library (libpkv.so) for
 * chunked prefill on AMD Instinct MI355X (gfx950).
 *
 * The operation (AReno PR #642, "What does this PR do?"): a prompt that is
 * prefilled in several chunks keeps its earlier chunks' K/V in a paged cache.
 * Each query token of the current chunk attends, through the page table, to
 * its request's cached prefix plus its own chunk, with the causal mask
 * aligned bottom-right: token i of a chunk that follows P cached tokens sees
 * key positions 0 .. P+i. New chunk K/V is appended into the pages first,
 * continuing inside the last partly filled page.
 *
 * Argument vocabulary follows the pages' statement of the problem (AstrAI
 * compare v1.3.12..925cbed: csrc/kernels/attn_types.cuh PagedAttentionParams,
 * astrai/extension/attention_ops.py attn_paged_prefill, and
 * astrai/inference/core/cache.py KVCache / PagePool.bind_tasks): paged K/V
 * pools, a per-request page table (req_to_token), qo_indptr / kv_indptr
 * prefix sums, prefix lengths, a window and the page size.
 *
 * Conventions shared by every entry point
 *   - Status codes only; no exception crosses the ABI. On a non-zero status
 *     pkv_last_error() returns a message for the calling thread. Every
 *     argument is validated before anything is launched.
 *   - The caller owns every buffer. The library never allocates device
 *     memory and keeps no per-call state; all device work is asynchronous on
 *     the given stream (a hipStream_t; NULL is the null stream).
 *   - Element layouts (all contiguous, row-major):
 *       q, out            [total_q, num_q_heads, head_dim]
 *       k_new, v_new      [total_q, num_kv_heads, head_dim]
 *       k_pool, v_pool    [num_pages, page_size, num_kv_heads, head_dim]
 *       page_table        int32 [rows, page_table_stride]; entry [r][p] is the
 *                         physical page holding logical page p (positions
 *                         p*page_size .. p*page_size+page_size-1) of the
 *                         request stored in row r. Row r of request b is
 *                         req_pool_indices[b], or b when req_pool_indices is
 *                         NULL. Only entries of positions < N_b are read.
 *     Tokens of the batch are in request order: request b owns q/out/k_new/
 *     v_new rows qo_indptr[b] .. qo_indptr[b+1]-1.
 *     q, out, k_new, v_new, the pools, q_out, rope_table and the workspace
 *     must be 16-byte aligned (the kernels move 16-byte vectors); a
 *     misaligned one is PKV_ERR_INVALID_ARGUMENT.
 *   - Element type: bf16 (round-to-nearest-even outputs, fp32 accumulation)
 *     or fp32, chosen by pkv_shape.dtype for all of q, pools, out.
 *   - Page ids read from the page table outside [0, num_pages) are never
 *     dereferenced: the attention reads such a key as zeros, the append drops
 *     the write, and either sets the plan's device status word to
 *     PKV_STATUS_BAD_PAGE (see pkv_read_status).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* pkv_stream_t; /* a hipStream_t */

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad length, inconsistent sizes   */
  PKV_ERR_UNSUPPORTED = -2,      /* head_dim/dtype/group size not built, not gfx950 */
  PKV_ERR_WORKSPACE = -3,        /* a caller buffer is smaller than required        */
  PKV_ERR_HIP = -4               /* the HIP runtime reported an error               */
};

enum { PKV_DTYPE_BF16 = 0, PKV_DTYPE_FP32 = 1 };

enum { PKV_STATUS_BAD_PAGE = 1 };

/* Flags of build_extend_metadata_ex. PKV_FLAG_NON_CAUSAL: every row of a
 * request sees all N_b of its keys, chunk rows after it included (AstrAI
 * compare v1.3.12..925cbed, attn_paged_prefill: is_causal=False gives a
 * causal offset of -1, no causal mask; attn_paged_test.cu tests it with
 * q_len = kv_len). Incompatible with a sliding window. */
enum { PKV_FLAG_NON_CAUSAL = 1 };

/* Largest number of KV splits of one tile of query rows. */
#define PKV_MAX_SPLITS 32

/* Geometry of one attention layer's cache. */
typedef struct pkv_shape {
  int32_t num_q_heads;  /* Hq                                                   */
  int32_t num_kv_heads; /* Hkv < 32768; Hq % Hkv == 0, G = Hq / Hkv <= 128      */
  int32_t head_dim;     /* D in {64, 128}                                       */
  int32_t page_size;    /* ps >= 1 tokens per page                              */
  int32_t num_pages;    /* pages in each pool                                   */
  int32_t dtype;        /* PKV_DTYPE_BF16 or PKV_DTYPE_FP32                     */
} pkv_shape;

/* Result of build_extend_metadata: host scalars plus device pointers into the
 * caller's meta_dev buffer. Plain data: copy it freely; it stays valid while
 * meta_dev does. Reuse it for every layer of the step. */
typedef struct pkv_plan {
  int32_t batch;          /* B                                                  */
  int32_t total_q;        /* sum of chunk lengths (rows of q / out)             */
  int32_t max_q_len;      /* longest chunk                                      */
  int32_t max_kv_len;     /* longest prefix + chunk                             */
  int32_t n_items;        /* attention work items (one workgroup each)          */
  int32_t n_split_rows;   /* query tokens computed as KV splits + combine       */
  int32_t max_splits;     /* split stride of the partial buffers                */
  int32_t window;         /* sliding window W (<= 0: none)                      */
  int32_t flags;          /* PKV_FLAG_* the plan was built with                 */
  int32_t slot_blocks;    /* estimated 64-key blocks of the busiest workgroup   */
                          /* slot: max(longest item, all items / slots)        */
  int32_t num_cus;        /* compute units the work list was sized for          */
  pkv_shape shape;        /* the shape the plan was built for                   */
  size_t workspace_bytes; /* scratch paged_extend_attn needs (0 if no splits)   */
  /* device pointers (NULL after a host-only build) */
  const int32_t* qo_indptr;   /* [B+1] exclusive prefix sum of chunk lengths    */
  const int32_t* kv_indptr;   /* [B+1] exclusive prefix sum of prefix + chunk   */
  const int32_t* prefix_lens; /* [B]                                            */
  const void* items;          /* work list (library-private format)             */
  const int32_t* split_rows;  /* [n_split_rows][2] token index, split count     */
  int32_t* status;            /* one int32, zeroed by the metadata copy         */
} pkv_plan;

/*
 * Size query for build_extend_metadata's buffers (host only: no device work;
 * the compute-unit count of the current HIP device is read as
 * build_extend_metadata reads it, so that both calls plan the same work list).
 *   prefix_lens_h, chunk_lens_h  host int32 [batch]: P_b >= 0, L_b >= 0
 *   window                       W (<= 0: none)
 *   decode_splits                KV splits for one-token chunks; 0 = choose
 *   meta_bytes      out: bytes of meta_host and of meta_dev (same layout)
 *   workspace_bytes out: bytes paged_extend_attn needs as workspace
 * Returns PKV_OK, PKV_ERR_INVALID_ARGUMENT or PKV_ERR_UNSUPPORTED.
 */
int pkv_extend_metadata_size(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                             const pkv_shape* shape, int32_t window, int32_t decode_splits,
                             size_t* meta_bytes, size_t* workspace_bytes);

/*
 * build_extend_metadata -- step a1: per-step metadata, built once on the host
 * and reused by every layer (AReno PR #642: prefix and total-KV lengths are
 * carried in scheduler metadata; AstrAI compare, cache.py: kv_indptr is the
 * prefix sum of per-request sequence lengths, precomputed once per step).
 *
 * Computes qo_indptr (exclusive cumsum of L_b), kv_indptr (exclusive cumsum
 * of N_b = P_b + L_b), a copy of prefix_lens and the attention work list into
 * meta_host, then enqueues one host-to-device copy of meta_host into meta_dev
 * on `stream`. No device synchronisation. The work list is sized for the
 * compute units of the current HIP device (AstrAI compare, csrc/kernels/
 * attn_dispatchers.cuh: get_sm_count caches the count per device and
 * compute_num_splits sizes the KV splits from it): its count is read once per
 * device and cached; with no current device (a host-only plan on a machine
 * without a GPU) the plan is sized for an MI355X's 256.
 *   meta_host   caller buffer of >= meta_bytes; it must stay unchanged until
 *               the copy has executed. Pinned memory (hipHostMalloc) is read
 *               in place by a small copy kernel on `stream`; other host
 *               memory goes through hipMemcpyAsync.
 *   meta_dev    device buffer of >= meta_bytes, 16-byte aligned, or NULL for
 *               a host-only plan (then no HIP call is made and the plan's
 *               device pointers are NULL: useful for inspecting the plan
 *               without a GPU).
 *   plan_out    receives the plan.
 * Errors: PKV_ERR_INVALID_ARGUMENT (null pointers, batch < 1, negative
 * lengths, int32 overflow of the sums, Hq % Hkv != 0, page_size < 1,
 * num_pages < 1, decode_splits outside 0..PKV_MAX_SPLITS),
 * PKV_ERR_UNSUPPORTED (head_dim not 64/128, dtype unknown, G > 128,
 * Hkv >= 32768, one token row of a pool >= 2^24 bytes or one page > 2^31-1
 * bytes, device not gfx950), PKV_ERR_WORKSPACE (a buffer too small),
 * PKV_ERR_HIP.
 */
int build_extend_metadata(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                          const pkv_shape* shape, int32_t window, int32_t decode_splits,
                          void* meta_host, size_t meta_host_bytes, void* meta_dev, size_t meta_dev_bytes,
                          pkv_plan* plan_out, pkv_stream_t stream);

/*
 * build_extend_metadata_ex, pkv_extend_metadata_size_ex -- the same with
 * `flags` and `num_cus` (flags 0 and num_cus 0 are build_extend_metadata).
 *   flags    PKV_FLAG_*. With PKV_FLAG_NON_CAUSAL each tile's key range is its
 *            request's whole [0, N_b) and the attention applies no causal
 *            bound; pkv_append and paged_extend_attn take the plan unchanged.
 *   num_cus  compute units to size the work list for (the KV splits fill
 *            num_cus resident workgroup slots); 0 = the current device's
 *            count as above. A plan sized for more units than the device has
 *            is still correct, only slower. At most 65536.
 * Errors as build_extend_metadata, plus PKV_ERR_INVALID_ARGUMENT for unknown
 * flags, a window with PKV_FLAG_NON_CAUSAL, or num_cus outside 0..65536.
 */
int build_extend_metadata_ex(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                             const pkv_shape* shape, int32_t window, int32_t flags, int32_t decode_splits,
                             int32_t num_cus, void* meta_host, size_t meta_host_bytes, void* meta_dev,
                             size_t meta_dev_bytes, pkv_plan* plan_out, pkv_stream_t stream);
int pkv_extend_metadata_size_ex(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                                const pkv_shape* shape, int32_t window, int32_t flags, int32_t decode_splits,
                                int32_t num_cus, size_t* meta_bytes, size_t* workspace_bytes);

/*
 * pkv_append -- step a2: write the chunk's new K/V into the pools
 * (AReno PR #642: continue prefill inside the last allocated KV page;
 * AstrAI compare, cache.py: the write slots of a prefill step are the
 * req_to_token entries of positions start_pos .. seq_len-1).
 *
 * For token i of request b (position p = P_b + i) copies k_new/v_new row
 * qo_indptr[b]+i into slot (page_table[row_b][p / page_size], p % page_size)
 * of k_pool/v_pool. Bit copy; no other pool byte is written.
 *   page_table_stride   entries per page-table row; must cover max_kv_len
 *   req_pool_indices    device int32 [batch] or NULL (row b = b); every
 *                       value must be a row of page_table (device data: not
 *                       checked, like the data pointers themselves)
 * Errors: PKV_ERR_INVALID_ARGUMENT (null pointer, plan/shape mismatch, stride
 * too small), PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
int pkv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* page_table,
               int32_t page_table_stride, const int32_t* req_pool_indices, const pkv_plan* plan,
               const pkv_shape* shape, pkv_stream_t stream);

/*
 * pkv_rope_append -- rotary position embedding of the chunk's new query and
 * key rows fused with the KV append (AstrAI compare v1.3.12..925cbed,
 * csrc/kernels/rotary_emb.cu: bf16 rows rotated with an fp32 (cos, sin)
 * table of [.., head_dim/2, 2]; the CUDA backend's prefill path then writes
 * the step's K/V into the cache slots; AReno PR #642: a later chunk's rows sit
 * at absolute positions behind the cached prefix).
 *
 * For token i of request b at absolute position p = P_b + i, pair j of every
 * head row (elements 2j, 2j+1) is rotated by row p of the table:
 *   (a, b) -> (a*cos - b*sin, a*sin + b*cos),  (cos, sin) = rope_table[p][j]
 * in fp32 and rounded once to the storage type (round to nearest even):
 *   q_out[t][h]                  rotated q[t][h] for every query head h
 *   k_pool slot of position p    rotated k_new[t][h] for every KV head h
 *   v_pool slot of position p    v_new[t][h], a bit copy
 * The slot of p is (page_table[row_b][p / page_size], p % page_size), as in
 * pkv_append; no other pool byte is written. Rotating every chunk at its
 * absolute positions makes a chunked prefill equal to one full prefill.
 *   q, q_out       [total_q, Hq, D]; q_out may equal q (in place), else the
 *                  two must not overlap; neither may overlap the pools
 *   rope_table     device fp32 [rope_table_len][D/2][2], 16-byte aligned
 *   rope_table_len positions the table holds; must be >= plan->max_kv_len
 * Errors: PKV_ERR_INVALID_ARGUMENT (null pointer, misaligned or too short
 * table, plan/shape mismatch, page-table stride too small),
 * PKV_ERR_UNSUPPORTED, PKV_ERR_HIP. A page id outside the pool sets
 * PKV_STATUS_BAD_PAGE and that token is skipped.
 */
int pkv_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, const float* rope_table,
                    int32_t rope_table_len, void* k_pool, void* v_pool, const int32_t* page_table,
                    int32_t page_table_stride, const int32_t* req_pool_indices, const pkv_plan* plan,
                    const pkv_shape* shape, pkv_stream_t stream);

/*
 * paged_extend_attn -- steps a3..a9: attention of every chunk row over its
 * request's prefix plus chunk (AReno PR #642; AstrAI compare,
 * attn_paged_test.cu CPU reference for paged prefill: query head h reads KV
 * head h / (Hq/Hkv); a request's causal offset is its total length minus its
 * chunk length).
 *
 * Row i of request b, query head h, sees key positions j with
 *   j <= P_b + i   and   (window <= 0 or j >= P_b + i - window + 1)
 * and gets softmax(sm_scale * q.k_j) weighted V of those keys (0 if none).
 *   qo_indptr, kv_indptr, prefix_lens   device int32 arrays ([B+1],[B+1],[B])
 *        describing the batch: each must be NULL or the plan's own device
 *        array (plan->qo_indptr, ...), which hold exactly these prefix sums
 *        and lengths (so prefix_lens[b] == kv_indptr[b+1] - kv_indptr[b] -
 *        (qo_indptr[b+1] - qo_indptr[b]) always holds). Any other pointer is
 *        rejected with PKV_ERR_INVALID_ARGUMENT: the work list carries every
 *        offset, and device arrays of the caller cannot be compared with the
 *        plan without a host synchronisation.
 *   window     must equal the plan's window.
 *   sm_scale   softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   out        [total_q, Hq, D] written for every row.
 *   workspace  device scratch of >= plan->workspace_bytes (may be NULL when
 *              that is 0): per-split partial results, combined by a second
 *              kernel launched here when the plan has split rows.
 * The pools must already hold the chunk's K/V (call pkv_append first).
 * Errors: PKV_ERR_INVALID_ARGUMENT, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE,
 * PKV_ERR_HIP.
 */
int paged_extend_attn(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                      int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                      const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                      const pkv_plan* plan, const pkv_shape* shape, void* out, void* workspace,
                      size_t workspace_bytes, pkv_stream_t stream);

/*
 * paged_extend_attn_masked -- paged_extend_attn with an explicit keep-mask
 * (AstrAI compare v1.3.12..925cbed, attn_paged_prefill: a bool mask, True =
 * keep, 2-D [batch, kv_len] or 4-D [batch, 1 or heads, 1 or q_len, kv_len],
 * applied together with the causal flag).
 *
 * A key j of row i (chunk row, 0-based) of request b, query head h, is visible
 * when it is visible for paged_extend_attn with the same plan (causal or not,
 * window) and mask[((b * mask_heads + hh) * mask_rows + ii) * mask_kv_stride + j]
 * is nonzero, with hh = h if mask_heads > 1 else 0 and ii = i if mask_rows > 1
 * else 0 (a 2-D mask is mask_heads = mask_rows = 1). A row that keeps no key
 * gets 0.
 *   mask            device bytes, 4-byte aligned
 *   mask_heads      1 or Hq
 *   mask_rows       1 or >= plan->max_q_len
 *   mask_kv_stride  bytes per mask row, a multiple of 4, >= plan->max_kv_len
 * Every other argument and error as paged_extend_attn, plus
 * PKV_ERR_INVALID_ARGUMENT for a NULL or malformed mask.
 */
int paged_extend_attn_masked(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                             const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                             const uint8_t* mask, int32_t mask_heads, int32_t mask_rows, int32_t mask_kv_stride,
                             const pkv_plan* plan, const pkv_shape* shape, void* out, void* workspace,
                             size_t workspace_bytes, pkv_stream_t stream);

/*
 * paged_extend_attn_append -- steps a2..a9 in one call: pkv_append of the
 * chunk's K/V and paged_extend_attn over the result (AReno PR #642: the chunk
 * continues inside its request's last page and attends to the cached prefix;
 * AstrAI compare, cache.py and the backend's prefill path: the step's K/V are
 * written to the slots of positions start_pos .. seq_len-1, then the paged
 * attention reads the cache). Output and every pool byte equal those of
 * pkv_append followed by paged_extend_attn, bit for bit.
 * bf16, when the plan's slot_blocks is at most 128: a single attention launch
 * does both. Its gather reads key positions >= P_b from k_new / v_new rather
 * than from the pool, and each new row is copied into its slot by one work
 * item of the query tile holding that token (of a tile cut into S key
 * splits, split k copies the tile's tokens k, k + S, ...; split-row combine
 * as usual). Otherwise (longer launches, where the
 * fused gather's per-lane addressing costs more than the launch it saves) and
 * for fp32: the append kernel runs first, then the attention.
 *   k_new, v_new   [total_q, Hkv, D]; must not overlap the pools
 *   k_pool, v_pool read at positions < P_b, written at P_b .. N_b - 1
 * The batch offsets are the plan's (qo_indptr, kv_indptr, prefix_lens).
 * Every other argument as paged_extend_attn. Errors as pkv_append and
 * paged_extend_attn, plus PKV_ERR_INVALID_ARGUMENT when k_new or v_new
 * overlaps a pool. A page id outside the pool sets PKV_STATUS_BAD_PAGE and that
 * row is not written.
 */
int paged_extend_attn_append(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                             const int32_t* page_table, int32_t page_table_stride, const int32_t* req_pool_indices,
                             int32_t window, float sm_scale, const pkv_plan* plan, const pkv_shape* shape,
                             void* out, void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/*
 * paged_extend_attn_noalloc -- paged_extend_attn without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The split
 * partials go to a static device array of PKV_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device for the life of the process; nothing is
 * allocated or freed by the call. All calls on one device share that array,
 * so calls that overlap in time on one device (other streams, other threads)
 * race and must not be made. The array needs no clearing between calls: every
 * byte a call reads was written earlier in the same call.
 * Every argument as paged_extend_attn. Errors as paged_extend_attn, plus
 * PKV_ERR_WORKSPACE when plan->workspace_bytes exceeds
 * PKV_NOALLOC_SCRATCH_BYTES (a plan with that many split partials needs
 * paged_extend_attn and a workspace), PKV_ERR_UNSUPPORTED for a device index
 * of 64 or more, and PKV_ERR_HIP when the array's address cannot be read.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int paged_extend_attn_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                              const pkv_plan* plan, const pkv_shape* shape, void* out, pkv_stream_t stream);

/* Copies the plan's device status word to *status_out after synchronising the
 * stream (a diagnostic; not needed on the hot path). */
int pkv_read_status(const pkv_plan* plan, int32_t* status_out, pkv_stream_t stream);

/* Message for the calling thread's last non-zero status ("" if none). */
const char* pkv_last_error(void);

/* 1 if `device` is a gfx950 GPU the library was built for, 0 if not,
 * negative status if the device cannot be queried. */
int pkv_device_supported(int device);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
