// KV append for chunked prefill: scatter each new token's K/V row into its
// page slot.
//
// AReno PR #642 ("What does this PR do?"): a later prefill chunk continues
// inside the last, partly filled KV page of its request. AstrAI compare
// v1.3.12..925cbed (astrai/inference/core/cache.py, PagePool.bind_tasks):
// the write slots of a prefill step are the page-table entries of positions
// start_pos .. seq_len-1, and the backend writes k_buffer[out_cache_loc] = k.
//
// A token's K (or V) row of Hkv*D elements is contiguous both in k_new and in
// its pool slot ([page][slot][Hkv][D]). A workgroup owns one token (blockIdx.x)
// and a span of its row's 16-byte vectors (blockIdx.y): the token's request,
// position and page are uniform, so they come from scalar loads, and the row
// loads are issued before the page lookup so that their latencies overlap.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pkv_internal.hpp"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct AppendParams {
  const u32x4* k_new;
  const u32x4* v_new;
  u32x4* k_pool;
  u32x4* v_pool;
  const int32_t* page_table;
  const int32_t* req_pool_indices;
  const int32_t* qo_indptr;
  const int32_t* prefix_lens;
  int32_t* status;
  int32_t vecs_per_token;  // Hkv * D * elem_bytes / 16
  int32_t batch;
  int32_t total_q;
  int32_t page_size;
  int32_t page_table_stride;
  int32_t num_pages;
};

// The index arrays are read-only here: reading them through the constant
// address space lets the (uniform) lookups use scalar loads.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ inline cint_ptr as_const(const int32_t* p) { return (cint_ptr)p; }

// Request owning global token t: the last b with qo_indptr[b] <= t (requests
// with an empty chunk share their qo_indptr value with the next request).
__device__ inline int find_request(cint_ptr qo_indptr, int batch, int t) {
  int lo = 0, hi = batch;  // invariant: qo_indptr[lo] <= t < qo_indptr[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qo_indptr[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  const int v = blockIdx.y * blockDim.x + threadIdx.x;   // vector within the token row
  const bool lane_live = v < p.vecs_per_token;
  for (int t = blockIdx.x; t < p.total_q; t += gridDim.x) {   // uniform per workgroup
    const int64_t src = int64_t(t) * p.vecs_per_token + v;
    u32x4 kv, vv;
    if (lane_live) {
      kv = p.k_new[src];
      vv = p.v_new[src];
    }
    const int b = find_request(as_const(p.qo_indptr), p.batch, t);
    const int pos = as_const(p.prefix_lens)[b] + (t - as_const(p.qo_indptr)[b]);
    const int col = pos / p.page_size;
    bool ok = pos >= 0 && col < p.page_table_stride;
    int page = -1;
    if (ok) {
      const int row = p.req_pool_indices ? as_const(p.req_pool_indices)[b] : b;
      page = as_const(p.page_table)[int64_t(row) * p.page_table_stride + col];
      ok = page >= 0 && page < p.num_pages;
    }
    if (!ok) {
      if (threadIdx.x == 0) atomicOr(p.status, PKV_STATUS_BAD_PAGE);
      continue;
    }
    if (lane_live) {
      const int64_t slot = int64_t(page) * p.page_size + (pos - col * p.page_size);
      const int64_t dst = slot * p.vecs_per_token + v;
      p.k_pool[dst] = kv;
      p.v_pool[dst] = vv;
    }
  }
}

// Rotary embedding of the token's query and key rows, fused with the append
// (AstrAI compare v1.3.12..925cbed, csrc/kernels/rotary_emb.cu: an fp32 table
// of (cos, sin) per pair of head dimensions, [.., head_dim/2, 2]; the backend's
// prefill path then writes K/V into the cache slots). Pair j of a head row is
// elements 2j and 2j+1: (a, b) -> (a cos - b sin, a sin + b cos), in fp32,
// rounded once to the storage type; the table row is the token's absolute
// position P_b + i. A workgroup owns one token; its lanes take the 16-byte
// vectors of the token's Q row, K row and V row in turn (V is copied as is).
struct RopeParams {
  AppendParams ap;
  const u32x4* q;
  u32x4* q_out;
  const float* table;
  int32_t table_len;
  int32_t head_dim;
  int32_t q_vecs;   // 16-byte vectors of a token's Q row (Hq * D * elem / 16)
};

template <bool BF16>
__global__ __launch_bounds__(1024) void rope_append_kernel(const RopeParams r) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const AppendParams& p = r.ap;
  constexpr int EPV = BF16 ? 8 : 4;   // elements per 16-byte vector
  const int kv_vecs = p.vecs_per_token;
  const int v = blockIdx.y * blockDim.x + threadIdx.x;   // slot: Q vectors, then K, then V
  const bool lane_live = v < r.q_vecs + 2 * kv_vecs;
  for (int t = blockIdx.x; t < p.total_q; t += gridDim.x) {   // uniform per workgroup
    const int b = find_request(as_const(p.qo_indptr), p.batch, t);
    const int pos = as_const(p.prefix_lens)[b] + (t - as_const(p.qo_indptr)[b]);
    const int col = pos / p.page_size;
    bool ok = pos >= 0 && col < p.page_table_stride && pos < r.table_len;
    int page = -1;
    if (ok) {
      const int row = p.req_pool_indices ? as_const(p.req_pool_indices)[b] : b;
      page = as_const(p.page_table)[int64_t(row) * p.page_table_stride + col];
      ok = page >= 0 && page < p.num_pages;
    }
    if (!ok) {
      if (threadIdx.x == 0 && blockIdx.y == 0) atomicOr(p.status, PKV_STATUS_BAD_PAGE);
      continue;
    }
    if (!lane_live) continue;
    const bool is_q = v < r.q_vecs, is_v = v >= r.q_vecs + kv_vecs;
    const int vec = is_q ? v : (is_v ? v - r.q_vecs - kv_vecs : v - r.q_vecs);
    const int64_t slot = int64_t(page) * p.page_size + (pos - col * p.page_size);
    if (is_v) {
      p.v_pool[slot * kv_vecs + vec] = p.v_new[int64_t(t) * kv_vecs + vec];
      continue;
    }
    const u32x4 raw = is_q ? r.q[int64_t(t) * r.q_vecs + vec] : p.k_new[int64_t(t) * kv_vecs + vec];
    // this vector's first pair within its head row, and the table row of the position
    const int pair0 = ((vec * EPV) % r.head_dim) / 2;
    const float* cs = r.table + (int64_t(pos) * (r.head_dim / 2) + pair0) * 2;
    float x[EPV], c[EPV];
    if constexpr (BF16) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = float(h[e]);
      const f32x8 tv = *reinterpret_cast<const f32x8*>(cs);   // 4 pairs' (cos, sin), 32-byte aligned
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = tv[e];
    } else {
      const f32x4 h = __builtin_bit_cast(f32x4, raw);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = h[e];
      const f32x4 tv = *reinterpret_cast<const f32x4*>(cs);   // 2 pairs' (cos, sin)
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = tv[e];
    }
    float y[EPV];
#pragma unroll
    for (int k = 0; k < EPV / 2; ++k) {
      const float a = x[2 * k], bb = x[2 * k + 1], co = c[2 * k], si = c[2 * k + 1];
      y[2 * k] = a * co - bb * si;
      y[2 * k + 1] = a * si + bb * co;
    }
    u32x4 res;
    if constexpr (BF16) {
      bf16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (__bf16)y[e];
      res = __builtin_bit_cast(u32x4, h);
    } else {
      const f32x4 h = {y[0], y[1], y[2], y[3]};
      res = __builtin_bit_cast(u32x4, h);
    }
    if (is_q)
      r.q_out[int64_t(t) * r.q_vecs + vec] = res;
    else
      p.k_pool[slot * kv_vecs + vec] = res;
  }
}

// Step metadata from the caller's pinned host buffer (read through its device
// mapping) into meta_dev: 16 bytes per lane, the buffer's size being a
// multiple of 256 bytes.
__global__ __launch_bounds__(256) void copy_meta_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int n16) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n16; i += gridDim.x * 256) dst[i] = src[i];
}

}  // namespace

int launch_meta_copy(const void* src_dev, void* dst, size_t bytes, void* stream) {
  const int n16 = int(bytes / 16);
  const int blocks = std::max(1, std::min(128, (n16 + 255) / 256));
  hipLaunchKernelGGL(copy_meta_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src_dev), static_cast<uint4*>(dst), n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "metadata copy failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int launch_append(const AppendArgs& a, void* stream) {
  const int esize = a.shape.dtype == PKV_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = int64_t(a.shape.num_kv_heads) * a.shape.head_dim * esize;
  if (row_bytes % 16) return set_error(PKV_ERR_UNSUPPORTED, "K/V token rows must be a multiple of 16 bytes");
  if (a.total_q == 0) return PKV_OK;
  AppendParams p;
  p.k_new = static_cast<const u32x4*>(a.k_new);
  p.v_new = static_cast<const u32x4*>(a.v_new);
  p.k_pool = static_cast<u32x4*>(a.k_pool);
  p.v_pool = static_cast<u32x4*>(a.v_pool);
  p.page_table = a.page_table;
  p.req_pool_indices = a.req_pool_indices;
  p.qo_indptr = a.qo_indptr;
  p.prefix_lens = a.prefix_lens;
  p.status = a.status;
  p.vecs_per_token = int32_t(row_bytes / 16);
  p.batch = a.batch;
  p.total_q = a.total_q;
  p.page_size = a.shape.page_size;
  p.page_table_stride = a.page_table_stride;
  p.num_pages = a.shape.num_pages;
  const int blocks = a.total_q < (1 << 20) ? a.total_q : (1 << 20);
  if (a.rope_table) {
    // x: tokens; y: spans of the token's Q, K and V vectors (up to 1024 lanes each)
    RopeParams r;
    r.ap = p;
    r.q = static_cast<const u32x4*>(a.q);
    r.q_out = static_cast<u32x4*>(a.q_out);
    r.table = a.rope_table;
    r.table_len = a.rope_table_len;
    r.head_dim = a.shape.head_dim;
    r.q_vecs = int32_t(int64_t(a.shape.num_q_heads) * a.shape.head_dim * esize / 16);
    const int total = r.q_vecs + 2 * p.vecs_per_token;
    const int threads = total >= 1024 ? 1024 : ((total + 63) / 64) * 64;
    const int spans = (total + threads - 1) / threads;
    if (a.shape.dtype == PKV_DTYPE_BF16)
      hipLaunchKernelGGL(rope_append_kernel<true>, dim3(blocks, spans), dim3(threads), 0,
                         static_cast<hipStream_t>(stream), r);
    else
      hipLaunchKernelGGL(rope_append_kernel<false>, dim3(blocks, spans), dim3(threads), 0,
                         static_cast<hipStream_t>(stream), r);
  } else {
    // x: tokens (one workgroup each, looping past 2^20); y: spans of a row's vectors
    const int threads = p.vecs_per_token >= 256 ? 256 : ((p.vecs_per_token + 63) / 64) * 64;
    const int spans = (p.vecs_per_token + threads - 1) / threads;
    hipLaunchKernelGGL(append_kernel, dim3(blocks, spans), dim3(threads), 0, static_cast<hipStream_t>(stream), p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv
