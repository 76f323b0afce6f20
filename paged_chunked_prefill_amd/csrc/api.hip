// C ABI of libpkv: argument validation, device checks and launches.
// Declarations and the contract of every function are in include/pkv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "pkv_internal.hpp"

namespace pkv {

namespace {
thread_local char g_error[512] = "";

// Per-device "is gfx950" cache; the property query costs far more than a launch.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

int query_device(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

int device_supported(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return query_device(dev);
  std::call_once(g_dev_once[dev], [dev] { g_dev_ok[dev] = query_device(dev); });
  return g_dev_ok[dev];
}

// Per-device compute-unit count, read once per device and cached (the
// planner sizes its KV splits from it). 0 when it cannot be read.
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

int query_cus(int dev) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();   // leave no error behind for the next launch check
    return 0;
  }
  return n > 0 ? n : 0;
}

// Compute units of the current HIP device, or kNominalCUs (an MI355X) when no
// device is current or its count cannot be read.
int current_device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return kNominalCUs;
  }
  int n;
  if (dev < 0 || dev >= kMaxDevices) {
    n = query_cus(dev);
  } else {
    std::call_once(g_cu_once[dev], [dev] { g_cu_count[dev] = query_cus(dev); });
    n = g_cu_count[dev];
  }
  return n > 0 ? n : kNominalCUs;
}

constexpr int32_t kMaxPlanCUs = 65536;

// Largest host-to-device copy the HIP runtime makes with a kernel of its own
// (beyond it, the DMA engine).
constexpr size_t kRuntimeKernelCopyBytes = 16 << 10;

int resolve_cus(int32_t num_cus, int32_t* out) {
  if (num_cus < 0 || num_cus > kMaxPlanCUs)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "num_cus must be in 0..%d (got %d)", kMaxPlanCUs, num_cus);
  *out = num_cus > 0 ? num_cus : current_device_cus();
  return PKV_OK;
}

int check_current_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "no current HIP device: %s", hipGetErrorString(e));
  const int ok = device_supported(dev);
  if (ok < 0) return set_error(PKV_ERR_HIP, "cannot query HIP device %d", dev);
  if (ok == 0) return set_error(PKV_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X); this library targets gfx950 only", dev);
  return PKV_OK;
}

bool same_shape(const pkv_shape& a, const pkv_shape& b) {
  return a.num_q_heads == b.num_q_heads && a.num_kv_heads == b.num_kv_heads && a.head_dim == b.head_dim &&
         a.page_size == b.page_size && a.num_pages == b.num_pages && a.dtype == b.dtype;
}

int check_plan(const pkv_plan* plan, const pkv_shape* shape, const char* who) {
  if (!plan) return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: plan is NULL", who);
  if (int st = validate_shape(shape)) return st;
  if (!same_shape(plan->shape, *shape))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: shape differs from the one the plan was built for", who);
  if (!plan->qo_indptr || !plan->kv_indptr || !plan->prefix_lens || !plan->items || !plan->status)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: plan has no device metadata (host-only build?)", who);
  return PKV_OK;
}

int check_page_table(const int32_t* page_table, int32_t stride, const pkv_plan* plan, const char* who) {
  if (!page_table) return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: page_table is NULL", who);
  const int64_t need = (int64_t(plan->max_kv_len) + plan->shape.page_size - 1) / plan->shape.page_size;
  if (stride < 1 || stride < need)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: page_table_stride %d cannot hold %lld pages (max_kv_len %d)",
                     who, stride, (long long)need, plan->max_kv_len);
  return PKV_OK;
}
}  // namespace

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace pkv

// Scratch of paged_extend_attn_noalloc: the split partials of one call, in a
// file-scope device array instead of a caller workspace. Each device holds its
// own copy for the life of the process; calls on one device share it. In host
// code the array's name is not a device address: the address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array.
int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "no current HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(PKV_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return set_error(PKV_ERR_HIP, "device %d: cannot get the scratch array's address: %s", dev,
                     hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_error; }

int pkv_device_supported(int device) {
  const int ok = device_supported(device);
  if (ok < 0) return set_error(PKV_ERR_HIP, "cannot query HIP device %d", device);
  return ok;
}

int pkv_extend_metadata_size_ex(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                                const pkv_shape* shape, int32_t window, int32_t flags, int32_t decode_splits,
                                int32_t num_cus, size_t* meta_bytes, size_t* workspace_bytes_out) {
  g_error[0] = 0;
  if (!meta_bytes || !workspace_bytes_out)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "pkv_extend_metadata_size: output pointers must not be NULL");
  int32_t cus = 0;
  int st = resolve_cus(num_cus, &cus);
  if (st) return st;
  pkv_plan plan;
  st = plan_extend(batch, prefix_lens_h, chunk_lens_h, shape, window, flags, decode_splits, cus, nullptr, 0, &plan,
                   meta_bytes);
  if (st) return st;
  *workspace_bytes_out = plan.workspace_bytes;
  return PKV_OK;
}

int pkv_extend_metadata_size(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                             const pkv_shape* shape, int32_t window, int32_t decode_splits, size_t* meta_bytes,
                             size_t* workspace_bytes_out) {
  return pkv_extend_metadata_size_ex(batch, prefix_lens_h, chunk_lens_h, shape, window, 0, decode_splits, 0,
                                     meta_bytes, workspace_bytes_out);
}

int build_extend_metadata(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                          const pkv_shape* shape, int32_t window, int32_t decode_splits, void* meta_host,
                          size_t meta_host_bytes, void* meta_dev, size_t meta_dev_bytes, pkv_plan* plan_out,
                          pkv_stream_t stream) {
  return build_extend_metadata_ex(batch, prefix_lens_h, chunk_lens_h, shape, window, 0, decode_splits, 0,
                                  meta_host, meta_host_bytes, meta_dev, meta_dev_bytes, plan_out, stream);
}

int build_extend_metadata_ex(int32_t batch, const int32_t* prefix_lens_h, const int32_t* chunk_lens_h,
                             const pkv_shape* shape, int32_t window, int32_t flags, int32_t decode_splits,
                             int32_t num_cus, void* meta_host, size_t meta_host_bytes, void* meta_dev,
                             size_t meta_dev_bytes, pkv_plan* plan_out, pkv_stream_t stream) {
  g_error[0] = 0;
  if (!meta_host || !plan_out)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "build_extend_metadata: meta_host and plan_out must not be NULL");
  int32_t cus = 0;
  int st = resolve_cus(num_cus, &cus);
  if (st) return st;
  size_t total = 0;
  pkv_plan plan;
  st = plan_extend(batch, prefix_lens_h, chunk_lens_h, shape, window, flags, decode_splits, cus, meta_host,
                   meta_host_bytes, &plan, &total);
  if (st) return st;
  if (meta_dev) {
    if (meta_dev_bytes < total)
      return set_error(PKV_ERR_WORKSPACE, "meta_dev holds %zu bytes, %zu needed", meta_dev_bytes, total);
    if (reinterpret_cast<uintptr_t>(meta_dev) & 15)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "meta_dev must be 16-byte aligned");
    if ((st = check_current_device())) return st;
    // The runtime copies up to 16 KiB from pinned memory with a copy kernel of
    // its own (2.7 us); above that it takes the DMA engine, and the next kernel
    // then starts 9-34 us after the copy ends. Larger pinned meta_host
    // (device-mapped host memory) is copied by a kernel that reads it in
    // place: one launch at any size. Other host memory takes the runtime copy.
    hipPointerAttribute_t attr;
    const void* src_dev = nullptr;
    if (total > kRuntimeKernelCopyBytes) {
      if (hipPointerGetAttributes(&attr, meta_host) == hipSuccess && attr.type == hipMemoryTypeHost &&
          !(reinterpret_cast<uintptr_t>(attr.devicePointer) & 15))
        src_dev = attr.devicePointer;
      else
        (void)hipGetLastError();   // not memory the runtime knows: leave no error behind
    }
    if (src_dev) {
      if ((st = launch_meta_copy(src_dev, meta_dev, total, stream))) return st;
    } else {
      const hipError_t e =
          hipMemcpyAsync(meta_dev, meta_host, total, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return set_error(PKV_ERR_HIP, "metadata copy failed: %s", hipGetErrorString(e));
    }
    const MetaLayout lay = meta_layout(batch, plan.n_items, plan.n_split_rows);
    char* d = static_cast<char*>(meta_dev);
    plan.qo_indptr = reinterpret_cast<const int32_t*>(d + lay.qo_indptr);
    plan.kv_indptr = reinterpret_cast<const int32_t*>(d + lay.kv_indptr);
    plan.prefix_lens = reinterpret_cast<const int32_t*>(d + lay.prefix_lens);
    plan.items = d + lay.items;
    plan.split_rows = plan.n_split_rows ? reinterpret_cast<const int32_t*>(d + lay.split_rows) : nullptr;
    plan.status = reinterpret_cast<int32_t*>(d + lay.status);
  }
  *plan_out = plan;
  return PKV_OK;
}

// Every kernel moves 16-byte vectors of these tensors.
static bool misaligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

int pkv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* page_table,
               int32_t page_table_stride, const int32_t* req_pool_indices, const pkv_plan* plan,
               const pkv_shape* shape, pkv_stream_t stream) {
  g_error[0] = 0;
  int st = check_plan(plan, shape, "pkv_append");
  if (st) return st;
  if ((st = check_page_table(page_table, page_table_stride, plan, "pkv_append"))) return st;
  if (plan->total_q > 0 && (!k_new || !v_new || !k_pool || !v_pool))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "pkv_append: K/V pointers must not be NULL");
  if (plan->total_q > 0 && (misaligned16(k_new) || misaligned16(v_new) || misaligned16(k_pool) || misaligned16(v_pool)))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "pkv_append: K/V pointers must be 16-byte aligned");
  if ((st = check_current_device())) return st;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.page_table_stride = page_table_stride;
  a.req_pool_indices = req_pool_indices;
  a.qo_indptr = plan->qo_indptr;
  a.prefix_lens = plan->prefix_lens;
  a.status = plan->status;
  a.batch = plan->batch;
  a.total_q = plan->total_q;
  a.shape = *shape;
  return launch_append(a, stream);
}

int pkv_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, const float* rope_table,
                    int32_t rope_table_len, void* k_pool, void* v_pool, const int32_t* page_table,
                    int32_t page_table_stride, const int32_t* req_pool_indices, const pkv_plan* plan,
                    const pkv_shape* shape, pkv_stream_t stream) {
  g_error[0] = 0;
  int st = check_plan(plan, shape, "pkv_rope_append");
  if (st) return st;
  if ((st = check_page_table(page_table, page_table_stride, plan, "pkv_rope_append"))) return st;
  if (plan->total_q > 0 && (!q || !q_out || !k_new || !v_new || !k_pool || !v_pool || !rope_table))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "pkv_rope_append: q, q_out, K/V, pools and rope_table must not be NULL");
  if (plan->total_q > 0 && (misaligned16(q) || misaligned16(q_out) || misaligned16(k_new) || misaligned16(v_new) ||
                            misaligned16(k_pool) || misaligned16(v_pool) || misaligned16(rope_table)))
    return set_error(PKV_ERR_INVALID_ARGUMENT,
                     "pkv_rope_append: q, q_out, K/V, pools and rope_table must be 16-byte aligned");
  if (plan->total_q > 0 && rope_table_len < plan->max_kv_len)
    return set_error(PKV_ERR_INVALID_ARGUMENT,
                     "pkv_rope_append: rope_table has %d positions, the batch reaches position %d", rope_table_len,
                     plan->max_kv_len - 1);
  if ((st = check_current_device())) return st;
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.page_table_stride = page_table_stride;
  a.req_pool_indices = req_pool_indices;
  a.qo_indptr = plan->qo_indptr;
  a.prefix_lens = plan->prefix_lens;
  a.status = plan->status;
  a.batch = plan->batch;
  a.total_q = plan->total_q;
  a.shape = *shape;
  a.q = q;
  a.q_out = q_out;
  a.rope_table = rope_table;   // non-NULL whenever there are rows (checked above)
  a.rope_table_len = rope_table_len;
  return launch_append(a, stream);
}

static int extend_attn_call(const char* name, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_table, int32_t page_table_stride, const int32_t* req_pool_indices,
                            const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* prefix_lens,
                            int32_t window, float sm_scale, const uint8_t* mask, int32_t mask_heads,
                            int32_t mask_rows, int32_t mask_kv_stride, const pkv_plan* plan, const pkv_shape* shape,
                            void* out, void* workspace, size_t workspace_bytes, pkv_stream_t stream,
                            const void* k_new = nullptr, const void* v_new = nullptr,
                            bool validate_only = false) {
  g_error[0] = 0;
  int st = check_plan(plan, shape, name);
  if (st) return st;
  if ((st = check_page_table(page_table, page_table_stride, plan, name))) return st;
  if (window != plan->window)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: window %d differs from the plan's %d", name, window,
                     plan->window);
  if (plan->total_q > 0 && (!q || !k_pool || !v_pool || !out))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: q, pools and out must not be NULL", name);
  if (plan->total_q > 0 && (misaligned16(q) || misaligned16(k_pool) || misaligned16(v_pool) || misaligned16(out) ||
                            misaligned16(workspace) || misaligned16(k_new) || misaligned16(v_new)))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: q, pools, out, workspace and new K/V must be 16-byte aligned",
                     name);
  if (!(std::isfinite(sm_scale)))
    return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: sm_scale is not finite", name);
  // the batch arrays: NULL or the plan's own device copies (the kernels take
  // every offset from the plan; caller device arrays cannot be compared with
  // it without a host synchronisation)
  auto planned = [](const void* given, const void* own) { return given == nullptr || given == own; };
  if (!planned(qo_indptr, plan->qo_indptr) || !planned(kv_indptr, plan->kv_indptr) ||
      !planned(prefix_lens, plan->prefix_lens))
    return set_error(PKV_ERR_INVALID_ARGUMENT,
                     "%s: qo_indptr, kv_indptr and prefix_lens must each be NULL or the plan's own device array",
                     name);
  if (mask && plan->total_q > 0) {
    if (mask_heads != 1 && mask_heads != shape->num_q_heads)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: mask_heads must be 1 or %d (got %d)", name,
                       shape->num_q_heads, mask_heads);
    if (mask_rows != 1 && mask_rows < plan->max_q_len)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: mask_rows must be 1 or >= the longest chunk %d (got %d)", name,
                       plan->max_q_len, mask_rows);
    if (mask_kv_stride < plan->max_kv_len || (mask_kv_stride & 3))
      return set_error(PKV_ERR_INVALID_ARGUMENT,
                       "%s: mask_kv_stride must be a multiple of 4 and >= the longest request %d (got %d)", name,
                       plan->max_kv_len, mask_kv_stride);
    if (reinterpret_cast<uintptr_t>(mask) & 3)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: mask must be 4-byte aligned", name);
    if (int64_t(plan->batch) * mask_heads * mask_rows * int64_t(mask_kv_stride) >= (int64_t(1) << 40))
      return set_error(PKV_ERR_UNSUPPORTED, "%s: mask too large", name);
  }
  if (plan->workspace_bytes > 0) {
    if (!workspace)
      return set_error(PKV_ERR_WORKSPACE, "%s: the plan needs %zu workspace bytes, got NULL", name,
                       plan->workspace_bytes);
    if (workspace_bytes < plan->workspace_bytes)
      return set_error(PKV_ERR_WORKSPACE, "%s: workspace holds %zu bytes, %zu needed", name,
                       workspace_bytes, plan->workspace_bytes);
  }
  if ((st = check_current_device())) return st;
  if (validate_only) return PKV_OK;
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt(float(shape->head_dim));
  AttnArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.page_table_stride = page_table_stride;
  a.req_pool_indices = req_pool_indices;
  a.qo_indptr = plan->qo_indptr;
  a.prefix_lens = plan->prefix_lens;
  a.items = static_cast<const WorkItem*>(plan->items);
  a.split_rows = plan->split_rows;
  a.status = plan->status;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.o_part = plan->n_split_rows ? ws : nullptr;
  a.ml_part = plan->n_split_rows
                  ? reinterpret_cast<float*>(ws + workspace_o_bytes(plan->n_split_rows, shape->num_q_heads,
                                                                    plan->max_splits, shape->head_dim,
                                                                    shape->dtype))
                  : nullptr;
  a.n_items = plan->n_items;
  a.n_split_rows = plan->n_split_rows;
  a.max_splits = plan->max_splits;
  a.total_q = plan->total_q;
  a.window = window;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.shape = *shape;
  a.mask = mask;
  a.mask_heads = mask_heads;
  a.mask_rows = mask_rows;
  a.mask_kv_stride = mask_kv_stride;
  if (k_new) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool_w = const_cast<void*>(k_pool);
    a.v_pool_w = const_cast<void*>(v_pool);
  }
  return launch_extend_attn(a, stream);
}

int paged_extend_attn(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                      int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                      const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                      const pkv_plan* plan, const pkv_shape* shape, void* out, void* workspace,
                      size_t workspace_bytes, pkv_stream_t stream) {
  return extend_attn_call("paged_extend_attn", q, k_pool, v_pool, page_table, page_table_stride, req_pool_indices,
                          qo_indptr, kv_indptr, prefix_lens, window, sm_scale, nullptr, 1, 1, 0, plan, shape, out,
                          workspace, workspace_bytes, stream);
}

int paged_extend_attn_masked(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                             const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                             const uint8_t* mask, int32_t mask_heads, int32_t mask_rows, int32_t mask_kv_stride,
                             const pkv_plan* plan, const pkv_shape* shape, void* out, void* workspace,
                             size_t workspace_bytes, pkv_stream_t stream) {
  if (!mask && plan && plan->total_q > 0) {
    g_error[0] = 0;
    return set_error(PKV_ERR_INVALID_ARGUMENT, "paged_extend_attn_masked: mask must not be NULL");
  }
  return extend_attn_call("paged_extend_attn_masked", q, k_pool, v_pool, page_table, page_table_stride,
                          req_pool_indices, qo_indptr, kv_indptr, prefix_lens, window, sm_scale, mask, mask_heads,
                          mask_rows, mask_kv_stride, plan, shape, out, workspace, workspace_bytes, stream);
}

int paged_extend_attn_append(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                             const int32_t* page_table, int32_t page_table_stride, const int32_t* req_pool_indices,
                             int32_t window, float sm_scale, const pkv_plan* plan, const pkv_shape* shape,
                             void* out, void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
  static const char* name = "paged_extend_attn_append";
  g_error[0] = 0;
  int st = check_plan(plan, shape, name);
  if (st) return st;
  if (plan->total_q > 0) {
    if (!k_new || !v_new || !k_pool || !v_pool)
      return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: K/V pointers must not be NULL", name);
    // the launch reads k_new / v_new while it writes the pools
    const size_t esize = shape->dtype == PKV_DTYPE_BF16 ? 2 : 4;
    const size_t row = size_t(shape->num_kv_heads) * shape->head_dim * esize;
    const size_t new_bytes = size_t(plan->total_q) * row;
    const size_t pool_bytes = size_t(shape->num_pages) * size_t(shape->page_size) * row;
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
      const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
      return x < y + nb && y < x + na;
    };
    for (const void* n : {k_new, v_new})
      for (const void* pl : {static_cast<const void*>(k_pool), static_cast<const void*>(v_pool)})
        if (overlap(n, new_bytes, pl, pool_bytes))
          return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: k_new / v_new overlap a pool", name);
  }
  if (shape->dtype != PKV_DTYPE_BF16 || plan->slot_blocks > kFuseMaxSlotBlocks) {
    // the append kernel first, then the attention: every argument of both is
    // checked before the append is launched
    if ((st = extend_attn_call(name, q, k_pool, v_pool, page_table, page_table_stride, req_pool_indices, nullptr,
                               nullptr, nullptr, window, sm_scale, nullptr, 1, 1, 0, plan, shape, out, workspace,
                               workspace_bytes, stream, nullptr, nullptr, true)))
      return st;
    if ((st = pkv_append(k_new, v_new, k_pool, v_pool, page_table, page_table_stride, req_pool_indices, plan, shape,
                         stream)))
      return st;
    return extend_attn_call(name, q, k_pool, v_pool, page_table, page_table_stride, req_pool_indices, nullptr,
                            nullptr, nullptr, window, sm_scale, nullptr, 1, 1, 0, plan, shape, out, workspace,
                            workspace_bytes, stream);
  }
  return extend_attn_call(name, q, k_pool, v_pool, page_table, page_table_stride, req_pool_indices, nullptr, nullptr,
                          nullptr, window, sm_scale, nullptr, 1, 1, 0, plan, shape, out, workspace, workspace_bytes,
                          stream, plan->total_q > 0 ? k_new : nullptr, v_new);
}

int paged_extend_attn_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* req_pool_indices, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* prefix_lens, int32_t window, float sm_scale,
                              const pkv_plan* plan, const pkv_shape* shape, void* out, pkv_stream_t stream) {
  static const char* name = "paged_extend_attn_noalloc";
  g_error[0] = 0;
  if (!plan) return set_error(PKV_ERR_INVALID_ARGUMENT, "%s: plan is NULL", name);
  if (plan->workspace_bytes > size_t(PKV_NOALLOC_SCRATCH_BYTES))
    return set_error(PKV_ERR_WORKSPACE, "%s: the plan needs %zu workspace bytes, more than the %zu-byte static scratch",
                     name, plan->workspace_bytes, size_t(PKV_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    int st = check_current_device();
    if (st) return st;
    if ((st = static_scratch(&ws))) return st;
  }
  return extend_attn_call(name, q, k_pool, v_pool, page_table, page_table_stride, req_pool_indices, qo_indptr,
                          kv_indptr, prefix_lens, window, sm_scale, nullptr, 1, 1, 0, plan, shape, out, ws,
                          ws ? size_t(PKV_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

int pkv_read_status(const pkv_plan* plan, int32_t* status_out, pkv_stream_t stream) {
  g_error[0] = 0;
  if (!plan || !plan->status || !status_out)
    return set_error(PKV_ERR_INVALID_ARGUMENT, "pkv_read_status: plan with device metadata and status_out needed");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(status_out, plan->status, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(PKV_ERR_HIP, "pkv_read_status: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
