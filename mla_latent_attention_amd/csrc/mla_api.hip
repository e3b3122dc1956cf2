// mla_api.hip - the extern "C" boundary declared in include/mla.h: argument
// validation, workspace sizing, the per-device property cache and launches.
// Every check runs before anything is enqueued; no HIP call is made for an
// invalid argument, so the error paths run without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"
#include "mla_plan.h"
#include "mla_plan_host.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// Compute units of the current device (cached), or 0 if HIP fails.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool shape_ok(int batch, int num_q_tokens, int num_heads, int max_seqlen_q) {
  if (batch < 1 || num_q_tokens < 1 || num_heads < 1) return false;
  if (max_seqlen_q < 1 || max_seqlen_q > 64) return false;
  if (num_q_tokens > (int64_t)batch * max_seqlen_q) return false;
  // token * heads * 576 must stay addressable with 64-bit offsets and the
  // combine grid (tokens * head groups) within one grid dimension.
  if ((int64_t)num_q_tokens * (num_heads / mla::kGroup) > 0x7FFFFFFF) return false;
  return true;
}

// Fixed device scratch for mla_decode_noalloc, the entry point for callers
// that cannot allocate: it holds the call's workspace (split descriptors and
// partials).  Each device holds its own copy of the array for the life of the
// process.  In host code `scratch` only names the symbol; its device address
// comes from hipGetSymbolAddress, per device, and only that address is ever
// handed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(20) << 20;  // 20 MiB
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address per device, once found

// Device address of this device's scratch (set up on the first call on the
// device, with that device current), or nullptr if HIP fails.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

#ifdef MLA_DEBUG_CHECKS
// The debug build's check result: one word per device, written by the check
// kernel and read back by the entry point that launched it.
static __device__ int debug_status;

// Runs the device-side index check on `stream`, waits for it, and returns
// MLA_ERR_BAD_INPUT if it found a violation (the debug build only: this
// synchronises, which the release entry points never do).
mla_status debug_check(mla::CheckParams c, void* stream) {
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_status)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return MLA_ERR_HIP;
  }
  c.status = static_cast<int*>(ptr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mla::launch_check_inputs(c, st) != hipSuccess) return MLA_ERR_HIP;
  int found = 0;
  if (hipMemcpyAsync(&found, ptr, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MLA_ERR_HIP;
  return found != 0 ? MLA_ERR_BAD_INPUT : MLA_OK;
}
#endif

mla::CheckParams check_params(const int32_t* qo_indptr, const int32_t* kv_indptr,
                              const int32_t* kv_indices, int64_t kv_indices_len,
                              const int32_t* last_page_lens, int page_shift, int64_t pool_entries,
                              int batch, int num_q_tokens, int max_seqlen_q,
                              const int32_t* g_kv_indptr, int cp_size, int cp_rank) {
  mla::CheckParams c;
  c.qo_indptr = qo_indptr;
  c.kv_indptr = kv_indptr;
  c.kv_indices = kv_indices;
  c.last_page_lens = last_page_lens;
  c.g_kv_indptr = g_kv_indptr;
  c.kv_indices_len = kv_indices_len;
  c.pool_entries = pool_entries;
  c.batch = batch;
  c.num_q_tokens = num_q_tokens;
  c.max_seqlen_q = max_seqlen_q;
  c.page_shift = page_shift;
  c.cp_size = g_kv_indptr != nullptr ? cp_size : 1;
  c.cp_rank = g_kv_indptr != nullptr ? cp_rank : 0;
  c.status = nullptr;
  return c;
}

using mla::kMaxWorkers;
constexpr int kMaxCpSize = 1024;  // DCP shards accepted by mla_decode_dcp
constexpr int kMaxPageShift = 12;  // page sizes accepted by mla_decode_paged: 1 .. 4096

// Partial slots per worker for a call shape (group mode applies to the fp8
// kernels; the layout is sized the same for both storage types).
int slots_for(int num_heads, int max_seqlen_q) {
  return mla::slots_per_worker(mla::use_group_mode(num_heads / mla::kGroup, max_seqlen_q));
}

// Default worker count: one per CU (both kernels run one workgroup per CU).
int workers_for(int num_heads, int max_seqlen_q, int cus) {
  (void)num_heads;
  (void)max_seqlen_q;
  return cus;
}

mla_status decode_impl(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                       int64_t pool_entries, void* o, const int32_t* qo_indptr,
                       const int32_t* kv_indptr, const int32_t* kv_indices, int64_t kv_indices_len,
                       int batch, int num_q_tokens, int num_heads, int max_seqlen_q,
                       float sm_scale, const float* q_scale, const float* kv_scale,
                       int return_lse, float* lse, const int32_t* g_kv_indptr, int cp_size,
                       int cp_rank, const int32_t* last_page_lens, int page_shift, void* workspace,
                       size_t workspace_bytes, int num_workers, void* stream, int o_fp32 = 0) {
  if (!q || !kv_pool || !o || !qo_indptr || !kv_indptr || !kv_indices)
    return MLA_ERR_NULL_POINTER;
  if (return_lse && !lse) return MLA_ERR_NULL_POINTER;
  if (q_dtype != kv_dtype) return MLA_ERR_BAD_DTYPE;
  if (q_dtype != MLA_DTYPE_FP8_E4M3FN && q_dtype != MLA_DTYPE_BF16) return MLA_ERR_BAD_DTYPE;
  if (num_heads % mla::kGroup != 0 || num_heads <= 0) return MLA_ERR_UNSUPPORTED;
  if (!shape_ok(batch, num_q_tokens, num_heads, max_seqlen_q)) return MLA_ERR_BAD_SHAPE;
  if (pool_entries < 1 || kv_indices_len < 0 || kv_indices_len > 0x7FFFFFFF)
    return MLA_ERR_BAD_SHAPE;
  if (num_workers < 0 || num_workers > kMaxWorkers) return MLA_ERR_BAD_SHAPE;
  const int64_t num_units = (int64_t)num_q_tokens * (num_heads / mla::kGroup);
  const int slots = slots_for(num_heads, max_seqlen_q);
  if (!workspace) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (num_workers > 0 && workspace_bytes < mla::workspace_bytes(num_workers, num_units, slots))
    return MLA_ERR_WORKSPACE_TOO_SMALL;

  const int kdt = (kv_dtype == MLA_DTYPE_FP8_E4M3FN) ? 0 : 1;
  const bool group_mode = kdt == 0 && mla::use_group_mode(num_heads / mla::kGroup, max_seqlen_q);
  if (num_workers == 0) {
    const int cus = current_cu_count();
    if (cus <= 0) return MLA_ERR_HIP;
    num_workers = workers_for(num_heads, max_seqlen_q, cus);
    if (workspace_bytes < mla::workspace_bytes(num_workers, num_units, slots))
      return MLA_ERR_WORKSPACE_TOO_SMALL;
  }

  mla::DecodeParams p;
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_pool);
  p.pool_entries = pool_entries;
  // An fp32 output (DCP shards to be merged) also keeps the split partials in
  // fp32, so the result carries no bf16 rounding before the merge's own.
  p.o = o_fp32 ? nullptr : static_cast<uint16_t*>(o);
  p.o32 = o_fp32 ? static_cast<float*>(o) : nullptr;
  p.part_fp32 = o_fp32 ? 1 : 0;
  p.qo_indptr = qo_indptr;
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.kv_indices_len = (int)kv_indices_len;
  p.batch = batch;
  p.num_tokens = num_q_tokens;
  p.num_heads = num_heads;
  p.sm_scale = sm_scale;
  p.q_scale = q_scale;
  p.kv_scale = kv_scale;
  p.lse = return_lse ? lse : nullptr;
  mla::set_workspace(p, static_cast<char*>(workspace), num_units, num_workers, slots);
  p.num_workers = num_workers;
  p.causal = 1;
  p.g_kv_indptr = g_kv_indptr;
  p.cp_size = cp_size;
  p.cp_rank = cp_rank;
  p.last_page_lens = page_shift > 0 ? last_page_lens : nullptr;
  p.page_shift = page_shift;
#ifdef MLA_DEBUG_CHECKS
  {
    const mla_status s = debug_check(
        check_params(qo_indptr, kv_indptr, kv_indices, kv_indices_len, p.last_page_lens,
                     page_shift, pool_entries, batch, num_q_tokens, max_seqlen_q, g_kv_indptr,
                     cp_size, cp_rank),
        stream);
    if (s != MLA_OK) return s;
  }
#endif
  if (mla::launch_decode(p, kdt, group_mode, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER: a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE: a size argument is out of range";
    case MLA_ERR_BAD_DTYPE: return "MLA_ERR_BAD_DTYPE: unsupported storage type combination";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: num_heads must be a multiple of 16";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MLA_ERR_SCRATCH_TOO_SMALL:
      return "MLA_ERR_SCRATCH_TOO_SMALL: the call needs more workspace than the fixed scratch "
             "of mla_decode_noalloc holds";
    case MLA_ERR_BAD_INPUT:
      return "MLA_ERR_BAD_INPUT: the index arguments break the call's contract (found by the "
             "device-side check)";
    default: return "MLA_ERR_UNKNOWN";
  }
}

size_t mla_decode_workspace_bytes_ex(int batch, int num_q_tokens, int num_heads,
                                     int max_seqlen_q, int num_workers) {
  if (!shape_ok(batch, num_q_tokens, num_heads, max_seqlen_q)) return 0;
  if (num_workers < 1 || num_workers > kMaxWorkers) return 0;
  return mla::workspace_bytes(num_workers, (int64_t)num_q_tokens * (num_heads / mla::kGroup),
                              slots_for(num_heads, max_seqlen_q));
}

size_t mla_decode_workspace_bytes(int batch, int num_q_tokens, int num_heads, int max_seqlen_q) {
  if (!shape_ok(batch, num_q_tokens, num_heads, max_seqlen_q)) return 0;
  const int cus = current_cu_count();
  if (cus <= 0) return 0;
  return mla::workspace_bytes(workers_for(num_heads, max_seqlen_q, cus),
                              (int64_t)num_q_tokens * (num_heads / mla::kGroup),
                              slots_for(num_heads, max_seqlen_q));
}

mla_status mla_decode_ex(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                         int64_t pool_entries, void* o, const int32_t* qo_indptr,
                         const int32_t* kv_indptr, const int32_t* kv_indices,
                         int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                         int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                         const float* q_scale, const float* kv_scale, int return_lse,
                         float* lse, void* workspace, size_t workspace_bytes, int num_workers,
                         void* stream) {
  (void)kv_last_page_lens;  // page_size 1: all ones by contract, never read
  return decode_impl(q, q_dtype, kv_pool, kv_dtype, pool_entries, o, qo_indptr, kv_indptr,
                     kv_indices, kv_indices_len, batch, num_q_tokens, num_heads, max_seqlen_q,
                     sm_scale, q_scale, kv_scale, return_lse, lse, nullptr, 1, 0, nullptr, 0,
                     workspace, workspace_bytes, num_workers, stream);
}

mla_status mla_decode_paged(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                            int64_t pool_entries, void* o, const int32_t* qo_indptr,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int64_t kv_indices_len, const int32_t* kv_last_page_lens,
                            int page_size, int batch, int num_q_tokens, int num_heads,
                            int max_seqlen_q, float sm_scale, const float* q_scale,
                            const float* kv_scale, int return_lse, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int shift = 0;
  while (shift <= kMaxPageShift && (1 << shift) != page_size) ++shift;
  if (page_size < 1 || shift > kMaxPageShift) return MLA_ERR_BAD_SHAPE;
  if (shift > 0 && !kv_last_page_lens) return MLA_ERR_NULL_POINTER;
  // Rows are page * page_size + slot: every page number must name whole rows
  // of the pool, and the largest row must stay a valid int32.
  if (shift > 0 && (pool_entries % page_size != 0 || pool_entries > 0x7FFFFFFF))
    return MLA_ERR_BAD_SHAPE;
  return decode_impl(q, q_dtype, kv_pool, kv_dtype, pool_entries, o, qo_indptr, kv_indptr,
                     kv_indices, kv_indices_len, batch, num_q_tokens, num_heads, max_seqlen_q,
                     sm_scale, q_scale, kv_scale, return_lse, lse, nullptr, 1, 0,
                     kv_last_page_lens, shift, workspace, workspace_bytes, 0, stream);
}

mla_status mla_decode_dcp(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                          int64_t pool_entries, void* o, const int32_t* qo_indptr,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                          int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                          const float* q_scale, const float* kv_scale, int return_lse,
                          float* lse, const int32_t* g_kv_indptr, int cp_world_size,
                          int cp_rank, int o_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  (void)kv_last_page_lens;
  if (!g_kv_indptr) return MLA_ERR_NULL_POINTER;
  if (o_dtype != MLA_DTYPE_BF16 && o_dtype != MLA_DTYPE_FP32) return MLA_ERR_BAD_DTYPE;
  if (cp_world_size < 1 || cp_world_size > kMaxCpSize || cp_rank < 0 || cp_rank >= cp_world_size)
    return MLA_ERR_BAD_SHAPE;
  return decode_impl(q, q_dtype, kv_pool, kv_dtype, pool_entries, o, qo_indptr, kv_indptr,
                     kv_indices, kv_indices_len, batch, num_q_tokens, num_heads, max_seqlen_q,
                     sm_scale, q_scale, kv_scale, return_lse, lse, g_kv_indptr, cp_world_size,
                     cp_rank, nullptr, 0, workspace, workspace_bytes, 0, stream,
                     o_dtype == MLA_DTYPE_FP32 ? 1 : 0);
}

mla_status mla_decode(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                      int64_t pool_entries, void* o, const int32_t* qo_indptr,
                      const int32_t* kv_indptr, const int32_t* kv_indices,
                      int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                      int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                      const float* q_scale, const float* kv_scale, int return_lse, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_ex(q, q_dtype, kv_pool, kv_dtype, pool_entries, o, qo_indptr, kv_indptr,
                       kv_indices, kv_indices_len, kv_last_page_lens, batch, num_q_tokens,
                       num_heads, max_seqlen_q, sm_scale, q_scale, kv_scale, return_lse, lse,
                       workspace, workspace_bytes, 0, stream);
}

mla_status mla_decode_noalloc(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                              int64_t pool_entries, void* o, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* kv_indices,
                              int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                              int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                              const float* q_scale, const float* kv_scale, int return_lse,
                              float* lse, void* stream) {
  // The same checks as mla_decode first (nothing below allocates), then the
  // size check against the fixed scratch.
  if (!q || !kv_pool || !o || !qo_indptr || !kv_indptr || !kv_indices)
    return MLA_ERR_NULL_POINTER;
  if (!shape_ok(batch, num_q_tokens, num_heads, max_seqlen_q)) return MLA_ERR_BAD_SHAPE;
  if (num_heads <= 0 || num_heads % mla::kGroup != 0) return MLA_ERR_UNSUPPORTED;
  const int cus = current_cu_count();
  if (cus <= 0) return MLA_ERR_HIP;
  const size_t need = mla::workspace_bytes(workers_for(num_heads, max_seqlen_q, cus),
                                           (int64_t)num_q_tokens * (num_heads / mla::kGroup),
                                           slots_for(num_heads, max_seqlen_q));
  if (need > kNoAllocScratchBytes) return MLA_ERR_SCRATCH_TOO_SMALL;
  void* ws = device_scratch();
  if (ws == nullptr) return MLA_ERR_HIP;
  (void)kv_last_page_lens;
  return decode_impl(q, q_dtype, kv_pool, kv_dtype, pool_entries, o, qo_indptr, kv_indptr,
                     kv_indices, kv_indices_len, batch, num_q_tokens, num_heads, max_seqlen_q,
                     sm_scale, q_scale, kv_scale, return_lse, lse, nullptr, 1, 0, nullptr, 0, ws,
                     kNoAllocScratchBytes, 0, stream);
}

size_t mla_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

namespace {

// The layer step's workspace after the decode's: the fp8 q rows (T, H_pad,
// 576) the prologue builds, then one plan per worker.
size_t step_q_bytes(int num_q_tokens, int num_heads_pad) {
  return mla::align256((size_t)num_q_tokens * num_heads_pad * mla::kRowDim);
}
size_t step_extra_bytes(int num_q_tokens, int num_heads_pad, int num_workers) {
  return step_q_bytes(num_q_tokens, num_heads_pad) +
         mla::align256((size_t)num_workers * sizeof(mla::WorkerPlan));
}

// Cascade workspace: the group-mode decode workspace for the one-launch call
// (2T virtual tokens), followed by its fp32 outputs, parts (2, T, H, 512) and
// lse_parts (2, T, H): prefix first, suffix second (fp32 keeps the merge from
// adding a third bf16 rounding to the result).
struct CascadeLayout {
  size_t decode_bytes, parts_off, lse_off, total;
};

// The cascade takes any head count (rows are packed 16 to a row group, so
// 12 real heads need no padding) within the plain call's other limits.
bool cascade_shape_ok(int batch, int num_q_tokens, int num_heads, int max_seqlen_q) {
  if (num_heads < 1 || num_heads > 4096) return false;
  const int padded = mla::kGroup * mla::group_slots_per_token(num_heads);
  return shape_ok(batch, num_q_tokens, padded, max_seqlen_q) &&
         (int64_t)2 * num_q_tokens * num_heads <= 0x7FFFFFFF;
}

CascadeLayout cascade_layout(int batch, int num_q_tokens, int num_heads, int max_seqlen_q,
                             int cus) {
  const int64_t units = 2 * (int64_t)num_q_tokens * mla::group_slots_per_token(num_heads);
  CascadeLayout l;
  l.decode_bytes = mla::align256(mla::workspace_bytes(cus, units, mla::slots_per_worker(true)));
  l.parts_off = l.decode_bytes;
  l.lse_off = l.parts_off + mla::align256((size_t)2 * num_q_tokens * num_heads * mla::kLatent * 4);
  l.total = l.lse_off + mla::align256((size_t)2 * num_q_tokens * num_heads * 4);
  (void)batch;
  (void)max_seqlen_q;
  return l;
}


}  // namespace

size_t mla_decode_cascade_workspace_bytes(int batch, int num_q_tokens, int num_heads,
                                          int max_seqlen_q) {
  if (!cascade_shape_ok(batch, num_q_tokens, num_heads, max_seqlen_q)) return 0;
  const int cus = current_cu_count();
  if (cus <= 0) return 0;
  return cascade_layout(batch, num_q_tokens, num_heads, max_seqlen_q, cus).total;
}

mla_status mla_decode_cascade(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                              int64_t pool_entries, void* o, const int32_t* qo_indptr,
                              const int32_t* prefix_indices, int64_t prefix_len,
                              const int32_t* suffix_indptr, const int32_t* suffix_indices,
                              int64_t suffix_indices_len, int batch, int num_q_tokens,
                              int num_heads, int max_seqlen_q, float sm_scale,
                              const float* q_scale, const float* kv_scale, int return_lse,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !kv_pool || !o || !qo_indptr || !suffix_indptr || !workspace)
    return MLA_ERR_NULL_POINTER;
  if (prefix_len > 0 && !prefix_indices) return MLA_ERR_NULL_POINTER;
  if (suffix_indices_len > 0 && !suffix_indices) return MLA_ERR_NULL_POINTER;
  if (return_lse && !lse) return MLA_ERR_NULL_POINTER;
  if (q_dtype != MLA_DTYPE_FP8_E4M3FN || kv_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_BAD_DTYPE;
  const int T = num_q_tokens;
  if (!cascade_shape_ok(batch, T, num_heads, max_seqlen_q)) return MLA_ERR_BAD_SHAPE;
  if (pool_entries < 1 || prefix_len < 0 || suffix_indices_len < 0 ||
      prefix_len + suffix_indices_len > 0x7FFFFFFF || T > (1 << 29) || batch > (1 << 29))
    return MLA_ERR_BAD_SHAPE;
  const int cus = current_cu_count();
  if (cus <= 0) return MLA_ERR_HIP;
  const CascadeLayout lay = cascade_layout(batch, T, num_heads, max_seqlen_q, cus);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const int64_t units = (int64_t)T * mla::group_slots_per_token(num_heads);
  char* ws = static_cast<char*>(workspace);
  float* parts = reinterpret_cast<float*>(ws + lay.parts_off);
  float* lse_parts = reinterpret_cast<float*>(ws + lay.lse_off);
  const int64_t rows = (int64_t)T * num_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);

  mla::DecodeParams p;
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_pool);
  p.pool_entries = pool_entries;
  p.num_tokens = T;
  p.num_heads = num_heads;
  p.sm_scale = sm_scale;
  p.q_scale = q_scale;
  p.kv_scale = kv_scale;
  p.num_workers = cus;

  // One group-mode launch over the cascade view (see ReqSource): request 0
  // is every token (virtual tokens 0 .. T-1) against the prefix, all entries
  // visible, so each prefix row is gathered once per eight row groups of the
  // whole batch; requests 1 .. B are the caller's requests again (virtual
  // tokens T .. 2T-1) against their suffixes, causal.  The two passes share
  // one balanced work stream and one split combine, and their fp32 outputs
  // land in parts[0] and parts[1].
  p.o = nullptr;
  p.o32 = parts;
  p.lse = lse_parts;
  p.qo_indptr = qo_indptr;
  p.kv_indptr = suffix_indptr;
  p.kv_indices = prefix_indices;
  p.kv_indices2 = suffix_indices;
  p.cascade_prefix = (int)prefix_len;
  p.kv_indices_len = (int)(prefix_len + suffix_indices_len);
  p.batch = batch + 1;
  p.num_tokens = 2 * T;
  p.causal = 1;
  mla::set_workspace(p, ws, 2 * units, p.num_workers, mla::slots_per_worker(true));
#ifdef MLA_DEBUG_CHECKS
  {
    // The suffix lists as the batch, then the prefix list whole.
    mla_status s = debug_check(check_params(qo_indptr, suffix_indptr, suffix_indices,
                                            suffix_indices_len, nullptr, 0, pool_entries, batch,
                                            T, max_seqlen_q, nullptr, 1, 0),
                               stream);
    if (s == MLA_OK && prefix_len > 0)
      s = debug_check(check_params(nullptr, nullptr, prefix_indices, prefix_len, nullptr, 0,
                                   pool_entries, 1, 0, 1, nullptr, 1, 0),
                      stream);
    if (s != MLA_OK) return s;
  }
#endif
  if (mla::launch_decode(p, 0, true, st) != hipSuccess) return MLA_ERR_HIP;

  // LSE merge of the two passes (a pass that saw nothing has lse = -inf).
  if (mla::launch_merge(parts, 1, lse_parts, 2, rows, static_cast<uint16_t*>(o),
                        return_lse ? lse : nullptr, st) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_merge_partials(const void* o_parts, int parts_dtype, const float* lse_parts,
                              int num_parts, int num_q_tokens, int num_heads, void* o,
                              float* lse, void* stream) {
  if (!o_parts || !lse_parts || !o) return MLA_ERR_NULL_POINTER;
  if (parts_dtype != MLA_DTYPE_FP32 && parts_dtype != MLA_DTYPE_BF16) return MLA_ERR_BAD_DTYPE;
  if (num_parts < 1 || num_q_tokens < 1 || num_heads < 1) return MLA_ERR_BAD_SHAPE;
  const int64_t rows = (int64_t)num_q_tokens * num_heads;
  if ((rows + 3) / 4 > 0x7FFFFFFF) return MLA_ERR_BAD_SHAPE;
  if (mla::launch_merge(o_parts, parts_dtype == MLA_DTYPE_FP32, lse_parts, num_parts, rows,
                        static_cast<uint16_t*>(o), lse,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int64_t mla_plan_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* g_kv_indptr, int batch, int num_heads, int num_workers,
                      int cp_world_size, int cp_rank, int64_t* out, int64_t out_cap) {
  return mla::plan_pieces_host(qo_indptr, kv_indptr, g_kv_indptr, batch, num_heads, num_workers,
                               cp_world_size, cp_rank, out, out_cap);
}

int64_t mla_plan_groups_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* g_kv_indptr, int batch, int num_heads,
                             int num_workers, int causal, int cp_world_size, int cp_rank,
                             int64_t* out, int64_t out_cap) {
  return mla::plan_group_pieces_host(qo_indptr, kv_indptr, g_kv_indptr, batch, num_heads,
                                     num_workers, causal, cp_world_size, cp_rank, out, out_cap);
}

mla_status mla_rope_quant_cache(const void* q_latent, const void* q_pe, const void* k_latent,
                                const void* k_pe, const int32_t* positions, const float* cos_sin,
                                int max_pos, int rope_style, void* q_out, int num_q_tokens,
                                int num_heads, int num_heads_pad, void* kv_pool,
                                int64_t pool_entries, const int32_t* slot_mapping,
                                const float* q_scale, const float* kv_scale, void* stream) {
  if (!q_latent || !q_pe || !k_latent || !k_pe || !positions || !cos_sin || !q_out || !kv_pool ||
      !slot_mapping)
    return MLA_ERR_NULL_POINTER;
  if (num_q_tokens < 1 || num_heads < 1 || num_heads_pad < num_heads || max_pos < 1 ||
      pool_entries < 1 || (rope_style != 0 && rope_style != 1))
    return MLA_ERR_BAD_SHAPE;
  if ((int64_t)(num_heads_pad + 1) * 72 > 0x7FFFFFFF) return MLA_ERR_BAD_SHAPE;
  if (mla::launch_rope_quant_cache(
          static_cast<const uint16_t*>(q_latent), static_cast<const uint16_t*>(q_pe),
          static_cast<const uint16_t*>(k_latent), static_cast<const uint16_t*>(k_pe), positions,
          cos_sin, max_pos, rope_style, static_cast<uint8_t*>(q_out), num_q_tokens, num_heads,
          num_heads_pad, static_cast<uint8_t*>(kv_pool), pool_entries, slot_mapping, q_scale,
          kv_scale, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

size_t mla_decode_step_workspace_bytes(int batch, int num_q_tokens, int num_heads_pad,
                                       int max_seqlen_q) {
  if (!shape_ok(batch, num_q_tokens, num_heads_pad, max_seqlen_q)) return 0;
  if (num_heads_pad % mla::kGroup != 0) return 0;
  const int cus = current_cu_count();
  if (cus <= 0) return 0;
  const int64_t num_units = (int64_t)num_q_tokens * (num_heads_pad / mla::kGroup);
  return mla::align256(mla::workspace_bytes(cus, num_units, mla::slots_per_worker(false))) +
         step_extra_bytes(num_q_tokens, num_heads_pad, cus);
}

mla_status mla_decode_step(const void* q_latent, const void* q_pe, const void* k_latent,
                           const void* k_pe, const int32_t* positions, const float* cos_sin,
                           int max_pos, int rope_style, const int32_t* slot_mapping,
                           void* kv_pool, int64_t pool_entries, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t kv_indices_len, int batch, int num_q_tokens, int num_heads,
                           int num_heads_pad, int max_seqlen_q, float sm_scale,
                           const float* q_scale, const float* kv_scale, const void* w_uv,
                           void* o_latent, void* out, int return_lse, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_latent || !q_pe || !k_latent || !k_pe || !positions || !cos_sin || !slot_mapping ||
      !kv_pool || !qo_indptr || !kv_indptr || !kv_indices || !w_uv || !o_latent || !out)
    return MLA_ERR_NULL_POINTER;
  if (return_lse && !lse) return MLA_ERR_NULL_POINTER;
  if (num_heads_pad <= 0 || num_heads_pad % mla::kGroup != 0) return MLA_ERR_UNSUPPORTED;
  if (num_heads < 1 || num_heads > num_heads_pad || max_pos < 1 ||
      (rope_style != 0 && rope_style != 1))
    return MLA_ERR_BAD_SHAPE;
  if (!shape_ok(batch, num_q_tokens, num_heads_pad, max_seqlen_q)) return MLA_ERR_BAD_SHAPE;
  if (pool_entries < 1 || kv_indices_len < 0 || kv_indices_len > 0x7FFFFFFF)
    return MLA_ERR_BAD_SHAPE;
  if ((int64_t)num_q_tokens * num_heads_pad > 0x7FFFFFFF) return MLA_ERR_BAD_SHAPE;
  const int cus = current_cu_count();
  if (cus <= 0) return MLA_ERR_HIP;
  const int G = num_heads_pad / mla::kGroup;
  const int64_t num_units = (int64_t)num_q_tokens * G;
  const int slots = mla::slots_per_worker(false);
  const size_t dec_bytes = mla::align256(mla::workspace_bytes(cus, num_units, slots));
  if (!workspace ||
      workspace_bytes < dec_bytes + step_extra_bytes(num_q_tokens, num_heads_pad, cus))
    return MLA_ERR_WORKSPACE_TOO_SMALL;

  mla::DecodeParams p;
  p.q_out = static_cast<uint8_t*>(workspace) + dec_bytes;  // built by the call
  p.q = p.q_out;
  p.plans = reinterpret_cast<mla::WorkerPlan*>(p.q_out + step_q_bytes(num_q_tokens, num_heads_pad));
  p.kv = static_cast<const uint8_t*>(kv_pool);
  p.kv_out = static_cast<uint8_t*>(kv_pool);
  p.pool_entries = pool_entries;
  p.o = static_cast<uint16_t*>(o_latent);
  p.o32 = nullptr;
  p.part_fp32 = 0;
  p.qo_indptr = qo_indptr;
  p.kv_indptr = kv_indptr;
  p.kv_indices = kv_indices;
  p.kv_indices_len = (int)kv_indices_len;
  p.batch = batch;
  p.num_tokens = num_q_tokens;
  p.num_heads = num_heads_pad;
  p.sm_scale = sm_scale;
  p.q_scale = q_scale;
  p.kv_scale = kv_scale;
  p.lse = return_lse ? lse : nullptr;
  mla::set_workspace(p, static_cast<char*>(workspace), num_units, cus, slots);
  p.num_workers = cus;
  p.causal = 1;
  p.q_latent = static_cast<const uint16_t*>(q_latent);
  p.q_pe = static_cast<const uint16_t*>(q_pe);
  p.k_latent = static_cast<const uint16_t*>(k_latent);
  p.k_pe = static_cast<const uint16_t*>(k_pe);
  p.positions = positions;
  p.cos_sin = cos_sin;
  p.max_pos = max_pos;
  p.rope_style = rope_style;
  p.real_heads = num_heads;
  p.slot_mapping = slot_mapping;
#ifdef MLA_DEBUG_CHECKS
  {
    const mla_status s = debug_check(
        check_params(qo_indptr, kv_indptr, kv_indices, kv_indices_len, nullptr, 0, pool_entries,
                     batch, num_q_tokens, max_seqlen_q, nullptr, 1, 0),
        stream);
    if (s != MLA_OK) return s;
  }
#endif
  if (mla::launch_decode_step(p, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out),
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_check_inputs(const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, int64_t kv_indices_len,
                            const int32_t* kv_last_page_lens, int page_size,
                            int64_t pool_entries, int batch, int num_q_tokens, int max_seqlen_q,
                            const int32_t* g_kv_indptr, int cp_world_size, int cp_rank,
                            int* status, void* stream) {
  if (!qo_indptr || !kv_indptr || !status || (kv_indices_len > 0 && !kv_indices))
    return MLA_ERR_NULL_POINTER;
  int shift = 0;
  while (shift <= kMaxPageShift && (1 << shift) != page_size) ++shift;
  if (page_size < 1 || shift > kMaxPageShift) return MLA_ERR_BAD_SHAPE;
  if (batch < 1 || num_q_tokens < 0 || max_seqlen_q < 1 || kv_indices_len < 0 ||
      pool_entries < 1)
    return MLA_ERR_BAD_SHAPE;
  if (g_kv_indptr != nullptr &&
      (cp_world_size < 1 || cp_world_size > kMaxCpSize || cp_rank < 0 || cp_rank >= cp_world_size))
    return MLA_ERR_BAD_SHAPE;
  mla::CheckParams c = check_params(qo_indptr, kv_indptr, kv_indices, kv_indices_len,
                                    kv_last_page_lens, shift, pool_entries, batch, num_q_tokens,
                                    max_seqlen_q, g_kv_indptr, cp_world_size, cp_rank);
  c.status = status;
  if (mla::launch_check_inputs(c, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_latent_to_v(const void* o_latent, const void* w_uv, void* out, int num_q_tokens,
                           int num_heads, int num_heads_pad, void* stream) {
  if (!o_latent || !w_uv || !out) return MLA_ERR_NULL_POINTER;
  if (num_q_tokens < 1 || num_heads < 1 || num_heads > 65535 || num_heads_pad < num_heads)
    return MLA_ERR_BAD_SHAPE;
  if (mla::launch_latent_to_v(static_cast<const uint16_t*>(o_latent),
                              static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out),
                              num_q_tokens, num_heads, num_heads_pad,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
