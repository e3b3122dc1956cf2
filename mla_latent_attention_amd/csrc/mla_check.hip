// mla_check.hip - device-side check of a decode call's index arguments.
//
// The decode kernels take the call's CSR description ("[Kimi-K3 MLA TP8] MLA
// performance", Sec. 4.1 "Arguments": qo_indptr, kv_indptr, kv_indices,
// kv_last_page_lens; Sec. 5.2: with page_size 1 the kv_indptr deltas are KV
// lengths and kv_indices holds one pool entry per token) on trust: they clamp
// every index to the buffer it addresses, so a broken description gives wrong
// numbers, never an out-of-bounds access.  This kernel reports such a
// description instead: one pass over the requests and the index list, with a
// bit per kind of violation OR-ed into a status word.  It reads each input
// only within the bounds the host passes (batch + 1 indptr entries,
// kv_indices_len indices), whatever the arrays hold.
#include <hip/hip_runtime.h>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace mla {

__global__ void mla_check_clear_kernel(int* status) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *status = 0;
}

__global__ __launch_bounds__(256) void mla_check_inputs_kernel(const CheckParams c) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int bad = 0;
  // Per request: both indptr arrays start at 0 and never decrease; the last
  // entries match the token count and fit the index list; a request holds at
  // most max_seqlen_q query tokens; a request with pages names how many
  // entries its last page holds; a DCP shard holds exactly its share of the
  // request's positions (every cp_size-th from cp_rank).
  // (No kv_indptr: the list is checked whole, as a cascade call's prefix.)
  const int nreq = c.kv_indptr != nullptr ? c.batch : 0;
  for (int64_t b = gid; b < nreq; b += stride) {
    const int64_t qa = c.qo_indptr[b], qb = c.qo_indptr[b + 1];
    if ((b == 0 && qa != 0) || qb < qa || qb - qa > c.max_seqlen_q) bad |= MLA_CHECK_QO_INDPTR;
    if (b == c.batch - 1 && qb != c.num_q_tokens) bad |= MLA_CHECK_QO_INDPTR;
    const int64_t ka = c.kv_indptr[b], kb = c.kv_indptr[b + 1];
    if ((b == 0 && ka != 0) || kb < ka) bad |= MLA_CHECK_KV_INDPTR;
    if (b == c.batch - 1 && kb > c.kv_indices_len) bad |= MLA_CHECK_KV_INDPTR;
    if (c.last_page_lens != nullptr) {
      const int lp = c.last_page_lens[b];
      const int page = 1 << c.page_shift;
      // page_size 1: every entry is a whole page, so the length is 1 (0 is
      // also taken for a request with no entries).
      const bool ok = c.page_shift == 0 ? (lp == 1 || (kb == ka && lp == 0))
                                        : (kb == ka || (lp >= 1 && lp <= page));
      if (!ok) bad |= MLA_CHECK_LAST_PAGE_LEN;
    }
    if (c.g_kv_indptr != nullptr) {
      const int64_t ga = c.g_kv_indptr[b], gb = c.g_kv_indptr[b + 1];
      if ((b == 0 && ga != 0) || gb < ga) bad |= MLA_CHECK_DCP_LENGTHS;
      const int64_t n = gb - ga;
      const int64_t share = n > c.cp_rank ? (n - c.cp_rank - 1) / c.cp_size + 1 : 0;
      if (kb - ka != share) bad |= MLA_CHECK_DCP_LENGTHS;
    }
  }
  // Every index the requests use names a row of the pool (a page of it when
  // the cache is paged).  kv_indptr[batch] is clamped to the list's length,
  // which the check above reports if it exceeds it.
  const int64_t used = c.kv_indptr != nullptr ? (int64_t)c.kv_indptr[c.batch] : c.kv_indices_len;
  const int64_t n = used < 0 ? 0 : (used < c.kv_indices_len ? used : c.kv_indices_len);
  const int64_t limit = c.pool_entries >> c.page_shift;
  for (int64_t i = gid; i < n; i += stride) {
    const int v = c.kv_indices[i];
    if (v < 0 || (int64_t)v >= limit) bad |= MLA_CHECK_KV_INDEX;
  }
  if (bad != 0) atomicOr(c.status, bad);
}

hipError_t launch_check_inputs(const CheckParams& c, hipStream_t stream) {
  hipLaunchKernelGGL(mla_check_clear_kernel, dim3(1), dim3(64), 0, stream, c.status);
  // Enough threads for one index each up to 256 blocks of 256, grid-stride
  // beyond; at least one block for the per-request checks.
  const int64_t items = c.kv_indices_len > c.batch ? c.kv_indices_len : c.batch;
  int64_t blocks = (items + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(mla_check_inputs_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, c);
  return hipGetLastError();
}

}  // namespace mla
