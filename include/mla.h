/*
 * mla.h - C ABI of the MI355X (gfx950) latent-MLA decode library.
 *
 * The operation: absorbed (latent) multi-head latent attention decode over a
 * token-major paged cache, as described on the page "[Kimi-K3 MLA TP8] MLA
 * performance" (ROCm/aiter issue 4541):
 *   - Sec. 2 "K3 MLA geometry": every cached token is one 576-wide latent row
 *     (512 latent + 64 rope) shared by all query heads; scores use all 576
 *     dims, the output is the softmax-weighted sum of the first 512 dims;
 *     sm_scale = 1/sqrt(192).
 *   - Sec. 3 "Entry point" and Sec. 4.1 "Arguments": the call's tensors
 *     (q, kv_buffer, o, qo_indptr, kv_indptr, kv_indices, kv_last_page_lens,
 *     sm_scale, q_scale, kv_scale, return_lse) and their layouts.
 *   - Sec. 5.2 "The kernel runs with page_size = 1": kv_indptr deltas are KV
 *     lengths in tokens, kv_indices holds one pool entry per token.
 * The merge of partial answers follows "Kimi K3 on AMD Instinct MI355X: vLLM
 * Serving Matches NVIDIA HGX B300 Throughput per GPU on AgentX", Sec. "1.
 * Cache: keep conversation state available for reuse" (partial answers carry
 * normalisation information and are merged with softmax weights).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *     row-major memory on the current HIP device.  The library allocates and
 *     frees nothing on the call path and keeps no state between calls other
 *     than a cached per-device property query.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and the call returns without synchronising.  The host
 *     never reads device memory, so the calls can be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     violation returns a status code and enqueues nothing.  A failed launch
 *     returns MLA_ERR_HIP.  No C++ exception crosses this interface.
 *   - Device-side contents (indptr monotonicity, index ranges) are the
 *     caller's contract.  The kernels clamp every index they read to the
 *     buffer it addresses, so a violation gives wrong numbers, never an
 *     out-of-bounds access.  mla_check_inputs reports violations on request;
 *     a library built with MLA_DEBUG_CHECKS defined (libmla_debug.so) runs
 *     that check inside every decode entry point, synchronises, and returns
 *     MLA_ERR_BAD_INPUT, enqueuing nothing else, when it finds one.
 *   - Concurrent calls on different streams need distinct workspaces.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types. FP8 is OCP float8_e4m3fn (the KV cache dtype of Sec. 1). */
typedef enum {
  MLA_DTYPE_FP8_E4M3FN = 0,
  MLA_DTYPE_BF16 = 1,
  MLA_DTYPE_FP32 = 2
} mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,
  MLA_ERR_BAD_SHAPE = 2,
  MLA_ERR_BAD_DTYPE = 3,
  MLA_ERR_UNSUPPORTED = 4,
  MLA_ERR_WORKSPACE_TOO_SMALL = 5,
  MLA_ERR_HIP = 6,
  MLA_ERR_SCRATCH_TOO_SMALL = 7,
  MLA_ERR_BAD_INPUT = 8
} mla_status;

/* Width of one cache row and of the output (Sec. 2 "K3 MLA geometry"). */
#define MLA_ROW_DIM 576
#define MLA_LATENT_DIM 512
/* Heads are processed in groups of 16; callers pad 12 -> 16 (Sec. 5.1). */
#define MLA_HEAD_GROUP 16

/*
 * Workspace bytes mla_decode needs on the current device for this call shape.
 * The workspace holds the partial answers of the KV splits (o rows and their
 * lse) and one 16-byte split descriptor per (query token, head group); its
 * size depends only on the device's compute-unit count and the arguments
 * below, not on KV lengths or the storage type.  Returns 0 for invalid shapes.
 *
 * Two kernels serve mla_decode.  The standard one gives each worker
 * workgroup a contiguous range of (token, head group) rows, at most two of
 * them partial (two 16x512 partial slots per worker), one worker per compute
 * unit.  When num_heads / 16 * max_seqlen_q >= 4 and the storage is FP8, the
 * group-mode kernel instead walks 8 row groups of one request over a single
 * shared KV range, so each gathered cache row feeds 128 query rows; it also
 * runs one worker per compute unit, with sixteen partial slots each.
 * Partial o rows are stored in fp16, divided by kv_scale, for an FP8 cache
 * with a bf16 output and in fp32 otherwise (a bf16 cache, or an fp32 output as
 * mla_decode_dcp can ask for); the slots are sized for fp32 either way.  The workspace is sized for
 * the group-mode layout whenever the shape qualifies.
 */
size_t mla_decode_workspace_bytes(int batch, int num_q_tokens, int num_heads, int max_seqlen_q);

/*
 * MLA decode (Sec. 3 entry point; Sec. 4.1 argument layouts).
 *
 *  q              (num_q_tokens, num_heads, 576) of q_dtype.  Heads beyond the
 *                 model's real count are caller padding; each head attends
 *                 independently, so padding never changes a real head.
 *  kv_pool        (pool_entries, 576) of kv_dtype, i.e. the (N,1,1,576) cache
 *                 viewed token-major (page_size 1).
 *  o              (num_q_tokens, num_heads, 512) bfloat16, written
 *                 (round to nearest even).
 *  qo_indptr      (batch+1) int32: request b owns query tokens
 *                 [qo_indptr[b], qo_indptr[b+1]); qo_indptr[batch] must equal
 *                 num_q_tokens and every request at most max_seqlen_q tokens.
 *  kv_indptr      (batch+1) int32 offsets into kv_indices; deltas are each
 *                 request's KV length in tokens.
 *  kv_indices     (kv_indices_len) int32 pool entry of every cached token.
 *  kv_last_page_lens (batch) int32, all ones for page_size 1; not read
 *                 (may be NULL).
 *  sm_scale       host float, the softmax scale (1/sqrt(192) for K3).
 *  q_scale, kv_scale  device fp32 scalars (0-d tensors); real = stored*scale.
 *                 NULL means 1.0.
 *  return_lse, lse  if return_lse != 0, lse (num_q_tokens, num_heads) fp32
 *                 receives ln(sum_i exp(s_i)) of each row; it may be NULL
 *                 otherwise.
 *  workspace      device scratch of at least
 *                 mla_decode_workspace_bytes(batch, num_q_tokens, num_heads,
 *                 max_seqlen_q) bytes, 256-byte aligned; contents on entry do
 *                 not matter (every byte read is written earlier in the call).
 *
 * Query token j of a request with qlen tokens and n cached entries sees the
 * first n - (qlen - 1 - j) entries (bottom-right causal alignment for
 * multi-token verification).  A row that sees nothing gets o = 0 and
 * lse = -inf.  Supported: q_dtype == kv_dtype, either FP8_E4M3FN or BF16;
 * num_heads a positive multiple of 16; 1 <= max_seqlen_q <= 64.
 */
mla_status mla_decode(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                      int64_t pool_entries, void* o, const int32_t* qo_indptr,
                      const int32_t* kv_indptr, const int32_t* kv_indices,
                      int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                      int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                      const float* q_scale, const float* kv_scale, int return_lse, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments and results as mla_decode, without the workspace.  The call
 * uses a fixed scratch array that the library holds on each device for the
 * life of the process (mla_decode_noalloc_scratch_bytes(), 20 MiB), and
 * allocates nothing, on the host or the device.
 *
 *  - A call whose workspace (mla_decode_workspace_bytes for its shape) exceeds
 *    the scratch returns MLA_ERR_SCRATCH_TOO_SMALL and enqueues nothing.  On
 *    MI355X (256 compute units) that admits standard-mode calls
 *    (num_heads / 16 * max_seqlen_q < 4, e.g. the 16-head single-token call)
 *    with up to about 250,000 (token, head group) units, and no group-mode call.
 *  - The scratch is shared by every call on one device, and no byte of it needs
 *    to be cleared between calls (each call writes every byte it reads), but
 *    calls that overlap on one device (concurrent streams) race on it: order
 *    them, or use mla_decode with separate workspaces.
 *  - The first call on a device looks up the scratch's device address
 *    (hipGetSymbolAddress) with that device current; an error there returns
 *    MLA_ERR_HIP.
 */
mla_status mla_decode_noalloc(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                              int64_t pool_entries, void* o, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, const int32_t* kv_indices,
                              int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                              int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                              const float* q_scale, const float* kv_scale, int return_lse,
                              float* lse, void* stream);

/* Bytes of the fixed scratch mla_decode_noalloc uses on each device. */
size_t mla_decode_noalloc_scratch_bytes(void);

/*
 * mla_decode with an explicit number of worker workgroups (0 = the library's
 * choice: one per compute unit).  The KV work is cut into
 * `num_workers` equal contiguous ranges; results agree with mla_decode within
 * rounding.  The workspace must hold mla_decode_workspace_bytes_ex(...,
 * num_workers) bytes.
 */
mla_status mla_decode_ex(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                         int64_t pool_entries, void* o, const int32_t* qo_indptr,
                         const int32_t* kv_indptr, const int32_t* kv_indices,
                         int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                         int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                         const float* q_scale, const float* kv_scale, int return_lse,
                         float* lse, void* workspace, size_t workspace_bytes, int num_workers,
                         void* stream);

size_t mla_decode_workspace_bytes_ex(int batch, int num_q_tokens, int num_heads,
                                     int max_seqlen_q, int num_workers);

/*
 * mla_decode over a paged cache with pages of page_size entries ("[Kimi-K3
 * MLA TP8] MLA performance", Sec. 3: the entry point's page_size and
 * kv_last_page_lens arguments; Sec. 5.2: the captured call runs with
 * page_size 1, and the allocator hands out blocks of 128 slots).
 *
 * Arguments as for mla_decode, except:
 *  kv_pool        (pool_entries, 576) rows, i.e. (pool_entries / page_size)
 *                 pages of page_size consecutive rows; page k holds rows
 *                 [k * page_size, (k + 1) * page_size).
 *  kv_indptr      (batch+1) int32 offsets into kv_indices, in pages.
 *  kv_indices     (kv_indices_len) int32 page numbers, request by request.
 *  kv_last_page_lens (batch) int32 device array: slots used in each request's
 *                 last page, 1..page_size.
 *  page_size      a power of two, 1..4096; for 1 the call is mla_decode and
 *                 kv_last_page_lens is not read.
 * Request b holds (pages_b - 1) * page_size + kv_last_page_lens[b] entries
 * (none if it has no pages); entry i is pool row
 * kv_indices[kv_indptr[b] + i / page_size] * page_size + i % page_size.  A
 * last-page length outside 1..page_size is clamped to it.  For
 * page_size > 1, pool_entries must be a multiple of page_size and at most
 * 2^31 - 1 (MLA_ERR_BAD_SHAPE), and kv_last_page_lens must not be NULL
 * (MLA_ERR_NULL_POINTER).  Same workspace, types, shapes and masking as
 * mla_decode.
 */
mla_status mla_decode_paged(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                            int64_t pool_entries, void* o, const int32_t* qo_indptr,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int64_t kv_indices_len, const int32_t* kv_last_page_lens,
                            int page_size, int batch, int num_q_tokens, int num_heads,
                            int max_seqlen_q, float sm_scale, const float* q_scale,
                            const float* kv_scale, int return_lse, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * One shard of decode context parallelism (DCP): "Kimi K3 on AMD Instinct
 * MI355X ...", Sec. "1. Cache: keep conversation state available for reuse"
 * (each of the GPUs keeps one eighth of the cached positions, runs the
 * exchanged queries of all heads against them, and the partial answers are
 * merged with softmax weights; multi-token verification under DCP), with the
 * shard arguments of the entry point in "[Kimi-K3 MLA TP8] MLA performance",
 * Sec. 3 (g_kv_indptr, cp_world_size, cp_rank).
 *
 * Arguments as for mla_decode, where kv_indptr / kv_indices describe this
 * shard's entries, plus:
 *  g_kv_indptr    (batch+1) int32 device offsets of the requests' full
 *                 (all-shard) lists: N_b = g_kv_indptr[b+1] - g_kv_indptr[b]
 *                 positions in total.
 *  cp_world_size  shards the positions are dealt over, 1..1024.
 *  cp_rank        this shard, 0 <= cp_rank < cp_world_size.
 *  o_dtype        MLA_DTYPE_BF16: o is (num_q_tokens, num_heads, 512) bf16, as
 *                 for mla_decode.  MLA_DTYPE_FP32: o is the same shape in fp32,
 *                 and the call's internal split partials are kept in fp32 too,
 *                 so a shard's answer reaches the merge unrounded; the merge
 *                 (mla_merge_partials with FP32 parts) then rounds once, to the
 *                 final bf16.  Any other value returns MLA_ERR_BAD_DTYPE.
 * Layout (caller's contract): positions are dealt round-robin, so this
 * shard's i-th entry of request b is the entry at full-list position
 * cp_rank + i * cp_world_size; it holds ceil((N_b - cp_rank) /
 * cp_world_size) entries.  Query token j of a request with qlen tokens sees
 * the local entries whose full-list position is <= N_b - qlen + j (the
 * bottom-right causal rule of mla_decode applied to full-list positions); a
 * row that sees nothing gets o = 0 and lse = -inf, which
 * mla_merge_partials gives weight 0.  With return_lse set, merging the
 * cp_world_size shards' (o, lse) with mla_merge_partials gives the result of
 * mla_decode over the full lists.  Same workspace as mla_decode; same
 * supported types and shapes.  A NULL g_kv_indptr returns
 * MLA_ERR_NULL_POINTER, a cp_world_size or cp_rank out of range
 * MLA_ERR_BAD_SHAPE.
 */
mla_status mla_decode_dcp(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                          int64_t pool_entries, void* o, const int32_t* qo_indptr,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          int64_t kv_indices_len, const int32_t* kv_last_page_lens, int batch,
                          int num_q_tokens, int num_heads, int max_seqlen_q, float sm_scale,
                          const float* q_scale, const float* kv_scale, int return_lse,
                          float* lse, const int32_t* g_kv_indptr, int cp_world_size,
                          int cp_rank, int o_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * LSE-weighted merge of partial answers over disjoint KV shards (the DCP
 * merge of the blog's Sec. 1; the same math combines the decode's own splits).
 *
 *  o_parts    (num_parts, num_q_tokens, num_heads, 512) of parts_dtype
 *             (BF16 or FP32), each shard's normalised output.
 *  lse_parts  (num_parts, num_q_tokens, num_heads) fp32, each shard's lse;
 *             -inf marks an empty shard: its o_parts row is read but given
 *             weight 0 by a select, so its contents (even NaN) never matter.
 *  o          (num_q_tokens, num_heads, 512) bf16, written.
 *  lse        (num_q_tokens, num_heads) fp32, written if not NULL.
 * For each row: M = max_s lse_s, L = M + ln sum_s exp(lse_s - M),
 * o = sum_s exp(lse_s - L) o_s, lse = L; a row empty in every shard gets
 * o = 0, lse = -inf.
 */
mla_status mla_merge_partials(const void* o_parts, int parts_dtype, const float* lse_parts,
                              int num_parts, int num_q_tokens, int num_heads, void* o,
                              float* lse, void* stream);

/* Static, human-readable name of a status code. */
const char* mla_status_string(int status);

/*
 * Device-side check of a decode call's index arguments, the parts of the call
 * the host validation cannot see (Sec. 4.1 "Arguments" and Sec. 5.2: CSR
 * qo_indptr / kv_indptr over a list of pool entries, or of page numbers for a
 * paged cache).  Enqueues, on `stream`, a write of 0 to *status followed by a
 * pass that ORs in one bit per kind of violation found:
 *   MLA_CHECK_QO_INDPTR      qo_indptr[0] != 0, a decrease, a request with
 *                            more than max_seqlen_q tokens, or
 *                            qo_indptr[batch] != num_q_tokens;
 *   MLA_CHECK_KV_INDPTR      kv_indptr[0] != 0, a decrease, or
 *                            kv_indptr[batch] > kv_indices_len;
 *   MLA_CHECK_KV_INDEX       an entry of kv_indices[0 .. kv_indptr[batch])
 *                            outside [0, pool_entries / page_size);
 *   MLA_CHECK_LAST_PAGE_LEN  (when kv_last_page_lens is given) page_size 1:
 *                            a length other than 1 (0 allowed for an empty
 *                            request); page_size > 1: a request with pages
 *                            whose length is outside 1 .. page_size;
 *   MLA_CHECK_DCP_LENGTHS    (when g_kv_indptr is given, as for
 *                            mla_decode_dcp) g_kv_indptr[0] != 0, a
 *                            decrease, or a request whose local list does not
 *                            hold exactly its share of positions (those p <
 *                            its global length with p mod cp_world_size ==
 *                            cp_rank).
 * 0 means none found.  Inputs are read only within the sizes passed (batch + 1
 * indptr entries, kv_indices_len indices), whatever they hold.  For
 * mla_decode_cascade, check the suffix lists as the batch and the prefix as a
 * batch of one request.  The call itself allocates nothing and does not
 * synchronise; read *status after the stream has reached it.
 *
 *  status  device int, written by the check (caller-owned).
 *  page_size 1, 2, 4, ..., 4096; pool_entries >= 1 (rows of the pool).
 *  g_kv_indptr may be NULL (then cp_world_size and cp_rank are ignored).
 *
 * Errors (nothing enqueued): MLA_ERR_NULL_POINTER (qo_indptr, kv_indptr,
 * status, or kv_indices with kv_indices_len > 0), MLA_ERR_BAD_SHAPE (batch <
 * 1, num_q_tokens < 0, max_seqlen_q < 1, kv_indices_len < 0, pool_entries <
 * 1, page_size not a power of two in range, cp_rank outside
 * 0 .. cp_world_size - 1).  MLA_ERR_HIP if the launch fails.
 */
#define MLA_CHECK_QO_INDPTR 1
#define MLA_CHECK_KV_INDPTR 2
#define MLA_CHECK_KV_INDEX 4
#define MLA_CHECK_LAST_PAGE_LEN 8
#define MLA_CHECK_DCP_LENGTHS 16
mla_status mla_check_inputs(const int32_t* qo_indptr, const int32_t* kv_indptr,
                            const int32_t* kv_indices, int64_t kv_indices_len,
                            const int32_t* kv_last_page_lens, int page_size,
                            int64_t pool_entries, int batch, int num_q_tokens, int max_seqlen_q,
                            const int32_t* g_kv_indptr, int cp_world_size, int cp_rank,
                            int* status, void* stream);

/*
 * Shared-prefix (cascade) decode ("[Kimi-K3 MLA TP8] MLA performance",
 * ROCm/aiter issue 4541, Sec. 5.4 on reuse of the prefix shared by the
 * batch's requests): the same result as mla_decode when request b's entry
 * list is prefix_indices (shared by every request) followed by its own
 * suffix_indices[suffix_indptr[b] .. suffix_indptr[b+1]).  The shared rows are
 * gathered once for eight row groups (all tokens, all heads) instead of once
 * per request and head group.
 *
 *  Arguments as for mla_decode, with kv_indptr / kv_indices replaced by
 *  prefix_indices (prefix_len) int32 and suffix_indptr (batch+1) /
 *  suffix_indices (suffix_indices_len) int32, all device memory.
 *  Supported: FP8 q and KV only.  num_heads may be any count from 1 to 4,096:
 *  the query rows (token, head) are packed 16 to a matrix tile whatever the
 *  head count, so a model's 12 real heads are passed unpadded, q
 *  (num_q_tokens, 12, 576) and o (num_q_tokens, 12, 512), and no tile row is
 *  spent on padding ("[Kimi-K3 MLA TP8] MLA performance", Sec. 5.1: with 12
 *  heads padded to 16, a quarter of the Q tile is zero).  Causal draft tokens: every request's suffix
 *  must hold at least qlen_b - 1 entries (a token's masked entries then all
 *  lie in the suffix); this is the caller's contract, not checked.
 *  workspace: at least mla_decode_cascade_workspace_bytes(...) bytes.
 *  Runs three kernels on `stream`: one group-mode decode launch that takes
 *  the prefix pass (every token against the shared prefix) and the suffix
 *  pass (each request against its own suffix) as one balanced work stream,
 *  writing fp32 o / lse for each pass into the workspace; its split combine;
 *  and an LSE merge of the two passes into o / lse.
 */
size_t mla_decode_cascade_workspace_bytes(int batch, int num_q_tokens, int num_heads,
                                          int max_seqlen_q);

mla_status mla_decode_cascade(const void* q, int q_dtype, const void* kv_pool, int kv_dtype,
                              int64_t pool_entries, void* o, const int32_t* qo_indptr,
                              const int32_t* prefix_indices, int64_t prefix_len,
                              const int32_t* suffix_indptr, const int32_t* suffix_indices,
                              int64_t suffix_indices_len, int batch, int num_q_tokens,
                              int num_heads, int max_seqlen_q, float sm_scale,
                              const float* q_scale, const float* kv_scale, int return_lse,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The step before the decode ("[Kimi-K3 MLA TP8] MLA performance", Sec. 3:
 * the decode's q is produced by one fused op that also writes the step's new
 * cache entry into the pool the decode reads; Sec. 2 geometry: 512 latent +
 * 64 rope dims).  For every token t:
 *   q_out[t, h]  = fp8((q_latent[t, h] ++ rope(q_pe[t, h], positions[t])) / q_scale)
 *                  for h < num_heads, all-zero codes for the pad heads
 *                  num_heads <= h < num_heads_pad;
 *   kv_pool[slot_mapping[t]] = fp8((k_latent[t] ++ rope(k_pe[t], positions[t])) / kv_scale)
 *                  unless slot_mapping[t] is negative or >= pool_entries (no write).
 *
 *  q_latent      (num_q_tokens, num_heads, 512) bf16: the absorbed q.
 *  q_pe          (num_q_tokens, num_heads, 64) bf16: q's rope dims before rotation.
 *  k_latent      (num_q_tokens, 512) bf16, k_pe (num_q_tokens, 64) bf16: the
 *                tokens' new cache entries before rotation and quantisation.
 *  positions     (num_q_tokens) int32, clamped to [0, max_pos).
 *  cos_sin       (max_pos, 64) fp32: cos of the 32 rotation angles of a
 *                position, then their sin.
 *  rope_style    0: dims (2j, 2j+1) rotate by angle j; 1: dims (j, j+32) do.
 *                A rotated dim is x_a cos - x_b sin or x_b cos + x_a sin with
 *                every product and sum rounded to fp32 (no fused multiply-add).
 *  q_out         (num_q_tokens, num_heads_pad, 576) fp8 e4m3fn, written.
 *  kv_pool       (pool_entries, 576) fp8 e4m3fn; only the slots named are written.
 *  q_scale, kv_scale  device fp32 scalars (NULL = 1.0); stored = real / scale,
 *                divided in fp32 (correctly rounded).
 * fp8 is round-to-nearest-even with finite values beyond 448 saturating to
 * +-448 (NaN stays NaN).  Tokens writing the same slot race.  Errors: NULL
 * pointers; num_q_tokens, num_heads or max_pos < 1, num_heads_pad <
 * num_heads, rope_style not 0 or 1 (MLA_ERR_BAD_SHAPE).
 */
mla_status mla_rope_quant_cache(const void* q_latent, const void* q_pe, const void* k_latent,
                                const void* k_pe, const int32_t* positions, const float* cos_sin,
                                int max_pos, int rope_style, void* q_out, int num_q_tokens,
                                int num_heads, int num_heads_pad, void* kv_pool,
                                int64_t pool_entries, const int32_t* slot_mapping,
                                const float* q_scale, const float* kv_scale, void* stream);

/*
 * The step after the decode ("[Kimi-K3 MLA TP8] MLA performance", Sec. 3: a
 * separate batched GEMM maps the 512-dim latent output back to v_head_dim;
 * Sec. 2: v_head_dim = 128):
 *   out[t, h, :] = o_latent[t, h, :] . w_uv[h]^T   for h < num_heads
 * with fp32 accumulation, rounded to bf16 (nearest even).
 *
 *  o_latent  (num_q_tokens, num_heads_pad, 512) bf16: mla_decode's o (the
 *            pad heads are not read).
 *  w_uv      (num_heads, 128, 512) bf16: each head's (out, in) weight.
 *  out       (num_q_tokens, num_heads, 128) bf16, written.
 * Errors: NULL pointers; num_q_tokens < 1, num_heads outside 1..65535 or
 * num_heads_pad < num_heads (MLA_ERR_BAD_SHAPE).
 */
mla_status mla_latent_to_v(const void* o_latent, const void* w_uv, void* out, int num_q_tokens,
                           int num_heads, int num_heads_pad, void* stream);

/*
 * One decode step of an MLA layer with the steps either side folded in
 * ("[Kimi-K3 MLA TP8] MLA performance", Sec. 3: the fused rope / concat /
 * fp8 op that produces q and writes the step's new cache entries, the decode,
 * and the batched GEMM to v_head_dim; Sec. 2 geometry).  The same results as
 *   mla_rope_quant_cache(q_latent, q_pe, k_latent, k_pe, positions, cos_sin,
 *                        max_pos, rope_style, q_fp8, num_q_tokens, num_heads,
 *                        num_heads_pad, kv_pool, pool_entries, slot_mapping,
 *                        q_scale, kv_scale);
 *   mla_decode(q_fp8, FP8, kv_pool, FP8, ..., o_latent, ..., num_heads_pad, ...);
 *   mla_latent_to_v(o_latent, w_uv, out, num_q_tokens, num_heads, num_heads_pad);
 * in three launches instead of four: a prologue kernel, one block per decode
 * worker, does a share of the rope / fp8 / cache-write step (q rows into the
 * workspace) and computes that worker's plan; the decode kernel starts from
 * the stored plan; one kernel after it merges split rows and applies w_uv.  The new cache entries, o_latent, lse and out equal the
 * three-call chain's bit for bit.
 *
 *  Arguments as for mla_rope_quant_cache (num_heads = the real heads,
 *  num_heads_pad a positive multiple of 16), mla_decode (FP8 cache, page_size
 *  1) and mla_latent_to_v, all device memory except the sizes and sm_scale.
 *  o_latent (num_q_tokens, num_heads_pad, 512) bf16 is written as mla_decode's
 *  o; out (num_q_tokens, num_heads, 128) bf16 as mla_latent_to_v's.
 *  Contract (not checked): token j of a request with qlen tokens and n
 *  entries has its new entry listed at position n - qlen + j of the request's
 *  kv_indices, and that index equals slot_mapping of the token (or the token's
 *  slot is negative or >= pool_entries, and nothing is written); other rows
 *  of the pool are not written during the call.
 *  workspace: at least mla_decode_step_workspace_bytes(batch, num_q_tokens,
 *  num_heads_pad, max_seqlen_q) bytes (the decode's workspace, the fp8 q
 *  rows and the workers' plans); contents on entry do not matter.
 * Errors: NULL pointers (MLA_ERR_NULL_POINTER); num_heads_pad not a positive
 * multiple of 16 (MLA_ERR_UNSUPPORTED); the shape checks of the three calls
 * (MLA_ERR_BAD_SHAPE); a small workspace (MLA_ERR_WORKSPACE_TOO_SMALL).
 */
size_t mla_decode_step_workspace_bytes(int batch, int num_q_tokens, int num_heads_pad,
                                       int max_seqlen_q);

mla_status mla_decode_step(const void* q_latent, const void* q_pe, const void* k_latent,
                           const void* k_pe, const int32_t* positions, const float* cos_sin,
                           int max_pos, int rope_style, const int32_t* slot_mapping,
                           void* kv_pool, int64_t pool_entries, const int32_t* qo_indptr,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t kv_indices_len, int batch, int num_q_tokens, int num_heads,
                           int num_heads_pad, int max_seqlen_q, float sm_scale,
                           const float* q_scale, const float* kv_scale, const void* w_uv,
                           void* o_latent, void* out, int return_lse, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host mirror of the work planner, for tests: given host copies of qo_indptr
 * and kv_indptr, fill `out` (capacity `out_cap` pieces, 8 int64 each:
 * worker, token, head_group, kv_begin, kv_end, unit_len, slot, is_complete)
 * with the pieces every worker processes, in worker order.  slot is the
 * partial-answer slot (-1 for complete pieces).  g_kv_indptr (host, may be
 * NULL), cp_world_size and cp_rank describe a DCP shard as for
 * mla_decode_dcp (NULL, 1, 0 without DCP).  Returns the number of pieces
 * (which may exceed out_cap; only out_cap are written), or -1 on bad input.
 */
int64_t mla_plan_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                      const int32_t* g_kv_indptr, int batch, int num_heads, int num_workers,
                      int cp_world_size, int cp_rank, int64_t* out, int64_t out_cap);

/*
 * Host mirror of the group-mode planner (the fp8 path when num_heads / 16 *
 * max_seqlen_q >= 4), for tests.  A unit is 8 consecutive row groups
 * rg = j * (num_heads / 16) + g of one request (token j, head group g), as
 * long as the last of them sees.  Records as for mla_plan_host but with
 * columns: worker, request, unit, kv_begin, kv_end, unit_len, slot_base,
 * is_complete; slot_base is the first of the piece's 8 partial slots (one per
 * row group), -1 for complete pieces.  causal = 0 lets every token see all of
 * its request's entries (the cascade's prefix pass).  DCP arguments and
 * return convention as for mla_plan_host.
 */
int64_t mla_plan_groups_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* g_kv_indptr, int batch, int num_heads,
                             int num_workers, int causal, int cp_world_size, int cp_rank,
                             int64_t* out, int64_t out_cap);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
