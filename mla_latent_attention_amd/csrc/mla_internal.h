// mla_internal.h - parameters shared between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla_plan.h"

namespace mla {

// A decode worker's share as the planner leaves it (the layer step's prologue
// kernel stores one per worker): stream range [p0, p1) and the cursor at p0;
// ok = 0: nothing to do.
struct WorkerPlan {
  int64_t p0, p1;
  Cursor c;
  int ok;
};

struct DecodeParams {
  const uint8_t* q;         // (T, H, 576) elements of the storage type
  const uint8_t* kv;        // (pool_entries, 576)
  int64_t pool_entries;
  uint16_t* o;              // (T, H, 512) bf16
  float* o32;               // if set, o is written here in fp32 instead (cascade passes,
                            // DCP shards asked for fp32 output)
  const int32_t* qo_indptr;  // (B+1)
  const int32_t* kv_indptr;  // (B+1)
  const int32_t* kv_indices;
  int kv_indices_len;
  int batch;
  int num_tokens;
  int num_heads;
  float sm_scale;
  const float* q_scale;     // device scalar or nullptr (1.0)
  const float* kv_scale;    // device scalar or nullptr (1.0)
  float* lse;               // (T, H) or nullptr
  float* part_o;            // workspace: (slots*num_workers, 16, 512) split partials
  int part_fp32 = 0;        // 1: partials in fp32; 0: fp32 for a bf16 cache, fp16 for an
                            // fp8 one (see the workspace layout below)
  float* part_lse;          // workspace: (slots*num_workers, 16) fp32
  int4* desc;               // workspace: (tokens * head groups) split-unit descriptors
  int2* desc_rows = nullptr;  // group mode: {first token, first head * 32 + rows} of each
                              // descriptor's row group (rows 1..16; packed heads)
  int num_workers;
  int causal;               // 1: bottom-right causal; 0: every token of a request sees all
                            // of its entries
  const int32_t* g_kv_indptr = nullptr;  // (B+1) full-list offsets under DCP, or nullptr
  int cp_size = 1;                        // DCP shards (1 without DCP)
  int cp_rank = 0;                        // this shard
  const int32_t* last_page_lens = nullptr;  // (B) paged caches: used slots of the last page
  int page_shift = 0;                     // log2(page_size); 0: kv_indices name entries
  // Shared-prefix (cascade) call in one group-mode launch (the ReqSource
  // cascade view): entries [0, cascade_prefix) come from kv_indices (the
  // prefix), the rest from kv_indices2 (the suffixes); -1: off.
  int cascade_prefix = -1;
  const int32_t* kv_indices2 = nullptr;
  // Layer step (mla_decode_step; only its prologue kernel reads these): the
  // rope / fp8 / cache-write step's inputs and outputs.
  const uint16_t* q_latent = nullptr;  // (T, real_heads, 512) bf16
  const uint16_t* q_pe = nullptr;      // (T, real_heads, 64) bf16, before rotation
  const uint16_t* k_latent = nullptr;  // (T, 512) bf16: the tokens' new entries
  const uint16_t* k_pe = nullptr;      // (T, 64) bf16, before rotation
  const int32_t* positions = nullptr;  // (T), clamped to [0, max_pos)
  const float* cos_sin = nullptr;      // (max_pos, 64): 32 cos then 32 sin
  int max_pos = 0;
  int rope_style = 0;                  // 0: dims (2j, 2j+1) rotate; 1: dims (j, j+32)
  int real_heads = 0;                  // heads of q_latent / q_pe; the rest are padding
  const int32_t* slot_mapping = nullptr;  // (T) pool slot of each token's new entry
  uint8_t* kv_out = nullptr;           // the pool again, writable
  uint8_t* q_out = nullptr;            // (T, H, 576) fp8 q built by the call (q reads it)
  WorkerPlan* plans = nullptr;         // (num_workers) plans of the planned decode build
};

// The planner's view of the call's requests.  Builds without kPaged /
// kCascade drop those fields as constants.
template <bool kPaged, bool kCascade = false>
__host__ __device__ inline ReqSource source_of(const DecodeParams& p) {
  ReqSource s;
  s.qo = p.qo_indptr;
  s.kvp = p.kv_indptr;
  s.gkvp = kCascade ? nullptr : p.g_kv_indptr;  // a cascade call is never a DCP shard
  s.kv_cap = p.kv_indices_len;
  s.T = p.num_tokens;
  s.causal = p.causal;
  s.cp_size = kCascade ? 1 : p.cp_size;
  s.cp_rank = kCascade ? 0 : p.cp_rank;
  s.lpl = kPaged ? p.last_page_lens : nullptr;
  s.page_shift = kPaged ? p.page_shift : 0;
  s.prefix_len = kCascade ? p.cascade_prefix : -1;
  return s;
}


// Workspace layout for `num_workers` workers, `slots` partial slots per worker
// and `num_units` = tokens * head groups (every byte the kernels read is
// written earlier in the same call, so no clearing is ever needed):
//   desc     (num_units) int4 per row group {first worker, last worker, slot
//            of the first worker, 1} for a row group split over several
//            workers, w = 0 else; then one spare entry (index num_units) that
//            takes the stores of lanes holding no descriptor, so that the
//            group kernel writes descriptors without a divergent branch
//   part_o   (slots * num_workers, 16, 512) fp32 partial outputs (calls on an
//            fp8 cache store them as fp16 divided by kv_scale, at the same
//            element indices, in the first half of the region, unless
//            part_fp32 is set)
//            (then, group mode, desc_rows: int2 per entry, the output rows of
//            the entry's row group, written with its descriptor)
//   part_lse (slots * num_workers, 16) fp32 partial lse
constexpr int kMaxWorkers = 1 << 16;
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t desc_entries_bytes(int64_t num_units) { return align256(size_t(num_units + 1) * 16); }
inline size_t desc_bytes(int64_t num_units) {
  return desc_entries_bytes(num_units) + align256(size_t(num_units + 1) * 8);
}
inline size_t part_o_bytes(int num_workers, int slots) {
  return align256(size_t(slots) * num_workers * 16 * 512 * 4);
}
inline size_t part_lse_bytes(int num_workers, int slots) {
  return align256(size_t(slots) * num_workers * 16 * 4);
}
inline size_t workspace_bytes(int num_workers, int64_t num_units, int slots) {
  return desc_bytes(num_units) + part_o_bytes(num_workers, slots) +
         part_lse_bytes(num_workers, slots);
}

// Points the call's descriptors, partials and their lse into workspace ws.
inline void set_workspace(DecodeParams& p, char* ws, int64_t num_units, int num_workers, int slots) {
  p.desc = reinterpret_cast<int4*>(ws);
  p.desc_rows = reinterpret_cast<int2*>(ws + desc_entries_bytes(num_units));
  p.part_o = reinterpret_cast<float*>(ws + desc_bytes(num_units));
  p.part_lse = reinterpret_cast<float*>(ws + desc_bytes(num_units) +
                                        part_o_bytes(num_workers, slots));
}

// kv_dtype: 0 = fp8 e4m3fn, 1 = bf16.  group_mode selects the group-mode
// kernels (fp8 only; the workspace then has 16 slots per worker).
hipError_t launch_decode(const DecodeParams& p, int kv_dtype, bool group_mode, hipStream_t stream);
// The group-mode decode kernel alone (mla_decode_groups.hip).
hipError_t launch_decode_groups(const DecodeParams& p, hipStream_t stream);

hipError_t launch_merge(const void* o_parts, int parts_fp32, const float* lse_parts, int num_parts,
                        int64_t rows, uint16_t* o, float* lse, hipStream_t stream);
// The fused layer step: the fused fp8 decode (standard kernel) and the
// combine + latent -> v kernel (mla_decode.hip).
hipError_t launch_decode_step(const DecodeParams& p, const uint16_t* w_uv, uint16_t* vout,
                              hipStream_t stream);

// Device-side check of a call's index arguments (mla_check.hip): bits of
// MLA_CHECK_* OR-ed into *status (cleared first).
struct CheckParams {
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* last_page_lens;  // nullptr: not checked
  const int32_t* g_kv_indptr;     // nullptr: not a DCP shard
  int64_t kv_indices_len;
  int64_t pool_entries;
  int batch;
  int num_q_tokens;
  int max_seqlen_q;
  int page_shift;
  int cp_size;
  int cp_rank;
  int* status;
};
hipError_t launch_check_inputs(const CheckParams& c, hipStream_t stream);

// Steps either side of the decode (mla_surround.hip).
hipError_t launch_rope_quant_cache(const uint16_t* q_latent, const uint16_t* q_pe,
                                   const uint16_t* k_latent, const uint16_t* k_pe,
                                   const int32_t* positions, const float* cos_sin, int max_pos,
                                   int rope_style, uint8_t* q_out, int T, int num_heads,
                                   int num_heads_pad, uint8_t* kv_pool, int64_t pool_entries,
                                   const int32_t* slot_mapping, const float* q_scale,
                                   const float* kv_scale, hipStream_t stream);
hipError_t launch_latent_to_v(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* out, int T,
                              int H, int H_pad, hipStream_t stream);

}  // namespace mla
