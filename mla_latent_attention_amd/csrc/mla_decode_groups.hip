// mla_decode_groups.hip - group-mode latent MLA decode for gfx950 (fp8).
//
// Same computation as mla_decode.hip ("[Kimi-K3 MLA TP8] MLA performance",
// ROCm/aiter issue 4541, Sec. 2 "K3 MLA geometry"), for calls whose requests
// hold several row groups (query token x 16 heads): many heads, or several
// draft tokens checked at once.  The DCP share of "Kimi K3 on AMD Instinct
// MI355X: vLLM Serving Matches NVIDIA HGX B300 Throughput per GPU on AgentX"
// (Sec. "1. Cache: keep conversation state available for reuse": all 96 heads
// of 4 tokens over one rank's slice of the history) has 24 row groups per
// request; with one unit per row group every cached row would be gathered 24
// times.
//
// Design (our own):
//   * A unit is four consecutive row groups of one request (mla_plan.h, group
//     mode); workers take equal, boundary-snapped shares of the unit stream as
//     in the standard mode.
//   * The four waves of a workgroup own the unit's four row groups and walk the
//     same KV range.  Tiles of 32 rows are gathered once by all 256 threads
//     with direct global->LDS loads (each lane 16 consecutive bytes of a row)
//     into a three-tile LDS ring with a 592-byte row stride; two tiles are in
//     flight while one is consumed.
//   * Two workgroups share a CU (two waves per SIMD, 250 registers each), so one
//     wave's softmax and LDS latency overlap the other wave's MFMAs.
//   * Each wave computes its row group over the shared tile: S^T = K.Q^T on
//     v_mfma_f32_16x16x32_fp8_fp8 with K read from LDS and q in registers, the
//     online softmax (masking the entries its token may not see), and
//     O^T += V^T.P^T on bf16 MFMA, with the V^T operand read from the
//     row-major tile by the LDS transpose read (ds_read_b64_tr_b8) and widened
//     exactly from fp8, and P in bf16: one MFMA per 16 dims and 32 rows
//     instead of two fp8 ones (P as hi + lo).  Every wave writes its own o (or
//     partial): there is no cross-wave merge.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

constexpr int kGTile = 32;                                    // KV rows per shared tile
constexpr int kGBlocks = kGTile / 16;                         // 16-row S^T blocks per tile
constexpr int kGHalves = kGTile / 32;                         // 32-row P.V steps per tile
constexpr int kGIdxSeg = 2048;                                // kv_indices staged per segment
constexpr int kGChunks = kRowDim / 16;                        // 16-byte chunks per row (36)
constexpr int kGRowSlots = kGChunks + 1;                      // + one pad slot per staged row
constexpr int kGStride = 16 * kGRowSlots;                     // LDS bytes per staged row (592)
constexpr int kGLoads = 5;                                    // load instructions per wave per tile
constexpr int kGTileBytes = kWaves * kGLoads * 64 * 16;       // 20,480 (>= 32 rows x 592)
constexpr int kGRing = 3;                                     // tiles in the LDS ring
static_assert(kGTile * kGStride <= kGTileBytes, "a tile's rows must fit its ring slot");
constexpr int kGSlotsPerPiece = kGroupsPerUnit;               // one partial slot per row group

// The ring's three tiles are separate LDS objects, always named statically:
// the compiler then knows which tile a direct-to-LDS load writes and which one
// an LDS read reads, and waits only for the loads of the tile being read
// (through one array it must wait for every outstanding load before any read).
__shared__ __attribute__((aligned(16))) uint8_t g_ring0[kGTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_ring1[kGTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_ring2[kGTileBytes];

template <int kB>
__device__ __forceinline__ uint8_t* ring() {
  if constexpr (kB == 0) return g_ring0;
  if constexpr (kB == 1) return g_ring1;
  return g_ring2;
}

struct alignas(16) GroupShared {
  int32_t idx[kGIdxSeg];  // kv_indices of the current segment of the piece
  int64_t red[kWaves];
  int pb[2];
  int64_t pcum[2];
};

typedef int v8i_t __attribute__((ext_vector_type(8)));

// q row lane%16 of the wave's row group, as the B operands of five
// 16x16x128 MFMA steps.  Step c < 4 (latent dims 128c .. 128c + 127): the
// lane holds dims 128c + 16gq + [0, 16) and 128c + 64 + 16gq + [0, 16)
// (gq = lane/16), the same bytes it reads of each K row, so the contraction
// pairs every q dim with the same K dim whatever order the instruction
// assigns to a lane's 32 bytes.  Step 4: rope dims 512 + 16gq + [0, 16), then
// 16 zero bytes (the K operand's matching half is any finite row data).
struct GroupQ {
  v8i_t part[5];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; all-ones leaves a counter unchecked).
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kVmcntOneTileOut = waitcnt_vm(kGLoads);  // all but the last tile's loads done
constexpr int kVmcntNone = waitcnt_vm(0);

__device__ __forceinline__ void uniformize(GCursor& c) {
  c.b = uniform(c.b);
  c.u = uniform(c.u);
  c.k = uniform(c.k);
  c.r.kv_base = uniform(c.r.kv_base);
  c.r.n = uniform(c.r.n);
  c.r.q_base = uniform(c.r.q_base);
  c.r.qlen = uniform(c.r.qlen);
}

__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// One direct global->LDS load: lane l's 16 bytes at `src` land at LDS address
// lds + 16l (the LDS base is taken from m0).  Written as inline assembly so the
// compiler does not track it: its own bookkeeping would wait for every such
// load before any LDS read.  The waits for these loads are explicit (a vmcnt
// wait before the barrier that publishes a tile); the compiler's own waits for
// its loads stay correct because the counter completes in order.
__device__ __forceinline__ void lds_dma_16(const uint8_t* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}

// LDS address (byte offset in the workgroup's LDS) of a shared object.
__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// Gathers tile `tile` of the current segment (rows at positions tile*32 + r,
// clamped to the segment's last row) straight into ring tile kB
// with global_load_lds_dwordx4: instruction k of wave wv writes LDS bytes
// [(5wv + k) * 1024, +1024), lane l the 16 bytes of slot s = 64(5wv + k) + l,
// which is staged row s / 37, chunk s % 37.  Lanes on a pad slot (chunk 36) or
// past the last row load a duplicate of a real chunk that is never read.
// Every load is unconditional, so the outstanding-load count is static.
template <int kB>
__device__ __forceinline__ void group_issue(const DecodeParams& p, const int32_t* sidx, int rows,
                                            int tile, int wv, int lane) {
  const uint32_t dst = lds_addr_of(ring<kB>()) + 1024u * (uint32_t)(uniform(wv) * kGLoads);
  const uint32_t last_row = (uint32_t)lmin(p.pool_entries - 1, 0x7FFFFFFF);
  // All source addresses first (their index reads overlap), then the loads
  // (each asm statement orders the memory operations around it).
  const uint8_t* src[kGLoads];
#pragma unroll
  for (int k = 0; k < kGLoads; ++k) {
    const int slot = (wv * kGLoads + k) * 64 + lane;
    const int row = imin(slot / kGRowSlots, kGTile - 1);
    const int ch = imin(slot - (slot / kGRowSlots) * kGRowSlots, kGChunks - 1);
    // Clamp to the pool without branches (a negative index becomes the last row).
    const uint32_t r = umin((uint32_t)sidx[imin(tile * kGTile + row, rows - 1)], last_row);
    src[k] = p.kv + (uint64_t)r * kRowDim + 16 * ch;
  }
#pragma unroll
  for (int k = 0; k < kGLoads; ++k) lds_dma_16(src[k], dst + 1024u * k);
}

// One shared 32-row tile for this wave's row group.  `base` is the piece
// position of the tile's first row; positions >= rows_w are masked.
template <int kB>
__device__ __forceinline__ void group_tile(WaveState& st, const GroupQ& q, int base, int rows_w,
                                           float cs, int n, int gq) {
  const uint8_t* buf = ring<kB>();
  // S^T for the tile's 16-row blocks, one independent MFMA chain each, all
  // on v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 operands, unit scales: E8M0
  // 127 = 2^0).  The chain must not mix MFMA kinds: a 16x16x32 fp8 step that
  // reads this 8-pass MFMA's result as its accumulator right behind it gets
  // garbage, and the compiler does not separate the two.
  v4f s[kGBlocks];
#pragma unroll
  for (int b = 0; b < kGBlocks; ++b) s[b] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 hi[kGBlocks];
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    v8i_t kc[kGBlocks];
#pragma unroll
    for (int b = 0; b < kGBlocks; ++b) {
      const uint8_t* row = buf + (16 * b + n) * kGStride + 128 * c + 16 * gq;
      const uint4 a0 = *(const uint4*)row;
      if (c < 4) hi[b] = *(const uint4*)(row + 64);  // step 4 reuses step 3's (q is zero there)
      kc[b] = v8i_t{(int)a0.x,    (int)a0.y,    (int)a0.z,    (int)a0.w,
                    (int)hi[b].x, (int)hi[b].y, (int)hi[b].z, (int)hi[b].w};
    }
#pragma unroll
    for (int b = 0; b < kGBlocks; ++b)
      s[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[b], q.part[c], s[b], 0, 0, 0,
                                                              127, 0, 127);
  }

  // Row lane%16; this lane holds kv rows 16b + 4gq + i of the tile.
  float x[4 * kGBlocks];
#pragma unroll
  for (int b = 0; b < kGBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[4 * b + i] = (base + 16 * b + 4 * gq + i < rows_w) ? s[b][i] * cs : neg_inf();
  softmax_update<4 * kGBlocks>(st, x);

  // O^T += V^T . P^T over the tile's 32-row steps on v_mfma_f32_16x16x32_bf16.
  // Within a step, operand element k = 8gq + j is kv row kappa(gq, j) =
  // 4gq + j (j < 4), 16 + 4gq + j - 4: the rows this lane's S^T holds, so P^T
  // is this lane's own probabilities in bf16 (about 16 significant bits).
  // V^T comes from the row-major tile through the LDS transpose read: within
  // each 16-lane group g, lane 2b + h addresses kv row kappa(g, b) at dims
  // 16*blk + 8h, and lane i receives byte i of the 16 dims from each of the
  // rows kappa(g, 0..7), i.e. its fp8 operand for dim 16*blk + i, widened
  // exactly to bf16.
#pragma unroll
  for (int h = 0; h < kGHalves; ++h) {
    v8bf_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)x[8 * h + i];
      pb[4 + i] = (__bf16)x[8 * h + 4 + i];
    }
    const int sl = n;  // lane within its 16-lane group
    const int jr = sl >> 1;
    const int krow = 32 * h + ((jr < 4) ? (4 * gq + jr) : (16 + 4 * gq + (jr - 4)));
    const uint8_t* vbase = buf + krow * kGStride + 8 * (sl & 1);
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      const v2i_t a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vbase + 16 * blk));
      const v2bf_t a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)a.x, 1.0f, false);
      const v2bf_t a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)a.x, 1.0f, true);
      const v2bf_t a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)a.y, 1.0f, false);
      const v2bf_t a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((u32)a.y, 1.0f, true);
      const v8bf_t va = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      st.O[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.O[blk], 0, 0, 0);
    }
  }
}

// Consume tile tt from ring tile kB after issuing tile tt+2 into ring tile
// (kB + 2) % 3 (the one every wave finished before this step's barrier).
template <int kB>
__device__ __forceinline__ void group_step(const DecodeParams& p, GroupShared& sh, WaveState& st,
                                           const GroupQ& q, int seg0, int srows, int ntiles,
                                           int tt, int rows_w, float cs, int wv, int lane, int n,
                                           int gq) {
  __builtin_amdgcn_s_waitcnt(kVmcntOneTileOut);
  __syncthreads();  // tile tt is in LDS; every wave is done with tile tt-1
  group_issue<(kB + 2) % kGRing>(p, sh.idx, srows, imin(tt + 2, ntiles - 1), wv, lane);
  const int base = seg0 + tt * kGTile;
  if (base < rows_w) group_tile<kB>(st, q, base, rows_w, cs, n, gq);
}

// One piece: positions [c.k, c.k + len) of unit c.u of request c.b (unit
// length L).  slot_base < 0: the piece is the whole unit and every wave writes
// o / lse; else wave wv writes partial slot slot_base + wv.
__device__ __forceinline__ void group_piece(const DecodeParams& p, GroupShared& sh,
                                            const GCursor& c, int G, int L, int len,
                                            int slot_base, int w, float cs, float ks) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  const int R = c.r.qlen * G;
  const int rg = kGroupsPerUnit * c.u + wv;
  const bool valid = rg < R;
  const int rgc = imin(rg, R - 1);
  const int j = rgc / G, g = rgc - j * G;
  const int t = c.r.q_base + j;
  const int vw = valid ? visible(c.r.n, c.r.qlen, j) : 0;
  const int rows_w = imax(0, imin(vw - c.k, len));  // positions this wave may see
  const bool complete = slot_base < 0;

  // Split-unit descriptor of this wave's row group (see mla_decode.hip):
  // written by the workers holding the unit's first and last pieces.
  if (lane == 0 && valid && vw > 0) {
    int* d = (int*)(p.desc + ((int64_t)t * G + g));
    if (c.k == 0) {
      d[0] = w;
      d[2] = complete ? 0 : slot_base + wv;
      d[3] = complete ? 0 : 1;
    }
    if (!complete && c.k + len == L) d[1] = w;
  }

  __syncthreads();  // the previous piece is done with the LDS tiles and indices

  // q of this wave's row group (registers) and the first index batch, in one
  // round trip.
  const int kv_pos0 = c.r.kv_base + c.k;
  GroupQ q;
  {
    const uint8_t* qrow = p.q + ((int64_t)t * p.num_heads + g * kGroup + n) * kRowDim + 16 * gq;
    uint4 xq[9];
#pragma unroll
    for (int cc = 0; cc < 9; ++cc) xq[cc] = *(const uint4*)(qrow + 64 * cc);
    stage_first_indices(sh.idx, p.kv_indices + kv_pos0, imin(len, kGIdxSeg));
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      const uint4 a0 = xq[2 * c], a1 = (c < 4) ? xq[2 * c + 1] : make_uint4(0, 0, 0, 0);
      q.part[c] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                        (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    // Nothing the compiler tracks may be outstanding once the untracked tile
    // loads start: a later wait for q would also wait for those.
    __builtin_amdgcn_s_waitcnt(kVmcntNone);
  }

  WaveState st;
#pragma unroll
  for (int b = 0; b < 32; ++b) st.O[b] = v4f{0.f, 0.f, 0.f, 0.f};
  st.m = neg_inf();
  st.l = 0.f;

  for (int seg0 = 0; seg0 < len; seg0 += kGIdxSeg) {
    const int srows = imin(kGIdxSeg, len - seg0);
    if (seg0 > 0) __syncthreads();  // the previous segment is done with the indices
    stage_indices(sh.idx, p.kv_indices + kv_pos0 + seg0, seg0 == 0 ? kIdxBatch * kThreads : 0,
                  srows);
    __syncthreads();
    const int ntiles = (srows + kGTile - 1) / kGTile;
    // Ring of three tiles: while tile tt is consumed, tiles tt+1 and tt+2 are
    // in flight.  Before the barrier that publishes tile tt, each wave waits
    // until its own loads of tile tt have landed (the 5 loads of tile tt+1,
    // issued later, may stay outstanding).  The loop is unrolled by the ring
    // size so that every ring tile is named statically.
    group_issue<0>(p, sh.idx, srows, 0, wv, lane);
    group_issue<1>(p, sh.idx, srows, imin(1, ntiles - 1), wv, lane);
    for (int tt = 0; tt < ntiles; tt += kGRing) {
      group_step<0>(p, sh, st, q, seg0, srows, ntiles, tt, rows_w, cs, wv, lane, n, gq);
      if (tt + 1 < ntiles)
        group_step<1>(p, sh, st, q, seg0, srows, ntiles, tt + 1, rows_w, cs, wv, lane, n, gq);
      if (tt + 2 < ntiles)
        group_step<2>(p, sh, st, q, seg0, srows, ntiles, tt + 2, rows_w, cs, wv, lane, n, gq);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntNone);  // drain the tail loads before LDS is reused
    __syncthreads();
  }

  if (!valid) return;
  float Lsum = st.l;
  Lsum += __shfl_xor(Lsum, 16);
  Lsum += __shfl_xor(Lsum, 32);
  if (complete && vw == 0) return;  // the row group sees nothing: o / lse written elsewhere

  // Lane (n, gq) holds dims 16*blk + 4gq + r of row n in O^T block blk,
  // element r.
  const bool empty = rows_w == 0;  // only in a split piece: contributes weight 0
  const float oscale = empty ? 0.f : ks / Lsum;
  const float lse_val = empty ? neg_inf() : (st.m + fast_log2(Lsum)) * kLn2;
  if (complete) {
    const int64_t orow = (int64_t)t * p.num_heads + g * kGroup + n;
    uint16_t* dst = p.o + orow * kLatent + 4 * gq;
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      uint2 pk;
      pk.x = bf16_bits(st.O[blk][0] * oscale) | (bf16_bits(st.O[blk][1] * oscale) << 16);
      pk.y = bf16_bits(st.O[blk][2] * oscale) | (bf16_bits(st.O[blk][3] * oscale) << 16);
      *(uint2*)(dst + 16 * blk) = pk;
    }
    if (p.lse != nullptr && gq == 0) p.lse[orow] = lse_val;
    return;
  }
  const int64_t slot = slot_base + wv;
  float* dst = p.part_o + (slot * kGroup + n) * kLatent + 4 * gq;
#pragma unroll
  for (int blk = 0; blk < 32; ++blk)
    *(float4*)(dst + 16 * blk) = make_float4(st.O[blk][0] * oscale, st.O[blk][1] * oscale,
                                             st.O[blk][2] * oscale, st.O[blk][3] * oscale);
  if (gq == 0) p.part_lse[slot * kGroup + n] = lse_val;
}

// One worker: locate its share of the group-mode stream and run its pieces.
__device__ __forceinline__ void group_worker(const DecodeParams& p, GroupShared& sh) {
  const int G = p.num_heads / kGroup;

  // Pass 1 over requests: stream length W; zero this block's empty tokens.
  int64_t acc = 0;
  for (int b = threadIdx.x; b < p.batch; b += kThreads) {
    const Req r = load_req(p.qo_indptr, p.kv_indptr, b, p.kv_indices_len, p.num_tokens);
    acc += group_request_rows(r, G);
    const int nempty = imin(r.qlen, imax(0, r.qlen - r.n));
    for (int jj = 0; jj < nempty; ++jj)
      if ((r.q_base + jj) % (int)gridDim.x == (int)blockIdx.x) zero_token(p, r.q_base + jj);
  }
  const int64_t W = uniform(block_sum_i64(acc, sh.red));
  const int w = blockIdx.x;
  if (W == 0) return;
  const int nw = effective_workers(W, p.num_workers);
  if (w >= nw) return;
  const int64_t x0 = worker_begin(w, W, nw), x1 = worker_begin(w + 1, W, nw);
  const int64_t xs[2] = {x0, x1 < W ? x1 : -1};
  plan_locate2(p, [G](const Req& r) { return group_request_rows(r, G); }, xs, sh.red, sh.pb,
               sh.pcum);
  const int b0 = uniform(sh.pb[0]), b1 = uniform(sh.pb[1]);
  if (b0 < 0 || b1 == -1) return;  // not reached with consistent indptr
  GCursor c;
  gcursor_in_request(c, b0, load_req(p.qo_indptr, p.kv_indptr, b0, p.kv_indices_len, p.num_tokens),
                     x0 - uniform(sh.pcum[0]), G);
  uniformize(c);
  int64_t p1 = W;
  if (x1 < W) {
    GCursor c1;
    gcursor_in_request(c1, b1,
                       load_req(p.qo_indptr, p.kv_indptr, b1, p.kv_indices_len, p.num_tokens),
                       x1 - uniform(sh.pcum[1]), G);
    uniformize(c1);
    p1 = gsnap_at(x1, c1, G);
  }
  const int64_t p0 = gsnap_at(x0, c, G);
  if (p0 >= p1) return;
  if (p0 < x0) {
    c.k = 0;
  } else if (p0 > x0) {
    if (!gcursor_next_unit(c, p.qo_indptr, p.kv_indptr, p.batch, p.kv_indices_len, p.num_tokens,
                           G))
      return;
    uniformize(c);
  }
  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;
  const float cs = p.sm_scale * kLog2e * qs * ks;

  int64_t pos = p0;
  int piece = 0;
  while (pos < p1) {
    const int L = group_unit_len(c.r, G, c.u);
    const int len = (int)lmin((int64_t)(L - c.k), p1 - pos);
    if (len <= 0) break;  // not reached with a consistent plan
    const bool complete = (c.k == 0 && len == L);
    const int slot_base =
        complete ? -1 : kGSlotsPerPiece * (2 * w + (piece == 0 ? 0 : 1));
    group_piece(p, sh, c, G, L, len, slot_base, w, cs, ks);
    pos += len;
    c.k += len;
    ++piece;
    if (pos < p1 && c.k == L) {
      if (!gcursor_next_unit(c, p.qo_indptr, p.kv_indptr, p.batch, p.kv_indices_len,
                             p.num_tokens, G))
        break;
      uniformize(c);
    }
  }
}

// Two workgroups per CU (two waves per SIMD): one wave's softmax and LDS
// latency overlap the other's MFMAs.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_groups_fp8_kernel(const DecodeParams p) {
  __shared__ GroupShared sh;
  group_worker(p, sh);
}

hipError_t launch_decode_groups(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(mla_decode_groups_fp8_kernel, dim3(p.num_workers), dim3(kThreads), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace mla
