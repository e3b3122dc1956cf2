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
// times, and the attention arithmetic (not HBM) sets the time.
//
// Design (our own):
//   * A unit is eight row groups of one request (mla_plan.h, group mode);
//     workers take equal, boundary-snapped shares of the unit stream as in
//     the standard mode.  One workgroup (four waves, one per SIMD) per CU.
//   * Wave wv owns the unit's row groups wv and wv + 4: 32 query rows, the N
//     dimension of 32x32 MFMAs, so every K and V element read from LDS
//     serves 32 rows.
//   * Tiles of 32 KV rows are gathered once by all 256 threads with direct
//     global->LDS loads (each lane 16 consecutive bytes of a row) into a
//     six-tile LDS ring with a 592-byte row stride; three later tiles are in
//     flight while one is consumed.
//   * Per tile and wave: S^T = K.Q^T on v_mfma_scale_f32_32x32x64_f8f6f4
//     (nine steps, K from LDS, q in registers), the online softmax (each
//     lane masks the entries its row's token may not see) and P packed as
//     fp8 hi + lo under an E8M0 scale per (query row, tile).  Every two
//     tiles, O^T += V^T.P^T on the same MFMA over 64 KV rows, with the V^T
//     operand read straight from the fp8 tiles by the LDS transpose read
//     (ds_read_b64_tr_b8).  Every wave writes its own o (or partials): there
//     is no cross-wave merge.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

constexpr int kGTile = 32;                               // KV rows per shared tile
constexpr int kGIdxSeg = 4096;                           // kv_indices staged per segment
constexpr int kGChunks = kRowDim / 16;                   // 16-byte chunks per row (36)
constexpr int kGRowSlots = kGChunks + 1;                 // + one pad slot per staged row
constexpr int kGStride = 16 * kGRowSlots;                // LDS bytes per staged row (592)
constexpr int kGLoads = 5;                               // load instructions per wave per tile
constexpr int kGTileBytes = kWaves * kGLoads * 64 * 16;  // 20,480 (>= 32 rows x 592)
constexpr int kGRing = 6;                                // tiles in the LDS ring
static_assert(kGTile * kGStride <= kGTileBytes, "a tile's rows must fit its ring slot");
static_assert(kGroupsPerUnit == 2 * kWaves, "each wave owns two row groups of a unit");
constexpr int kGSlotsPerPiece = kGroupsPerUnit;          // one partial slot per row group
// P = 2^(s - m) with m a row's first visible score: P may grow to 2^kPBig
// before the piece is redone with m = the row's true max (see wide_tile).
constexpr float kPBig = 64.0f;

__shared__ __attribute__((aligned(16))) uint8_t g_ring[kGRing * kGTileBytes];

struct alignas(16) GroupShared {
  int32_t idx[kGIdxSeg];  // kv_indices of the current segment of the piece
  int flag[kWaves];       // per-wave "redo the piece" votes
  int64_t red[kWaves];
  PlanHit hits[2];
};

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; all-ones leaves a counter unchecked).
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kVmcntNone = waitcnt_vm(0);

// Waits until at most `tiles` tiles of this wave's ring loads are in flight
// (kGLoads loads each; loads complete in order).
__device__ __forceinline__ void wait_tiles_in_flight(int tiles) {
  static_assert(kGRing - 3 == 3, "one case per possible count");
  switch (tiles) {
    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(1 * kGLoads)); break;
    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kGLoads)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kGLoads)); break;
  }
}

__device__ __forceinline__ void uniformize(GCursor& c) {
  c.b = uniform(c.b);
  c.u = uniform(c.u);
  c.k = uniform(c.k);
  uniformize(c.r);
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
// clamped to the segment's last row) straight into ring slot `slot` with
// global_load_lds_dwordx4: instruction k of wave wv writes LDS bytes
// [(5wv + k) * 1024, +1024) of the slot, lane l the 16 bytes of slot position
// s = 64(5wv + k) + l, which is staged row s / 37, chunk s % 37.  Lanes on a
// pad position (chunk 36) or past the last row load a duplicate of a real
// chunk that is never read.  Every load is unconditional, so the
// outstanding-load count is static.
__device__ __forceinline__ void group_issue(const DecodeParams& p, const int32_t* sidx, int rows,
                                            int tile, int slot, int wv, int lane) {
  const uint32_t dst = lds_addr_of(g_ring) + (uint32_t)(uniform(slot) * kGTileBytes) +
                       1024u * (uint32_t)(uniform(wv) * kGLoads);
  const uint32_t last_row = (uint32_t)lmin(p.pool_entries - 1, 0x7FFFFFFF);
  // All source addresses first (their index reads overlap), then the loads
  // (each asm statement orders the memory operations around it).
  const uint8_t* src[kGLoads];
#pragma unroll
  for (int k = 0; k < kGLoads; ++k) {
    const int s = (wv * kGLoads + k) * 64 + lane;
    const int row = imin(s / kGRowSlots, kGTile - 1);
    const int ch = imin(s - (s / kGRowSlots) * kGRowSlots, kGChunks - 1);
    // Clamp to the pool without branches (a negative index becomes the last row).
    const uint32_t r = umin((uint32_t)sidx[imin(tile * kGTile + row, rows - 1)], last_row);
    src[k] = p.kv + (uint64_t)r * kRowDim + 16 * ch;
  }
#pragma unroll
  for (int k = 0; k < kGLoads; ++k) lds_dma_16(src[k], dst + 1024u * k);
}

// Per-wave state: O^T for the wave's 32 query rows (32x32 MFMA layout: lane l
// holds row lane%32, dims 32*blk + 8*(v/4) + 4*(l/32) + v%4 in O[blk][v]);
// for row lane%32 (equal in lanes l and l^32) the reference m of P = 2^(s - m),
// the largest score seen and whether a score exceeded m + kPBig; this lane's
// partial sum of P.
struct WideState {
  v16f O[16];
  float m;
  float mx;
  float l;   // sum of P (the lse's)
  float lw;  // sum of the weights the MFMAs use, hi + lo (o's normaliser)
  bool big;
};

// P^T operands of one 64-row P.V step (two tiles), as fp8 hi + lo parts.
// Byte 16*tau + v of a lane is the lane's value v of tile tau of the pair
// (KV row 8*(v/4) + 4*(lane/32) + v%4 of that tile).  On the MFMA's k axis a
// 32-value scale block is bytes 16b .. 16b+15 of lanes n and n+32, i.e. one
// tile of one query row, with its E8M0 scale in lane n + 32b: e[tau] is the
// row's exponent for tile tau.
struct PairP {
  v8i_t hi, lo;
  int e[2];
};

// Lane-specific LDS offsets within a ring slot.
struct TileOffsets {
  int k;     // K operand: row lane%32, bytes 32*(lane/32) of each 64-byte chunk
  int v[2];  // V^T transpose-read source for the two 16-row halves of a tile
};

// S^T = bias + K.Q^T as a chain of nine v_mfma_scale_f32_32x32x64_f8f6f4
// steps (unit E8M0 scales in `sc` = 127) with the accumulator in vector
// registers; bias is 0, or -inf for the entries a row may not see.  Written
// as inline assembly because the compiler puts an MFMA result in the
// accumulator registers, which here all hold O^T: it would then move a block
// of O^T out and back on every tile.  Same-kind steps may feed each other
// back to back.  Steps [kC0, kC0 + 3) here, K operands of those steps in k.
template <int kC0>
__device__ __forceinline__ void qk_steps(v16f& s, const v8i_t (&k)[3], const v8i_t (&q)[9], int sc,
                                         const v16f& bias) {
  if (kC0 == 0) {
    // The leading wait states separate the vector ALU's last writes of the
    // bias registers from the MFMA's read of them (the compiler inserts no
    // wait for an MFMA it cannot see).
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %4, %3, %3 op_sel_hi:[0,0,0]"
                 : "=&v"(s)
                 : "v"(k[0]), "v"(q[0]), "v"(sc), "v"(bias));
  } else {
    // bias is an (unused) input of the next steps so that its registers stay
    // untouched while the first step may still read it (an MFMA reads its
    // accumulator input late in its passes).
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(s)
                 : "v"(k[0]), "v"(q[kC0]), "v"(sc), "v"(bias));
  }
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
               : "+v"(s)
               : "v"(k[1]), "v"(q[kC0 + 1]), "v"(sc));
  if (kC0 < 6) {
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(s)
                 : "v"(k[2]), "v"(q[kC0 + 2]), "v"(sc));
  } else {
    // The trailing 20 wait states cover the latency of the last step's result
    // before the vector ALU reads it.
    asm volatile(
        "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]\n\t"
        "s_nop 15\n\ts_nop 3"
        : "+v"(s)
        : "v"(k[2]), "v"(q[kC0 + 2]), "v"(sc));
  }
}

// K operands of steps [kC0, kC0 + 3) of a tile (row lane%32, bytes
// 64c + 32*(lane/32) .. +32 of the 576-byte row).
template <int kC0>
__device__ __forceinline__ void read_k3(v8i_t (&k)[3], const uint8_t* buf, const TileOffsets& off) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint8_t* kp = buf + off.k + 64 * (kC0 + i);
    const uint4 a0 = *(const uint4*)kp, a1 = *(const uint4*)(kp + 16);
    k[i] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                 (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  }
}

// S^T of one shared 32-row tile for this wave's 32 query rows.  The K
// operands are read three steps at a time (24 registers live, not 72).
__device__ __forceinline__ v16f tile_qk(const v8i_t (&q)[9], const uint8_t* buf,
                                        const TileOffsets& off, int sc, const v16f& bias) {
  v16f s;
  v8i_t k[3];
  read_k3<0>(k, buf, off);
  qk_steps<0>(s, k, q, sc, bias);
  read_k3<3>(k, buf, off);
  qk_steps<3>(s, k, q, sc, bias);
  read_k3<6>(k, buf, off);
  qk_steps<6>(s, k, q, sc, bias);
  return s;
}

// The online-softmax step of one tile from its raw scores s (masked entries
// already -inf) and the tile's P operand.  Value v of this lane is KV row
// 8*(v/4) + 4h + v%4 of the tile.  cs > 0 is the base-2 score scale, so a
// tile's scaled maximum is its raw maximum scaled, and each exponent is one
// fused multiply-add.  Straight-line code: no branch splits it from the P.V
// steps it is interleaved with.
template <int kTau>
__device__ __forceinline__ void tile_softmax(WideState& st, PairP& pp, const v16f& s, float cs) {
  float r[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) r[v] = s[v];
  float tr = r[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) tr = fmaxf(tr, r[v]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tr), __float_as_uint(tr),
                                                     false, false);
    tr = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max over lanes l, l^32
  }
  const float tmax = tr * cs;
  // The reference m is fixed at a row's first visible score maximum and never
  // raised, so O is never rescaled inside the tile loop (O lives in the
  // accumulator registers, where a rescale would cost a copy of all of it).
  // P = 2^(s - m) may exceed 1; a row whose scores rise more than 2^kPBig
  // above m sets `big` and the piece is redone with m = its true maximum.
  // Before its first visible score m is -FLT_MAX (finite), which keeps
  // P = 2^(-inf) = 0 for masked entries instead of NaN.
  st.mx = fmaxf(st.mx, tmax);
  st.m = (st.m == -__FLT_MAX__ && tmax > neg_inf()) ? tmax : st.m;
  st.big = st.big || (tmax > st.m + kPBig);
  // The tile's block exponent: P' = P * 2^-e <= 2^8 for the tile's row max,
  // within fp8 range; entries far below it lose nothing that matters next to
  // the block maximum (the hi + lo pair keeps about 8 significant bits).
  // A row that sees none of the tile (tmax = -inf) gets e = -127 and P = 0.
  const float rel = tmax - st.m;
  int e = (int)__builtin_ceilf(fminf(fmaxf(rel, -200.f), 200.f)) - 8;
  e = imin(imax(e, -127), 127);
  const float nref = -(st.m + (float)e);
  // (Sums start at -0, which x + -0 = x lets the compiler drop.)
  float x[16], ps[4] = {-0.f, -0.f, -0.f, -0.f}, dw = -0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    x[v] = fast_exp2(__builtin_fmaf(r[v], cs, nref));
    ps[v & 3] += x[v];
  }
  pp.e[kTau] = e;
  // fp8 hi part, then the residual as fp8 lo (same block scale).  Each
  // packing's first write keeps the upper half of its destination, given a
  // register that is dead by then, so no zeroing move is needed.  o is
  // normalised by the sum of the weights the MFMAs use (hi + lo, not P): the
  // split's rounding then moves o towards the entries it favours instead of
  // scaling it, an error bounded by |V - o| rather than |V|.  The lse keeps
  // the sum of P.
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 0], x[4 * w + 1], __float_as_int(r[4 * w]),
                                             false);
    hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], hw, true);
    const v2f_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
    const v2f_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
    const float d0 = x[4 * w + 0] - h01[0], d1 = x[4 * w + 1] - h01[1];
    const float d2 = x[4 * w + 2] - h23[0], d3 = x[4 * w + 3] - h23[1];
    int lw = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, __float_as_int(x[4 * w]), false);
    lw = __builtin_amdgcn_cvt_pk_fp8_f32(d2, d3, lw, true);
    dw = add_fp8x4(lw, dw) - ((d0 + d1) + (d2 + d3));
    pp.hi[4 * kTau + w] = hw;
    pp.lo[4 * kTau + w] = lw;
  }
  const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  st.l += __builtin_ldexpf(psum, e);
  st.lw += __builtin_ldexpf(psum + dw, e);
}

// O^T += V^T . P^T over the pair's 64 rows for dim blocks [kB0, kB0 + 8) on
// v_mfma_scale_f32_32x32x64_f8f6f4 (hi and lo parts of P, one step each per
// 32-dim block).  The A operand is V^T straight from the row-major fp8 tiles
// by the LDS transpose read: read (tile tau, half u) gives lane l byte j =
// V[kappa(l/32, 8u + j)][32*blk + l%32], operand bytes 16*tau + 8*u + j, the
// same KV rows as the P bytes.
template <int kB0>
__device__ __forceinline__ void pair_pv(WideState& st, const PairP& pp, const uint8_t* buf0,
                                        const uint8_t* buf1, const TileOffsets& off, int h) {
  const int sc = 127 + (h ? pp.e[1] : pp.e[0]);  // block tau's scale sits in lanes with l/32 = tau
#pragma unroll
  for (int blk = kB0; blk < kB0 + 8; ++blk) {
    const v2i_t a0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf0 + off.v[0] + 32 * blk));
    const v2i_t a1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf0 + off.v[1] + 32 * blk));
    const v2i_t a2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf1 + off.v[0] + 32 * blk));
    const v2i_t a3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf1 + off.v[1] + 32 * blk));
    const v8i_t va = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
    st.O[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pp.hi, st.O[blk], 0, 0, 0, 127,
                                                                0, sc);
    st.O[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pp.lo, st.O[blk], 0, 0, 0, 127,
                                                                0, sc);
    // Only vector and scalar ALU work may cross (the softmax it runs beside):
    // hoisting later blocks' V reads would hold their registers early.
    __builtin_amdgcn_sched_barrier(0x0406);
  }
}

// Score bias of one tile for row lane%32: 0 for the first lim rows, -inf for
// the rest.  Value v of this lane is KV row 8*(v/4) + 4h + v%4.
__device__ __forceinline__ v16f mask_bias(int lim, int h) {
  v16f c;
#pragma unroll
  for (int v = 0; v < 16; ++v) c[v] = (8 * (v >> 2) + 4 * h + (v & 3) < lim) ? 0.f : neg_inf();
  return c;
}

// One step of the tile loop: S^T of the two tiles of a new pair, their
// softmax and P operands (cur), and the previous pair's P.V (prev, still in
// its ring slots p0 / p1), half of it after each tile's scores.  Row lane%32
// sees the first lim0 / lim1 rows of the two tiles; full: all rows of both.
__device__ __forceinline__ void pair_step(WideState& st, PairP& cur, const PairP& prev,
                                          const v8i_t (&q)[9], const uint8_t* b0,
                                          const uint8_t* b1, const uint8_t* p0, const uint8_t* p1,
                                          const TileOffsets& off, int sc, int lim0, int lim1,
                                          bool full, float cs, int h) {
  // Each half is one basic block (the mask's branch comes before it).
  v16f c0 = {};
  if (!full) c0 = mask_bias(lim0, h);
  const v16f s0 = tile_qk(q, b0, off, sc, c0);
  tile_softmax<0>(st, cur, s0, cs);
  pair_pv<0>(st, prev, p0, p1, off, h);
  v16f c1 = {};
  if (!full) c1 = mask_bias(lim1, h);
  const v16f s1 = tile_qk(q, b1, off, sc, c1);
  tile_softmax<1>(st, cur, s1, cs);
  pair_pv<8>(st, prev, p0, p1, off, h);
}

// The 32 partial rows of a wave (O^T * oscale, as fp16 or fp32) go to global
// memory through LDS: a lane holds 16-byte pieces of its row scattered over 16
// blocks, so storing them directly makes every store instruction touch 32 rows
// 1 KB apart, which issues slowly; staged, each store writes two whole
// 512-byte row pieces.  The rows pass in chunks of 512 bytes per row: two
// halves of 256 dims in fp16, four quarters of 128 dims in fp32.  Row
// r = lane%32 of the wave is head r%16 of row group wv + 4*(r/16), whose
// partial slot is slot_base + wv + 4*(r/16).  Uses ring bytes
// [wv * kStageBytes, +kStageBytes): no wave reads the ring after its tile
// loop, and the next piece waits for every wave before refilling it.
constexpr int kStageStride = 528;                 // 512 bytes of a row chunk + 16 (bank spread)
constexpr int kStageBytes = 32 * kStageStride;  // one wave's 32 rows
static_assert(kWaves * kStageBytes <= kGRing * kGTileBytes, "staging fits in the ring");

template <bool kF32>
__device__ __forceinline__ void store_partials(const WideState& st, float oscale, void* part,
                                               int64_t slot_base, int wv, int lane) {
  constexpr int kChunks = kF32 ? 4 : 2;    // passes over the staging rows
  constexpr int kBlocks = 16 / kChunks;    // O^T blocks (32 dims each) per pass
  constexpr int kElem = kF32 ? 4 : 2;      // bytes per stored value
  uint8_t* stage = g_ring + wv * kStageBytes;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int chunk = 0; chunk < kChunks; ++chunk) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int blk = kBlocks * chunk + b;
        uint8_t* dst = stage + r * kStageStride + kElem * (32 * b + 8 * q4 + 4 * h);
        const float a0 = st.O[blk][4 * q4 + 0] * oscale, a1 = st.O[blk][4 * q4 + 1] * oscale;
        const float a2 = st.O[blk][4 * q4 + 2] * oscale, a3 = st.O[blk][4 * q4 + 3] * oscale;
        if constexpr (kF32) {
          *(float4*)dst = make_float4(a0, a1, a2, a3);
        } else {
          uint2 pk;
          pk.x = pack_f16x2(a0, a1);
          pk.y = pack_f16x2(a2, a3);
          *(uint2*)dst = pk;
        }
      }
    wave_lds_sync();  // the wave's writes are in LDS before any lane reads another's
#pragma unroll
    for (int it = 0; it < 16; ++it) {  // two rows per instruction, 32 lanes x 16 bytes each
      const int rr = 2 * it + (lane >> 5), c = lane & 31;
      const uint4 v = *(const uint4*)(stage + rr * kStageStride + 16 * c);
      const int64_t slot = slot_base + wv + kWaves * (rr >> 4);
      const int64_t e0 = (slot * kGroup + (rr & 15)) * kLatent + (kLatent / kChunks) * chunk;
      if constexpr (kF32)
        *(uint4*)((float*)part + e0 + 4 * c) = v;
      else
        *(uint4*)((uint16_t*)part + e0 + 8 * c) = v;
    }
    wave_lds_sync();  // reads done before the next chunk overwrites the rows
  }
}

// One piece: entries [k0, k0 + len) of unit c.u of request c.b (unit
// length L; H heads, the request's rows packed 16 to a row group).
// slot_base < 0: the piece is the whole unit and every row writes o / lse;
// else row group i of the unit writes partial slot slot_base + i.
template <bool kPaged, bool kCascade>
__device__ __forceinline__ void group_piece(const DecodeParams& p, GroupShared& sh,
                                            const GCursor& c, int k0, int H, int L, int len,
                                            int slot_base, int w, float cs, float ks) {
  const int tid = threadIdx.x, wv = uniform(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, hq = lane & 31, half = hq >> 4, n16 = hq & 15;
  const int NR = c.r.qlen * H;              // the request's query rows
  const int RG = group_row_groups(c.r, H);  // and row groups
  const bool complete = slot_base < 0;

  // The wave's two row groups (uniform): the entries their last rows see
  // (the most any of their rows sees) and their first rows see (the fewest;
  // 0 if the row group is not full).  Rows are token-major, so a row group's
  // visible counts rise from its first row to its last.
  int rows_h[2], vis_h[2], first_h[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int rgk = kGroupsPerUnit * c.u + wv + kWaves * k;
    const bool ok = rgk < RG;
    vis_h[k] = ok ? req_visible(c.r, group_last_token(c.r, H, rgk)) : 0;
    const int vfirst = (ok && kGroup * rgk + kGroup <= NR)
                           ? req_visible(c.r, imin(kGroup * rgk, NR - 1) / H) : 0;
    rows_h[k] = imax(0, imin(vis_h[k] - k0, len));
    first_h[k] = imax(0, imin(vfirst - k0, len));
  }
  const int wave_rows = uniform(imax(rows_h[0], rows_h[1]));
  const int full_rows = uniform(imin(first_h[0], first_h[1]));
  const int ulocal = wv + kWaves * half;  // this lane's row group within the unit
  const int rg = kGroupsPerUnit * c.u + ulocal;
  const int row = kGroup * rg + n16;      // this lane's query row within the request
  const bool valid = row < NR;
  const int rowc = imin(row, NR - 1);
  const int j = rowc / H, hh = rowc - j * H;  // its token and head
  const int t = c.r.q_base + j;
  // The q row: in a one-launch cascade call tokens T .. 2T-1 (the suffix
  // requests) are the caller's tokens 0 .. T-1 again.
  const int qtok = (kCascade && t >= (p.num_tokens >> 1)) ? t - (p.num_tokens >> 1) : t;
  const int vw = valid ? req_visible(c.r, j) : 0;
  const int rows_w = imax(0, imin(vw - k0, len));

  // Split-unit descriptor of each row group (see mla_decode.hip): written by
  // the workers holding the unit's first and last pieces, with the row
  // group's output rows (its first token and head, and its row count).
  // Every lane stores (the conditions are uniform); lanes that hold no row
  // group's descriptor store to the spare entry after the last, so that no
  // divergent branch exists here: the compiler has placed a register spill
  // under such a branch's narrowed exec mask, saving only the branch's lanes.
  {
    const int Gs = group_slots_per_token(H);
    const bool mine = (lane == 0 || lane == 16) && rg < RG && (half ? vis_h[1] : vis_h[0]) > 0;
    const int64_t e = mine ? (int64_t)c.r.q_base * Gs + rg : (int64_t)p.num_tokens * Gs;
    int* d = (int*)(p.desc + e);
    if (k0 == 0) {
      d[0] = w;
      d[2] = complete ? 0 : slot_base + ulocal;
      d[3] = complete ? 0 : 1;
      p.desc_rows[e] = make_int2(t, hh * 32 + imin(kGroup, NR - kGroup * rg));
    }
    if (!complete && k0 + len == L) d[1] = w;
  }

  __syncthreads();  // the previous piece is done with the LDS ring and indices

  // q rows of this lane's row group (registers) and the first index batch, in
  // one round trip.  Step c: head n16's bytes [64c + 32h, +32).
  const RowSrc src = row_src<kPaged>(c.r, k0);
  v8i_t q[9];
  {
    const uint8_t* qrow = p.q + ((int64_t)qtok * H + hh) * kRowDim + 32 * h;
    uint4 xq[18];
#pragma unroll
    for (int i = 0; i < 18; ++i) xq[i] = *(const uint4*)(qrow + 64 * (i >> 1) + 16 * (i & 1));
    stage_first_indices<kPaged, kThreads, kCascade>(sh.idx, p, src, imin(len, kGIdxSeg));
#pragma unroll
    for (int cc = 0; cc < 9; ++cc) {
      const uint4 a0 = xq[2 * cc], a1 = xq[2 * cc + 1];
      q[cc] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                    (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    // The softmax scales raw scores by a positive factor: a negative scale
    // moves onto q, whose fp8 sign bits flip exactly.
    if (cs < 0.f) {
#pragma unroll
      for (int cc = 0; cc < 9; ++cc) q[cc] ^= (int)0x80808080u;
    }
    // Nothing the compiler tracks may be outstanding once the untracked tile
    // loads start: a later wait for q would also wait for those.
    __builtin_amdgcn_s_waitcnt(kVmcntNone);
  }
  // |cs|, kept >= the smallest normal so that a masked score (-inf) still
  // scales to -inf (a NaN scale stays NaN).
  const float csa = fabsf(cs) < __FLT_MIN__ ? __FLT_MIN__ : fabsf(cs);

  TileOffsets off;
  off.k = hq * kGStride + 32 * h;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // Transpose-read source: 16-lane group gg = lane/16, position i = lane%16
    // supplies KV row kappa(gg/2, i/2) at dims 16*(gg%2) + 8*(i%2) of the block.
    const int gg = lane >> 4, i = lane & 15, b = i >> 1;
    const int krow = 16 * u + 8 * (b >> 2) + 4 * (gg >> 1) + (b & 3);
    off.v[u] = krow * kGStride + 16 * (gg & 1) + 8 * (i & 1);
  }

  const int sc = uniform(127);  // E8M0 scale 2^0 for both MFMA operands
  WideState st;
  st.m = -__FLT_MAX__;
  st.mx = neg_inf();
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
  for (int b = 0; b < 16; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.O[b][i] = 0.f;
  st.l = 0.f;
  st.lw = 0.f;
  st.big = false;

  for (int seg0 = 0; seg0 < len; seg0 += kGIdxSeg) {
    const int srows = imin(kGIdxSeg, len - seg0);
    if (seg0 > 0) __syncthreads();  // the previous segment is done with the indices
    // The first kIdxBatch * kThreads indices of segment 0 came with q, but
    // only for the first pass: a redo after a piece of several segments finds
    // the last segment's indices there.
    stage_indices<kPaged, kThreads, kCascade>(sh.idx, p, src.template at<kPaged>(seg0),
                                              (seg0 == 0 && pass == 0) ? kIdxBatch * kThreads : 0,
                                              srows);
    __syncthreads();
    const int ntiles = (srows + kGTile - 1) / kGTile;
    // Ring of six tiles, consumed in pairs (P.V takes two tiles per step).  At
    // the step of pair (t, t+1) one barrier publishes both tiles and shows
    // every wave done with pair (t-4, t-3) (its P.V ran at the previous step),
    // whose slots then take pair (t+2, t+3): the pair is scored and pair
    // (t-2, t-1) goes through P.V while the next pair is in flight.  Before
    // the barrier each wave waits until its own loads of tiles t and t+1 have
    // landed.  An odd last tile pairs with itself at P = 0.
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (i < ntiles) group_issue(p, sh.idx, srows, i, i, wv, lane);
    // One straight-line step per pair, so that its softmax (vector ALU) and
    // the previous pair's P.V (matrix cores), which are independent, can issue
    // interleaved.  A tile past this wave's rows is scored fully masked (P = 0
    // changes no state), and the first step's P.V runs with P = 0.
    // The P operands of consecutive pairs alternate between pa and pb (the
    // loop runs two pairs per iteration), so no step copies one into the other.
    PairP pa, pb;
    pb.hi = v8i_t{};
    pb.lo = v8i_t{};
    pb.e[0] = pb.e[1] = 0;
    const uint8_t* pb0 = g_ring;
    const uint8_t* pb1 = g_ring;
    auto step = [&](int t, PairP& cur, const PairP& prev) {
      wait_tiles_in_flight(0);  // this wave's loads of tiles t, t+1 (the last it issued)
      __syncthreads();  // tiles t, t+1 are in LDS; every wave is done with t-4, t-3
#pragma unroll
      for (int k = 2; k < 4; ++k)
        if (t + k < ntiles) group_issue(p, sh.idx, srows, t + k, (t + k) % kGRing, wv, lane);
      const uint8_t* b0 = g_ring + (t % kGRing) * kGTileBytes;
      const uint8_t* b1 = t + 1 < ntiles ? g_ring + ((t + 1) % kGRing) * kGTileBytes : b0;
      const int base0 = seg0 + t * kGTile, base1 = base0 + kGTile;
      // lim1 <= 0 also masks a missing odd tile: its rows lie past the piece.
      const int lim1 = t + 1 < ntiles ? rows_w - base1 : 0;
      pair_step(st, cur, prev, q, b0, b1, pb0, pb1, off, sc, rows_w - base0, lim1,
                t + 1 < ntiles && base1 + kGTile <= full_rows, csa, h);
      pb0 = b0;
      pb1 = b1;
    };
    bool last_in_a = false;  // which of pa, pb holds the last pair's P
    for (int t = 0; t < ntiles; t += 4) {
      step(t, pa, pb);
      if (t + 2 >= ntiles) {
        last_in_a = true;
        break;
      }
      step(t + 2, pb, pa);
    }
    if (last_in_a) pb = pa;
    if (seg0 + (((ntiles - 1) >> 1) << 1) * kGTile < wave_rows) {  // the last pair
      pair_pv<0>(st, pb, pb0, pb1, off, h);
      pair_pv<8>(st, pb, pb0, pb1, off, h);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntNone);  // every ring load has landed
    __syncthreads();
  }
  // Redo the piece (all waves: the tiles are gathered together) if any row's
  // scores rose too far above its reference; then m is the row's maximum.
  if (pass == 0) {
    if ((tid & 63) == 0) sh.flag[wv] = __any(st.big) ? 1 : 0;
    __syncthreads();
    const int redo = sh.flag[0] | sh.flag[1] | sh.flag[2] | sh.flag[3];
    __syncthreads();
    if (!redo) break;
    st.m = (st.mx == neg_inf()) ? -__FLT_MAX__ : st.mx;
  }
  }

  float Lsum = st.l, Wsum = st.lw;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(Lsum), __float_as_uint(Lsum),
                                                     false, false);
    Lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(Wsum), __float_as_uint(Wsum),
                                                     false, false);
    Wsum = __uint_as_float(sv[0]) + __uint_as_float(sv[1]);
  }
  const bool empty = rows_w == 0;  // in a split piece: contributes weight 0
  const float oscale = empty ? 0.f : ks / Wsum;
  // The lane's row, rebuilt here from an opaque copy of the thread id, so that
  // none of its indices stays live across the tile loop.
  const int elane = opaque(tid) & 63;
  const int eh = elane >> 5, en16 = elane & 15;
  const int eulocal = wv + kWaves * ((elane & 31) >> 4);
  const int erow = kGroup * (kGroupsPerUnit * c.u + eulocal) + en16;
  const int erowc = imin(erow, NR - 1);
  const int ej = erowc / H;
  const int64_t eorow = (int64_t)(c.r.q_base + ej) * H + (erowc - ej * H);
  const float lse_val = empty ? neg_inf() : (st.m + fast_log2(Lsum)) * kLn2;
  if (!complete) {
    // Partials are stored in fp16 (round to nearest even), without the kv
    // scale (the combine applies it), unless the call asks for fp32 ones (an
    // fp32 output): every worker writes eight row groups of them at the end
    // of a split piece, and their bytes, written and read back by the
    // combine, rival the attention arithmetic.  Every lane takes part: the
    // rows of a row group past the request's last (empty, weight 0) land in
    // that row group's own slot, which the combine never reads.  Lanes l and
    // l+32 store the same lse.
    if (p.part_fp32)
      store_partials<true>(st, oscale, p.part_o, slot_base, wv, elane);
    else
      store_partials<false>(st, empty ? 0.f : 1.0f / Wsum, p.part_o, slot_base, wv, elane);
    p.part_lse[(slot_base + eulocal) * kGroup + en16] = lse_val;
    return;
  }
  if (erow >= NR) return;
  if (req_visible(c.r, ej) == 0) return;  // the row sees nothing: o / lse written elsewhere
  {
    const int64_t orow = eorow;
    const int h = eh;
    if (p.o32 != nullptr) {
      float* d32 = p.o32 + orow * kLatent + 4 * h;
#pragma unroll
      for (int blk = 0; blk < 16; ++blk)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(float4*)(d32 + 32 * blk + 8 * q4) =
              make_float4(st.O[blk][4 * q4 + 0] * oscale, st.O[blk][4 * q4 + 1] * oscale,
                          st.O[blk][4 * q4 + 2] * oscale, st.O[blk][4 * q4 + 3] * oscale);
      if (p.lse != nullptr && h == 0) p.lse[orow] = lse_val;
      return;
    }
    uint16_t* dst = p.o + orow * kLatent + 4 * h;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 pk;
        pk.x = pack_bf16x2(st.O[blk][4 * q4 + 0] * oscale, st.O[blk][4 * q4 + 1] * oscale);
        pk.y = pack_bf16x2(st.O[blk][4 * q4 + 2] * oscale, st.O[blk][4 * q4 + 3] * oscale);
        *(uint2*)(dst + 32 * blk + 8 * q4) = pk;
      }
    if (p.lse != nullptr && h == 0) p.lse[orow] = lse_val;
    return;
  }
}

// One worker: locate its share of the group-mode stream and run its pieces.
template <bool kPaged, bool kCascade>
__device__ __forceinline__ void group_worker(const DecodeParams& p, GroupShared& sh) {
  const int H = p.num_heads;
  // The scales first: their loads overlap the planner's.
  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;

  const int w = blockIdx.x;
  int64_t W, x0, x1;
  int nw;
  PlanHit hit[2];
  if (!plan_lookup<kPaged, kThreads, kCascade>(
          p, [H](const Req& r) { return group_request_rows(r, H); },
          [&p, H](const Req& r) { clear_group_request(p, r, H); },
          w, sh.red, sh.hits, W, nw, x0, x1, hit))
    return;
  if (hit[0].b < 0 || (x1 < W && hit[1].b < 0)) return;  // not reached with consistent indptr
  const ReqSource src = source_of<kPaged, kCascade>(p);
  GCursor c;
  gcursor_in_request(c, hit[0].b, hit[0].r, x0 - hit[0].cum, H);
  uniformize(c);
  int64_t p1 = W;
  if (x1 < W) {
    GCursor c1;
    gcursor_in_request(c1, hit[1].b, hit[1].r, x1 - hit[1].cum, H);
    uniformize(c1);
    p1 = gsnap_at(x1, c1, H);
  }
  const int64_t p0 = gsnap_at(x0, c, H);
  if (p0 >= p1) return;
  if (p0 < x0) {
    c.k = 0;
  } else if (p0 > x0) {
    if (!gcursor_next_unit(c, src, p.batch, H)) return;
    uniformize(c);
  }
  const float cs = p.sm_scale * kLog2e * qs * ks;

  // Walk the share in stream rows (unit spans); each span's leading
  // kGroupPieceRows rows hold no entries, so a share may end with rows that
  // only charge a unit's start: no piece there.
  int64_t pos = p0;
  int piece = 0;
  while (pos < p1) {
    const int L = group_unit_len(c.r, H, c.u);
    const int span = L + kGroupPieceRows;
    const int n = (int)lmin((int64_t)(span - c.k), p1 - pos);
    if (n <= 0) break;  // not reached with a consistent plan
    int k0, len;
    group_piece_entries(c.k, n, k0, len);
    if (len > 0) {
      const bool complete = (k0 == 0 && len == L);
      const int slot_base =
          complete ? -1 : kGSlotsPerPiece * (2 * w + (piece == 0 ? 0 : 1));
      group_piece<kPaged, kCascade>(p, sh, c, uniform(k0), H, L, uniform(len), slot_base, w, cs,
                                    ks);
      ++piece;
    }
    pos += n;
    c.k += n;
    if (pos < p1 && c.k == span) {
      if (!gcursor_next_unit(c, src, p.batch, H)) break;
      uniformize(c);
    }
  }
}

// One workgroup per CU: the four waves (one per SIMD) each hold 256 O^T
// accumulators and use the whole register file.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_groups_fp8_kernel(const DecodeParams p) {
  __shared__ GroupShared sh;
  group_worker<false, false>(p, sh);
}

// The paged-cache build (page_size > 1).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_groups_fp8_paged_kernel(const DecodeParams p) {
  __shared__ GroupShared sh;
  group_worker<true, false>(p, sh);
}

// The one-launch shared-prefix (cascade) build.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_groups_fp8_cascade_kernel(const DecodeParams p) {
  __shared__ GroupShared sh;
  group_worker<false, true>(p, sh);
}

hipError_t launch_decode_groups(const DecodeParams& p, hipStream_t stream) {
  if (p.cascade_prefix >= 0)
    hipLaunchKernelGGL(mla_decode_groups_fp8_cascade_kernel, dim3(p.num_workers), dim3(kThreads), 0,
                       stream, p);
  else if (p.page_shift > 0)
    hipLaunchKernelGGL(mla_decode_groups_fp8_paged_kernel, dim3(p.num_workers), dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(mla_decode_groups_fp8_kernel, dim3(p.num_workers), dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace mla
