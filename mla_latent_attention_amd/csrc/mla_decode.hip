// mla_decode.hip - split-KV latent MLA decode for gfx950 (MI355X / CDNA4).
//
// What is computed ("[Kimi-K3 MLA TP8] MLA performance", ROCm/aiter issue
// 4541, Sec. 2 "K3 MLA geometry" and Sec. 5.2 "The kernel runs with
// page_size = 1"): for every query row (token t, head h) of request b,
//   s_i = sm_scale * q_scale * kv_scale * sum_{d<576} q[t,h,d] * pool[L_b[i], d]
//   o[t,h,:] = kv_scale * sum_i softmax(s)_i * pool[L_b[i], 0:512]
// over the entries L_b[i] the token may see, with lse = ln sum_i exp(s_i).
//
// Design (our own; the pages' assembly kernel is not available):
//   * One workgroup (4 waves, one per SIMD) per worker; the planner in
//     mla_plan.h hands each worker an equal share of the KV stream.
//   * Inside a piece the 4 waves take interleaved tiles of 18 KB of gathered
//     rows (32 fp8 rows or 16 bf16 rows) and run independent online softmaxes,
//     merged through LDS at the piece's end.
//   * Per tile a wave gathers its rows with 16-byte loads straight into VGPRs,
//     two tiles ahead of use, laid out as the A operand of the QK MFMA, so
//     Q.K^T runs from registers as S^T (kv x 16 rows) = K (kv x 576) . Q^T.
//   * The latent part of each row goes to a per-wave LDS tile (row-major,
//     padded stride); P.V reads it back transposed into the V^T A operand
//     (v_perm byte or half-word selects), so the contraction runs as
//     O^T (512 x 16 rows) += V^T . P^T on MFMA.
//   * P is fed as two terms, P = hi + lo (e4m3 for the fp8 path, bf16 for the
//     bf16 path), so the contraction sees ~8 (fp8) or ~16 (bf16) significant
//     bits of P; a single e4m3 P (4 bits) would not meet the output tolerance.
//   * Scores are kept in base 2 (log2(e) folded into the scale).  The running
//     max is only raised when a row's max grows by more than 2x, so the O^T
//     accumulators are rescaled on few tiles.
//   * Every load of the tile loop is unconditional (tail positions repeat the
//     piece's last entry and are masked), so the outstanding-load count is
//     static and the two-tile prefetch survives compilation.
//   * Split-KV partials are merged by a second, small kernel: each worker
//     leaves a descriptor for the split unit that starts in it, and the
//     combine kernel merges exactly those units by LSE.  (Merging inside the
//     decode would need device-scope fences, which write back and invalidate
//     the L2 of every XCD under the still-running workers.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_rope.h"

namespace mla {

// ---------------------------------------------------------------- tile loop

struct alignas(16) DecodeShared {
  uint8_t buf[kCombBytes];  // V staging during the tile loop, O^T exchange after it
  int32_t idx[kIdxSeg];     // kv_indices of the current segment of the piece
  int64_t red[kWaves];
  float m[kWaves][16];
  float l[kWaves][16];
  float dl[kWaves][16];
  PlanHit hits[2];
};

// The unit (query token, head group) a piece belongs to.
struct UnitRef {
  int t, g;
};

struct TileIdx {
  int i0, i1;  // pool rows this lane gathers: tile row (lane%16) and, for
               // 32-row tiles, tile row (16 + lane%16)
};

// Clamped address of byte 16*gq of pool row idx.
template <int kRowBytes>
__device__ __forceinline__ const uint8_t* row_ptr(const uint8_t* kv, int64_t pool_entries, int idx,
                                                  int gq) {
  int64_t r = idx < 0 ? 0 : (int64_t)idx;
  r = r < pool_entries ? r : pool_entries - 1;
  return kv + r * kRowBytes + 16 * gq;
}

// Copies a head group's 16 q rows (kLoads 16-byte loads per lane, row stride
// kRowBytes) from q0 into LDS at dst in lane order: entry 64c + l holds row
// l%16, bytes [64c + 16*(l/16), +16).  All loads are issued before the first
// store (the tail rereads the last entry).  Returns this lane's entry 0.
//
// The first kIdxBatch * kThreads kv_indices of the piece (n of them, n >= 1)
// are copied to idx_dst in the same pass, so the piece's start costs one
// memory round trip; the caller copies the rest.
template <int kLoads, int kRowBytes, bool kPaged>
__device__ __forceinline__ const uint4* stage_q(uint8_t* dst_bytes, const uint8_t* q0,
                                                int32_t* idx_dst, const DecodeParams& p,
                                                RowSrc idx_src, int n) {
  // Thread (wave wv, lane l) copies entries 64c + l for c = wv, wv + 4, ...:
  // one per-lane base address plus a wave-uniform offset per load.  Waves
  // past the last c repeat it (the same value to the same entry).
  uint4* dst = (uint4*)dst_bytes;
  constexpr int kPer = (kLoads + kWaves - 1) / kWaves;
  const int lane = threadIdx.x & 63, wv = uniform((int)(threadIdx.x >> 6));
  const uint8_t* src = q0 + (lane & 15) * kRowBytes + 16 * (lane >> 4);
  uint4 v[kPer];
  int32_t iv[kIdxBatch];
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = *(const uint4*)(src + 64 * imin(kWaves * k + wv, kLoads - 1));
  const int32_t* ibase = p.kv_indices + idx_src.ib;
  if constexpr (!kPaged) {
#pragma unroll
    for (int j = 0; j < kIdxBatch; ++j) iv[j] = ibase[imin(j * kThreads + (int)threadIdx.x, n - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < kIdxBatch; ++j)
      iv[j] = paged_row(ibase, p.page_shift,
                        idx_src.k0 + imin(j * kThreads + (int)threadIdx.x, n - 1));
  }
  // Stores are unconditional too (past-the-end lanes rewrite the last entry
  // with the value its owner writes): a conditional store would let the
  // compiler sink each load into its branch and serialise the round trips.
#pragma unroll
  for (int k = 0; k < kPer; ++k) dst[64 * imin(kWaves * k + wv, kLoads - 1) + lane] = v[k];
#pragma unroll
  for (int j = 0; j < kIdxBatch; ++j) idx_dst[imin(j * kThreads + (int)threadIdx.x, n - 1)] = iv[j];
  return dst + lane;
}

// ---- fp8 e4m3 path: 32-row tiles of 576-byte rows.
//
// Lane l (row n = l%16, group g = l/16) gathers tile rows n and 16 + n: for
// s = 0..3 the 32 bytes [128s + 32g, +32) of the latent dims, the operand of
// one v_mfma_scale_f32_16x16x128_f8f6f4 step (unit E8M0 scales), and the 16
// rope bytes [512 + 16g, +16), the operands of two v_mfma_f32_16x16x32_fp8_fp8
// steps, so Q.K^T runs from registers as S^T (kv x 16 rows) = K . Q^T in
// 4 x 32 + 2 x 16 = 160 cycles per 16 kv rows (eighteen 16x16x32 steps took
// 288).  q holds the same bytes of its rows, so the dims pair up whatever
// order the matrix cores sum them in.  The two step kinds keep separate
// accumulators (an MFMA must not read another kind's result as its
// accumulator), added at the end.  The latent 512 bytes go to a per-wave LDS
// tile; P.V reads 16 bytes from each of 8 rows and transposes 4x4 byte blocks
// (v_perm) into the V^T A operand: O^T (512 x 16 rows) += V^T . P^T.  P enters
// as two e4m3 terms, P*128 = hi + lo, which keeps ~8 significant bits of P (a
// single e4m3 P, 4 bits, would not meet the output tolerance).

constexpr int kFp8Tile = 32;
constexpr int kFp8VStride = 528;  // LDS bytes per staged V row (512 + pad)

__device__ __forceinline__ TileIdx fp8_fetch_idx(const int32_t* sidx, int rows, int tile, int n) {
  const int e0 = imin(tile * kFp8Tile + n, rows - 1);
  const int e1 = imin(tile * kFp8Tile + 16 + n, rows - 1);
  TileIdx t;
  t.i0 = sidx[e0];
  t.i1 = sidx[e1];
  return t;
}

// Byte offset of load c (0..8) of a row for lane group g: latent bytes
// [128(c/2) + 32g + 16(c%2), +16) for c < 8, rope bytes [512 + 16g, +16).
__device__ __forceinline__ int fp8_load_offset(int c, int g) {
  return c < 8 ? 128 * (c >> 1) + 32 * g + 16 * (c & 1) : kLatent + 16 * g;
}

__device__ __forceinline__ void fp8_issue_rows(uint4 (&B)[18], const uint8_t* kv,
                                               int64_t pool_entries, TileIdx ti, int gq) {
  const uint8_t* s0 = row_ptr<kRowDim>(kv, pool_entries, ti.i0, 0);
  const uint8_t* s1 = row_ptr<kRowDim>(kv, pool_entries, ti.i1, 0);
#pragma unroll
  for (int c = 0; c < 9; ++c) B[c] = *(const uint4*)(s0 + fp8_load_offset(c, gq));
#pragma unroll
  for (int c = 0; c < 9; ++c) B[9 + c] = *(const uint4*)(s1 + fp8_load_offset(c, gq));
}

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i as_v8i(uint4 a, uint4 b) {
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

struct Fp8Q {
  v8i m[4];   // q row lane%16, latent bytes [128s + 32*(lane/16), +32)
  long r[2];  // its rope bytes [512 + 16*(lane/16), +8) and [+8, +16)
};

// One 32-row tile: S^T = K.Q^T, online softmax, O^T += V^T.P^T.  With kRefill,
// B is refilled with the rows of `next` (two tiles ahead for this wave) right
// after its contents are consumed, and the indices four tiles ahead are fetched.
template <bool kRefill>
__device__ __forceinline__ void fp8_tile(WaveState& st, uint4 (&B)[18], TileIdx& next,
                                         const Fp8Q& q, uint8_t* vst, const DecodeParams& p,
                                         const int32_t* sidx, int rows, int tile, float cs, int n,
                                         int gq) {
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  v4f t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_v8i(B[2 * k], B[2 * k + 1]), q.m[k],
                                                           s0, 0, 0, 0, 127, 0, 127);
    s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_v8i(B[9 + 2 * k], B[10 + 2 * k]),
                                                           q.m[k], s1, 0, 0, 0, 127, 0, 127);
  }
  t0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(B[8].x, B[8].y), q.r[0], t0, 0, 0, 0);
  t1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(B[17].x, B[17].y), q.r[0], t1, 0, 0, 0);
  t0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(B[8].z, B[8].w), q.r[1], t0, 0, 0, 0);
  t1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(B[17].z, B[17].w), q.r[1], t1, 0, 0, 0);

  // Stage the latent 512 bytes of both 16-row blocks in this wave's LDS tile.
  wave_lds_sync();  // the previous tile's V reads are complete
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    *(uint4*)(vst + n * kFp8VStride + fp8_load_offset(c, gq)) = B[c];
    *(uint4*)(vst + (16 + n) * kFp8VStride + fp8_load_offset(c, gq)) = B[9 + c];
  }
  s0 += t0;
  s1 += t1;
  if constexpr (kRefill) {
    fp8_issue_rows(B, p.kv, p.pool_entries, next, gq);
    next = fp8_fetch_idx(sidx, rows, tile + 4 * kWaves, n);
  }

  // Row lane%16; this lane holds kv rows 4gq+i and 16+4gq+i.
  const int base = tile * kFp8Tile + 4 * gq;
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (base + i < rows) ? s0[i] * cs : neg_inf();
    x[4 + i] = (base + 16 + i < rows) ? s1[i] * cs : neg_inf();
  }
  softmax_update<8>(st, x);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= 128.0f;  // P * 128 <= 2^kLazy * 128 = 256 < 448

  // P*128 = hi + lo in e4m3; byte k of the operand = kv row kappa(gq, k).
  u32 h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h0, true);
  u32 h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
  h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], h1, true);
  float r[8];
  {
    const v2f32_t a = __builtin_amdgcn_cvt_pk_f32_fp8(h0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(h0, true);
    const v2f32_t c = __builtin_amdgcn_cvt_pk_f32_fp8(h1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(h1, true);
    r[0] = x[0] - a[0];
    r[1] = x[1] - a[1];
    r[2] = x[2] - b[0];
    r[3] = x[3] - b[1];
    r[4] = x[4] - c[0];
    r[5] = x[5] - c[1];
    r[6] = x[6] - d[0];
    r[7] = x[7] - d[1];
  }
  u32 l0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
  l0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], l0, true);
  u32 l1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[4], r[5], 0, false);
  l1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[6], r[7], l1, true);
  const long phi = as_long(h0, h1), plo = as_long(l0, l1);
  // o is normalised by the sum of the weights the MFMAs use (hi + lo, not P):
  // the split's rounding then moves o towards the entries it favours instead
  // of scaling it, an error bounded by |V - o| rather than |V|.  The lse
  // keeps the sum of P.
  st.dl = add_fp8x4(l1, add_fp8x4(l0, st.dl)) -
          (((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7])));

  // O^T += V^T . P^T; the kv row of operand byte k is kappa(gq, k):
  // 4gq + k for k < 4, 16 + 4gq + (k - 4) otherwise.
  wave_lds_sync();  // all lanes' V writes are in LDS
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = (k < 4) ? (4 * gq + k) : (16 + 4 * gq + (k - 4));
      v[k] = *(const uint4*)(vst + row * kFp8VStride + 16 * n + 256 * half);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      u32 a0, a1, a2, a3, b0, b1, b2, b3;
      const u32* w0 = (const u32*)&v[0];
      const u32* w1 = (const u32*)&v[1];
      const u32* w2 = (const u32*)&v[2];
      const u32* w3 = (const u32*)&v[3];
      const u32* w4 = (const u32*)&v[4];
      const u32* w5 = (const u32*)&v[5];
      const u32* w6 = (const u32*)&v[6];
      const u32* w7 = (const u32*)&v[7];
      transpose4x4(w0[qq], w1[qq], w2[qq], w3[qq], a0, a1, a2, a3);
      transpose4x4(w4[qq], w5[qq], w6[qq], w7[qq], b0, b1, b2, b3);
      const long A[4] = {as_long(a0, b0), as_long(a1, b1), as_long(a2, b2), as_long(a3, b3)};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int blk = half * 16 + 4 * qq + bb;
        st.O[blk] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(A[bb], phi, st.O[blk], 0, 0, 0);
        st.O[blk] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(A[bb], plo, st.O[blk], 0, 0, 0);
      }
    }
  }
}

struct Fp8Path {
  // Split partials in fp16 without the kv scale (pack_f16x2): half the bytes
  // of fp32 to write and read back, within the gate for the merged rows.
  static constexpr bool kHalfParts = true;
  static constexpr int kRowBytes = kRowDim;
  static constexpr int kTile = kFp8Tile;
  static constexpr int kVStride = kFp8VStride;
  static constexpr float kPScale = 128.0f;
  using Q = Fp8Q;
  // Q stays in registers (lane l: row l%16 of the unit's head group); its
  // loads go out with the piece's first index batch.
  template <bool kPaged>
  static __device__ __forceinline__ void load_q(Q& q, const DecodeParams& p, DecodeShared& sh,
                                                const UnitRef& u, RowSrc idx, int n) {
    const int lane = opaque((int)threadIdx.x) & 63;  // address built here, not held
    const uint8_t* qrow =
        p.q + ((int64_t)u.t * p.num_heads + u.g * kGroup + (lane & 15)) * kRowBytes;
    uint4 x[9];
#pragma unroll
    for (int c = 0; c < 9; ++c) x[c] = *(const uint4*)(qrow + fp8_load_offset(c, lane >> 4));
    stage_first_indices<kPaged>(sh.idx, p, idx, n);
#pragma unroll
    for (int k = 0; k < 4; ++k) q.m[k] = as_v8i(x[2 * k], x[2 * k + 1]);
    q.r[0] = as_long(x[8].x, x[8].y);
    q.r[1] = as_long(x[8].z, x[8].w);
  }
  static __device__ __forceinline__ TileIdx fetch_idx(const int32_t* sidx, int rows, int tile,
                                                      int n) {
    return fp8_fetch_idx(sidx, rows, tile, n);
  }
  static __device__ __forceinline__ void issue_rows(uint4 (&B)[18], const uint8_t* kv,
                                                    int64_t pool_entries, TileIdx ti, int gq) {
    fp8_issue_rows(B, kv, pool_entries, ti, gq);
  }
  template <bool kRefill>
  static __device__ __forceinline__ void tile(WaveState& st, uint4 (&B)[18], TileIdx& next,
                                              const Q& q, uint8_t* vst, const DecodeParams& p,
                                              const int32_t* sidx, int rows, int t, float cs,
                                              int n, int gq) {
    fp8_tile<kRefill>(st, B, next, q, vst, p, sidx, rows, t, cs, n, gq);
  }
  // O^T block b = 16*half + 4*qq + bb, element i, at lane (n, gq) is dim
  // 256*half + 64*gq + 16*i + 4*qq + bb.  Wave wv owns blocks [8wv, 8wv + 8):
  // dims first_dim(wv, gq) + kDimStride*i + (block - 8wv).
  static constexpr int kDimStride = 16;
  static __device__ __forceinline__ int first_dim(int wv, int gq) {
    return 256 * (wv >> 1) + 64 * gq + 8 * (wv & 1);
  }
};

// ---- bf16 path: 16-row tiles of 1152-byte rows (the same 18 KB per tile).
//
// Lane l gathers tile row (l%16), bytes [64c + 16*(l/16), +16) for c = 0..17:
// eight bf16 dims 32c + 8*(l/16) + j, the A operand of v_mfma_f32_16x16x32_bf16
// for K-block c, so S^T (16 kv x 16 rows) = K . Q^T runs from registers.  The
// S^T accumulator (lane holds kv rows 4*(l/16) + i of row l%16) is exactly the
// B operand of v_mfma_f32_16x16x16_bf16 (P^T), so P needs no reshuffle; the
// V^T A operand (dim l%16 of a block, kv rows 4*(l/16) + j) comes from four
// 16-byte LDS reads per lane and 16-bit v_perm selects.  P enters as
// P = hi + lo in bf16 (~16 significant bits).

constexpr int kBf16Tile = 16;
constexpr int kBf16RowBytes = 2 * kRowDim;  // 1152
constexpr int kBf16VStride = 1040;          // LDS bytes per staged V row (1024 + pad)

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef u32 v4u __attribute__((ext_vector_type(4)));
typedef u32 v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8bf as_v8bf(uint4 x) {
  return __builtin_bit_cast(v8bf, v4u{x.x, x.y, x.z, x.w});
}
__device__ __forceinline__ v4s as_v4s(u32 lo, u32 hi) {
  return __builtin_bit_cast(v4s, v2u{lo, hi});
}

__device__ __forceinline__ TileIdx bf16_fetch_idx(const int32_t* sidx, int rows, int tile, int n) {
  TileIdx t;
  t.i0 = sidx[imin(tile * kBf16Tile + n, rows - 1)];
  t.i1 = t.i0;
  return t;
}

__device__ __forceinline__ void bf16_issue_rows(uint4 (&B)[18], const uint8_t* kv,
                                                int64_t pool_entries, TileIdx ti, int gq) {
  const uint8_t* s0 = row_ptr<kBf16RowBytes>(kv, pool_entries, ti.i0, gq);
#pragma unroll
  for (int c = 0; c < 18; ++c) B[c] = *(const uint4*)(s0 + 64 * c);
}

// Q is staged once per piece in LDS, past the V tiles, in lane order: entry
// 64c + l holds q row l%16, bytes [64c + 16*(l/16), +16), so a wave reads the
// B operand of K-block c as 64 consecutive 16-byte words.  (Kept in registers
// it would cost 72 VGPRs per lane, which this path does not have.)
constexpr int kBf16QOffset = kWaves * kBf16Tile * kBf16VStride;  // 66,560
struct Bf16Q {
  const uint4* lds;  // this lane's entry of K-block 0
};

template <bool kRefill>
__device__ __forceinline__ void bf16_tile(WaveState& st, uint4 (&B)[18], TileIdx& next,
                                          const Bf16Q& q, uint8_t* vst, const DecodeParams& p,
                                          const int32_t* sidx, int rows, int tile, float cs, int n,
                                          int gq) {
  // Q operands come from LDS in groups of 6 K-blocks; the scheduling fences
  // keep the compiler from hoisting all 18 reads (72 VGPRs) at once.
  v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c0 = 0; c0 < 9; c0 += 3) {
#pragma unroll
    for (int c = c0; c < c0 + 3; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(B[c]), as_v8bf(q.lds[64 * c]), s0, 0, 0,
                                                   0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(B[9 + c]), as_v8bf(q.lds[64 * (9 + c)]),
                                                   s1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stage the latent 1024 bytes of the 16 rows in this wave's LDS tile.
  wave_lds_sync();  // the previous tile's V reads are complete
#pragma unroll
  for (int c = 0; c < 16; ++c) *(uint4*)(vst + n * kBf16VStride + 64 * c + 16 * gq) = B[c];
  if constexpr (kRefill) {
    bf16_issue_rows(B, p.kv, p.pool_entries, next, gq);
    next = bf16_fetch_idx(sidx, rows, tile + 4 * kWaves, n);
  }

  // Row lane%16; this lane holds kv rows 4gq+i.
  const int base = tile * kBf16Tile + 4 * gq;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (base + i < rows) ? (s0[i] + s1[i]) * cs : neg_inf();
  softmax_update<4>(st, x);

  // P = hi + lo, both bf16; element j of the operand is kv row 4gq + j.
  const u32 h01 = pack_bf16x2(x[0], x[1]), h23 = pack_bf16x2(x[2], x[3]);
  const u32 l01 = pack_bf16x2(x[0] - __uint_as_float(h01 << 16), x[1] - __uint_as_float(h01 & 0xFFFF0000u));
  const u32 l23 = pack_bf16x2(x[2] - __uint_as_float(h23 << 16), x[3] - __uint_as_float(h23 & 0xFFFF0000u));
  const v4s phi = as_v4s(h01, h23);
  const v4s plo = as_v4s(l01, l23);

  // O^T += V^T . P^T.  For c = 0..3 the lane reads dims [8m, 8m + 8) with
  // m = n + 16c of kv rows 4gq + j; word w of those 16 bytes holds dims 8m + 2w
  // (low half) and 8m + 2w + 1 (high half).  Block 8c + t takes dim 8m + t,
  // so O^T block 8c + t, element i, at lane (n, gq) is dim
  // 8 * (4gq + i + 16c) + t.
  wave_lds_sync();  // all lanes' V writes are in LDS
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *(const uint4*)(vst + (4 * gq + j) * kBf16VStride + 16 * n + 256 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32 r0 = ((const u32*)&v[0])[w], r1 = ((const u32*)&v[1])[w];
      const u32 r2 = ((const u32*)&v[2])[w], r3 = ((const u32*)&v[3])[w];
      const v4s ae = as_v4s(__builtin_amdgcn_perm(r1, r0, 0x05040100u),
                            __builtin_amdgcn_perm(r3, r2, 0x05040100u));
      const v4s ao = as_v4s(__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                            __builtin_amdgcn_perm(r3, r2, 0x07060302u));
      const int be = 8 * c + 2 * w, bo = be + 1;
      st.O[be] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, phi, st.O[be], 0, 0, 0);
      st.O[bo] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, phi, st.O[bo], 0, 0, 0);
      st.O[be] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, plo, st.O[be], 0, 0, 0);
      st.O[bo] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, plo, st.O[bo], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct Bf16Path {
  // Split partials in fp32: a bf16 cache's rows are not bounded by the e4m3
  // range that keeps fp16 partials finite.
  static constexpr bool kHalfParts = false;
  static constexpr int kRowBytes = kBf16RowBytes;
  static constexpr int kTile = kBf16Tile;
  static constexpr int kVStride = kBf16VStride;
  static constexpr float kPScale = 1.0f;
  using Q = Bf16Q;
  // Cooperative copy of the unit's 16 q rows into LDS; the caller synchronises
  // the block before the first tile reads it.
  template <bool kPaged>
  static __device__ __forceinline__ void load_q(Q& q, const DecodeParams& p, DecodeShared& sh,
                                                const UnitRef& u, RowSrc idx, int n) {
    q.lds = stage_q<18, kRowBytes, kPaged>(sh.buf + kBf16QOffset,
                                   p.q + ((int64_t)u.t * p.num_heads + u.g * kGroup) * kRowBytes,
                                   sh.idx, p, idx, n);
  }
  static __device__ __forceinline__ TileIdx fetch_idx(const int32_t* sidx, int rows, int tile,
                                                      int n) {
    return bf16_fetch_idx(sidx, rows, tile, n);
  }
  static __device__ __forceinline__ void issue_rows(uint4 (&B)[18], const uint8_t* kv,
                                                    int64_t pool_entries, TileIdx ti, int gq) {
    bf16_issue_rows(B, kv, pool_entries, ti, gq);
  }
  template <bool kRefill>
  static __device__ __forceinline__ void tile(WaveState& st, uint4 (&B)[18], TileIdx& next,
                                              const Q& q, uint8_t* vst, const DecodeParams& p,
                                              const int32_t* sidx, int rows, int t, float cs,
                                              int n, int gq) {
    bf16_tile<kRefill>(st, B, next, q, vst, p, sidx, rows, t, cs, n, gq);
  }
  // Block 8c + t, element i, at lane (n, gq) is dim 128c + 32gq + 8i + t; wave
  // wv owns blocks [8wv, 8wv + 8), i.e. c = wv.
  static constexpr int kDimStride = 8;
  static __device__ __forceinline__ int first_dim(int wv, int gq) { return 128 * wv + 32 * gq; }
};

static_assert(kWaves * kFp8Tile * kFp8VStride <= kCombBytes, "fp8 V staging must fit in LDS");
static_assert(kBf16QOffset + 18 * 64 * 16 <= kCombBytes, "bf16 V staging and Q must fit in LDS");

// ---------------------------------------------------------------- pieces

// One piece: the `rows` entries of unit u whose pool rows `src` gives.  slot < 0
// means the piece is the whole unit and o / lse are written directly.
//
// The 4 waves take interleaved tiles (wave wv: tiles wv, wv + 4, ...) and run
// independent online softmaxes over them, merged through LDS at the end.  A
// wave keeps two tiles of rows in flight in registers (bufA / bufB), each
// refilled right after its contents are consumed; every load is unconditional
// (positions past the segment repeat its last index and are masked), so the
// outstanding-load count stays static and the prefetch survives compilation.
// Indices are staged in LDS per segment, off the vector-memory counter.
template <class Path, bool kPaged>
__device__ __forceinline__ void decode_piece(const DecodeParams& p, DecodeShared& sh,
                                             const UnitRef& u, RowSrc src, int rows, int slot,
                                             float cs, float ks) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, gq = lane >> 4;
  __syncthreads();  // the previous piece is done with the LDS buffer

  typename Path::Q q;
  Path::template load_q<kPaged>(q, p, sh, u, src, imin(rows, kIdxSeg));

  WaveState st;
#pragma unroll
  for (int b = 0; b < 32; ++b) st.O[b] = v4f{0.f, 0.f, 0.f, 0.f};
  st.m = neg_inf();
  st.l = 0.f;
  st.dl = 0.f;

  uint8_t* vst = sh.buf + wv * Path::kTile * Path::kVStride;
  for (int seg0 = 0; seg0 < rows; seg0 += kIdxSeg) {
    const int srows = imin(kIdxSeg, rows - seg0);
    if (seg0 > 0) __syncthreads();  // the previous segment's index reads are done
    // The first kIdxBatch * kThreads indices of segment 0 came with Q.
    stage_indices<kPaged>(sh.idx, p, src.template at<kPaged>(seg0),
                          seg0 == 0 ? kIdxBatch * kThreads : 0, srows);
    __syncthreads();
    const int32_t* sidx = sh.idx;
    const int ntiles = (srows + Path::kTile - 1) / Path::kTile;
    const int m = ntiles > wv ? (ntiles - wv + kWaves - 1) / kWaves : 0;  // this wave's tiles
    if (m > 0) {
      // wave tile k is tile wv + 4k; even k live in bufA, odd k in bufB.
      uint4 bufA[18], bufB[18];
      TileIdx nextA, nextB;
      {
        const TileIdx t0 = Path::fetch_idx(sidx, srows, wv, n);
        const TileIdx t1 = Path::fetch_idx(sidx, srows, wv + kWaves, n);
        Path::issue_rows(bufA, p.kv, p.pool_entries, t0, gq);
        Path::issue_rows(bufB, p.kv, p.pool_entries, t1, gq);
        nextA = Path::fetch_idx(sidx, srows, wv + 2 * kWaves, n);
        nextB = Path::fetch_idx(sidx, srows, wv + 3 * kWaves, n);
      }
      int k = 0;
      for (; k + 3 < m; k += 2) {
        Path::template tile<true>(st, bufA, nextA, q, vst, p, sidx, srows, wv + kWaves * k, cs, n,
                                  gq);
        Path::template tile<true>(st, bufB, nextB, q, vst, p, sidx, srows, wv + kWaves * (k + 1),
                                  cs, n, gq);
      }
      const int rem = m - k;
      if (rem == 3) {
        Path::template tile<true>(st, bufA, nextA, q, vst, p, sidx, srows, wv + kWaves * k, cs, n,
                                  gq);
        Path::template tile<false>(st, bufB, nextB, q, vst, p, sidx, srows, wv + kWaves * (k + 1),
                                   cs, n, gq);
        Path::template tile<false>(st, bufA, nextA, q, vst, p, sidx, srows, wv + kWaves * (k + 2),
                                   cs, n, gq);
      } else if (rem == 2) {
        Path::template tile<false>(st, bufA, nextA, q, vst, p, sidx, srows, wv + kWaves * k, cs, n,
                                   gq);
        Path::template tile<false>(st, bufB, nextB, q, vst, p, sidx, srows, wv + kWaves * (k + 1),
                                   cs, n, gq);
      } else if (rem == 1) {
        Path::template tile<false>(st, bufA, nextA, q, vst, p, sidx, srows, wv + kWaves * k, cs, n,
                                   gq);
      }
    }
  }

  // ---- merge the 4 waves' online-softmax states
  // The per-lane LDS and output addresses from here on are rebuilt from an
  // opaque thread id.
  const int etid = opaque(tid), elane = etid & 63, ewv = etid >> 6, en = elane & 15,
            egq = elane >> 4;
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
  st.dl += __shfl_xor(st.dl, 16);
  st.dl += __shfl_xor(st.dl, 32);
  __syncthreads();  // every wave is done with its V staging
  if (egq == 0) {
    sh.m[ewv][en] = st.m;
    sh.l[ewv][en] = st.l;
    sh.dl[ewv][en] = st.dl;
  }
  v4f* comb = (v4f*)sh.buf;
#pragma unroll
  for (int b = 0; b < 32; ++b) comb[(ewv * 32 + b) * 64 + elane] = st.O[b];
  __syncthreads();

  float mw[kWaves], M = neg_inf();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = sh.m[w][en];
    M = fmaxf(M, mw[w]);
  }
  float fw[kWaves], L = 0.f, DL = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    fw[w] = (mw[w] == neg_inf()) ? 0.f : fast_exp2(mw[w] - M);
    L += sh.l[w][en] * fw[w];
    DL += sh.dl[w][en] * fw[w];
  }
  // fp16 split partials leave out the kv scale (the combine applies it).
  // o over the weights' sum, L * kPScale + DL (the lse takes L).
  const bool half_parts = Path::kHalfParts && slot >= 0 && !p.part_fp32;
  const float oscale = (half_parts ? 1.0f : ks) / __builtin_fmaf(Path::kPScale, L, DL);

  // This wave writes O^T blocks [8wv, 8wv + 8); element i of block 8wv + bb is
  // dim first_dim + kDimStride*i + bb.
  float acc[4][8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += fw[w] * comb[(w * 32 + 8 * ewv + bb) * 64 + elane];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][bb] = a[i] * oscale;
  }
  const int dim0 = Path::first_dim(ewv, egq);
  const float lse_val = (M + fast_log2(L)) * kLn2;
  if (slot < 0) {
    const int64_t orow = (int64_t)u.t * p.num_heads + u.g * kGroup + en;
    if (p.o32 != nullptr) {
      float* d32 = p.o32 + orow * kLatent + dim0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* d = d32 + Path::kDimStride * i;
        *(float4*)d = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        *(float4*)(d + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
      }
    } else {
      uint16_t* dst = p.o + orow * kLatent + dim0;
#pragma unroll
      for (int i = 0; i < 4; ++i) store_bf16x8(dst + Path::kDimStride * i, acc[i]);
    }
    if (p.lse != nullptr && ewv == 0 && egq == 0) p.lse[orow] = lse_val;
    return;
  }
  if (half_parts) {
    // fp16 at the fp32 layout's element indices, in the first half of the
    // region.
    uint16_t* dst = (uint16_t*)p.part_o + ((int64_t)slot * kGroup + en) * kLatent + dim0;
#pragma unroll
    for (int i = 0; i < 4; ++i) store_f16x8(dst + Path::kDimStride * i, acc[i]);
  } else {
    float* dst = p.part_o + ((int64_t)slot * kGroup + en) * kLatent + dim0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* d = dst + Path::kDimStride * i;
      *(float4*)d = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      *(float4*)(d + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
  }
  if (ewv == 0 && egq == 0) p.part_lse[(int64_t)slot * kGroup + en] = lse_val;
}

// One worker: locate its share of the KV stream and run its pieces.
// This worker's range [p0, p1) of the stream and the cursor at p0: the
// equal-share boundaries, each snapped to a unit boundary within kSnapRows
// (0 and W are boundaries already).  The lookup also zeroes the empty tokens
// this block owns.  False: the worker has nothing to do.  All threads call it.
template <bool kPaged>
__device__ __forceinline__ bool plan_worker(const DecodeParams& p, int64_t* red, PlanHit* hits,
                                            Cursor& c, int64_t& p0, int64_t& p1) {
  const int G = p.num_heads / kGroup;
  const int w = blockIdx.x;
  int64_t W, x0, x1;
  int nw;
  PlanHit hit[2];
  if (!plan_lookup<kPaged, kThreads, false>(
          p, [G](const Req& r) { return (int64_t)G * request_rows(r); },
          [&p](const Req& r) {
            const int nempty = req_empty_tokens(r);
            for (int j = 0; j < nempty; ++j)
              if ((r.q_base + j) % p.num_workers == (int)blockIdx.x) zero_token(p, r.q_base + j);
          },
          w, red, hits, W, nw, x0, x1, hit))
    return false;
  if (hit[0].b < 0 || (x1 < W && hit[1].b < 0)) return false;  // not with consistent indptr
  const ReqSource src = source_of<kPaged>(p);
  cursor_in_request(c, hit[0].b, hit[0].r, x0 - hit[0].cum, G);
  uniformize(c);
  p1 = W;
  if (x1 < W) {
    Cursor c1;
    cursor_in_request(c1, hit[1].b, hit[1].r, x1 - hit[1].cum, G);
    uniformize(c1);
    p1 = snap_at(x1, c1);
  }
  p0 = snap_at(x0, c);
  if (p0 >= p1) return false;
  if (p0 < x0) {
    c.k = 0;  // moved back to the start of its unit
  } else if (p0 > x0) {  // moved forward past the end of its unit
    if (!cursor_next_unit(c, src, p.batch, G)) return false;
    uniformize(c);
  }
  return true;
}

// kPlanned: the plan comes from p.plans (the layer step's prologue kernel
// computed it) instead of the planner.
template <class Path, bool kPaged, bool kPlanned = false>
__device__ __forceinline__ void decode_worker(const DecodeParams& p, DecodeShared& sh) {
  const int G = p.num_heads / kGroup;
  // The scales first: their loads overlap the planner's.
  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;
  const int w = blockIdx.x;
  Cursor c;
  int64_t p0, p1;
  if constexpr (kPlanned) {
    const WorkerPlan& wp = p.plans[w];
    if (!uniform(wp.ok)) return;
    p0 = uniform(wp.p0);
    p1 = uniform(wp.p1);
    c = wp.c;
    uniformize(c);
  } else {
    if (!plan_worker<kPaged>(p, sh.red, sh.hits, c, p0, p1)) return;
  }
  const ReqSource src = source_of<kPaged>(p);
  const float cs = p.sm_scale * kLog2e * qs * ks;

  int64_t pos = p0;
  int piece = 0;
  while (pos < p1) {
    const int v = req_visible(c.r, c.j);
    const int len = (int)lmin((int64_t)(v - c.k), p1 - pos);
    if (len <= 0) break;  // not reached with a consistent plan
    const bool complete = (c.k == 0 && len == v);
    const int slot = complete ? -1 : (piece == 0 ? 2 * w : 2 * w + 1);
    UnitRef u;
    u.t = c.r.q_base + c.j;
    u.g = c.g;
    if (threadIdx.x == 0) {
      // Split-unit descriptor for the combine pass {first worker, last worker,
      // slot of the first worker, split?}: the worker holding the unit's first
      // piece writes fields 0, 2 and 3, the one holding its last piece field 1.
      // The unit is merged from the first worker's slot and slot 2w' of every
      // later worker w' up to the last.  (Written before the piece runs, so
      // none of this stays live across its tile loop.)
      int* d = (int*)(p.desc + ((int64_t)u.t * G + u.g));
      const int wv = opaque(w);  // moved to a vector register here, not held
      if (c.k == 0) {
        d[0] = wv;
        d[2] = slot;
        d[3] = complete ? 0 : 1;
      }
      if (!complete && c.k + len == v) d[1] = wv;
    }
    decode_piece<Path, kPaged>(p, sh, u, row_src<kPaged>(c.r, c.k), len, slot, cs, ks);
    pos += len;
    c.k += len;
    ++piece;
    if (pos < p1 && c.k == v) {
      if (!cursor_next_unit(c, src, p.batch, G)) break;
      uniformize(c);
    }
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8_kernel(const DecodeParams p) {
  __shared__ DecodeShared sh;
  decode_worker<Fp8Path, false>(p, sh);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_bf16_kernel(const DecodeParams p) {
  __shared__ DecodeShared sh;
  decode_worker<Bf16Path, false>(p, sh);
}

// The layer step's decode (fp8, page_size 1): the standard kernel on the plan
// and q rows the step's prologue kernel left in the workspace.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8_planned_kernel(const DecodeParams p) {
  __shared__ DecodeShared sh;
  decode_worker<Fp8Path, false, true>(p, sh);
}

// The layer step's prologue: blocks 0 .. num_workers-1 compute and store the
// decode workers' plans (and zero the empty tokens, as the decode's planner
// does); the blocks after them do the rope / fp8 / cache-write step, one
// chunk of 8 codes per thread (q rows of every padded head, then each token's
// new cache entry), so both run side by side.  The stores reach the decode at
// the kernel boundary.
struct PrologueShared {
  int64_t red[kWaves];
  PlanHit hits[2];
};

__global__ __launch_bounds__(kThreads) void mla_step_prologue_kernel(const DecodeParams p) {
  __shared__ PrologueShared sh;
  if ((int)blockIdx.x >= p.num_workers) {
    const int Hp = p.num_heads;
    const int per_token = (Hp + 1) * kChunksPerRow;
    const int64_t it = (int64_t)(blockIdx.x - p.num_workers) * kThreads + threadIdx.x;
    if (it >= (int64_t)p.num_tokens * per_token) return;
    const int t = (int)(it / per_token);
    const int rem = (int)(it - (int64_t)t * per_token);
    const int row = rem / kChunksPerRow;
    rope_quant_item(p.q_latent, p.q_pe, p.k_latent, p.k_pe, p.positions, p.cos_sin, p.max_pos,
                    p.rope_style, p.q_out, p.real_heads, Hp, p.kv_out, p.pool_entries,
                    p.slot_mapping, p.q_scale, p.kv_scale, t, row, rem - row * kChunksPerRow);
    return;
  }
  Cursor c;
  int64_t p0 = 0, p1 = 0;
  const bool ok = plan_worker<false>(p, sh.red, sh.hits, c, p0, p1);
  if (threadIdx.x == 0) {
    WorkerPlan& wp = p.plans[blockIdx.x];
    wp.ok = ok ? 1 : 0;
    wp.p0 = p0;
    wp.p1 = p1;
    wp.c = c;
  }
}

// Paged-cache builds (page_size > 1).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8_paged_kernel(const DecodeParams p) {
  __shared__ DecodeShared sh;
  decode_worker<Fp8Path, true>(p, sh);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_bf16_paged_kernel(const DecodeParams p) {
  __shared__ DecodeShared sh;
  decode_worker<Bf16Path, true>(p, sh);
}

// ---------------------------------------------------------------- split combine

// grid (units, 32) of four-wave blocks: block (u, 2n + h) merges row n, dims
// [256h, 256h + 256) of unit u = t * G + g if it was split, 4 dims per lane:
// M = max lse_s, o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// The slots are the first worker's own and, for each later worker w', the
// slot of its first piece: kSlots * w' + (position of the row group within
// its piece), i.e. first_slot mod (kSlots / 2) (0 in the standard mode, with
// kSlots = 2; the row group within the unit in group mode, with kSlots = 16).
// Up to 16 slots are merged by the first wave alone; beyond that wave wv takes
// batches wv, wv + 4, ... of 16 slots and the four partial merges are merged
// once more through LDS, so a unit split over many workers costs a quarter of
// the dependent load rounds.
constexpr int kCombineWaves = 4;
constexpr int kCombineThreads = 64 * kCombineWaves;
constexpr int kCombineBatch = 16;

template <int kHalves>
struct CombineShared {
  float4 acc[kCombineWaves][kHalves][64];
  float m[kCombineWaves];
  float sum[kCombineWaves];
};

// The merge of row n of split unit d (its descriptor) over its slots, for
// kHalves consecutive 256-dim halves from h0: lane l takes dims
// 256 (h0 + i) + 4l .. + 3 of half i.  On return the wave that holds the
// result (wave 0; the return value says which) has the unnormalised sums in
// acc, the row's running maximum in M and its weight sum in sum.  All four
// waves of the block must call it (the many-slot path meets at a barrier);
// every element goes through the same operations whatever kHalves is.
template <int kSlots, bool kHalfParts, int kHalves>
__device__ __forceinline__ bool combine_row(const DecodeParams& p, CombineShared<kHalves>& sh,
                                            const int4 d, int n, int h0,
                                            float4 (&acc)[kHalves], float& M, float& sum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int w0 = d.x, S = d.y - d.x + 1;
  const bool many = S > kCombineBatch;  // uniform over the block
  const int pos = d.z % (kSlots / 2);
  auto slot_of = [&](int i) -> int64_t {
    return i == 0 ? (int64_t)d.z : (int64_t)kSlots * (w0 + i) + pos;
  };

  // Slots in batches: every load of a batch is issued before any is used,
  // with an online rescale across batches.  A slot whose lse is -inf (its
  // piece held none of the row's visible entries) gets weight 0.  With at
  // most kCombineBatch slots only wave 0 has a batch.
  M = neg_inf();
  sum = 0.f;
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) acc[hf] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int step = many ? kCombineWaves * kCombineBatch : kCombineBatch;
  for (int i0 = wv * kCombineBatch; i0 < S; i0 += step) {
    float4 x[kCombineBatch][kHalves];
    float ls[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {  // past-the-end slots reload the last one, weight 0
      const int64_t slot = slot_of(imin(i0 + j, S - 1));
      ls[j] = p.part_lse[slot * kGroup + n];
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        const int64_t e0 = (slot * kGroup + n) * kLatent + 256 * (h0 + hf) + 4 * lane;
        if constexpr (kHalfParts) {
          const uint2 b = *(const uint2*)((const uint16_t*)p.part_o + e0);
          const float2 lo = unpack_f16x2(b.x), hi = unpack_f16x2(b.y);
          x[j][hf] = make_float4(lo.x, lo.y, hi.x, hi.y);
        } else {
          x[j][hf] = *(const float4*)(p.part_o + e0);
        }
      }
    }
    // Keep the scheduler from interleaving these loads with their uses, which
    // would leave only a couple in flight at a time.
    __builtin_amdgcn_sched_barrier(0);
    float bm = M;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j)
      if (i0 + j < S) bm = fmaxf(bm, ls[j]);
    if (bm == neg_inf()) continue;  // nothing visible yet: acc and sum stay 0
    const float alpha = (M == neg_inf()) ? 0.f : fast_exp2((M - bm) * kLog2e);
    sum *= alpha;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      acc[hf].x *= alpha;
      acc[hf].y *= alpha;
      acc[hf].z *= alpha;
      acc[hf].w *= alpha;
    }
    M = bm;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const float wt = (i0 + j < S) ? fast_exp2((ls[j] - M) * kLog2e) : 0.f;
      sum += wt;
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        acc[hf].x += wt * x[j][hf].x;
        acc[hf].y += wt * x[j][hf].y;
        acc[hf].z += wt * x[j][hf].z;
        acc[hf].w += wt * x[j][hf].w;
      }
    }
  }
  if (many) {
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) sh.acc[wv][hf][lane] = acc[hf];
    if (lane == 0) {
      sh.m[wv] = M;
      sh.sum[wv] = sum;
    }
    __syncthreads();
    if (wv != 0) return false;
    M = neg_inf();
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) M = fmaxf(M, sh.m[i]);
    sum = 0.f;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) acc[hf] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) {
      const float wt = (sh.m[i] == neg_inf()) ? 0.f : fast_exp2((sh.m[i] - M) * kLog2e);
      sum += wt * sh.sum[i];
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        const float4 a = sh.acc[i][hf][lane];
        acc[hf].x += wt * a.x;
        acc[hf].y += wt * a.y;
        acc[hf].z += wt * a.z;
        acc[hf].w += wt * a.w;
      }
    }
  }
  return wv == 0;
}

template <int kSlots, bool kHalfParts>
__device__ __forceinline__ void combine_unit(const DecodeParams& p, CombineShared<1>& sh) {
  const int64_t u = blockIdx.x;
  const int4 d = p.desc[u];
  // Group mode: the row group's first token and head and its row count (rows
  // are packed when the head count is not a multiple of 16), loaded beside
  // the descriptor rather than after it.
  int2 rr = make_int2(0, 0);
  if constexpr (kSlots != 2) rr = p.desc_rows[u];
  if (d.w == 0) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = blockIdx.y >> 1, h = blockIdx.y & 1;
  // The row's place in o: unit u = token * G + head group in the standard
  // kernels, the descriptor's rows in group mode.
  int64_t orow;
  if constexpr (kSlots == 2) {
    const int G = p.num_heads / kGroup;
    orow = (u / G) * p.num_heads + (u % G) * kGroup + n;
  } else {
    if (n >= (rr.y & 31)) return;  // past the last row of a partial row group
    orow = (int64_t)rr.x * p.num_heads + (rr.y >> 5) + n;
  }
  if (d.y - d.x + 1 <= kCombineBatch && wv != 0) return;  // one wave merges up to a batch
  float4 acc[1];
  float M, sum;
  if (!combine_row<kSlots, kHalfParts, 1>(p, sh, d, n, h, acc, M, sum)) return;
  // fp16 partials carry no kv scale: applied here, with the normalisation.
  const float ks = kHalfParts && p.kv_scale != nullptr ? *p.kv_scale : 1.0f;
  const float inv = sum > 0.f ? ks / sum : 0.f;  // a row that sees nothing: o = 0, lse = -inf
  if (p.o32 != nullptr) {
    *(float4*)(p.o32 + orow * kLatent + 256 * h + 4 * lane) =
        make_float4(acc[0].x * inv, acc[0].y * inv, acc[0].z * inv, acc[0].w * inv);
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(acc[0].x * inv, acc[0].y * inv);
    pk.y = pack_bf16x2(acc[0].z * inv, acc[0].w * inv);
    *(uint2*)(p.o + orow * kLatent + 256 * h + 4 * lane) = pk;
  }
  if (p.lse != nullptr && h == 0 && lane == 0)
    p.lse[orow] = sum > 0.f ? M + fast_log2(sum) * kLn2 : neg_inf();
}

// The standard kernels' split combine: fp8 caches leave fp16 partials, bf16
// caches fp32 ones.
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(const DecodeParams p) {
  __shared__ CombineShared<1> sh;
  combine_unit<2, true>(p, sh);
}

__global__ __launch_bounds__(kCombineThreads) void mla_combine_fp32_kernel(const DecodeParams p) {
  __shared__ CombineShared<1> sh;
  combine_unit<2, false>(p, sh);
}

__global__ __launch_bounds__(kCombineThreads) void mla_combine_groups_kernel(const DecodeParams p) {
  __shared__ CombineShared<1> sh;
  combine_unit<2 * kGroupsPerUnit, true>(p, sh);
}

// Group mode with fp32 partials (calls whose output is fp32).
__global__ __launch_bounds__(kCombineThreads) void mla_combine_groups_fp32_kernel(
    const DecodeParams p) {
  __shared__ CombineShared<1> sh;
  combine_unit<2 * kGroupsPerUnit, false>(p, sh);
}

// The fused layer step's tail: the split combine and the latent -> v map in
// one launch ("[Kimi-K3 MLA TP8] MLA performance", Sec. 3: a batched GEMM maps
// each head's 512-dim latent output to v_head_dim = 128, Sec. 2).  grid
// (T * H_pad) blocks of four waves, block (t, h): row h of token t's unit is
// merged from its partials if the unit was split (the same arithmetic as
// mla_combine_kernel, written to o and lse) or read back from o if the decode
// wrote it whole; then, for a real head, out[t, h, :] = o[t, h, :] . W[h]^T on
// v_mfma_f32_16x16x32_bf16 with the bf16 row in every A row and the same
// operand order and k steps as mla_latent_to_v_kernel, so each output is the
// one that kernel gives for this row.  Wave w computes outputs
// [32w, 32w + 32); its W operands are in flight from the block's start.
__global__ __launch_bounds__(kCombineThreads) void mla_combine_v_kernel(const DecodeParams p,
                                                                        const uint16_t* w_uv,
                                                                        uint16_t* vout) {
  __shared__ CombineShared<2> sh;
  __shared__ __align__(16) uint16_t orow[kLatent];
  const int Hp = p.num_heads, G = Hp / kGroup;
  const int t = blockIdx.x / Hp, h = blockIdx.x - t * Hp;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool real = h < p.real_heads;

  uint4 b[2][16];
  if (real) {
    const uint16_t* wrow = w_uv + ((int64_t)h * 128 + 32 * wv + (lane & 15)) * kLatent + 8 * (lane >> 4);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < 16; ++s) b[nt][s] = *(const uint4*)(wrow + nt * 16 * kLatent + 32 * s);
  }

  const int64_t u = (int64_t)t * G + h / kGroup;
  const int n = h % kGroup;
  const int64_t orow_g = (int64_t)t * Hp + h;
  const int4 d = p.desc[u];
  if (d.w == 0) {  // a complete unit: the decode wrote the row
    if (wv == 0) *(uint4*)(orow + 8 * lane) = *(const uint4*)(p.o + orow_g * kLatent + 8 * lane);
  } else {
    float4 acc[2];
    float M, sum;
    if (combine_row<2, true, 2>(p, sh, d, n, 0, acc, M, sum)) {
      const float ks = p.kv_scale != nullptr ? *p.kv_scale : 1.0f;  // fp16 partials carry none
      const float inv = sum > 0.f ? ks / sum : 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[hf].x * inv, acc[hf].y * inv);
        pk.y = pack_bf16x2(acc[hf].z * inv, acc[hf].w * inv);
        *(uint2*)(p.o + orow_g * kLatent + 256 * hf + 4 * lane) = pk;
        *(uint2*)(orow + 256 * hf + 4 * lane) = pk;
      }
      if (p.lse != nullptr && lane == 0)
        p.lse[orow_g] = sum > 0.f ? M + fast_log2(sum) * kLn2 : neg_inf();
    }
  }
  __syncthreads();
  if (!real) return;
  v4f acc2[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const uint4 a = *(const uint4*)(orow + 8 * (lane >> 4) + 32 * s);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      acc2[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(a), as_v8bf(b[nt][s]), acc2[nt],
                                                         0, 0, 0);
  }
  // Element 0 of lanes 0..15: A row 0, output dim 32 wv + 16 nt + lane.
  if (lane < 16) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint32_t x = __float_as_uint(acc2[nt][0]);
      x += 0x7FFFu + ((x >> 16) & 1u);  // round to nearest even
      vout[((int64_t)t * p.real_heads + h) * 128 + 32 * wv + 16 * nt + lane] = (uint16_t)(x >> 16);
    }
  }
}

// ---------------------------------------------------------------- shard merge

// One wave per (token, head) row, 8 dims per lane.  Shards are taken in
// batches of kMergeBatch: all lse loads of a batch, then all row loads, are in
// flight before any is used (indices past S reload shard S-1 with weight 0),
// with an online rescale across batches.  An empty shard (lse = -inf) gets
// weight 0 through a select, so whatever its row holds (even NaN) is ignored.
constexpr int kMergeBatch = 8;

template <bool kFp32Parts>
__device__ __forceinline__ void load_part_row(const void* o_parts, int64_t off, float (&x)[8]) {
  if constexpr (kFp32Parts) {
    const float* src = (const float*)o_parts + off;
    const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 v = *(const uint4*)((const uint16_t*)o_parts + off);
    const u32 wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(wds[k] << 16);
      x[2 * k + 1] = __uint_as_float(wds[k] & 0xFFFF0000u);
    }
  }
}

template <bool kFp32Parts>
__global__ __launch_bounds__(kThreads) void mla_merge_kernel(const void* o_parts,
                                                             const float* lse_parts, int S,
                                                             int64_t rows, uint16_t* o,
                                                             float* lse) {
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float M = neg_inf(), sum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
    float ls[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      ls[j] = lse_parts[(int64_t)imin(s0 + j, S - 1) * rows + row];
    float x[kMergeBatch][8];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      load_part_row<kFp32Parts>(o_parts, ((int64_t)imin(s0 + j, S - 1) * rows + row) * kLatent +
                                             8 * lane, x[j]);
    __builtin_amdgcn_sched_barrier(0);
    float bm = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (s0 + j < S) bm = fmaxf(bm, ls[j]);
    if (bm == neg_inf()) continue;  // every shard so far is empty
    const float alpha = (M == neg_inf()) ? 0.f : fast_exp2((M - bm) * kLog2e);
    sum *= alpha;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= alpha;
    M = bm;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool live = (s0 + j < S) && ls[j] != neg_inf();
      const float wt = live ? fast_exp2((ls[j] - M) * kLog2e) : 0.f;
      sum += wt;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += live ? wt * x[j][d] : 0.f;
    }
  }
  uint16_t* dst = o + row * kLatent + 8 * lane;
  if (M == neg_inf()) {
    *(uint4*)dst = make_uint4(0, 0, 0, 0);
    if (lse != nullptr && lane == 0) lse[row] = neg_inf();
    return;
  }
  const float inv = 1.0f / sum;
  uint4 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *(uint4*)dst = pk;
  if (lse != nullptr && lane == 0) lse[row] = M + fast_log2(sum) * kLn2;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, bool group_mode, hipStream_t stream) {
  hipError_t e;
  if (group_mode && kv_dtype == 0)
    e = launch_decode_groups(p, stream);
  else if (kv_dtype == 0 || kv_dtype == 1) {
    const bool paged = p.page_shift > 0;
    if (kv_dtype == 0 && !paged)
      hipLaunchKernelGGL(mla_decode_fp8_kernel, dim3(p.num_workers), dim3(kThreads), 0, stream, p);
    else if (kv_dtype == 0)
      hipLaunchKernelGGL(mla_decode_fp8_paged_kernel, dim3(p.num_workers), dim3(kThreads), 0,
                         stream, p);
    else if (!paged)
      hipLaunchKernelGGL(mla_decode_bf16_kernel, dim3(p.num_workers), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(mla_decode_bf16_paged_kernel, dim3(p.num_workers), dim3(kThreads), 0,
                         stream, p);
    e = hipGetLastError();
  } else {
    return hipErrorNotSupported;
  }
  if (e != hipSuccess) return e;
  const unsigned units =
      (unsigned)(p.num_tokens * (group_mode ? group_slots_per_token(p.num_heads)
                                            : p.num_heads / kGroup));
  if (group_mode && kv_dtype == 0 && p.part_fp32)
    hipLaunchKernelGGL(mla_combine_groups_fp32_kernel, dim3(units, 2 * kGroup),
                       dim3(kCombineThreads), 0, stream, p);
  else if (group_mode && kv_dtype == 0)
    hipLaunchKernelGGL(mla_combine_groups_kernel, dim3(units, 2 * kGroup), dim3(kCombineThreads), 0,
                       stream, p);
  else if (kv_dtype == 0 && !p.part_fp32)
    hipLaunchKernelGGL(mla_combine_kernel, dim3(units, 2 * kGroup), dim3(kCombineThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(mla_combine_fp32_kernel, dim3(units, 2 * kGroup), dim3(kCombineThreads), 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeParams& p, const uint16_t* w_uv, uint16_t* vout,
                              hipStream_t stream) {
  const int64_t rope_items = (int64_t)p.num_tokens * (p.num_heads + 1) * kChunksPerRow;
  const int64_t blocks = p.num_workers + (rope_items + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_step_prologue_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_decode_fp8_planned_kernel, dim3(p.num_workers), dim3(kThreads), 0, stream,
                     p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_v_kernel, dim3((unsigned)(p.num_tokens * p.num_heads)),
                     dim3(kCombineThreads), 0, stream, p, w_uv, vout);
  return hipGetLastError();
}

hipError_t launch_merge(const void* o_parts, int parts_fp32, const float* lse_parts, int num_parts,
                        int64_t rows, uint16_t* o, float* lse, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + kWaves - 1) / kWaves);
  if (parts_fp32)
    hipLaunchKernelGGL(mla_merge_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, o_parts,
                       lse_parts, num_parts, rows, o, lse);
  else
    hipLaunchKernelGGL(mla_merge_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, o_parts,
                       lse_parts, num_parts, rows, o, lse);
  return hipGetLastError();
}

}  // namespace mla
