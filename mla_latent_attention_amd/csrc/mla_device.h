// mla_device.h - device helpers shared by the decode kernels: arithmetic
// helpers, block-wide scans, the planner's request lookup, the online-softmax
// state and the staging of q and kv_indices.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"
#include "mla_plan.h"

namespace mla {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCombBytes = kWaves * 32 * 64 * 16;  // 131,072: every wave's O^T
constexpr int kIdxSeg = 7168;                      // kv_indices staged in LDS per segment
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLazy = 1.0f;                       // rescale when a row max grows > 2^kLazy

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef float v2f32_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 bits with integer operations (finite
// inputs).
__device__ __forceinline__ u32 bf16_rne_bits(float f) {
  u32 u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats as packed bf16 bits (a in the low half), rounded to nearest even
// by one hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32 pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(u32, __builtin_convertvector(v2f32_t{a, b}, v2bf16_t));
}

// Split partials of the fp8 kernels are stored as fp16 (11 significant bits,
// against bf16's 8: with a bf16 partial the merged row carries two bf16
// roundings, up to one bf16 unit, 0.0156 at |o| in [2, 4), where the 1e-2
// bound allows one; with fp16 the pair stays under 0.0098), of values
// without the kv scale, so that they stay within fp16's range (|o / kv_scale|
// <= 448, the largest e4m3 value).  Round to nearest even.
// (Two scalar conversions, not the packed one: with the packed conversion the
// standard fp8 kernel's epilogue no longer fits its registers.)
__device__ __forceinline__ u32 pack_f16x2(float a, float b) {
  return (u32)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((u32)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ float2 unpack_f16x2(u32 w) {
  return make_float2((float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)));
}

__device__ __forceinline__ long as_long(u32 lo, u32 hi) {
  return (long)((uint64_t)lo | ((uint64_t)hi << 32));
}

// Orders this wave's LDS accesses (writes by some lanes, reads by others).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// 4x4 byte transpose: out_k = (a.byte k, b.byte k, c.byte k, d.byte k).
__device__ __forceinline__ void transpose4x4(u32 a, u32 b, u32 c, u32 d, u32& o0, u32& o1, u32& o2,
                                             u32& o3) {
  const u32 t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const u32 t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const u32 t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const u32 t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);           // a0 b0 c0 d0
  o1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);           // a1 b1 c1 d1
  o2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);           // a2 b2 c2 d2
  o3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);           // a3 b3 c3 d3
}

// ---------------------------------------------------------------- block helpers

// Block-uniform values read from memory arrive in vector registers; moving
// them to scalar registers keeps the planner state (live across the whole
// tile loop) out of the vector register budget of the loop.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
// A value the compiler cannot see through.  Per-lane address arithmetic of an
// epilogue built from it stays in the epilogue instead of being hoisted out of
// the enclosing loop, where it would hold vector registers the tile loop needs.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void uniformize(Req& r) {
  r.kv_base = uniform(r.kv_base);
  r.n = uniform(r.n);
  r.q_base = uniform(r.q_base);
  r.qlen = uniform(r.qlen);
  r.causal = uniform(r.causal);
  r.vbase = uniform(r.vbase);
  r.vstep = uniform(r.vstep);
}

__device__ __forceinline__ void uniformize(Cursor& c) {
  c.b = uniform(c.b);
  c.j = uniform(c.j);
  c.g = uniform(c.g);
  c.k = uniform(c.k);
  uniformize(c.r);
}

// Block-wide helpers for blocks of kT threads (red: kT/64 entries).
template <int kT = kThreads>
__device__ int64_t block_sum_i64(int64_t v, int64_t* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  int64_t s = 0;
  for (int i = 0; i < kT / 64; ++i) s += red[i];
  return s;
}

// Exclusive prefix sum over the block's kT values; `total` gets the sum.
template <int kT = kThreads>
__device__ int64_t block_excl_scan_i64(int64_t v, int64_t* red, int64_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int64_t x = v;
  for (int off = 1; off < 64; off <<= 1) {
    int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) red[wv] = x;
  __syncthreads();
  int64_t before = 0;
  total = 0;
  for (int i = 0; i < kT / 64; ++i) {
    if (i < wv) before += red[i];
    total += red[i];
  }
  return before + x - v;
}

// Requests containing stream positions x[0] and x[1] (a negative position is
// not looked up), where request r holds rows_of(r) stream rows: sb[i] =
// request (-1 if not found, -2 if not looked up) and scum[i] = that request's
// first stream position.
template <bool kPaged, int kT = kThreads, bool kCascade = false, class RowsOf>
__device__ void plan_locate2(const DecodeParams& p, RowsOf rows_of, const int64_t (&x)[2],
                             int64_t* red, int* sb, int64_t* scum) {
  if (threadIdx.x < 2) sb[threadIdx.x] = x[threadIdx.x] < 0 ? -2 : -1;
  const ReqSource src = source_of<kPaged, kCascade>(p);
  int64_t carry = 0;
  for (int b0 = 0; b0 < p.batch; b0 += kT) {
    const int b = b0 + threadIdx.x;
    int64_t R = 0;
    if (b < p.batch) {
      R = rows_of(load_req(src, b));
    }
    int64_t total;
    const int64_t cum = carry + block_excl_scan_i64<kT>(R, red, total);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (R > 0 && x[i] >= cum && x[i] < cum + R) {
        sb[i] = b;
        scum[i] = cum;
      }
    }
    carry += total;
    __syncthreads();
    if (sb[0] != -1 && sb[1] != -1) break;
  }
  __syncthreads();
}

// The requests holding stream positions x0 = worker_begin(w, W, nw) and x1
// (the next worker's start), where request b holds rows_of(b) stream rows.
// Batches of at most kT requests take one request per thread: one read of
// each request, one block-wide scan that gives W and every request's first
// stream position, and the two requests handed over through LDS (bounds
// included), so the lookup costs one memory round trip.  Larger batches scan
// twice (plan_locate2) and read the two requests again.  Empty tokens of the
// requests this block reads are zeroed on the way (zero_empty).  Returns
// false if this worker has nothing to do (W == 0 or w >= nw).
struct PlanHit {
  int b;        // request (-1: none)
  int64_t cum;  // its first stream position
  Req r;
};

template <bool kPaged, int kT, bool kCascade, class RowsOf, class ZeroEmpty>
__device__ __forceinline__ bool plan_lookup(const DecodeParams& p, RowsOf rows_of,
                                            ZeroEmpty zero_empty, int w, int64_t* red,
                                            PlanHit* hits, int64_t& W, int& nw, int64_t& x0,
                                            int64_t& x1, PlanHit (&out)[2]) {
  const ReqSource src = source_of<kPaged, kCascade>(p);
  if (p.batch <= kT) {
    const int b = threadIdx.x;
    Req r{};
    int64_t R = 0;
    if (b < p.batch) {
      r = load_req(src, b);
      R = rows_of(r);
      zero_empty(r);
    }
    int64_t total;
    const int64_t cum = block_excl_scan_i64<kT>(R, red, total);
    W = uniform(total);
    if (W == 0) return false;
    nw = effective_workers(W, p.num_workers);
    if (w >= nw) return false;
    x0 = worker_begin(w, W, nw);
    x1 = worker_begin(w + 1, W, nw);
    if (threadIdx.x < 2) hits[threadIdx.x].b = -1;
    __syncthreads();
    if (R > 0 && x0 >= cum && x0 < cum + R) hits[0] = PlanHit{b, cum, r};
    if (R > 0 && x1 < W && x1 >= cum && x1 < cum + R) hits[1] = PlanHit{b, cum, r};
    __syncthreads();
  } else {
    int64_t acc = 0;
    for (int b = threadIdx.x; b < p.batch; b += kT) {
      const Req r = load_req(src, b);
      acc += rows_of(r);
      zero_empty(r);
    }
    W = uniform(block_sum_i64<kT>(acc, red));
    if (W == 0) return false;
    nw = effective_workers(W, p.num_workers);
    if (w >= nw) return false;
    x0 = worker_begin(w, W, nw);
    x1 = worker_begin(w + 1, W, nw);
    const int64_t xs[2] = {x0, x1 < W ? x1 : -1};
    __shared__ int lb[2];
    __shared__ int64_t lcum[2];
    plan_locate2<kPaged, kT, kCascade>(p, rows_of, xs, red, lb, lcum);
    // Threads 0 and 1 fetch the two requests found.
    if (threadIdx.x < 2) {
      const int i = threadIdx.x;
      const int b = lb[i];
      hits[i].b = b;
      hits[i].cum = lcum[i];
      if (b >= 0) hits[i].r = load_req(src, b);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    out[i].b = uniform(hits[i].b);
    out[i].cum = uniform(hits[i].cum);
    out[i].r = hits[i].r;
    uniformize(out[i].r);
  }
  return true;
}

// ---------------------------------------------------------------- softmax state

struct WaveState {
  v4f O[32];  // O^T blocks (the dim of each element depends on the path);
              // scaled by the path's kPScale
  float m;    // (possibly stale) running max of base-2 scores of row lane%16
  float l;    // this lane's partial sum of 2^(s - m)
  float dl;   // fp8 path: this lane's sum of (hi + lo) - P * kPScale, the split's
              // rounding of the weights (o is normalised by l + dl / kPScale,
              // the lse takes l)
};

// Online-softmax update for row lane%16 from this lane's N scores (already
// masked to -inf past the piece).  Returns P = 2^(s - m) in x.  The running
// max is only raised when a row's max grows by more than 2^kLazy, so P stays
// <= 2^kLazy and the accumulators are rescaled on few tiles.
template <int N>
__device__ __forceinline__ void softmax_update(WaveState& st, float (&x)[N]) {
  float tmax = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) tmax = fmaxf(tmax, x[i]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const bool grow = tmax > st.m + kLazy;  // first tile: m = -inf
  if (__any(grow)) {
    const float mset = grow ? tmax : st.m;
    const float alpha = fast_exp2(st.m - mset);  // 1 for rows that keep m, 0 on the first tile
#pragma unroll
    for (int b = 0; b < 32; ++b) st.O[b] *= alpha;
    st.l *= alpha;
    st.dl *= alpha;
    st.m = mset;
  }
  float psum = -0.f;  // x + -0 = x: the first add folds away
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = fast_exp2(x[i] - st.m);
    psum += x[i];
  }
  st.l += psum;
}

// ---------------------------------------------------------------- staging

// kv_indices loads issued per thread before the first store.
constexpr int kIdxBatch = 8;

// Pool rows of a piece's entries.  Entry i of the piece is entry k0 + i of its
// request.  One entry per index (page_shift 0): the row is kv_indices[ib + i],
// ib being the piece's first index.  Paged cache (page_size 2^page_shift): ib
// is the request's first page number's index and the row is page * page_size
// + slot of entry k0 + i.  Consecutive entries share a page number, so a
// page's index is fetched from memory once and served from cache to the
// others.  (Two integers, so the pieces' long loops keep little extra state.)
struct RowSrc {
  int ib;
  int k0;

  template <bool kPaged>
  __device__ __forceinline__ RowSrc at(int i) const {  // the same source from entry i on
    RowSrc r = *this;
    if constexpr (kPaged)
      r.k0 += i;
    else
      r.ib += i;
    return r;
  }
};

// Kernels come in two builds: kPaged = false (one entry per index) and true
// (paged cache), so the common build carries none of the paging state.
template <bool kPaged>
__device__ __forceinline__ RowSrc row_src(const Req& r, int k) {
  RowSrc s;
  s.ib = r.kv_base + (kPaged ? 0 : k);
  s.k0 = k;
  return s;
}

// Pool row of entry e of a request whose page numbers start at `pages` (a
// page number out of range gives a row that the row loads clamp).
__device__ __forceinline__ int32_t paged_row(const int32_t* pages, int shift, int e) {
  return (int32_t)(((uint32_t)pages[e >> shift] << shift) | (uint32_t)(e & ((1 << shift) - 1)));
}

// Where index ib lives: kv_indices, or in a one-launch cascade call the
// suffixes' buffer past the prefix (a piece never straddles the two).
template <bool kCascade>
__device__ __forceinline__ const int32_t* index_base(const DecodeParams& p, int ib) {
  if constexpr (kCascade)
    return ib < p.cascade_prefix ? p.kv_indices + ib : p.kv_indices2 + (ib - p.cascade_prefix);
  return p.kv_indices + ib;
}

// Rows of entries [0, n) of src (first kIdxBatch * kT of them) to idx_dst.
template <bool kPaged, int kT = kThreads, bool kCascade = false>
__device__ __forceinline__ void stage_first_indices(int32_t* idx_dst, const DecodeParams& p,
                                                    RowSrc src, int n) {
  int32_t iv[kIdxBatch];
  const int32_t* base = index_base<kCascade>(p, src.ib);
  if constexpr (!kPaged) {
#pragma unroll
    for (int j = 0; j < kIdxBatch; ++j) iv[j] = base[imin(j * kT + (int)threadIdx.x, n - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < kIdxBatch; ++j)
      iv[j] = paged_row(base, p.page_shift, src.k0 + imin(j * kT + (int)threadIdx.x, n - 1));
  }
#pragma unroll
  for (int j = 0; j < kIdxBatch; ++j) idx_dst[imin(j * kT + (int)threadIdx.x, n - 1)] = iv[j];
}

// acc plus the four e4m3 values packed in w: each pair widened to f16 (exact)
// and summed by an f32 dot product with (1, 1).
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_fp8x4(u32 w, float acc) {
  const v2h_t one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false), one, acc,
                               false);
  return __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true), one, acc,
                                false);
}

__device__ __forceinline__ void store_f16x8(uint16_t* dst, const float (&a)[8]) {
  uint4 pk;
  pk.x = pack_f16x2(a[0], a[1]);
  pk.y = pack_f16x2(a[2], a[3]);
  pk.z = pack_f16x2(a[4], a[5]);
  pk.w = pack_f16x2(a[6], a[7]);
  *(uint4*)dst = pk;
}

__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float (&a)[8]) {
  uint4 pk;
  // Integer rounding here, not pack_bf16x2: with the conversion instruction
  // the standard fp8 kernel's register allocation spills (same results: both
  // round to nearest even).
  pk.x = bf16_rne_bits(a[0]) | (bf16_rne_bits(a[1]) << 16);
  pk.y = bf16_rne_bits(a[2]) | (bf16_rne_bits(a[3]) << 16);
  pk.z = bf16_rne_bits(a[4]) | (bf16_rne_bits(a[5]) << 16);
  pk.w = bf16_rne_bits(a[6]) | (bf16_rne_bits(a[7]) << 16);
  *(uint4*)dst = pk;
}

// Copies the rows of entries [from, n) of src (n >= 1) to the same positions
// of dst.  Each thread issues kIdxBatch loads before its first store
// (past-the-end positions reload the last index), so a segment costs one
// memory round trip per 2048 indices instead of one per 256.
template <bool kPaged, int kT = kThreads, bool kCascade = false>
__device__ __forceinline__ void stage_indices(int32_t* dst, const DecodeParams& p, RowSrc src,
                                              int from, int n) {
  const int32_t* base = index_base<kCascade>(p, src.ib);
  for (int i0 = from; i0 < n; i0 += kT * kIdxBatch) {
    int32_t v[kIdxBatch];
    if constexpr (!kPaged) {
#pragma unroll
      for (int j = 0; j < kIdxBatch; ++j) v[j] = base[imin(i0 + j * kT + (int)threadIdx.x, n - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < kIdxBatch; ++j)
        v[j] = paged_row(base, p.page_shift, src.k0 + imin(i0 + j * kT + (int)threadIdx.x, n - 1));
    }
#pragma unroll
    for (int j = 0; j < kIdxBatch; ++j) dst[imin(i0 + j * kT + (int)threadIdx.x, n - 1)] = v[j];
  }
}

// Query rows that see no entry get o = 0, lse = -inf; the block owning token t
// (t mod gridDim.x) writes them.  Rare: empty requests or early draft tokens.
// o = 0 and lse = -inf for every head of token t (a token that sees nothing).
__device__ void zero_token_rows(const DecodeParams& p, int t) {
  for (int h = 0; h < p.num_heads; ++h) {
    const int64_t orow = (int64_t)t * p.num_heads + h;
    if (p.o32 != nullptr) {
      float4* d32 = (float4*)(p.o32 + orow * kLatent);
      for (int k = 0; k < kLatent / 4; ++k) d32[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      uint4* dst = (uint4*)(p.o + orow * kLatent);
      for (int k = 0; k < kLatent / 8; ++k) dst[k] = make_uint4(0, 0, 0, 0);
    }
    if (p.lse != nullptr) p.lse[orow] = neg_inf();
  }
}

// The standard kernels' empty token: its head groups' descriptors say
// "not split", and its rows are zeroed.
__device__ void zero_token(const DecodeParams& p, int t) {
  const int G = p.num_heads / kGroup;
  for (int g = 0; g < G; ++g) p.desc[(int64_t)t * G + g] = make_int4(0, 0, 0, 0);
  zero_token_rows(p, t);
}

// Group mode's empty-row bookkeeping for request r (H heads): the rows of its
// tokens that see nothing, and "not split" descriptors for the entries no
// piece writes: its leading row groups whose rows all see nothing (only when
// some of its tokens see nothing; visible counts rise with the token) and its
// unused entries (entry q_base * Gs + rg, rg in [row groups, qlen * Gs)).
// Each token and entry is dealt to one block (index mod the worker count).
__device__ void clear_group_request(const DecodeParams& p, const Req& r, int H) {
  const int nempty = req_empty_tokens(r);
  for (int j = 0; j < nempty; ++j)
    if ((r.q_base + j) % p.num_workers == (int)blockIdx.x) zero_token_rows(p, r.q_base + j);
  const int Gs = group_slots_per_token(H);
  const int RG = group_row_groups(r, H);
  int dark = 0;  // leading row groups that see nothing
  if (nempty > 0)
    while (dark < RG && group_last_token(r, H, dark) < nempty) ++dark;
  const int base = r.q_base * Gs;
  for (int rg = 0; rg < dark; ++rg)
    if ((base + rg) % p.num_workers == (int)blockIdx.x) p.desc[base + rg] = make_int4(0, 0, 0, 0);
  for (int rg = RG; rg < r.qlen * Gs; ++rg)
    if ((base + rg) % p.num_workers == (int)blockIdx.x) p.desc[base + rg] = make_int4(0, 0, 0, 0);
}

}  // namespace mla
