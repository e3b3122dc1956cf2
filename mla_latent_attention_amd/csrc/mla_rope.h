// mla_rope.h - the arithmetic of the step before the decode: the rotary
// embedding of the 64 rope dims and the fp8 quantisation of a 576-wide row
// ("[Kimi-K3 MLA TP8] MLA performance", Sec. 3: one fused op produces the
// decode's q and writes the step's new cache entry; Sec. 2 geometry).  Shared
// by the standalone kernel and the decode's fused build, so that both produce
// the same codes bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

constexpr int kRopeDim = 64;
constexpr int kRopeHalf = 32;
constexpr int kChunk = 8;                      // outputs per thread
constexpr int kChunksPerRow = kRowDim / kChunk;  // 72

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> OCP e4m3fn code, round to nearest even, finite values beyond the
// largest (448) saturate to it, NaN stays NaN.  Integer arithmetic on the
// fp32 bits, so the result does not depend on a hardware conversion mode.
__device__ __forceinline__ uint32_t e4m3fn_code(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |f| >= 448 (and inf): saturate
  const int e = (int)(a >> 23) - 127;
  if (e < -6) {
    // Subnormal range: multiples of 2^-9.  |f| * 2^9 is exact; rint rounds
    // half to even; 8 * 2^-9 = 2^-6 is code 0x08, the smallest normal.
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)m;
  }
  uint32_t mant = a & 0x7FFFFFu;
  uint32_t m3 = mant >> 20;
  const uint32_t rest = mant & 0xFFFFFu;  // the 20 dropped bits
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
  uint32_t code = ((uint32_t)(e + 7) << 3) + m3;  // a mantissa carry bumps the exponent
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// The rotated value of rope dim i (0..63) of row x at a position whose
// cos / sin of angle j are cs[j] / cs[32 + j].  style 0: dims (2j, 2j+1)
// rotate together; style 1: dims (j, j+32).  Products and sums are rounded
// one at a time (no fused multiply-add), so the value, and the fp8 code it
// rounds to, is the same on any device.
__device__ __forceinline__ float rope_dim(const uint16_t* x, const float* cs, int i, int style) {
#pragma clang fp contract(off)
  int j, a, b;
  if (style == 0) {
    j = i >> 1;
    a = 2 * j;
    b = 2 * j + 1;
  } else {
    j = i & (kRopeHalf - 1);
    a = j;
    b = j + kRopeHalf;
  }
  const float c = cs[j], s = cs[kRopeHalf + j];
  const float xa = bf16_to_f32(x[a]), xb = bf16_to_f32(x[b]);
  if (i == a) return xa * c - xb * s;
  return xb * c + xa * s;
}

// Codes of dims [d0, d0 + 8) of one row (d0 a multiple of 8): latent dims
// from lat (bf16), rope dims rotated from pe (bf16) at the angles in cs,
// each divided by scale and quantised.  Packed little-endian, dim d0 first.
__device__ __forceinline__ uint2 row_codes8(const uint16_t* lat, const uint16_t* pe,
                                            const float* cs, int style, float scale, int d0) {
  uint32_t codes[kChunk];
#pragma unroll
  for (int e = 0; e < kChunk; ++e) {
    const int d = d0 + e;
    const float v = d < kLatent ? bf16_to_f32(lat[d]) : rope_dim(pe, cs, d - kLatent, style);
    codes[e] = e4m3fn_code(v / scale);  // stored = real / scale, correctly rounded
  }
  uint2 pk;
  pk.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
  pk.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
  return pk;
}

// One item of the step: chunk ch (8 codes, dims 8ch ..) of q row `row` of
// token t for row < num_heads_pad (the real heads' codes from q_latent / q_pe
// at the token's position over q_scale, zero codes for the pad heads), or, for
// row == num_heads_pad, of the token's new cache entry from k_latent / k_pe
// over kv_scale, written at slot_mapping[t] unless that is outside the pool.
__device__ __forceinline__ void rope_quant_item(
    const uint16_t* q_latent, const uint16_t* q_pe, const uint16_t* k_latent,
    const uint16_t* k_pe, const int32_t* positions, const float* cos_sin, int max_pos,
    int rope_style, uint8_t* q_out, int num_heads, int num_heads_pad, uint8_t* kv_pool,
    int64_t pool_entries, const int32_t* slot_mapping, const float* q_scale,
    const float* kv_scale, int t, int row, int ch) {
  const int d0 = ch * kChunk;
  const uint16_t* lat;  // this row's 512 latent dims
  const uint16_t* pe;   // and its 64 rope dims
  uint8_t* dst;
  float scale;
  if (row < num_heads_pad) {
    dst = q_out + ((int64_t)t * num_heads_pad + row) * kRowDim + d0;
    if (row >= num_heads) {  // pad head: zero codes
      *(uint2*)dst = make_uint2(0u, 0u);
      return;
    }
    lat = q_latent + ((int64_t)t * num_heads + row) * kLatent;
    pe = q_pe + ((int64_t)t * num_heads + row) * kRopeDim;
    scale = q_scale ? *q_scale : 1.0f;
  } else {
    const int slot = slot_mapping[t];
    if (slot < 0 || slot >= pool_entries) return;  // no cache write for this token
    dst = kv_pool + (int64_t)slot * kRowDim + d0;
    lat = k_latent + (int64_t)t * kLatent;
    pe = k_pe + (int64_t)t * kRopeDim;
    scale = kv_scale ? *kv_scale : 1.0f;
  }
  int pos = positions[t];
  pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
  *(uint2*)dst = row_codes8(lat, pe, cos_sin + (int64_t)pos * kRopeDim, rope_style, scale, d0);
}

}  // namespace mla
