// mla_surround.hip - the steps either side of the latent decode.
//
// "[Kimi-K3 MLA TP8] MLA performance", Sec. 3 (after the dispatched binary):
// the decode's q comes from one fused op that applies the rotary embedding to
// the 64 rope dims, concatenates them with the 512 latent dims, quantises to
// fp8 and writes the step's new cache entry into the same pool the decode
// reads; after the decode, a separate batched GEMM maps each head's 512-dim
// latent output to v_head_dim = 128 (Sec. 2 "K3 MLA geometry").
//
//   * mla_rope_quant_cache_kernel: one block per (token, chunk of outputs); a
//     thread produces 8 consecutive fp8 codes of one q row (real heads from
//     the inputs, pad heads zero) or of the token's new cache row.  Pure
//     element work: launch-bound at decode batch sizes.
//   * mla_latent_to_v_kernel: out[t, h, :] = o[t, h, :] . W[h]^T on
//     v_mfma_f32_16x16x32_bf16, one wave per (16 tokens, head, 16 output
//     dims), K = 512 in 16 steps; W is (heads, 128, 512) with the 512-dim
//     axis contiguous (a linear layer's (out, in) weight), so both operands
//     are 16-byte loads along K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

constexpr int kRopeDim = 64;
constexpr int kRopeHalf = 32;
constexpr int kChunk = 8;                      // outputs per thread
constexpr int kChunksPerRow = kRowDim / kChunk;  // 72
constexpr int kRopeThreads = 256;

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

}  // namespace

// grid (T, chunks / 256): item k of token t is chunk k % 72 of q row
// k / 72 (heads 0..H_pad-1) or, for k / 72 == H_pad, of the new cache row.
__global__ __launch_bounds__(kRopeThreads) void mla_rope_quant_cache_kernel(
    const uint16_t* q_latent, const uint16_t* q_pe, const uint16_t* k_latent,
    const uint16_t* k_pe, const int32_t* positions, const float* cos_sin, int max_pos,
    int rope_style, uint8_t* q_out, int num_heads, int num_heads_pad, uint8_t* kv_pool,
    int64_t pool_entries, const int32_t* slot_mapping, const float* q_scale,
    const float* kv_scale) {
  const int t = blockIdx.x;
  const int k = blockIdx.y * kRopeThreads + threadIdx.x;
  const int row = k / kChunksPerRow, chunk = k - row * kChunksPerRow;
  if (row > num_heads_pad) return;
  const int d0 = chunk * kChunk;
  int pos = positions[t];
  pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
  const float* cs = cos_sin + (int64_t)pos * kRopeDim;

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
  uint32_t codes[kChunk];
#pragma unroll
  for (int e = 0; e < kChunk; ++e) {
    const int d = d0 + e;
    const float v = d < kLatent ? bf16_to_f32(lat[d]) : rope_dim(pe, cs, d - kLatent, rope_style);
    codes[e] = e4m3fn_code(v / scale);  // stored = real / scale, correctly rounded
  }
  uint2 pk;
  pk.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
  pk.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
  *(uint2*)dst = pk;
}

// grid (ceil(T / 16), H, 2), block 256: wave wv of block (mt, h, nh) computes
// output dims [16 (4 nh + wv), +16) of tokens [16 mt, +16) of head h.
__global__ __launch_bounds__(256) void mla_latent_to_v_kernel(const uint16_t* o_latent,
                                                              const uint16_t* w_uv,
                                                              uint16_t* out, int T, int H,
                                                              int H_pad) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int n0 = 16 * (4 * blockIdx.z + wv);
  const int t0 = 16 * blockIdx.x;
  const int ta = t0 + (lane & 15) < T ? t0 + (lane & 15) : T - 1;  // A row (clamped)
  const int kq = 8 * (lane >> 4);
  const uint16_t* arow = o_latent + ((int64_t)ta * H_pad + h) * kLatent + kq;
  const uint16_t* brow = w_uv + ((int64_t)h * 128 + n0 + (lane & 15)) * kLatent + kq;
  uint4 a[16], b[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    a[s] = *(const uint4*)(arow + 32 * s);
    b[s] = *(const uint4*)(brow + 32 * s);
  }
  v4f_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(v8bf_t, v4u_t{a[s].x, a[s].y, a[s].z, a[s].w}),
        __builtin_bit_cast(v8bf_t, v4u_t{b[s].x, b[s].y, b[s].z, b[s].w}), acc, 0, 0, 0);
  // acc[i]: token t0 + 4 (lane / 16) + i, output dim n0 + lane % 16.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * (lane >> 4) + i;
    if (t < T) {
      uint32_t u = __float_as_uint(acc[i]);
      u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
      out[((int64_t)t * H + h) * 128 + n0 + (lane & 15)] = (uint16_t)(u >> 16);
    }
  }
}

hipError_t launch_rope_quant_cache(const uint16_t* q_latent, const uint16_t* q_pe,
                                   const uint16_t* k_latent, const uint16_t* k_pe,
                                   const int32_t* positions, const float* cos_sin, int max_pos,
                                   int rope_style, uint8_t* q_out, int T, int num_heads,
                                   int num_heads_pad, uint8_t* kv_pool, int64_t pool_entries,
                                   const int32_t* slot_mapping, const float* q_scale,
                                   const float* kv_scale, hipStream_t stream) {
  const int items = (num_heads_pad + 1) * kChunksPerRow;
  const dim3 grid(T, (items + kRopeThreads - 1) / kRopeThreads);
  hipLaunchKernelGGL(mla_rope_quant_cache_kernel, grid, dim3(kRopeThreads), 0, stream, q_latent,
                     q_pe, k_latent, k_pe, positions, cos_sin, max_pos, rope_style, q_out,
                     num_heads, num_heads_pad, kv_pool, pool_entries, slot_mapping, q_scale,
                     kv_scale);
  return hipGetLastError();
}

hipError_t launch_latent_to_v(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* out, int T,
                              int H, int H_pad, hipStream_t stream) {
  const dim3 grid((T + 15) / 16, H, 2);
  hipLaunchKernelGGL(mla_latent_to_v_kernel, grid, dim3(256), 0, stream, o_latent, w_uv, out, T, H,
                     H_pad);
  return hipGetLastError();
}

}  // namespace mla
