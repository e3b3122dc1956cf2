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
#include "mla_rope.h"

namespace mla {

namespace {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

constexpr int kRopeThreads = 256;

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
  rope_quant_item(q_latent, q_pe, k_latent, k_pe, positions, cos_sin, max_pos, rope_style, q_out,
                  num_heads, num_heads_pad, kv_pool, pool_entries, slot_mapping, q_scale, kv_scale,
                  t, row, chunk);
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
