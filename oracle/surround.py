"""The steps either side of the latent decode, written out plainly (oracle side).

Test infrastructure, like the rest of ``oracle``: only the tests, the smoke
check and the benchmark's CPU baseline use it.

What the pages fix ("[Kimi-K3 MLA TP8] MLA performance"):

* Sec. 3: the decode's q comes from one fused op that rotates the rope part,
  concatenates it with the latent part and quantises to fp8, and that op also
  writes the step's new cache entry into the pool the decode reads.  After
  the decode a separate batched GEMM maps each head's 512-dim latent output
  back to v_head_dim.
* Sec. 2 "K3 MLA geometry": kv_lora_rank 512, qk_rope_head_dim 64,
  v_head_dim 128; the cache entry is 512 latent + 64 rope dims, fp8 e4m3fn
  (Sec. 1).

Readings where the pages are silent (listed in the design notes):

1. Rotary embedding: the 64 rope dims form 32 pairs, pair j turning by the
   angle whose cos / sin the caller's table gives for the token's position.
   Style 0 pairs dims (2j, 2j+1), style 1 pairs (j, j+32).  The rotated pair
   is (a cos - b sin, b cos + a sin).  It is computed in binary32 with every
   product and sum rounded on its own, because the result then picks an fp8
   code and both sides must take that decision in the same arithmetic.
2. Quantisation: stored = real / scale (binary32 division, correctly
   rounded), then the nearest e4m3fn value, ties to the even code, finite
   values beyond 448 saturating to +-448, NaN staying NaN.
3. Pad heads (num_heads .. num_heads_pad-1) of q are all-zero codes.
4. latent -> v: out[t, h] = sum_k o[t, h, k] * W[h, n, k], with W stored
   (heads, 128, 512) like a linear layer's (out, in) weight.
"""

from __future__ import annotations

import numpy as np

from . import codecs

ROPE_DIM = 64
LATENT_DIM = 512
V_HEAD_DIM = 128

# Non-negative finite e4m3fn codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = codecs.E4M3FN_TABLE[:0x7F]


def quantize_e4m3fn(x) -> np.ndarray:
    """Reading 2: the nearest e4m3fn code of each binary32 value (uint8 array)."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    a = np.abs(flat)
    sign = np.where(np.signbit(flat), 0x80, 0).astype(np.int64)
    # Candidates: the first value >= a and the one below it.
    idx = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(idx, 0x7E)
    lo = np.maximum(idx - 1, 0)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi,
                                              np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= codecs.E4M3FN_MAX, 0x7E, pick)  # saturate (and inf)
    code = sign | _POS_CODES[pick]
    code = np.where(np.isnan(flat), sign | 0x7F, code)
    return code.astype(np.uint8).reshape(x.shape)


def rope(x, cos, sin, style: int) -> np.ndarray:
    """Reading 1: rotate the last axis (64 dims) of binary32 ``x`` by angles
    with the given cos / sin (broadcast over x's leading axes, 32 each)."""
    x = np.asarray(x, dtype=np.float32)
    cos = np.asarray(cos, dtype=np.float32)
    sin = np.asarray(sin, dtype=np.float32)
    j = np.arange(ROPE_DIM // 2)
    if style == 0:
        ia, ib = 2 * j, 2 * j + 1
    elif style == 1:
        ia, ib = j, j + ROPE_DIM // 2
    else:
        raise ValueError("style must be 0 or 1")
    a, b = x[..., ia], x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = (a * cos) - (b * sin)  # each numpy float32 op rounds once
    out[..., ib] = (b * cos) + (a * sin)
    return out


def rope_quant_cache(q_latent, q_pe, k_latent, k_pe, positions, cos_sin, rope_style: int,
                     num_heads_pad: int, q_scale: float, kv_scale: float):
    """The fused step before the decode.

    Args (bf16 inputs as uint16 codes):
      q_latent (T, H, 512), q_pe (T, H, 64), k_latent (T, 512), k_pe (T, 64);
      positions (T,) ints (clamped to the table); cos_sin (max_pos, 64)
      binary32, cos of the 32 angles then their sin; q_scale / kv_scale the
      binary32 scales.

    Returns (q_out (T, num_heads_pad, 576) uint8 codes, cache_rows (T, 576)
    uint8 codes: what is written to each token's slot).
    """
    ql = codecs.decode_bf16(np.asarray(q_latent)).astype(np.float32)
    qp = codecs.decode_bf16(np.asarray(q_pe)).astype(np.float32)
    kl = codecs.decode_bf16(np.asarray(k_latent)).astype(np.float32)
    kp = codecs.decode_bf16(np.asarray(k_pe)).astype(np.float32)
    cos_sin = np.asarray(cos_sin, dtype=np.float32)
    pos = np.clip(np.asarray(positions, dtype=np.int64), 0, cos_sin.shape[0] - 1)
    T, H, _ = ql.shape
    cos = cos_sin[pos, : ROPE_DIM // 2]  # (T, 32)
    sin = cos_sin[pos, ROPE_DIM // 2:]
    q_rot = rope(qp, cos[:, None, :], sin[:, None, :], rope_style)
    k_rot = rope(kp, cos, sin, rope_style)
    qs, ks = np.float32(q_scale), np.float32(kv_scale)
    q_real = np.concatenate([ql, q_rot], axis=-1)  # (T, H, 576)
    k_real = np.concatenate([kl, k_rot], axis=-1)  # (T, 576)
    q_out = np.zeros((T, num_heads_pad, LATENT_DIM + ROPE_DIM), dtype=np.uint8)
    q_out[:, :H] = quantize_e4m3fn(q_real / qs)
    return q_out, quantize_e4m3fn(k_real / ks)


def latent_to_v(o_latent, w_uv) -> np.ndarray:
    """Reading 4: out (T, H, 128) float64 from o (T, >= H, 512) and W (H, 128, 512)."""
    o = np.asarray(o_latent, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    H = w.shape[0]
    return np.einsum("thk,hnk->thn", o[:, :H], w)
