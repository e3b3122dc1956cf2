"""Scalar brute force used only to pin ``oracle.mla`` on tiny inputs.

It follows the same definition (see ``oracle.mla``) by a deliberately different
route, so that a mistake in one is unlikely to be repeated in the other:

* its own decoder maps every float8_e4m3fn / bfloat16 code to an exact integer
  times a fixed power of two (no lookup table, no float64);
* dot products over the 576 dims are exact integer sums;
* max, exp, sum and log run in 50-digit mpmath;
* the softmax-weighted sum over the 512 latent dims is an exact integer sum of
  fixed-point weights (2^-200 resolution) times the exact integer V codes.

The result is exact up to ~1e-45 relative, far below float64 resolution.
Python loops: keep the inputs tiny (a few hundred rows at most).
"""

from __future__ import annotations

import mpmath
import numpy as np

LATENT_DIM = 512
ROW_DIM = 576

# float8_e4m3fn values are integers times 2^-9; bfloat16 values are integers
# times 2^-133 (the smallest bf16 subnormal).
_E4M3_SHIFT = 9
_BF16_SHIFT = 133
_FIXED_BITS = 200


def e4m3fn_to_int(code: int) -> int:
    """Exact value of an e4m3fn code as an integer multiple of 2^-9."""
    code = int(code)
    neg = code >= 128
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN code in brute-force input")
    mag = m if e == 0 else (8 + m) << (e - 1)  # (1+m/8)*2^(e-7) = (8+m)*2^(e-1)*2^-9
    return -mag if neg else mag


def bf16_to_int(code: int) -> int:
    """Exact value of a bfloat16 code as an integer multiple of 2^-133."""
    code = int(code)
    neg = code >= 0x8000
    e = (code >> 7) & 0xFF
    m = code & 0x7F
    if e == 0xFF:
        raise ValueError("Inf/NaN code in brute-force input")
    # subnormal: m * 2^-133; normal: (128 + m) * 2^(e - 127 - 7)
    mag = m if e == 0 else (128 + m) << (e - 1)
    return -mag if neg else mag


def _decoder(dtype: str):
    if dtype == "fp8":
        return e4m3fn_to_int, _E4M3_SHIFT
    if dtype == "bf16":
        return bf16_to_int, _BF16_SHIFT
    raise ValueError(dtype)


def brute_decode(
    q, kv_pool, qo_indptr, kv_indptr, kv_indices, sm_scale, q_scale=1.0, kv_scale=1.0,
    dtype="fp8", digits=50,
):
    """Same contract as ``oracle.mla.mla_decode``; returns float64 arrays."""
    to_int, shift = _decoder(dtype)
    q = np.asarray(q)
    T, H, _ = q.shape
    B = len(qo_indptr) - 1
    o = np.zeros((T, H, LATENT_DIM), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    with mpmath.workdps(digits):
        scale = mpmath.mpf(float(sm_scale)) * mpmath.mpf(float(q_scale)) * mpmath.mpf(
            float(kv_scale)
        ) * mpmath.ldexp(1, -2 * shift)
        vscale = mpmath.mpf(float(kv_scale)) * mpmath.ldexp(1, -shift)
        for b in range(B):
            t0, t1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
            qlen = t1 - t0
            rows = [int(r) for r in kv_indices[int(kv_indptr[b]) : int(kv_indptr[b + 1])]]
            n = len(rows)
            kint = [[to_int(c) for c in kv_pool[r]] for r in rows]
            for j in range(qlen):
                t = t0 + j
                vis = n - (qlen - 1 - j)
                if vis <= 0:
                    continue
                for h in range(H):
                    qint = [to_int(c) for c in q[t, h]]
                    scores = []
                    for i in range(vis):
                        dot = 0
                        ki = kint[i]
                        for d in range(ROW_DIM):
                            dot += qint[d] * ki[d]
                        scores.append(scale * dot)
                    m = max(scores)
                    w = [mpmath.exp(s - m) for s in scores]
                    total = mpmath.fsum(w)
                    lse[t, h] = float(m + mpmath.log(total))
                    wfix = [int(mpmath.floor(x * mpmath.ldexp(1, _FIXED_BITS))) for x in w]
                    wsum = sum(wfix)
                    for d in range(LATENT_DIM):
                        acc = 0
                        for i in range(vis):
                            acc += wfix[i] * kint[i][d]
                        o[t, h, d] = float(mpmath.mpf(acc) * vscale / wsum)
    return o, lse


def brute_merge(o_parts, lse_parts, digits=50):
    """Scalar LSE merge over the leading axis, in mpmath."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    S = lse_parts.shape[0]
    rest = lse_parts.shape[1:]
    D = o_parts.shape[-1]
    o = np.zeros(rest + (D,), dtype=np.float64)
    lse = np.full(rest, -np.inf, dtype=np.float64)
    with mpmath.workdps(digits):
        for idx in np.ndindex(*rest):
            live = [s for s in range(S) if not np.isneginf(lse_parts[(s,) + idx])]
            if not live:
                continue
            ls = [mpmath.mpf(float(lse_parts[(s,) + idx])) for s in live]
            total = mpmath.fsum(mpmath.exp(x) for x in ls)
            lse[idx] = float(mpmath.log(total))
            for d in range(D):
                acc = mpmath.fsum(
                    mpmath.exp(x) * mpmath.mpf(float(o_parts[(s,) + idx + (d,)]))
                    for s, x in zip(live, ls)
                )
                o[idx + (d,)] = float(acc / total)
    return o, lse
