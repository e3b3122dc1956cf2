"""Pins for the oracle of the steps either side of the decode (oracle.surround).

* Quantisation: every finite e4m3fn value maps to its own code; points
  halfway between neighbours go to the even code; values beyond 448 saturate;
  in range it agrees with torch's float32 -> float8_e4m3fn cast (round to
  nearest even), an implementation written elsewhere.
* Rotary embedding: angle 0 is the identity, a quarter turn maps (a, b) to
  (-b, a) exactly, every pair keeps its length, two rotations compose to the
  sum of their angles, and the two pairings are the same rotation up to a
  fixed permutation of the dims.
* latent -> v: a weight that picks dims returns those dims exactly, and the
  product equals a plain triple loop on a small case.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import codecs, surround


def test_finite_codes_map_to_themselves():
    v = codecs.E4M3FN_TABLE.astype(np.float32)
    ok = np.isfinite(v)
    codes = surround.quantize_e4m3fn(v[ok])
    assert np.array_equal(codes, np.arange(256)[ok].astype(np.uint8))


def test_midpoints_round_to_the_even_code():
    vals = codecs.E4M3FN_TABLE[:0x7F]
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2  # exact in binary32
        want = c if c % 2 == 0 else c + 1
        assert surround.quantize_e4m3fn(np.array([mid]))[0] == want, c
        assert surround.quantize_e4m3fn(np.array([-mid]))[0] == 0x80 | want, c


def test_saturation_nan_and_signed_zero():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e30, np.inf, -1e9, np.nan, 0.0, -0.0, -1e-30],
                 dtype=np.float32)
    c = surround.quantize_e4m3fn(x).tolist()
    assert c[:7] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert c[7] & 0x7F == 0x7F
    assert c[8:] == [0x00, 0x80, 0x80]


def test_agrees_with_torch_cast_in_range():
    x = np.random.default_rng(1).standard_normal(1 << 18).astype(np.float32)
    x *= np.float32(2.0) ** np.random.default_rng(2).integers(-12, 9, size=x.size).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(surround.quantize_e4m3fn(x), ref)


def _angles(theta):
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_identity_quarter_turn_and_lengths(style):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    one, zero = np.ones(32, np.float32), np.zeros(32, np.float32)
    assert np.array_equal(surround.rope(x, one, zero, style), x)
    r = surround.rope(x, zero, one, style)
    j = np.arange(32)
    ia, ib = (2 * j, 2 * j + 1) if style == 0 else (j, j + 32)
    assert np.array_equal(r[:, ia], -x[:, ib]) and np.array_equal(r[:, ib], x[:, ia])
    c, s = _angles(rng.uniform(0, 2 * math.pi, 32))
    r = surround.rope(x, c, s, style).astype(np.float64)
    n0 = np.hypot(x[:, ia], x[:, ib])
    n1 = np.hypot(r[:, ia], r[:, ib])
    assert np.max(np.abs(n1 - n0) / n0) < 1e-6


@pytest.mark.parametrize("style", [0, 1])
def test_rope_rotations_compose(style):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    t1, t2 = rng.uniform(0, 3, 32), rng.uniform(0, 3, 32)
    two = surround.rope(surround.rope(x, *_angles(t1), style), *_angles(t2), style)
    once = surround.rope(x, *_angles(t1 + t2), style)
    assert np.max(np.abs(two.astype(np.float64) - once)) < 1e-5


def test_the_two_pairings_differ_by_a_permutation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    c, s = _angles(rng.uniform(0, 6, 32))
    j = np.arange(32)
    perm = np.empty(64, dtype=np.int64)  # interleaved position -> halves position
    perm[2 * j], perm[2 * j + 1] = j, j + 32
    halves = np.empty_like(x)
    halves[:, perm] = x
    a = surround.rope(x, c, s, 0)
    b = surround.rope(halves, c, s, 1)
    assert np.array_equal(a, b[:, perm])


def test_rope_quant_cache_pads_zero_and_uses_each_tokens_position():
    s = workloads.surround(3, 2, 50, 64, seed=7)
    q, k = (surround.rope_quant_cache(
        s.q_latent.view(torch.int16).numpy().view(np.uint16), s.q_pe.view(torch.int16).numpy().view(np.uint16),
        s.k_latent.view(torch.int16).numpy().view(np.uint16), s.k_pe.view(torch.int16).numpy().view(np.uint16),
        s.positions.numpy(), s.cos_sin.numpy(), 0, 4, 1.0, 1.0))
    assert q.shape == (3, 4, 576) and np.all(q[:, 2:] == 0)
    # token 1's rope dims, rotated by hand at its own position
    p = int(s.positions[1])
    x = s.q_pe[1, 0].float().numpy()
    c, sn = s.cos_sin[p, :32].numpy(), s.cos_sin[p, 32:].numpy()
    a, b = x[0::2], x[1::2]
    want = np.empty(64, np.float32)
    want[0::2], want[1::2] = a * c - b * sn, b * c + a * sn
    assert np.array_equal(q[1, 0, 512:], surround.quantize_e4m3fn(want))
    assert np.array_equal(k[1, :512], surround.quantize_e4m3fn(s.k_latent[1].float().numpy()))


def test_latent_to_v_picks_dims_and_matches_a_loop():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((3, 4, 512))
    pick = np.zeros((2, 128, 512))
    pick[0, np.arange(128), np.arange(128)] = 1.0
    pick[1, np.arange(128), 384 + np.arange(128)] = 1.0
    out = surround.latent_to_v(o, pick)
    assert np.array_equal(out[:, 0], o[:, 0, :128]) and np.array_equal(out[:, 1], o[:, 1, 384:])
    w = rng.standard_normal((2, 128, 512))
    out = surround.latent_to_v(o, w)
    for t in range(3):
        for h in range(2):
            for n in (0, 77, 127):
                acc = 0.0
                for kk in range(512):
                    acc += o[t, h, kk] * w[h, n, kk]
                assert abs(out[t, h, n] - acc) < 1e-9
