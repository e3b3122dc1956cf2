"""Pins for the oracle's decoders: exhaustive comparison with torch's casts.

[Kimi-K3 MLA TP8] MLA performance, Sec. 1 "Environment": the KV cache dtype is
float8_e4m3fn; o is bfloat16.  torch's own float8_e4m3fn / bfloat16 -> float64
casts are an independent implementation of the same formats.
"""

import math

import numpy as np
import pytest
import torch

from oracle import brute, codecs


def test_e4m3fn_all_256_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.decode_e4m3fn(codes.numpy())
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert sorted(np.flatnonzero(nan_ref).tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0  # largest finite
    assert got[0x01] == 2.0 ** -9  # smallest subnormal


def test_bf16_all_65536_codes_match_torch():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.decode_bf16(codes.numpy().view(np.uint16))
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])


def test_brute_integer_decoder_matches_table():
    for c in range(256):
        v = codecs.E4M3FN_TABLE[c]
        if math.isnan(v):
            with pytest.raises(ValueError):
                brute.e4m3fn_to_int(c)
            continue
        assert math.ldexp(brute.e4m3fn_to_int(c), -9) == v


def test_brute_bf16_decoder_matches_torch_sampled():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 65536, size=4000).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for c, r in zip(codes, ref):
        if not np.isfinite(r):
            continue
        assert math.ldexp(brute.bf16_to_int(int(c)), -133) == r


def test_input_cast_clamps_before_e4m3fn():
    """The generator clamps to +-448 because torch's cast gives NaN beyond range."""
    x = torch.tensor([500.0, -500.0, 448.0, 464.0])
    assert torch.isnan(x.to(torch.float8_e4m3fn).to(torch.float32)).any()
    y = x.clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float32)
    assert torch.equal(y, torch.tensor([448.0, -448.0, 448.0, 448.0]))
