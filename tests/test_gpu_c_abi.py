"""GPU: the library called from plain C.

tests/native/c_abi_decode.c (built by build(): gcc, C11, linked against
libmla.so and the HIP runtime) allocates its buffers with hipMalloc, calls
mla_decode and mla_merge_partials through include/mla.h with no PyTorch in the
process, and writes its inputs and outputs to files.  Here the float64 oracle
reads the same inputs and the outputs are held to the parity gate: a request
with no cached entries, one of 5 (a ragged first tile), and two that span
several tiles and are split over workers; a merge with empty shards and a row
empty in every shard."""

import math
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle.mla import merge_partials as oracle_merge
from oracle.mla import mla_decode as oracle_decode
from tests.parity import assert_gate, metrics

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "native", "c_abi_decode")
LENGTHS = [0, 5, 300, 1500]
T, H, POOL, PARTS = 4, 16, 2048, 3


def _bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_plain_c_caller_matches_oracle(tmp_path):
    assert os.path.exists(DRIVER), f"{DRIVER} is missing: run __graft_entry__.build() first"
    print("[c-abi] running the plain-C caller", file=sys.stderr, flush=True)
    res = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"exit {res.returncode}: {res.stderr}"

    def load(name, dtype):
        return np.fromfile(tmp_path / name, dtype=dtype)

    q = load("q.u8", np.uint8).reshape(T, H, 576)
    kv = load("kv.u8", np.uint8).reshape(POOL, 576)
    kv_indptr = load("kv_indptr.i32", np.int32)
    kv_indices = load("kv_indices.i32", np.int32)
    assert list(np.diff(kv_indptr)) == LENGTHS
    # The caller's arguments as the device saw them: sm_scale = 1/sqrt(192)
    # rounded to binary32 (sqrtf and the division are correctly rounded).
    sm_scale = float(np.float32(1.0) / np.sqrt(np.float32(192.0)))
    o_ref, lse_ref = oracle_decode(q, kv, np.arange(T + 1), kv_indptr, kv_indices, sm_scale,
                                   q_scale=0.75, kv_scale=1.25, dtype="fp8")
    o = _bf16(load("o.u16", np.uint16)).reshape(T, H, 512)
    lse = load("lse.f32", np.float32).reshape(T, H)
    m = metrics(o, o_ref, lse, lse_ref)
    print(f"[c-abi] mla_decode {m}", file=sys.stderr, flush=True)
    assert_gate(m, "plain-C mla_decode")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])), "the empty request"

    parts = load("parts.f32", np.float32).reshape(PARTS, T, H, 512)
    lse_parts = load("lse_parts.f32", np.float32).reshape(PARTS, T, H)
    mo_ref, mlse_ref = oracle_merge(parts, lse_parts)
    mo = _bf16(load("merged_o.u16", np.uint16)).reshape(T, H, 512)
    mlse = load("merged_lse.f32", np.float32).reshape(T, H)
    mm = metrics(mo, mo_ref, mlse, mlse_ref)
    print(f"[c-abi] mla_merge_partials {mm}", file=sys.stderr, flush=True)
    assert_gate(mm, "plain-C mla_merge_partials")
    assert np.all(mo[1, 3] == 0) and math.isinf(mlse[1, 3]) and mlse[1, 3] < 0, "empty row"
