"""The oracle's pins have teeth: plausible mistakes planted in a copy of the
oracle (on the CPU) are each caught by the brute-force comparison.

Each mutant rewrites one line of ``oracle.mla.mla_decode``'s source and runs the
same comparison the pins use; the pin must fail for every mutant.
"""

import inspect
import textwrap

import numpy as np
import pytest

import workloads
from oracle import brute, codecs, mla
from oracle import io as oio

MUTANTS = {
    "rope dims dropped from the score": ("Q @ K[:vis].T", "Q[:, :512] @ K[:vis, :512].T"),
    "V taken from the wrong slice": ("V = K[:, :LATENT_DIM]", "V = K[:, ROPE_DIM:]"),
    "lse in log2": ("np.log(denom[:, 0])", "np.log2(denom[:, 0])"),
    "causal mask off by one": ("vis = visible_length(n, qlen, j)", "vis = min(n, visible_length(n, qlen, j) + 1)"),
    "q_scale dropped": ("Q = q_scale * codecs.decode", "Q = codecs.decode"),
    "kv_scale dropped from V": ("V = K[:, :LATENT_DIM]", "V = K[:, :LATENT_DIM] / kv_scale"),
    "softmax without the 1/sum": ("o[t] = (e @ V[:vis]) / denom", "o[t] = (e @ V[:vis])"),
}


def _mutant(old, new):
    src = textwrap.dedent(inspect.getsource(mla.mla_decode))
    assert old in src, old
    ns = dict(vars(mla))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["mla_decode"]


def _case():
    w = workloads.build(
        "mutant-case", [9, 6], num_heads=16, real_heads=16, qlens=[3, 1], pool_entries=64,
        dtype="fp8", kv_std=1.0, q_std=2.0, scale_range=(0.5, 2.0), seed=31,
    )
    a = oio.workload_args(w)
    a.pop("tokens")
    return a


@pytest.fixture(scope="module")
def case_and_truth():
    a = _case()
    return a, brute.brute_decode(**a)


def test_unmutated_oracle_passes_the_pin(case_and_truth):
    a, (ob, lseb) = case_and_truth
    o, lse = mla.mla_decode(**a)
    fin = np.isfinite(lseb)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse[fin] - lseb[fin])) < 1e-12


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(case_and_truth, name):
    a, (ob, lseb) = case_and_truth
    fn = _mutant(*MUTANTS[name])
    o, lse = fn(**a)
    fin = np.isfinite(lseb) & np.isfinite(lse)
    err = max(float(np.max(np.abs(o - ob))),
              float(np.max(np.abs(lse[fin] - lseb[fin]))) if fin.any() else 0.0,
              0.0 if np.array_equal(np.isneginf(lse), np.isneginf(lseb)) else np.inf)
    assert err > 1e-6, f"mutant '{name}' slipped through (err {err:.2e})"


def test_flushed_subnormals_are_caught_by_the_codec_pin():
    import torch
    mutated = codecs.E4M3FN_TABLE.copy()
    mutated[1:8] = 0.0
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    ok = np.isfinite(ref)
    assert not np.array_equal(mutated[ok], ref[ok])
