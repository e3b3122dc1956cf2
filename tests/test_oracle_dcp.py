"""Pins for the oracle's DCP shard rule (reading 6 of ``oracle.mla``).

"Kimi K3 on AMD Instinct MI355X ...", Sec. 1: under DCP each GPU keeps an
eighth of a request's cached positions, the partial answers carry their
normalisation and are merged with softmax weights, and multi-token
verification runs on the shards.  Two facts fix the shard rule independently
of how the oracle writes it:

* dealing a request's positions over W shards, decoding each shard and
  merging the shards by LSE must give the full call (bottom-right causal on
  the full list), for any W, draft length and ragged length;
* one shard's answer for draft token j is attention over exactly the entries
  of the full list at positions p <= N - qlen + j with p mod W == rank, a set
  built here from the full list, not from the shard's own list.

The planted mistakes at the end show that both checks catch the plausible
wrong rules (the local list's own bottom-right mask, an off-by-one).
"""

import inspect
import textwrap

import numpy as np
import pytest

import workloads
from oracle import io as oio
from oracle import mla

LENGTHS = [0, 1, 3, 5, 7, 40, 61]
QLENS = [1, 4, 2, 3, 4, 2, 4]


def _args(w):
    a = oio.workload_args(w)
    a.pop("tokens")
    return a


def _full(seed=40):
    return workloads.build("dcp-pin", LENGTHS, num_heads=16, qlens=QLENS, pool_entries=256,
                           q_std=2.0, scale_range=(0.5, 2.0), seed=seed)


def _merge_shards(fn, full, W):
    parts = [fn(**_args(workloads.dcp_shard(full, W, r))) for r in range(W)]
    return mla.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


def _assert_same(o, lse, o_ref, lse_ref, rel=1e-12):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.max(np.abs(lse[fin] - lse_ref[fin])) <= rel * max(1.0, np.max(np.abs(lse_ref[fin])))
    assert np.max(np.abs(o - o_ref)) <= rel * max(1.0, np.max(np.abs(o_ref)))


@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_shards_merged_equal_the_full_causal_call(W):
    full = _full()
    o, lse = mla.mla_decode(**_args(full))
    om, lsem = _merge_shards(mla.mla_decode, full, W)
    _assert_same(om, lsem, o, lse)


def test_one_shard_is_attention_over_the_explicit_visible_set():
    full = _full(41)
    W, r = 3, 2
    shard = workloads.dcp_shard(full, W, r)
    o, lse = mla.mla_decode(**_args(shard))
    a = _args(full)
    kvp, qo = a["kv_indptr"], a["qo_indptr"]
    for b in range(len(LENGTHS)):
        N = int(kvp[b + 1] - kvp[b])
        qlen = int(qo[b + 1] - qo[b])
        for j in range(qlen):
            t = int(qo[b]) + j
            keep = [p for p in range(N) if p <= N - qlen + j and p % W == r]
            if not keep:
                assert np.all(o[t] == 0) and np.all(np.isneginf(lse[t]))
                continue
            one = dict(a, q=a["q"][t:t + 1], qo_indptr=np.array([0, 1]),
                       kv_indptr=np.array([0, len(keep)]),
                       kv_indices=a["kv_indices"][int(kvp[b]) + np.array(keep)])
            oj, lsej = mla.mla_decode(**one)
            _assert_same(o[t:t + 1], lse[t:t + 1], oj, lsej, rel=1e-14)


def test_shard_with_fewer_positions_than_ranks_is_empty():
    full = workloads.build("dcp-short", [3], num_heads=16, qlens=[1], pool_entries=16, seed=42)
    for r in range(8):
        o, lse = mla.mla_decode(**_args(workloads.dcp_shard(full, 8, r)))
        if r < 3:
            assert np.all(np.isfinite(lse))
        else:
            assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_single_shard_is_the_plain_call():
    full = _full(43)
    o, lse = mla.mla_decode(**_args(full))
    o1, lse1 = mla.mla_decode(**_args(workloads.dcp_shard(full, 1, 0)))
    assert np.array_equal(o, o1) and np.array_equal(lse, lse1)


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "the shard's own bottom-right mask": (
        "mla_decode", "vis = dcp_visible_length(n_full, n, qlen, j, cp_size, cp_rank)",
        "vis = visible_length(n, qlen, j)"),
    "last visible position off by one": ("dcp_visible_length", "last = n_full - qlen + j",
                                         "last = n_full - qlen + j + 1"),
    "rank ignored in the positions": ("dcp_visible_length", "positions = cp_rank + cp_size *",
                                      "positions = cp_size *"),
}


def _mutant(where, old, new):
    ns = dict(vars(mla))
    for name in ("dcp_visible_length", "mla_decode"):
        src = textwrap.dedent(inspect.getsource(getattr(mla, name)))
        if name == where:
            assert old in src, old
            src = src.replace(old, new)
        exec(compile(src, "<mutant>", "exec"), ns)
    return ns["mla_decode"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_breaks_the_shard_identity(name):
    full = _full()
    o, lse = mla.mla_decode(**_args(full))
    om, lsem = _merge_shards(_mutant(*MUTANTS[name]), full, 8)
    fin = np.isfinite(lse) & np.isfinite(lsem)
    err = max(float(np.max(np.abs(om - o))), float(np.max(np.abs(lsem[fin] - lse[fin]))),
              0.0 if np.array_equal(np.isneginf(lsem), np.isneginf(lse)) else np.inf)
    assert err > 1e-6, f"mutant '{name}' slipped through (err {err:.2e})"
