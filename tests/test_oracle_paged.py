"""Pins for the oracle's paged-cache addressing (reading 7 of ``oracle.mla``).

"[Kimi-K3 MLA TP8] MLA performance", Sec. 5.2: the captured call runs with
page_size 1 (per-entry indices, all-ones last-page lengths), while
block-granular addressing would use the allocator's 128-slot blocks, i.e. one
index per block.  What fixes the mapping independently of how the oracle
writes it:

* a worked example by hand (below);
* page_size 1 is the per-entry form itself;
* a paged call equals the per-entry call over a list built here by walking
  pages and slots in order, for random page tables and ragged last pages.

Planted mistakes at the end show the checks catch the plausible wrong
mappings.
"""

import inspect
import textwrap

import numpy as np
import pytest

import workloads
from oracle import io as oio
from oracle import mla


def test_worked_example():
    """Two requests over pages of 4 slots: request 0 has pages [3, 0] with 2
    slots used in the last (6 entries: rows 12..15, 0, 1); request 1 has no
    pages; request 2 has page [5] with all 4 slots used (rows 20..23)."""
    indptr, rows = mla.paged_entry_rows([0, 2, 2, 3], [3, 0, 5], [2, 1, 4], 4)
    assert indptr.tolist() == [0, 6, 6, 10]
    assert rows.tolist() == [12, 13, 14, 15, 0, 1, 20, 21, 22, 23]


def test_page_size_one_is_the_per_entry_form():
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 1000, size=37)
    indptr, rows = mla.paged_entry_rows([0, 10, 10, 37], idx, [1, 1, 1], 1)
    assert indptr.tolist() == [0, 10, 10, 37]
    assert np.array_equal(rows, idx)


def _walk_pages(kvp, pages, last, P):
    """Per-entry rows by walking each request's pages and their used slots."""
    out_rows, out_ptr = [], [0]
    for b in range(len(kvp) - 1):
        mine = pages[kvp[b]: kvp[b + 1]]
        for k, page in enumerate(mine):
            used = int(last[b]) if k == len(mine) - 1 else P
            for slot in range(used):
                out_rows.append(int(page) * P + slot)
        out_ptr.append(len(out_rows))
    return np.array(out_ptr), np.array(out_rows, dtype=np.int64)


@pytest.mark.parametrize("P,seed", [(2, 0), (16, 1), (128, 2)])
def test_paged_call_equals_the_walked_per_entry_call(P, seed):
    lengths = [0, 1, P - 1, P, P + 1, 3 * P + 5]
    w = workloads.build("paged-pin", lengths, num_heads=16, qlens=[1, 2, 1, 3, 1, 4],
                        pool_entries=64 * P, q_std=2.0, scale_range=(0.5, 2.0),
                        shared_prefix=P + 1, seed=60 + seed, page_size=P)
    a = oio.workload_args(w)
    a.pop("tokens")
    o, lse = mla.mla_decode(**a)
    kvp = w.kv_indptr.numpy()
    ptr, rows = _walk_pages(kvp, w.kv_indices.numpy(), w.kv_last_page_lens.numpy(), P)
    assert np.diff(ptr).tolist() == lengths
    flat = dict(a, kv_indptr=ptr, kv_indices=rows,
                kv_pool=oio.codes(w.kv_pool))  # the whole pool, addressed by row
    o2, lse2 = mla.mla_decode(**flat)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse2))
    assert np.max(np.abs(o - o2)) < 1e-12
    fin = np.isfinite(lse)
    assert np.max(np.abs(lse[fin] - lse2[fin])) < 1e-12


def test_prefix_pages_are_shared_and_the_rest_disjoint():
    w = workloads.build("paged-share", [700, 900, 300], num_heads=16, pool_entries=128 * 40,
                        shared_prefix=600, seed=65, page_size=128)
    kvp = w.kv_indptr.tolist()
    pages = [w.kv_indices[kvp[b]: kvp[b + 1]].tolist() for b in range(3)]
    assert pages[0][:4] == pages[1][:4]  # 600 // 128 = 4 whole shared pages
    assert len(set(pages[2]) & set(pages[0])) == 0  # 300 < 512: no whole prefix
    assert len(set(pages[0][4:]) & set(pages[1][4:])) == 0
    assert w.kv_last_page_lens.tolist() == [700 - 5 * 128, 900 - 7 * 128, 300 - 2 * 128]


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "page and slot swapped": ("pages[i // P] * P + i % P", "pages[i % P] * P + i // P"),
    "last page counted whole": ("(len(pages) - 1) * P + int(last[b])", "len(pages) * P"),
    "page number used as a row": ("pages[i // P] * P + i % P", "pages[i // P] + i % P"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(mla.paged_entry_rows))
    assert old in src
    ns = dict(vars(mla))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    fn = ns["paged_entry_rows"]
    caught = False
    try:
        indptr, rows = fn([0, 2, 2, 3], [3, 0, 5], [2, 1, 4], 4)
        caught = (indptr.tolist() != [0, 6, 6, 10]
                  or rows.tolist() != [12, 13, 14, 15, 0, 1, 20, 21, 22, 23])
    except (IndexError, ValueError):
        caught = True
    assert caught, f"mutant '{name}' slipped through"
