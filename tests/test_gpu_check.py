"""GPU: the device-side check of a call's index arguments (mla_check_inputs)
and the MLA_DEBUG_CHECKS build of the library (libmla_debug.so), whose decode
entry points run that check first and refuse a call that breaks its contract.

Each case breaks one part of the contract the header states and expects
exactly that part's bit; the valid calls expect none.  Every broken input
stays inside the buffers the host passes (the check reads nothing else, and
the refused calls launch no decode)."""

import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_attention_amd as mla  # noqa: E402
from mla_latent_attention_amd import _lib  # noqa: E402

DEV = torch.device("cuda:0")
LENGTHS = [700, 1300, 5, 2100]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _w(qlens=None, page_size=1, seed=170):
    return workloads.build("check", LENGTHS, num_heads=16, real_heads=12, qlens=qlens,
                           pool_entries=8192, kv_std=0.5, seed=seed, device=DEV,
                           page_size=page_size)


def _check(w, *, qo=None, kvp=None, idx=None, lpl="same", page_size=1, max_seqlen_q=None, **kw):
    return mla.check_inputs(
        w.qo_indptr if qo is None else qo, w.kv_indptr if kvp is None else kvp,
        w.kv_indices if idx is None else idx, w.kv_pool.view(-1, 576).shape[0],
        max_seqlen_q=w.max_seqlen_q if max_seqlen_q is None else max_seqlen_q,
        num_q_tokens=w.num_tokens, kv_last_page_lens=w.kv_last_page_lens if lpl == "same" else lpl,
        page_size=page_size, **kw)


def test_valid_calls_report_nothing():
    say("[check] valid: plain, draft tokens, paged, DCP shard")
    assert _check(_w()) == set()
    d = _w(qlens=[2, 1, 3, 1])
    assert _check(d) == set()
    pg = _w(page_size=128)
    assert _check(pg, page_size=128) == set()
    full = _w(qlens=[3, 2, 1, 1])
    sh = workloads.dcp_shard(full, 4, 3)
    assert _check(sh, g_kv_indptr=sh.g_kv_indptr, cp_world_size=4, cp_rank=3) == set()


def test_index_outside_the_pool():
    w = _w()
    pool = w.kv_pool.shape[0]
    for bad in (pool, pool + 5, -1):
        idx = w.kv_indices.clone()
        idx[int(w.kv_indptr[1])] = bad  # request 1's first entry
        assert _check(w, idx=idx) == {"MLA_CHECK_KV_INDEX"}, bad
    # Entries past kv_indptr[batch] are not part of the call.
    idx = torch.cat([w.kv_indices, torch.tensor([-7, pool], dtype=torch.int32, device=DEV)])
    assert _check(w, idx=idx) == set()


def test_broken_kv_indptr():
    w = _w()
    kvp = w.kv_indptr.clone()
    kvp[2] = kvp[1] - 1  # request 1 ends before it starts
    assert "MLA_CHECK_KV_INDPTR" in _check(w, kvp=kvp)
    kvp = w.kv_indptr.clone()
    kvp[-1] += 10  # past the end of the index list (read no further than its length)
    assert _check(w, kvp=kvp) == {"MLA_CHECK_KV_INDPTR"}
    kvp = w.kv_indptr.clone()
    kvp[0] = 1
    assert "MLA_CHECK_KV_INDPTR" in _check(w, kvp=kvp)


def test_broken_qo_indptr():
    w = _w(qlens=[2, 1, 3, 1])
    assert _check(w, max_seqlen_q=2) == {"MLA_CHECK_QO_INDPTR"}  # request 2 holds 3 tokens
    qo = w.qo_indptr.clone()
    qo[-1] += 1  # more tokens than the call says
    assert _check(w, qo=qo) == {"MLA_CHECK_QO_INDPTR"}
    qo = w.qo_indptr.clone()
    qo[1], qo[2] = qo[2].clone(), qo[1].clone()  # a decrease
    assert "MLA_CHECK_QO_INDPTR" in _check(w, qo=qo)


def test_last_page_lengths():
    w = _w()
    lpl = torch.ones(len(LENGTHS), dtype=torch.int32, device=DEV)
    assert _check(w, lpl=lpl) == set()
    lpl[2] = 2  # page_size 1: every length is 1
    assert _check(w, lpl=lpl) == {"MLA_CHECK_LAST_PAGE_LEN"}
    pg = _w(page_size=128)
    for bad in (0, 129):
        lpl = pg.kv_last_page_lens.clone()
        lpl[1] = bad
        assert _check(pg, lpl=lpl, page_size=128) == {"MLA_CHECK_LAST_PAGE_LEN"}, bad
    # A paged list holds page numbers: one past the last page is out of range.
    idx = pg.kv_indices.clone()
    idx[0] = pg.kv_pool.view(-1, 576).shape[0] // 128
    assert _check(pg, idx=idx, page_size=128) == {"MLA_CHECK_KV_INDEX"}


def test_dcp_shard_lengths():
    full = _w(qlens=[3, 2, 1, 1])
    sh = workloads.dcp_shard(full, 4, 3)
    g = sh.g_kv_indptr.clone()
    g[-1] += 4  # the last request's global list grows by 4: its share by one
    assert _check(sh, g_kv_indptr=g, cp_world_size=4, cp_rank=3) == {"MLA_CHECK_DCP_LENGTHS"}
    # The shard of rank 3 is not rank 0's share (the 5-entry request differs).
    assert _check(sh, g_kv_indptr=sh.g_kv_indptr, cp_world_size=4, cp_rank=0) == {
        "MLA_CHECK_DCP_LENGTHS"}


def test_violations_accumulate_and_the_check_replays_in_a_graph():
    w = _w()
    idx = w.kv_indices.clone()
    qo = w.qo_indptr.clone()
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)

    def run():
        mla.check_inputs(qo, w.kv_indptr, idx, w.kv_pool.shape[0], max_seqlen_q=1,
                         num_q_tokens=w.num_tokens, status=status)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep, (bad_idx, bad_qo, want) in enumerate([(True, False, 4), (True, True, 5),
                                                    (False, False, 0), (False, True, 1)]):
        idx.copy_(w.kv_indices)
        qo.copy_(w.qo_indptr)
        if bad_idx:
            idx[3] = -2
        if bad_qo:
            qo[-1] += 1
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == want, rep


def _args(w):
    return (w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
            w.sm_scale, w.q_scale, w.kv_scale)


def test_debug_build_matches_release_and_refuses_broken_calls(monkeypatch):
    w = _w(qlens=[2, 1, 3, 1])
    o_rel, lse_rel = mla.decode(*_args(w), return_lse=True, max_seqlen_q=3)
    torch.cuda.synchronize()
    monkeypatch.setattr(_lib, "lib", _lib.debug_lib)
    say("[check] debug library: valid call, then a broken index")
    o_dbg, lse_dbg = mla.decode(*_args(w), return_lse=True, max_seqlen_q=3)
    torch.cuda.synchronize()
    assert torch.equal(o_rel, o_dbg) and torch.equal(lse_rel, lse_dbg)
    bad = workloads.Workload(**{**w.__dict__, "kv_indices": w.kv_indices.clone()})
    bad.kv_indices[10] = w.kv_pool.shape[0] + 3
    o = torch.full_like(o_rel, 1.5)
    with pytest.raises(mla.MLAError) as e:
        mla.decode(*_args(bad), return_lse=True, max_seqlen_q=3, o=o)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((o == 1.5).all()), "a refused call writes nothing"
    # The cascade checks its suffix lists and its prefix.
    c = workloads.build("check-cascade", [900, 1000], num_heads=16, real_heads=12,
                        pool_entries=4096, kv_std=0.5, shared_prefix=600, seed=171, device=DEV)
    pre, sptr, suf = workloads.split_prefix(c, 600)
    mla.decode_cascade(c.q, c.kv_pool, c.qo_indptr, pre, sptr, suf, c.sm_scale, c.q_scale,
                       c.kv_scale, max_seqlen_q=1)
    pre_bad = pre.clone()
    pre_bad[-1] = -3
    with pytest.raises(mla.MLAError) as e:
        mla.decode_cascade(c.q, c.kv_pool, c.qo_indptr, pre_bad, sptr, suf, c.sm_scale,
                           c.q_scale, c.kv_scale, max_seqlen_q=1)
    assert e.value.status == 8
