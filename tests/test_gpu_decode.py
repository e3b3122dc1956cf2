"""GPU parity of mla_decode / mla_merge_partials against the float64 oracle.

Every call goes through the C ABI (libmla.so via the ctypes binding).  Inputs
come from the shared seeded generators; the oracle reads back exactly the
bytes the kernels consumed.  Small cases are compared in full; the full-size
workloads are compared on sampled requests in the launch configuration the
benchmark times (one worker per compute unit).
"""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import io as oio
from oracle import mla as omla
from tests.parity import assert_gate, bf16_abs_tol, metrics

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_attention_amd as mla  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run(w, num_workers=0, return_lse=True, q=None, o_dtype=torch.bfloat16):
    """decode() on w's inputs; decode_paged() for a paged cache, decode_dcp()
    for one DCP shard (o_dtype: the shard's output type)."""
    torch.cuda.synchronize()
    args = (w.q if q is None else q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
            w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale)
    if w.page_size > 1:
        assert num_workers == 0
        out = mla.decode_paged(*args, return_lse=return_lse, page_size=w.page_size,
                               max_seqlen_q=w.max_seqlen_q)
    elif w.g_kv_indptr is not None:
        assert num_workers == 0
        out = mla.decode_dcp(*args, return_lse=return_lse, g_kv_indptr=w.g_kv_indptr,
                             cp_world_size=w.cp_size, cp_rank=w.cp_rank, o_dtype=o_dtype,
                             max_seqlen_q=w.max_seqlen_q)
    else:
        out = mla.decode(*args, return_lse=return_lse, max_seqlen_q=w.max_seqlen_q,
                         num_workers=num_workers)
    torch.cuda.synchronize()
    return out


def oracle(w, requests=None):
    a = oio.workload_args(w, requests)
    toks = a["tokens"]
    o, lse = oio.call_decode(a)
    return toks, o, lse


def check(w, requests=None, num_workers=0, where="", bf16_ulp_abs=False,
          o_dtype=torch.bfloat16):
    """Compare with the oracle.  bf16_ulp_abs widens the absolute bound to one
    bf16 unit in the last place at the largest |o| where |o| >= 4 (only for
    cases whose outputs leave the benchmark distributions)."""
    say(f"[parity] {w.name} requests={requests} workers={num_workers}")
    o, lse = run(w, num_workers, o_dtype=o_dtype)
    toks, o_ref, lse_ref = oracle(w, requests)
    m = metrics(o[toks], o_ref, lse[toks], lse_ref)
    say(f"[parity] {w.name}: {m}")
    if bf16_ulp_abs:
        assert_gate(m, where or w.name, abs_tol=bf16_abs_tol(m["ref_absmax"]))
    else:
        assert_gate(m, where or w.name)
    return o, lse, m


# ------------------------------------------------------------------ small cases


def test_tiny_workload_full():
    check(workloads.tiny(DEV))


def small_shared(seed=0, B=4, H=16, qlens=None, real_heads=12):
    rng = np.random.default_rng(seed)
    lengths = [2000 + 1100 + int(x) for x in rng.integers(0, 400, size=B)]
    return workloads.build(
        f"small-shared-{seed}", lengths, num_heads=H, real_heads=real_heads, qlens=qlens,
        pool_entries=1 << 15, kv_std=0.5, q_std=1.0, scale_range=(0.5, 2.0), shared_prefix=2000,
        seed=100 + seed, device=DEV,
    )


@pytest.mark.parametrize("nw", [0, 1, 2, 3, 16, 256])
def test_small_shared_prefix_any_worker_count(nw):
    check(small_shared(), num_workers=nw, where=f"small nw={nw}")


# Ragged group-mode call (96 heads, draft tokens): with 23, 37 or 58 workers
# some share boundaries fall inside a unit's leading charge rows (checked on
# the CPU in test_plan.py), so a worker is charged for a unit start it does
# not run and the next worker takes the unit from its first entry.
CHARGE_LENGTHS = [700, 1900, 260, 3000, 45, 1200]
CHARGE_QLENS = [4, 2, 3, 1, 4, 2]


@pytest.mark.parametrize("nw", [5, 23, 37, 58])
def test_group_mode_share_boundaries_in_charge_rows(nw):
    w = workloads.build("charge", CHARGE_LENGTHS, num_heads=96, real_heads=96, qlens=CHARGE_QLENS,
                        pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0), seed=131,
                        device=DEV)
    check(w, num_workers=nw, where=f"charge rows nw={nw}")


@pytest.mark.parametrize("heads", [16, 96])
def test_one_long_request_split_over_many_workers(heads):
    """One request split over ~100-150 workers: the combine merges more than 16
    partials per row, which takes its four-wave path (standard and group mode)."""
    n = 40_000 if heads == 16 else 30_000
    w = workloads.build(f"long-{heads}", [n], num_heads=heads, real_heads=heads,
                        pool_entries=1 << 16, kv_std=0.5, scale_range=(0.5, 2.0), seed=61,
                        device=DEV)
    check(w, num_workers=256, where=f"one long request, {heads} heads")


def test_ragged_lengths_and_empty_requests():
    lengths = [0, 1, 31, 32, 33, 100, 1000, 4097, 0, 2]
    qlens = [1, 1, 1, 1, 1, 1, 1, 1, 1, 1]
    w = workloads.build("ragged", lengths, num_heads=16, real_heads=12, qlens=qlens,
                        pool_entries=8192, kv_std=1.0, scale_range=(0.5, 2.0), seed=7, device=DEV)
    for nw in (0, 5):
        o, lse, _ = check(w, num_workers=nw, where=f"ragged nw={nw}")
        assert torch.all(o[0] == 0) and torch.all(o[8] == 0)
        assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[8]))


def test_multi_token_causal_many_heads():
    w = workloads.build("mt-96", [700, 1333, 3], num_heads=96, real_heads=96, qlens=[4, 3, 4],
                        pool_entries=4096, kv_std=0.5, scale_range=(0.5, 2.0), seed=8, device=DEV)
    for nw in (0, 7):
        check(w, num_workers=nw, where=f"mt-96 nw={nw}")


@pytest.mark.parametrize("dtype,heads", [("fp8", 16), ("fp8", 96), ("bf16", 16)])
def test_multi_token_call_equals_truncated_single_token_calls(dtype, heads):
    """Draft token j of qlen sees the first n - (qlen - 1 - j) entries: the
    multi-token call and single-token calls over those prefixes (different
    kernels: group mode vs the standard one for fp8) must both match the
    oracle's row for that token.  (Each is compared with the oracle, not with
    the other: two bf16 results can differ by twice the gate.)"""
    w = workloads.build(f"trunc-{dtype}-{heads}", [1500, 2999], num_heads=heads,
                        real_heads=heads, qlens=[4, 3], pool_entries=8192, kv_std=0.5,
                        scale_range=(0.5, 2.0), dtype=dtype, seed=17, device=DEV)
    o, lse = run(w)
    toks, o_ref, lse_ref = oracle(w)
    assert list(toks) == list(range(w.num_tokens))
    assert_gate(metrics(o, o_ref, lse, lse_ref), f"{dtype} {heads} heads: multi-token call")
    kvp = w.kv_indptr.cpu().tolist()
    qo = w.qo_indptr.cpu().tolist()
    for b in range(2):
        n, ql = kvp[b + 1] - kvp[b], qo[b + 1] - qo[b]
        for j in range(ql):
            vis = n - (ql - 1 - j)
            t = qo[b] + j
            one = workloads.Workload(**{
                **w.__dict__, "q": w.q[t:t + 1].contiguous(),
                "qo_indptr": torch.tensor([0, 1], dtype=torch.int32, device=DEV),
                "kv_indptr": torch.tensor([0, vis], dtype=torch.int32, device=DEV),
                "kv_indices": w.kv_indices[kvp[b]: kvp[b] + vis].contiguous(),
                "kv_last_page_lens": w.kv_last_page_lens[:1], "lengths": [vis], "qlens": [1],
                "max_seqlen_q": 1})
            o1, l1 = run(one)
            m = metrics(o1, o_ref[t:t + 1], l1, lse_ref[t:t + 1])
            assert_gate(m, f"{dtype} {heads} heads: request {b} token {j} as a single-token call")


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_largest_draft_length_and_head_count(dtype):
    """max_seqlen_q = 64 (the largest accepted) with 128 heads: early draft
    tokens of short requests see nothing; fp8 runs in group mode (64 row
    groups of 8 head groups), bf16 in the standard kernel."""
    w = workloads.build(f"max-{dtype}", [5000, 70, 40, 0], num_heads=128, real_heads=128,
                        qlens=[64, 1, 33, 2], pool_entries=8192, kv_std=0.5,
                        scale_range=(0.5, 2.0), dtype=dtype, seed=27, device=DEV)
    o, lse, _ = check(w, where=f"qlen 64, 128 heads, {dtype}")
    T0 = 64 + 1  # request 2's first token
    assert torch.all(torch.isfinite(lse[T0 + 32]))  # its last token sees all 40 entries
    assert torch.all(lse[-2:] == -float("inf"))  # request 3 has no entries


def test_many_requests_span_several_planner_chunks():
    """700 requests (the planner scans requests 256 at a time per workgroup)
    with ragged lengths, some empty."""
    rng = np.random.default_rng(29)
    lengths = [int(x) for x in rng.integers(0, 400, size=700)]
    for i in range(0, 700, 37):
        lengths[i] = 0
    w = workloads.build("many-requests", lengths, num_heads=16, real_heads=12,
                        pool_entries=1 << 18, kv_std=0.5, scale_range=(0.5, 2.0), seed=28,
                        device=DEV)
    check(w, requests=[0, 1, 255, 256, 257, 511, 512, 699], where="700 requests")


def test_peaky_scores():
    """Stress case outside the benchmark distributions: |o| reaches ~5, where a
    bf16 unit in the last place (2^-5) exceeds 1e-2, so the absolute bound is
    bf16's own resolution at that magnitude; row-relative and lse gates hold."""
    w = workloads.build("peaky", [5000, 77], num_heads=32, real_heads=32, pool_entries=8192,
                        kv_std=2.0, q_std=4.0, scale_range=(0.5, 2.0), seed=9, device=DEV)
    o, lse = run(w)
    _, o_ref, lse_ref = oracle(w)
    m = metrics(o, o_ref, lse, lse_ref)
    say(f"[parity] peaky: {m}")
    assert_gate(m, "peaky", abs_tol=bf16_abs_tol(m["ref_absmax"]))


# ------------------------------------------------------------------ group mode
# fp8 calls with num_heads / 16 * max_seqlen_q >= 4 run the group-mode kernel:
# one workgroup walks 4 row groups of one request over a shared KV range.


def group_ragged():
    lengths = [0, 1, 31, 32, 33, 100, 1000, 4097, 0, 2, 20000]
    return workloads.build("group-ragged", lengths, num_heads=64, real_heads=60,
                           pool_entries=1 << 15, kv_std=1.0, scale_range=(0.5, 2.0), seed=21,
                           device=DEV)


@pytest.mark.parametrize("nw", [0, 1, 3, 37, 512])
def test_group_mode_ragged_any_worker_count(nw):
    """64 heads, one token per request: a unit is the token's 4 head groups.
    Requests of 1-2 entries return (scaled) V rows themselves, up to |o| ~ 4,
    where bf16's own rounding exceeds 1e-2: the absolute bound is one bf16
    unit in the last place at that magnitude (row-relative and lse gates as
    everywhere)."""
    o, lse, _ = check(group_ragged(), num_workers=nw, where=f"group ragged nw={nw}",
                      bf16_ulp_abs=True)
    for t in (0, 8):
        assert torch.all(o[t] == 0) and torch.all(torch.isneginf(lse[t]))


@pytest.mark.parametrize("nw", [0, 1, 5, 100])
def test_group_mode_units_span_tokens(nw):
    """16 heads, several query tokens: a unit holds 4 consecutive tokens, each
    wave masking its own causal limit; early draft tokens see nothing."""
    w = workloads.build("group-tokens", [5000, 10, 2, 3000, 1], num_heads=16, real_heads=12,
                        qlens=[4, 1, 3, 4, 2], pool_entries=16384, kv_std=0.5,
                        scale_range=(0.5, 2.0), seed=22, device=DEV)
    o, lse, _ = check(w, num_workers=nw, where=f"group tokens nw={nw}")
    qo = w.qo_indptr.cpu().tolist()
    empty = [qo[2], qo[4]]  # (n=2, qlen=3) token 0; (n=1, qlen=2) token 0
    for t in empty:
        assert torch.all(o[t] == 0) and torch.all(torch.isneginf(lse[t]))


@pytest.mark.parametrize("nw", [0, 3])
def test_group_mode_single_row_group_requests(nw):
    """16 heads with one 4-token request forces group mode; the single-token
    requests then form units of one row group (seven of eight idle)."""
    w = workloads.build("group-r1", [900, 2100, 5, 0, 3001, 1], num_heads=16, real_heads=12,
                        qlens=[1, 4, 1, 1, 1, 1], pool_entries=8192, kv_std=0.5,
                        scale_range=(0.5, 2.0), seed=19, device=DEV)
    check(w, num_workers=nw, where=f"group mode, one-row-group units, nw={nw}")


@pytest.mark.parametrize("nw", [1, 2, 0])
@pytest.mark.parametrize("heads", [64, 16])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_scores_rising_far_above_the_first_tiles(sign, heads, nw):
    """Request 0's later entries score ~426 base-2 units above its first 4,500.
    With 64 heads (group mode) a piece that sees this redoes its pass with the
    row's true maximum: one piece over both index segments (nw=1, 6,000
    entries > 4,096 staged per segment), a piece straddling the jump (nw=2), or
    the default split.  sign = -1 runs the same with a negative sm_scale (the
    kernel moves the sign onto q).  With 16 heads the standard kernel's running
    maximum takes the same jump."""
    w = workloads.redo_case(sign, heads, device=DEV)
    w.sm_scale = sign * w.sm_scale
    _, _, m = check(w, num_workers=nw, where=f"redo sign={sign} heads={heads} nw={nw}")
    assert m["ref_absmax"] > 0


@pytest.mark.parametrize("heads", [16, 64])
def test_zero_score_scale_gives_the_mean_of_v(heads):
    """sm_scale = 0: every score is 0, so o is the mean of the visible V rows
    and lse = ln n."""
    w = workloads.build(f"zero-scale-h{heads}", [1, 700, 5000], num_heads=heads,
                        real_heads=heads, pool_entries=1 << 13, kv_std=0.5, seed=93, device=DEV)
    w.sm_scale = 0.0
    check(w, where=f"zero scale heads={heads}")


def test_group_mode_pad_heads_bitwise_and_deterministic():
    w = workloads.build("group-pad", [3000, 1234, 77], num_heads=64, real_heads=60,
                        qlens=[2, 1, 2], pool_entries=8192, seed=23, device=DEV)
    o_zero, lse_zero = run(w)
    o_again, lse_again = run(w)
    assert torch.equal(o_zero, o_again) and torch.equal(lse_zero, lse_again)
    q_rand = w.q.clone()
    g = torch.Generator(device=DEV).manual_seed(8)
    noise = torch.randn(q_rand[:, 60:].shape, generator=g, device=DEV).clamp(-448, 448)
    q_rand[:, 60:] = noise.to(torch.float8_e4m3fn)
    o_r, lse_r = run(w, q=q_rand)
    assert torch.equal(o_r[:, :60], o_zero[:, :60])
    assert torch.equal(lse_r[:, :60], lse_zero[:, :60])


def test_group_mode_graph_replay_matches_eager_bitwise():
    w = workloads.build("group-graph", [2500, 900, 4000], num_heads=32, real_heads=32,
                        qlens=[2, 2, 1], pool_entries=8192, seed=24, device=DEV)
    o_eager, lse_eager = run(w)
    o = torch.empty_like(o_eager)
    lse = torch.empty_like(lse_eager)
    ws = mla.new_workspace(mla.workspace_bytes(w.batch, w.num_tokens, w.num_heads, 2), DEV)

    def call():
        mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
                   w.sm_scale, w.q_scale, w.kv_scale, return_lse=True, o=o, lse=lse,
                   max_seqlen_q=2, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_()
        lse.fill_(7.0)
        run(group_ragged())  # unrelated eager work on the same device
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), f"replay {rep}"
        assert torch.equal(lse, lse_eager), f"replay {rep}"


# ------------------------------------------------------------------ cascade
# decode_cascade(q, prefix + per-request suffixes) must equal decode() over the
# concatenated lists.


def run_cascade(w, prefix, return_lse=True):
    pre, sptr, suf = workloads.split_prefix(w, prefix)
    torch.cuda.synchronize()
    out = mla.decode_cascade(w.q, w.kv_pool, w.qo_indptr, pre, sptr, suf, w.sm_scale, w.q_scale,
                             w.kv_scale, return_lse=return_lse, max_seqlen_q=w.max_seqlen_q)
    torch.cuda.synchronize()
    return out


def check_cascade(w, prefix, requests=None, where="", bf16_ulp_abs=False):
    say(f"[cascade] {w.name} prefix={prefix} requests={requests}")
    o, lse = run_cascade(w, prefix)
    toks, o_ref, lse_ref = oracle(w, requests)
    m = metrics(o[toks], o_ref, lse[toks], lse_ref)
    say(f"[cascade] {w.name}: {m}")
    tol = {"abs_tol": bf16_abs_tol(m["ref_absmax"])} if bf16_ulp_abs else {}
    assert_gate(m, where or f"cascade {w.name}", **tol)
    return o, lse


def test_cascade_small_matches_oracle_and_plain_call():
    w = small_shared(11)
    o, lse = check_cascade(w, 2000)
    o2, lse2 = run(w)
    m = metrics(o, o2.float().cpu().numpy().astype(np.float64), lse, lse2.cpu().numpy())
    assert_gate(m, "cascade vs plain decode")


def test_cascade_edge_cases():
    """No prefix; empty suffixes; a request that is prefix only."""
    w = workloads.build("casc-edge", [1500, 1200, 1200, 2900], num_heads=32, real_heads=32,
                        pool_entries=8192, kv_std=0.5, scale_range=(0.5, 2.0), shared_prefix=1200,
                        seed=31, device=DEV)
    check_cascade(w, 1200, where="cascade: suffixes 300, 0, 0, 1700")
    check_cascade(w, 0, where="cascade: no prefix")
    v = workloads.build("casc-pre-only", [900, 900], num_heads=16, real_heads=12, pool_entries=4096,
                        shared_prefix=900, seed=32, device=DEV)
    check_cascade(v, 900, where="cascade: every suffix empty")


def test_cascade_multi_token_many_heads():
    """Draft tokens with 64 heads: the suffix pass runs in group mode, and every
    suffix holds at least qlen - 1 entries."""
    w = workloads.build("casc-mt", [2500, 2003, 2600], num_heads=64, real_heads=64,
                        qlens=[2, 4, 1], pool_entries=8192, kv_std=0.5, scale_range=(0.5, 2.0),
                        shared_prefix=2000, seed=33, device=DEV)
    check_cascade(w, 2000)


@pytest.mark.parametrize("H,qlens", [(12, None), (12, [2, 1, 3, 1]), (20, [1, 2, 1, 1]),
                                     (1, [3, 1, 1, 2]), (44, None)])
def test_cascade_unpadded_heads_match_oracle(H, qlens):
    """Any head count, unpadded: query rows (token, head) are packed 16 to a
    row group, so a row group can hold rows of two or more tokens (each masked
    by its own token's visible count under draft tokens)."""
    w = workloads.build(f"casc-h{H}", [2600, 2100, 3300, 2050], num_heads=H, real_heads=H,
                        qlens=qlens, pool_entries=16384, kv_std=0.5, scale_range=(0.5, 2.0),
                        shared_prefix=2000, seed=40 + H, device=DEV)
    check_cascade(w, 2000, where=f"cascade, {H} unpadded heads, qlens {qlens}")


def test_cascade_unpadded_12_heads_equal_the_padded_call_on_the_real_heads():
    """12 unpadded heads against the same q padded to 16 with zero heads: the
    real heads agree within the gate (different tile packings, same rows)."""
    w = workloads.build("casc-pad", [2600, 2100, 3300, 2050], num_heads=16, real_heads=12,
                        pool_entries=16384, kv_std=0.5, scale_range=(0.5, 2.0),
                        shared_prefix=2000, seed=51, device=DEV)
    w12 = workloads.Workload(**{**w.__dict__, "q": w.q[:, :12].contiguous(), "num_heads": 12,
                                "real_heads": 12, "name": "casc-pad-12"})
    o16, lse16 = run_cascade(w, 2000)
    o12, lse12 = run_cascade(w12, 2000)
    m = metrics(o12, o16[:, :12].float().cpu().numpy().astype(np.float64), lse12,
                lse16[:, :12].cpu().numpy())
    say(f"[cascade 12 vs 16] {m}")
    assert_gate(m, "cascade 12 unpadded heads vs padded to 16")


def test_cascade_graph_replay_matches_eager_bitwise():
    w = small_shared(12)
    pre, sptr, suf = workloads.split_prefix(w, 2000)
    o_e, lse_e = run_cascade(w, 2000)
    o = torch.empty_like(o_e)
    lse = torch.empty_like(lse_e)
    ws = mla.new_workspace(mla.cascade_workspace_bytes(w.batch, w.num_tokens, w.num_heads, 1), DEV)

    def call():
        mla.decode_cascade(w.q, w.kv_pool, w.qo_indptr, pre, sptr, suf, w.sm_scale, w.q_scale,
                           w.kv_scale, return_lse=True, o=o, lse=lse, max_seqlen_q=1, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_()
        lse.fill_(7.0)
        run(small_shared(8))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), f"replay {rep}"
        assert torch.equal(lse, lse_e), f"replay {rep}"


# ------------------------------------------------------------------ bf16 storage


def test_tiny_workload_bf16_full():
    w = workloads.build("tiny-bf16", [64, 100], num_heads=16, real_heads=12, pool_entries=256,
                        dtype="bf16", seed=1, device=DEV)
    check(w)


@pytest.mark.parametrize("nw", [0, 1, 3, 256])
def test_small_bf16_any_worker_count(nw):
    rng = np.random.default_rng(11)
    lengths = [1500 + int(x) for x in rng.integers(0, 900, size=5)]
    w = workloads.build("small-bf16", lengths, num_heads=32, real_heads=28, pool_entries=1 << 14,
                        dtype="bf16", kv_std=1.0, scale_range=(0.5, 2.0), shared_prefix=1200,
                        seed=111, device=DEV)
    check(w, num_workers=nw, where=f"small bf16 nw={nw}")


def test_ragged_lengths_bf16():
    """Lengths around the 16-row bf16 tile and the 4-wave tile interleave.

    A one-entry request returns kv_scale times its bf16 V row, |o| up to ~7,
    where bf16's own rounding (half a unit in the last place = 2^-6) exceeds
    1e-2: the absolute bound there is bf16's resolution; the row-relative and
    lse gates are unchanged."""
    lengths = [0, 1, 15, 16, 17, 63, 64, 65, 129, 2049, 0, 3]
    w = workloads.build("ragged-bf16", lengths, num_heads=16, real_heads=12, pool_entries=8192,
                        dtype="bf16", scale_range=(0.5, 2.0), seed=17, device=DEV)
    for nw in (0, 5):
        o, lse, _ = check(w, num_workers=nw, where=f"ragged bf16 nw={nw}", bf16_ulp_abs=True)
        assert torch.all(o[0] == 0) and torch.all(o[10] == 0)
        assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[10]))


def test_multi_token_causal_bf16():
    w = workloads.build("mt-bf16", [700, 1333, 3], num_heads=96, real_heads=96, qlens=[4, 3, 4],
                        pool_entries=4096, dtype="bf16", scale_range=(0.5, 2.0), seed=18,
                        device=DEV)
    for nw in (0, 7):
        check(w, num_workers=nw, where=f"mt-bf16 nw={nw}")


def test_pad_heads_bf16_bitwise():
    w = workloads.build("pad-bf16", [3000, 1234], num_heads=16, real_heads=12, pool_entries=8192,
                        dtype="bf16", seed=19, device=DEV)
    o_zero, lse_zero = run(w)
    q_rand = w.q.clone()
    g = torch.Generator(device=DEV).manual_seed(6)
    q_rand[:, 12:] = torch.randn(q_rand[:, 12:].shape, generator=g, device=DEV).to(torch.bfloat16)
    o_r, lse_r = run(w, q=q_rand)
    assert torch.equal(o_r[:, :12], o_zero[:, :12])
    assert torch.equal(lse_r[:, :12], lse_zero[:, :12])


# ------------------------------------------------------------------ invariants


def test_pad_heads_do_not_change_real_heads_bitwise():
    w = small_shared(1)
    o_zero, lse_zero = run(w)
    q_rand = w.q.clone()
    g = torch.Generator(device=DEV).manual_seed(5)
    noise = torch.randn(q_rand[:, 12:].shape, generator=g, device=DEV).clamp(-448, 448)
    q_rand[:, 12:] = noise.to(torch.float8_e4m3fn)
    o_r, lse_r = run(w, q=q_rand)
    assert torch.equal(o_r[:, :12], o_zero[:, :12])
    assert torch.equal(lse_r[:, :12], lse_zero[:, :12])


def test_workspace_reused_across_calls():
    """One workspace serves consecutive calls of different shapes and worker
    counts (nothing in it survives from one call to the next)."""
    ws = mla.new_workspace(mla.workspace_bytes(64, 64, 96, 4, num_workers=300), DEV)
    cases = [(small_shared(5), 300), (small_shared(6, B=3), 37), (small_shared(5), 300),
             (workloads.build("reuse-mt", [900, 40], num_heads=32, real_heads=32, qlens=[2, 4],
                              pool_entries=4096, scale_range=(0.5, 2.0), seed=12, device=DEV), 11)]
    for w, nw in cases:
        o, lse = mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                            w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                            return_lse=True, max_seqlen_q=w.max_seqlen_q, workspace=ws,
                            num_workers=nw)
        torch.cuda.synchronize()
        _, o_ref, lse_ref = oracle(w)
        assert_gate(metrics(o, o_ref, lse, lse_ref), f"reuse {w.name} nw={nw}")


def test_graph_replay_matches_eager_bitwise():
    """A decode captured in a HIP graph and replayed (with eager work between
    replays) gives the eager result bit for bit on every replay."""
    w = small_shared(7)
    o_eager, lse_eager = run(w)
    o = torch.empty_like(o_eager)
    lse = torch.empty_like(lse_eager)
    ws = mla.new_workspace(mla.workspace_bytes(w.batch, w.num_tokens, w.num_heads, 1), DEV)

    def call():
        mla.decode(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
                   w.sm_scale, w.q_scale, w.kv_scale, return_lse=True, o=o, lse=lse,
                   max_seqlen_q=1, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_()
        lse.fill_(7.0)
        run(small_shared(8))  # unrelated eager work on the same device
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), f"replay {rep}"
        assert torch.equal(lse, lse_eager), f"replay {rep}"


def test_run_to_run_bitwise_deterministic():
    w = small_shared(2)
    a = run(w)
    b = run(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_power_of_two_scale_exchange_is_bitwise():
    w = small_shared(3)
    o1, lse1 = run(w)
    w2 = workloads.Workload(**{**w.__dict__, "kv_scale": w.kv_scale * 2, "sm_scale": w.sm_scale / 2})
    o2, lse2 = run(w2)
    assert torch.equal(o2.float(), 2 * o1.float())
    assert torch.equal(lse2, lse1)


def test_kv_permutation_within_requests():
    w = small_shared(4)
    o1, lse1 = run(w)
    idx = w.kv_indices.clone()
    kvp = w.kv_indptr.cpu().tolist()
    g = torch.Generator(device=DEV).manual_seed(3)
    for b in range(w.batch):
        s, e = kvp[b], kvp[b + 1]
        idx[s:e] = idx[s:e][torch.randperm(e - s, generator=g, device=DEV)]
    w2 = workloads.Workload(**{**w.__dict__, "kv_indices": idx})
    o2, lse2 = run(w2)
    m = metrics(o2, o1.float().cpu().numpy().astype(np.float64), lse2, lse1.cpu().numpy())
    assert_gate(m, "permutation")


def test_dcp_shards_plus_merge_equal_the_full_call():
    """8 KV shards decoded with return_lse, merged by mla_merge_partials."""
    full = workloads.build("dcp-mini", [1600, 2400], num_heads=32, real_heads=32, qlens=[1, 1],
                           pool_entries=8192, kv_std=0.5, scale_range=(0.5, 2.0), seed=10, device=DEV)
    o_full, lse_full = run(full)
    kvp = full.kv_indptr.cpu().tolist()
    S = 8
    parts_o, parts_l = [], []
    for s in range(S):
        pieces, lens = [], []
        for b in range(full.batch):
            n = kvp[b + 1] - kvp[b]
            lo, hi = n * s // S, n * (s + 1) // S
            pieces.append(full.kv_indices[kvp[b] + lo: kvp[b] + hi])
            lens.append(hi - lo)
        ind = torch.cat(pieces)
        kv_indptr = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
        ws = workloads.Workload(**{**full.__dict__, "kv_indices": ind, "kv_indptr": kv_indptr, "lengths": lens})
        o_s, l_s = run(ws)
        parts_o.append(o_s)
        parts_l.append(l_s)
    o_m, lse_m = mla.merge_partials(torch.stack(parts_o), torch.stack(parts_l))
    toks, o_ref, lse_ref = oracle(full)
    assert_gate(metrics(o_m, o_ref, lse_m, lse_ref), "dcp merged vs oracle")
    assert_gate(metrics(o_full, o_ref, lse_full, lse_ref), "dcp full vs oracle")


# ------------------------------------------------------------------ DCP shards
# Positions dealt round-robin over the shards (mla_decode_dcp): every shard
# against the oracle's shard rule, and the merged shards against the full call.

DCP_CASES = {
    "fp8-16heads-standard": dict(num_heads=16, real_heads=12, qlens=[1, 3, 2, 3, 1, 3, 2],
                                 dtype="fp8"),
    "fp8-96heads-group": dict(num_heads=96, real_heads=96, qlens=[4, 1, 3, 4, 2, 4, 4],
                              dtype="fp8"),
    "bf16-16heads": dict(num_heads=16, real_heads=12, qlens=[4, 1, 3, 4, 2, 4, 4], dtype="bf16"),
}


@pytest.mark.parametrize("case", sorted(DCP_CASES))
def test_dcp_interleaved_shards_and_merge(case):
    """Every shard against the oracle's shard rule, then the 8 shards merged
    against the full call.  The shards return fp32 o (and keep fp32 split
    partials), so the merged bf16 answer is rounded once, by the merge, and is
    held to the same gate as a single call."""
    kw = DCP_CASES[case]
    full = workloads.build(f"dcp-{case}", [0, 3, 9, 700, 2501, 4096, 5003], pool_entries=1 << 14,
                           kv_std=0.5, scale_range=(0.5, 2.0), seed=71, device=DEV, **kw)
    W = 8
    parts_o, parts_l = [], []
    for r in range(W):
        shard = workloads.dcp_shard(full, W, r)
        o, lse, _ = check(shard, where=f"dcp {case} rank {r}", o_dtype=torch.float32)
        assert o.dtype == torch.float32
        parts_o.append(o)
        parts_l.append(lse)
    o_m, lse_m = mla.merge_partials(torch.stack(parts_o), torch.stack(parts_l))
    toks, o_ref, lse_ref = oracle(full)
    m = metrics(o_m, o_ref, lse_m, lse_ref)
    say(f"[dcp] {case} merged: {m}")
    assert_gate(m, f"dcp {case}: 8 shards merged vs the full call")


@pytest.mark.parametrize("case", sorted(DCP_CASES))
def test_dcp_bf16_shard_outputs(case):
    """The shards' default bf16 output: each shard is one call, held to the gate."""
    kw = DCP_CASES[case]
    full = workloads.build(f"dcp16-{case}", [0, 3, 9, 700, 2501, 4096, 5003],
                           pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0), seed=72,
                           device=DEV, **kw)
    for r in (0, 5, 7):
        o, _, _ = check(workloads.dcp_shard(full, 8, r), where=f"dcp bf16 out {case} rank {r}")
        assert o.dtype == torch.bfloat16


def test_dcp_bad_arguments_are_rejected():
    w = workloads.dcp_shard(workloads.tiny(DEV), 2, 1)
    for cps, cpr in ((2, 2), (0, 0), (2, -1)):
        with pytest.raises(mla.MLAError):
            mla.decode_dcp(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, None,
                           w.sm_scale, g_kv_indptr=w.g_kv_indptr, cp_world_size=cps, cp_rank=cpr)


# ------------------------------------------------------------------ paged cache
# mla_decode_paged: kv_indices hold page numbers; ragged last pages, empty
# requests, draft tokens, both storage types and both kernels.

PAGED_CASES = {
    "fp8-p128-16heads": dict(page_size=128, num_heads=16, real_heads=12, qlens=None, dtype="fp8"),
    "fp8-p2-16heads-draft": dict(page_size=2, num_heads=16, real_heads=12,
                                 qlens=[1, 3, 2, 1, 3, 2, 3], dtype="fp8"),
    "fp8-p16-96heads-group": dict(page_size=16, num_heads=96, real_heads=96,
                                  qlens=[4, 1, 3, 4, 2, 4, 4], dtype="fp8"),
    "bf16-p128-draft": dict(page_size=128, num_heads=16, real_heads=12,
                            qlens=[4, 1, 3, 4, 2, 4, 4], dtype="bf16"),
}


@pytest.mark.parametrize("case", sorted(PAGED_CASES))
def test_paged_cache_matches_oracle(case):
    kw = dict(PAGED_CASES[case])
    P = kw["page_size"]
    w = workloads.build(f"paged-{case}", [0, 1, 127, 128, 129, 1000, 5003],
                        pool_entries=P * max(64, (1 << 15) // P), kv_std=0.5,
                        scale_range=(0.5, 2.0), shared_prefix=300, seed=81, device=DEV, **kw)
    o, lse, _ = check(w, where=f"paged {case}")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_paged_bad_arguments_are_rejected():
    w = workloads.build("paged-bad", [200], num_heads=16, pool_entries=1024, seed=82, device=DEV,
                        page_size=128)
    for P in (3, 8192, 0):
        with pytest.raises(mla.MLAError):
            mla.decode_paged(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                             w.kv_last_page_lens, w.sm_scale, page_size=P)
    with pytest.raises(mla.MLAError):  # the pool is not a whole number of pages
        mla.decode_paged(w.q, w.kv_pool[:1000], w.qo_indptr, w.kv_indptr, w.kv_indices,
                         w.kv_last_page_lens, w.sm_scale, page_size=128)


# ------------------------------------------------------------------ merge


@pytest.mark.parametrize("parts_dtype", ["fp32", "bf16"])
def test_merge_partials_full_size(parts_dtype):
    o_p, lse_p = workloads.merge_shards(parts_dtype=parts_dtype, device=DEV)
    o, lse = mla.merge_partials(o_p, lse_p)
    torch.cuda.synchronize()
    ref_o, ref_lse = omla.merge_partials(oio.codes(o_p).astype(np.float64) if parts_dtype == "fp32"
                                         else _bf16_to_f64(o_p), lse_p.cpu().numpy().astype(np.float64))
    m = metrics(o, ref_o, lse, ref_lse)
    say(f"[merge] {parts_dtype}: {m}")
    assert_gate(m, f"merge {parts_dtype}")


@pytest.mark.parametrize("parts_dtype", ["fp32", "bf16"])
def test_merge_ignores_empty_shard_rows(parts_dtype):
    """Rows of shards marked empty (lse = -inf) may hold anything, NaN included."""
    o_p, lse_p = workloads.merge_shards(num_parts=11, num_tokens=5, num_heads=32,
                                        parts_dtype=parts_dtype, seed=77, device=DEV)
    o_ref_in = o_p.clone()
    o_p[torch.isneginf(lse_p)] = float("nan")
    o, lse = mla.merge_partials(o_p, lse_p)
    o2, lse2 = mla.merge_partials(o_ref_in, lse_p)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    ref_o, ref_lse = omla.merge_partials(
        oio.codes(o_ref_in).astype(np.float64) if parts_dtype == "fp32" else _bf16_to_f64(o_ref_in),
        lse_p.cpu().numpy().astype(np.float64))
    assert_gate(metrics(o, ref_o, lse, ref_lse), f"merge empty rows {parts_dtype}")


def _bf16_to_f64(t):
    from oracle import codecs
    return codecs.decode_bf16(oio.codes(t))


# ------------------------------------------------------------------ full sizes (sampled)


def test_headline_batch16_sampled():
    w = workloads.c16(DEV, "shared", return_lse=True)
    check(w, requests=[0, 7, 15])
    del w


def test_headline_batch16_unshared_prefix_sampled():
    w = workloads.c16(DEV, "unshared", return_lse=True)
    check(w, requests=[3, 12])


def test_batch24_sampled():
    w = workloads.c24(DEV, return_lse=True)
    check(w, requests=[0, 11, 23])


def test_mixed_lengths_fp8_sampled():
    w = workloads.mixed(DEV, "fp8", return_lse=True)
    L = np.array(w.lengths)
    check(w, requests=[int(L.argmax()), int(L.argmin()), 17])


def test_mixed_lengths_bf16_sampled():
    w = workloads.mixed(DEV, "bf16", return_lse=True)
    L = np.array(w.lengths)
    check(w, requests=[int(L.argmax()), int(L.argmin()), 17])
    del w


def test_dcp_share_sampled():
    """One DCP8 rank at full size (rank 7 of 142,000 positions per request)."""
    w = workloads.dcp_share(DEV)
    check(w, requests=[0, 5])


def test_dcp_local_share_sampled():
    """The DCP8-shaped share with the bottom-right mask on the shard's own list
    (batch 8, 96 heads, 4 draft tokens, 17,750 entries per request), sampled."""
    w = workloads.dcp_local(DEV)
    check(w, requests=[0, 6])


def test_headline_batch16_paged128_sampled():
    """The headline call as a page table of 128-slot pages (mla_decode_paged)."""
    w = workloads.c16(DEV, "paged128", return_lse=True)
    check(w, requests=[0, 9])
    del w


def test_headline_batch16_cascade_sampled():
    w = workloads.c16(DEV, "shared", return_lse=True)
    check_cascade(w, workloads.SHARED_PREFIX, requests=[0, 7, 15])
    del w


def test_headline_batch16_cascade_12_unpadded_heads_sampled():
    """The batch-16 call's 12 real heads passed unpadded to the cascade (its
    prefix pass packs 16 tokens x 12 heads into 12 row groups, not 16)."""
    w = workloads.c16(DEV, "shared", return_lse=True)
    w12 = workloads.Workload(**{**w.__dict__, "q": w.q[:, :12].contiguous(), "num_heads": 12,
                                "real_heads": 12, "name": "c16-12heads"})
    del w
    check_cascade(w12, workloads.SHARED_PREFIX, requests=[0, 7, 15])
    del w12


def test_captured_argument_layout_is_accepted():
    """The exact tensors of the captured call, including the (N,1,1,576) view."""
    w = workloads.c16(DEV, "shared")
    kv4 = w.kv_pool.view(-1, 1, 1, 576)
    assert tuple(kv4.stride()) == (576, 576, 576, 1)
    o = mla.decode(w.q, kv4, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
                   w.sm_scale, w.q_scale, w.kv_scale, max_seqlen_q=1)
    torch.cuda.synchronize()
    assert o.shape == (16, 16, 512) and o.dtype == torch.bfloat16 and o.stride() == (8192, 512, 1)
    assert w.kv_indices.numel() == workloads.INDEX_BUFFER
