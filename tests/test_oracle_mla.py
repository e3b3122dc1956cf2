"""Pins for the float64 oracle (CPU only).

Each test fixes the oracle against something other than itself: a scalar
brute force with exact integer dot products and 50-digit softmax, closed forms,
and invariants the pages state.  Pages: "[Kimi-K3 MLA TP8] MLA performance"
([Issue]) and "Kimi K3 on AMD Instinct MI355X: vLLM Serving Matches NVIDIA HGX
B300 Throughput per GPU on AgentX" ([Blog]).
"""

import math

import numpy as np
import pytest

import workloads
from oracle import brute, codecs
from oracle import io as oio
from oracle import mla

REL = 1e-12


def _close(a, b, rel=REL):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    scale = max(1.0, float(np.max(np.abs(b[fin])))) if fin.any() else 1.0
    err = float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0
    assert err <= rel * scale, f"max abs diff {err:.3e} > {rel:.1e} * {scale:.3e}"


def _args(w):
    a = oio.workload_args(w)
    a.pop("tokens")
    return a


# ---------------------------------------------------------------- brute force


def test_oracle_matches_brute_force_on_tiny_workload():
    """Full tiny workload (2 requests, 16 heads, kv 64/100, zero pad heads)."""
    a = _args(workloads.tiny())
    o, lse = mla.mla_decode(**a)
    ob, lseb = brute.brute_decode(**a)
    _close(o, ob)
    _close(lse, lseb)


def test_oracle_matches_brute_force_bf16_causal_scaled():
    """bf16 storage, 4 query tokens (causal), non-unit scales, a 1-entry request."""
    w = workloads.build(
        "bf16-causal", [7, 1, 12], num_heads=16, real_heads=16, qlens=[4, 1, 3],
        pool_entries=64, dtype="bf16", kv_std=0.8, q_std=1.3, scale_range=(0.5, 2.0), seed=11,
    )
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    ob, lseb = brute.brute_decode(**a)
    _close(o, ob)
    _close(lse, lseb)


def test_oracle_matches_brute_force_fp8_large_scores():
    """Wide score range (q_std 4): softmax dominated by a few entries."""
    w = workloads.build(
        "fp8-peaky", [40, 23], num_heads=16, real_heads=16, pool_entries=128, dtype="fp8",
        kv_std=2.0, q_std=4.0, scale_range=(0.5, 2.0), seed=12,
    )
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    ob, lseb = brute.brute_decode(**a)
    _close(o, ob)
    _close(lse, lseb)


# ---------------------------------------------------------------- closed forms


def _exact_scores(a, t, h, rows):
    """s_i with exact integer dots (brute decoder) and fsum, for closed forms."""
    qi = [brute.e4m3fn_to_int(c) for c in a["q"][t, h]]
    out = []
    for r in rows:
        ki = [brute.e4m3fn_to_int(c) for c in a["kv_pool"][r]]
        dot = sum(x * y for x, y in zip(qi, ki))
        out.append(a["sm_scale"] * a["q_scale"] * a["kv_scale"] * math.ldexp(dot, -18))
    return out


def test_single_entry_history_returns_its_value_row():
    w = workloads.build("n1", [1, 1], num_heads=16, pool_entries=16, scale_range=(0.5, 2), seed=3)
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    for b in range(2):
        r = a["kv_indices"][b]
        V = a["kv_scale"] * codecs.decode_e4m3fn(a["kv_pool"][r, :512])
        for h in range(16):
            assert np.array_equal(o[b, h], V)
            (s0,) = _exact_scores(a, b, h, [r])
            assert abs(lse[b, h] - s0) <= 1e-14 * max(1.0, abs(s0))


def test_equal_scores_give_mean_of_values_and_log_n():
    """Zero query rows (the pad heads) score every entry 0."""
    w = workloads.tiny()
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    for b, n in enumerate(w.lengths):
        rows = a["kv_indices"][a["kv_indptr"][b] : a["kv_indptr"][b + 1]]
        V = codecs.decode_e4m3fn(a["kv_pool"][rows, :512])
        mean = np.array([math.fsum(V[:, d]) / n for d in range(512)])
        for h in range(12, 16):
            _close(o[b, h], mean, rel=1e-14)
            assert abs(lse[b, h] - math.log(n)) <= 1e-14 * math.log(n)


def test_two_entries_follow_the_logistic_weights():
    w = workloads.build("n2", [2], num_heads=16, pool_entries=16, q_std=2.0, seed=5)
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    r0, r1 = a["kv_indices"][0], a["kv_indices"][1]
    V0 = codecs.decode_e4m3fn(a["kv_pool"][r0, :512])
    V1 = codecs.decode_e4m3fn(a["kv_pool"][r1, :512])
    for h in range(16):
        s0, s1 = _exact_scores(a, 0, h, [r0, r1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        _close(o[0, h], w0 * V0 + w1 * V1, rel=1e-14)
        hi = max(s0, s1)
        assert abs(lse[0, h] - (hi + math.log1p(math.exp(-abs(s0 - s1))))) <= 1e-14 * max(1, abs(hi))


# ---------------------------------------------------------------- invariants


def test_padding_heads_leave_real_heads_unchanged():
    """[Blog] Sec. 4: adding a head does not change another head's softmax."""
    a = _args(workloads.tiny())
    o16, lse16 = mla.mla_decode(**a)
    a12 = dict(a, q=np.ascontiguousarray(a["q"][:, :12]))
    o12, lse12 = mla.mla_decode(**a12)
    _close(o16[:, :12], o12, rel=1e-15)
    _close(lse16[:, :12], lse12, rel=1e-15)
    # and the pad rows' content does not matter either
    rng = np.random.default_rng(1)
    q_rand = a["q"].copy()
    q_rand[:, 12:] = rng.integers(0, 0x7E, size=q_rand[:, 12:].shape, dtype=np.uint8)
    o_r, lse_r = mla.mla_decode(**dict(a, q=q_rand))
    _close(o_r[:, :12], o12, rel=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merging_any_kv_split_equals_the_unsplit_result(seed):
    """[Blog] Sec. 1 / Sec. 4: partial answers merged by their softmax weights."""
    w = workloads.build("split", [97], num_heads=16, pool_entries=256, q_std=2.0,
                        scale_range=(0.5, 2.0), seed=20 + seed)
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, 97), size=3 + seed, replace=False))
    bounds = np.concatenate([[0], cuts, [97]])
    S = len(bounds) - 1
    # every shard is a separate "request" with the same query token
    parts = dict(a)
    parts["q"] = np.repeat(a["q"], S, axis=0)
    parts["qo_indptr"] = np.arange(S + 1)
    parts["kv_indptr"] = bounds
    o_p, lse_p = mla.mla_decode(**parts)
    om, lsem = mla.merge_partials(o_p[:, None], lse_p[:, None])
    _close(om, o, rel=1e-13)
    _close(lsem, lse, rel=1e-13)
    # empty shards (lse = -inf) are ignored
    o_p2 = np.concatenate([o_p, np.full_like(o_p[:1], np.nan)])
    lse_p2 = np.concatenate([lse_p, np.full_like(lse_p[:1], -np.inf)])
    om2, lsem2 = mla.merge_partials(o_p2[:, None], lse_p2[:, None])
    _close(om2, o, rel=1e-13)


def test_permuting_a_requests_entries_changes_nothing():
    a = _args(workloads.tiny())
    o, lse = mla.mla_decode(**a)
    rng = np.random.default_rng(4)
    idx = a["kv_indices"].copy()
    for b in range(2):
        s, e = a["kv_indptr"][b], a["kv_indptr"][b + 1]
        idx[s:e] = rng.permutation(idx[s:e])
    o2, lse2 = mla.mla_decode(**dict(a, kv_indices=idx))
    _close(o2, o, rel=1e-13)
    _close(lse2, lse, rel=1e-13)


def test_power_of_two_scale_exchange_is_exact():
    """(kv_scale * 2, sm_scale / 2) keeps every score and doubles o exactly."""
    a = _args(workloads.tiny())
    o, lse = mla.mla_decode(**a)
    o2, lse2 = mla.mla_decode(**dict(a, kv_scale=a["kv_scale"] * 2, sm_scale=a["sm_scale"] / 2))
    assert np.array_equal(o2, 2 * o)
    assert np.array_equal(lse2, lse)


def test_multi_token_call_equals_truncated_single_token_calls():
    w = workloads.build("mt", [50], num_heads=16, qlens=[4], pool_entries=128, seed=6)
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    rows = a["kv_indices"]
    for j in range(4):
        vis = 50 - (3 - j)
        aj = dict(a, q=a["q"][j : j + 1], qo_indptr=np.array([0, 1]),
                  kv_indptr=np.array([0, vis]), kv_indices=rows[:vis])
        oj, lsej = mla.mla_decode(**aj)
        _close(o[j], oj[0], rel=1e-15)
        _close(lse[j], lsej[0], rel=1e-15)


def test_empty_history_and_invisible_tokens():
    w = workloads.build("empty", [0, 2, 5], num_heads=16, qlens=[1, 4, 1], pool_entries=32, seed=7)
    a = _args(w)
    o, lse = mla.mla_decode(**a)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    # request 1: 4 draft tokens over 2 entries -> tokens 0 and 1 see nothing
    assert np.all(o[1:3] == 0) and np.all(np.isneginf(lse[1:3]))
    assert np.all(np.isfinite(lse[3:5]))
    assert np.all(np.isfinite(lse[5]))


# ---------------------------------------------------------------- merge


def test_merge_matches_brute_force_with_empty_shards():
    rng = np.random.default_rng(9)
    S, T, H, D = 5, 3, 4, 16
    o = rng.standard_normal((S, T, H, D))
    lse = rng.standard_normal((S, T, H)) * 3 + 5
    lse[1, 0, 0] = -np.inf
    lse[:, 2, 3] = -np.inf  # a row empty in every shard
    lse[:, 1, 1] = -np.inf
    lse[3, 1, 1] = 2.5  # exactly one live shard
    om, lsem = mla.merge_partials(o, lse)
    ob, lseb = brute.brute_merge(o, lse)
    _close(om, ob, rel=1e-14)
    _close(lsem, lseb, rel=1e-14)
    assert np.all(om[2, 3] == 0) and np.isneginf(lsem[2, 3])
    assert np.array_equal(om[1, 1], o[3, 1, 1]) and lsem[1, 1] == 2.5


# ---------------------------------------------------------------- page values


def test_sm_scale_and_geometry_match_the_printed_values(golden):
    g = golden("issue_geometry.json")
    assert repr(workloads.SM_SCALE_F64) == g["sm_scale_printed"]
    assert mla.QK_HEAD_DIM == g["qk_nope_head_dim"] + g["qk_rope_head_dim"] == g["qk_head_dim"]
    assert mla.ROW_DIM == g["kv_lora_rank"] + g["qk_rope_head_dim"] == g["kv_entry_width"]
    assert mla.LATENT_DIM == g["kv_lora_rank"]
    # 1/sqrt(192) and 192**-0.5 name the same binary32 value the device sees
    assert workloads.fp32(1 / math.sqrt(192)) == workloads.SM_SCALE
