"""Properties of the work planner (host mirror of the device planner; no GPU).

Every unit (query token, head group) must be covered exactly once by pieces,
every worker must get an equal share of the stream, partial pieces may only sit
at a worker's two ends, and the split combine's slot rule must name exactly the
slots the decode workers write.
"""

import numpy as np
import pytest

import workloads
from mla_latent_attention_amd import plan_groups_host, plan_host

MIN_WORKER_ROWS = 256
SNAP_ROWS = 64
GROUPS_PER_UNIT = 8  # group mode: row groups per unit
GROUP_SLOTS = 16  # group mode: partial slots per worker (two pieces x 8 row groups)
GROUP_PIECE_ROWS = 320  # group mode: a unit's span is its entries plus these leading rows


def visible(n, qlen, j):
    return max(0, n - (qlen - 1 - j))


def dcp_rule(gkv, cps, cpr):
    """Visible count on a DCP shard, by enumeration: local entry i is full-list
    position cpr + i * cps; token j of qlen sees positions <= N - qlen + j."""
    def vis(b, n, qlen, j):
        N = gkv[b + 1] - gkv[b]
        return sum(1 for i in range(n) if cpr + i * cps <= N - qlen + j)
    return vis


def units(qo, kv, G, rule=None):
    """(token, group, length, stream start) in stream order, skipping nothing."""
    out, pos = [], 0
    for b in range(len(qo) - 1):
        n, ql = kv[b + 1] - kv[b], qo[b + 1] - qo[b]
        for j in range(ql):
            v = visible(n, ql, j) if rule is None else rule(b, n, ql, j)
            for g in range(G):
                out.append((qo[b] + j, g, v, pos))
                pos += v
    return out, pos


def group_units(qo, kv, H, causal=True, rule=None):
    """Group mode: (request, unit, length, stream start, span) in stream order.
    A request's ql * H query rows (token j, head h) are numbered j * H + h and
    cut into row groups of 16; unit u covers row groups 8u..8u+7 and is as
    long as its last row sees; in the stream it takes GROUP_PIECE_ROWS more
    rows (ahead of its entries) when non-empty."""
    out, pos = [], 0
    U = GROUPS_PER_UNIT
    for b in range(len(qo) - 1):
        n, ql = kv[b + 1] - kv[b], qo[b + 1] - qo[b]
        R = -(-(ql * H) // 16)
        for u in range(-(-R // U)):
            last_rg = min(U * u + U - 1, R - 1)
            tok = min(16 * last_rg + 15, ql * H - 1) // H
            if not causal:
                v = n
            elif rule is None:
                v = visible(n, ql, tok)
            else:
                v = rule(b, n, ql, tok)
            span = v + GROUP_PIECE_ROWS if v > 0 else 0
            out.append((b, u, v, pos, span))
            pos += span
    return out, pos


def spans_of(us):
    """(stream start, stream length) of each non-empty unit: the span in group
    mode, the length otherwise."""
    return [(e[3], e[4] if len(e) > 4 else e[2]) for e in us if e[2] > 0]


def snapped_bounds(us, W, nw):
    """Worker boundaries: w*W//nw, moved onto a unit boundary within SNAP_ROWS
    (the nearer one; back on a tie)."""
    starts = [st for st, _ in spans_of(us)]
    lens = [n for _, n in spans_of(us)]
    bounds = [0]
    for w in range(1, nw):
        x = w * W // nw
        i = int(np.searchsorted(starts, x, side="right")) - 1
        k, v = x - starts[i], lens[i]
        if k == 0:
            bounds.append(x)
        elif k <= SNAP_ROWS and k <= v - k:
            bounds.append(x - k)
        elif v - k <= SNAP_ROWS:
            bounds.append(x + v - k)
        else:
            bounds.append(x)
    bounds.append(W)
    return bounds


def check_plan(qo, kv, H, nw_req, dcp=None):
    """dcp = (g_kv_indptr, cp_world_size, cp_rank) for a DCP shard's call."""
    G = H // 16
    rule = None if dcp is None else dcp_rule(*dcp)
    us, W = units(qo, kv, G, rule)
    kw = {} if dcp is None else dict(g_kv_indptr=dcp[0], cp_world_size=dcp[1], cp_rank=dcp[2])
    pieces = plan_host(qo, kv, H, nw_req, **kw)
    if W == 0:
        assert len(pieces) == 0
        return pieces
    nw = min(nw_req, max(1, W // MIN_WORKER_ROWS))
    S = snapped_bounds(us, W, nw)
    assert all(a < b for a, b in zip(S, S[1:]))
    cover = {}
    for w, t, g, kb, ke, ul, slot, comp in pieces:
        assert 0 <= kb < ke <= ul
        cover.setdefault((t, g), []).append((kb, ke, w, slot, comp))
    # coverage: each non-empty unit exactly tiled, in worker order
    for t, g, v, start in us:
        if v == 0:
            assert (t, g) not in cover
            continue
        segs = sorted(cover[(t, g)])
        assert segs[0][0] == 0 and segs[-1][1] == v
        for (a0, a1, *_), (b0, b1, *_) in zip(segs, segs[1:]):
            assert a1 == b0
        if len(segs) == 1:
            assert segs[0][4] == 1 and segs[0][3] == -1
        else:
            assert all(s[4] == 0 for s in segs)
            # the combine's rule: worker range [wlo, whi]; slot 2w+1 only for a
            # first worker that started before the unit
            begin = lambda w: S[w]  # noqa: E731
            owner = lambda p: int(np.searchsorted(S, p, side="right")) - 1  # noqa: E731
            wlo, whi = owner(start), owner(start + v - 1)
            want = {(2 * w + 1) if (w == wlo and begin(w) < start) else 2 * w for w in range(wlo, whi + 1)}
            assert {s[3] for s in segs} == want
            assert [s[2] for s in segs] == list(range(wlo, whi + 1))
    # balance: worker w processes exactly its stream share
    per_worker = np.zeros(nw, dtype=np.int64)
    for w, t, g, kb, ke, *_ in pieces:
        per_worker[w] += ke - kb
    shares = np.array([S[w + 1] - S[w] for w in range(nw)])
    assert np.array_equal(per_worker, shares)
    assert np.all(np.abs(shares - W / nw) <= 2 * SNAP_ROWS + 1)
    # no piece starts or ends within SNAP_ROWS of an interior unit boundary
    for w, t, g, kb, ke, ul, *_ in pieces:
        if kb > 0:
            assert kb > SNAP_ROWS and ul - kb > SNAP_ROWS
        if ke < ul:
            assert ke > SNAP_ROWS and ul - ke > SNAP_ROWS
    # partial pieces only at a worker's ends; slots unique
    slots = [p[6] for p in pieces if p[6] >= 0]
    assert len(slots) == len(set(slots))
    for w in range(nw):
        mine = pieces[pieces[:, 0] == w]
        for i, p in enumerate(mine):
            if p[7] == 0:
                assert i in (0, len(mine) - 1)
                assert p[6] == (2 * w if i == 0 else 2 * w + 1)
    return pieces


def indptr(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


@pytest.mark.parametrize("nw", [1, 7, 256])
def test_headline_batch(nw):
    L = workloads.c16_lengths()
    p = check_plan(indptr([1] * 16), indptr(L), 16, nw)
    if nw == 256:
        w_rows = sum(L) // 256
        assert abs(w_rows - 4276) <= 1
        # 16 workers per request, one piece each: no worker pays for a sliver
        assert len(p) == 256 and sorted(p[:, 0].tolist()) == list(range(256))


def test_c24_and_mixed_lengths():
    check_plan(indptr([1] * 24), indptr(workloads.c24_lengths()), 16, 256)
    check_plan(indptr([1] * 64), indptr(workloads.mixed_lengths()), 16, 256)


def test_dcp_share_multi_token_many_heads():
    pieces = check_plan(indptr([4] * 8), indptr([17_750] * 8), 96, 256)
    assert pieces[:, 2].max() == 5


@pytest.mark.parametrize("seed", range(12))
def test_random_ragged_plans(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lengths = rng.integers(0, 3000, size=B)
    lengths[rng.random(B) < 0.2] = 0
    qlens = rng.integers(1, 5, size=B)
    H = 16 * int(rng.integers(1, 4))
    check_plan(indptr(qlens), indptr(lengths), H, int(rng.integers(1, 300)))


def test_empty_and_tiny_inputs():
    check_plan(indptr([1, 1]), indptr([0, 0]), 16, 256)
    p = check_plan(indptr([1, 1]), indptr([64, 100]), 16, 256)
    assert len(p) == 2 and all(p[:, 7] == 1)  # one worker does everything
    check_plan(indptr([4, 3]), indptr([2, 1]), 16, 8)  # early draft tokens see nothing


def test_rejects_bad_planner_input():
    with pytest.raises(ValueError):
        plan_host(indptr([1]), indptr([10]), 12, 4)


# ---------------------------------------------------------------- group mode


def check_group_plan(qo, kv, H, nw_req, causal=True, dcp=None):
    """The host planner's group-mode pieces equal the model's: worker w's
    snapped share of the span stream, intersected with each unit's entries
    (its span less the GROUP_PIECE_ROWS leading rows, which only charge the
    unit's start), with the slot rule the combine relies on."""
    rule = None if dcp is None else dcp_rule(*dcp)
    us, W = group_units(qo, kv, H, causal, rule)
    kw = {} if dcp is None else dict(g_kv_indptr=dcp[0], cp_world_size=dcp[1], cp_rank=dcp[2])
    pieces = plan_groups_host(qo, kv, H, nw_req, causal, **kw)
    if W == 0:
        assert len(pieces) == 0
        return pieces
    nw = min(nw_req, max(1, W // MIN_WORKER_ROWS))
    S = snapped_bounds(us, W, nw)
    assert all(a < b for a, b in zip(S, S[1:]))
    want = []
    for w in range(nw):
        k = 0  # this worker's pieces so far
        for b, u, v, st, span in us:
            if v == 0:
                continue
            lo, hi = max(S[w], st + GROUP_PIECE_ROWS), min(S[w + 1], st + span)
            if lo >= hi:
                continue
            k0, k1 = lo - st - GROUP_PIECE_ROWS, hi - st - GROUP_PIECE_ROWS
            complete = k0 == 0 and k1 == v
            slot = -1 if complete else GROUP_SLOTS * w + (0 if k == 0 else GROUP_SLOTS // 2)
            want.append((w, b, u, k0, k1, v, slot, int(complete)))
            k += 1
    got = [tuple(int(x) for x in p) for p in pieces]
    assert got == want
    # every non-empty unit is tiled once, and a split unit's later workers
    # hold it as their first piece, in consecutive order (the group combine
    # reads slot 16 * w + row group of each of them)
    cover = {}
    for w, b, u, kb, ke, ul, slot, comp in got:
        cover.setdefault((b, u), []).append((kb, ke, w, slot))
    for b, u, v, st, span in us:
        if v == 0:
            assert (b, u) not in cover
            continue
        segs = sorted(cover[(b, u)])
        assert segs[0][0] == 0 and segs[-1][1] == v
        assert all(x[1] == y[0] for x, y in zip(segs, segs[1:]))
        assert [x[2] for x in segs] == list(range(segs[0][2], segs[0][2] + len(segs)))
        assert [x[3] for x in segs[1:]] == [GROUP_SLOTS * x[2] for x in segs[1:]]
    # equal shares, and no boundary within SNAP_ROWS of a span's ends
    shares = np.diff(np.array(S))
    assert np.all(np.abs(shares - W / nw) <= 2 * SNAP_ROWS + 1)
    starts = [st for st, _ in spans_of(us)]
    lens = [n for _, n in spans_of(us)]
    for x in S[1:-1]:
        i = int(np.searchsorted(starts, x, side="right")) - 1
        kx = x - starts[i]
        assert kx == 0 or (kx > SNAP_ROWS and lens[i] - kx > SNAP_ROWS)
    slots = [p[6] for p in got if p[6] >= 0]
    assert len(slots) == len(set(slots))
    return pieces


def test_group_plan_dcp_share_workload():
    """96 heads, 4 query tokens per request, 8 requests of 17,750 entries: 24
    row groups per request, 3 units each, 256 workers."""
    pieces = check_group_plan(indptr([4] * 8), indptr([17_750] * 8), 96, 256)
    assert pieces[:, 2].max() == 2
    # causal: a unit is as long as the token of its last row group sees
    # (row groups 0-7 end in token 1, 8-15 in token 2, 16-23 in token 3)
    lens = sorted(set(pieces[:, 5].tolist()))
    assert lens == [17_748, 17_749, 17_750]


def test_group_plan_charges_each_unit_start():
    """DCP share: the 16 workers whose share crosses a unit boundary run two
    pieces; each unit's leading GROUP_PIECE_ROWS rows give them that many
    fewer entries than a worker inside one unit."""
    p = plan_groups_host(indptr([4] * 8), indptr([17_750] * 8), 96, 256, True)
    entries, pieces = np.zeros(256, np.int64), np.zeros(256, np.int64)
    for r in p:
        entries[r[0]] += r[4] - r[3]
        pieces[r[0]] += 1
    assert np.bincount(pieces).tolist() == [0, 240, 16]
    assert entries[pieces == 1].max() - entries[pieces == 2].max() >= GROUP_PIECE_ROWS - 2 * SNAP_ROWS


def test_group_boundaries_fall_inside_charge_rows():
    """The ragged call of the GPU test for charge rows: with 23, 37 and 58
    workers some snapped share boundaries lie strictly inside a unit's
    leading GROUP_PIECE_ROWS rows (and the plan is still exact)."""
    qo, kv = indptr([4, 2, 3, 1, 4, 2]), indptr([700, 1900, 260, 3000, 45, 1200])
    us, W = group_units(qo, kv, 96)
    for nw_req in (23, 37, 58):
        nw = min(nw_req, max(1, W // MIN_WORKER_ROWS))
        S = snapped_bounds(us, W, nw)
        inside = sum(1 for x in S[1:-1] for b, u, v, st, span in us
                     if v > 0 and st < x < st + GROUP_PIECE_ROWS)
        assert inside > 0, nw_req
        check_group_plan(qo, kv, 96, nw_req)


def test_model_constants_match_the_planner_header():
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "mla_latent_attention_amd", "csrc",
                            "mla_plan.h")).read()
    for name, val in (("kMinWorkerRows", MIN_WORKER_ROWS), ("kSnapRows", SNAP_ROWS),
                      ("kGroupsPerUnit", GROUPS_PER_UNIT), ("kGroupPieceRows", GROUP_PIECE_ROWS)):
        m = re.search(r"constexpr int %s = (\d+);" % name, src)
        assert m and int(m.group(1)) == val, name


def test_group_units_mask_within_unit():
    """With 16 heads and 4 tokens, one unit holds all four tokens; its length
    is the last token's visible count, the others see fewer."""
    us, W = group_units(indptr([4]), indptr([100]), 16)
    assert [(u, v) for _, u, v, *_ in us] == [(0, 100)]
    us, W = group_units(indptr([5]), indptr([100]), 32)  # 10 row groups: units of 8 and 2
    assert [(u, v) for _, u, v, *_ in us] == [(0, 99), (1, 100)]


def test_group_units_pack_unpadded_heads():
    """12 heads: token j's rows are 12j .. 12j + 11, so row group 0 holds token 0
    and the first four heads of token 1; 16 tokens make 12 row groups (1.5
    units) instead of 16; a unit's length is its last row's token's."""
    us, W = group_units(indptr([16]), indptr([1000]), 12, causal=False)
    assert [(u, v) for _, u, v, *_ in us] == [(0, 1000), (1, 1000)]
    us, W = group_units(indptr([11]), indptr([1000]), 12)  # 132 rows: 9 row groups
    # unit 0: row groups 0-7 end at row 127, token 10; unit 1: row group 8, token 10
    assert [(u, v) for _, u, v, *_ in us] == [(0, 1000), (1, 1000)]
    us, W = group_units(indptr([3]), indptr([50]), 12)  # 36 rows: 3 row groups, one unit
    assert [(u, v) for _, u, v, *_ in us] == [(0, 50)]
    us, W = group_units(indptr([1, 1]), indptr([30, 40]), 20)  # 20 rows: two row groups each
    assert [(b, u, v) for b, u, v, *_ in us] == [(0, 0, 30), (1, 0, 40)]


@pytest.mark.parametrize("seed", range(12))
def test_group_random_ragged_plans(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 40))
    lengths = rng.integers(0, 5000, size=B)
    lengths[rng.random(B) < 0.2] = 0
    qlens = rng.integers(1, 6, size=B)
    H = 16 * int(rng.integers(1, 7)) if seed % 2 == 0 else int(rng.integers(1, 100))
    check_group_plan(indptr(qlens), indptr(lengths), H, int(rng.integers(1, 600)))


def test_group_empty_and_tiny_inputs():
    check_group_plan(indptr([4, 4]), indptr([0, 0]), 16, 512)
    p = check_group_plan(indptr([4]), indptr([200]), 16, 512)
    assert len(p) == 1 and p[0, 7] == 1
    check_group_plan(indptr([4, 3]), indptr([2, 1]), 32, 8)  # early draft tokens see nothing


def test_group_plan_without_causal_mask():
    """The cascade's prefix pass: one request holding every token, all of which
    see every entry; units are as long as the request."""
    pieces = check_group_plan(indptr([16]), indptr([63_911]), 16, 256, causal=False)
    assert set(pieces[:, 5].tolist()) == {63_911}
    check_group_plan(indptr([7]), indptr([5000]), 64, 37, causal=False)
    check_group_plan(indptr([3]), indptr([0]), 32, 8, causal=False)
    us, _ = group_units(indptr([4]), indptr([100]), 16, causal=False)
    assert [(u, v) for _, u, v, *_ in us] == [(0, 100)]
    # the cascade's prefix pass with 12 unpadded heads: 16 tokens, 192 rows
    pieces = check_group_plan(indptr([16]), indptr([63_911]), 12, 256, causal=False)
    assert set(pieces[:, 2].tolist()) == {0, 1}


# ---------------------------------------------------------------- DCP shards


def shard_lengths(full, cps, cpr):
    return [max(0, -(-(N - cpr) // cps)) for N in full]


@pytest.mark.parametrize("seed", range(10))
def test_random_dcp_shard_plans(seed):
    """Positions dealt round-robin over cps shards; the planner's unit lengths
    follow the shard's visibility rule (standard and group mode)."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 20))
    full = rng.integers(0, 4000, size=B)
    full[rng.random(B) < 0.2] = int(rng.integers(0, 9))
    qlens = rng.integers(1, 5, size=B)
    cps = int(rng.integers(1, 9))
    cpr = int(rng.integers(0, cps))
    kv = indptr(shard_lengths(full, cps, cpr))
    dcp = (indptr(full), cps, cpr)
    check_plan(indptr(qlens), kv, 16, int(rng.integers(1, 300)), dcp=dcp)
    check_group_plan(indptr(qlens), kv, 16 * int(rng.integers(1, 7)), int(rng.integers(1, 300)),
                     dcp=dcp)


def test_group_plan_dcp_share_interleaved():
    """The benchmark's DCP share: 142,000 positions per request dealt over 8
    shards, rank 7 (17,750 each).  Row groups 0-7 end in token 1, 8-15 in token
    2, 16-23 in token 3, which see positions up to 141,997, 141,998, 141,999."""
    full = [142_000] * 8
    kv = indptr(shard_lengths(full, 8, 7))
    pieces = check_group_plan(indptr([4] * 8), kv, 96, 256, dcp=(indptr(full), 8, 7))
    assert sorted(set(pieces[:, 5].tolist())) == [17_749, 17_750]
    pieces = check_group_plan(indptr([4] * 8), indptr(shard_lengths(full, 8, 0)), 96, 256,
                              dcp=(indptr(full), 8, 0))
    assert sorted(set(pieces[:, 5].tolist())) == [17_750]


def test_dcp_rejects_bad_rank():
    with pytest.raises(ValueError):
        plan_host(indptr([1]), indptr([10]), 16, 4, g_kv_indptr=indptr([80]), cp_world_size=8,
                  cp_rank=8)
