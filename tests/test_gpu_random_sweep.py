"""GPU parity over seeded random call shapes, every entry point against the
oracle (through the C ABI).

Each case draws a call: the entry point (plain with a forced worker count,
paged, one DCP shard, shared-prefix cascade), the storage type, batch, KV
lengths (some empty), draft-token counts, head count (padded or not) and page
size, builds the inputs with the seeded generators, and holds the result to
the parity gate on every request.  The cases are small enough for the oracle
to finish each in a second or two, and together they reach shapes the
hand-written tests do not enumerate (odd head counts with draft tokens in group
mode, DCP shards of ragged lists, worker counts that cut units into slivers)."""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import io as oio
from tests.parity import assert_gate, bf16_abs_tol, metrics

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_attention_amd as mla  # noqa: E402

DEV = torch.device("cuda:0")
MODES = ["plain", "plain", "paged", "dcp", "cascade"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw(seed):
    """The call of case `seed`: (mode, builder kwargs, extra)."""
    rng = np.random.default_rng(7100 + seed)
    mode = MODES[int(rng.integers(0, len(MODES)))]
    B = int(rng.integers(1, 9))
    qlens = [int(x) for x in rng.integers(1, 5, size=B)]
    if rng.random() < 0.4:
        qlens = [1] * B
    lengths = [int(x) for x in rng.integers(0, 4000, size=B)]
    for b in range(B):
        if rng.random() < 0.15:
            lengths[b] = int(rng.integers(0, 4))
    dtype = "bf16" if mode in ("plain", "paged", "dcp") and rng.random() < 0.3 else "fp8"
    if mode == "cascade":
        H = int(rng.choice([1, 12, 16, 20, 32, 48, 64]))
        real = H
    else:
        H = int(rng.choice([16, 32, 64, 96, 128]))
        real = int(rng.choice([H, max(1, H - 4)]))
    kw = dict(num_heads=H, real_heads=real, qlens=qlens, dtype=dtype, kv_std=0.5,
              scale_range=(0.5, 2.0), seed=7200 + seed)
    extra = {}
    if mode == "plain":
        extra["num_workers"] = int(rng.choice([0, 1, 3, 17, 256]))
    elif mode == "paged":
        kw["page_size"] = int(rng.choice([2, 16, 128]))
    elif mode == "dcp":
        extra["cp"] = int(rng.choice([2, 4, 8]))
        extra["rank"] = int(rng.integers(0, extra["cp"]))
    else:
        # Every suffix must hold at least qlen - 1 entries (the call's contract).
        room = min(n - (q - 1) for n, q in zip(lengths, qlens))
        if room < 0:
            lengths = [max(n, q - 1) for n, q in zip(lengths, qlens)]
            room = min(n - (q - 1) for n, q in zip(lengths, qlens))
        extra["prefix"] = int(rng.integers(0, room + 1))
        kw["shared_prefix"] = extra["prefix"]
    return mode, lengths, kw, extra


def run_case(seed):
    """Run case `seed` through the C ABI and the oracle: (metrics, mode, kwargs)."""
    mode, lengths, kw, extra = draw(seed)
    say(f"[sweep {seed}] {mode} lengths={lengths} {kw} {extra}")
    P = kw.get("page_size", 1)
    pool = P * max(64, (1 << 16) // P)
    w = workloads.build(f"sweep-{seed}", lengths, pool_entries=pool, device=DEV, **kw)
    args = (w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
            w.sm_scale, w.q_scale, w.kv_scale)
    torch.cuda.synchronize()
    if mode == "plain":
        o, lse = mla.decode(*args, return_lse=True, max_seqlen_q=w.max_seqlen_q,
                            num_workers=extra["num_workers"])
    elif mode == "paged":
        o, lse = mla.decode_paged(*args, return_lse=True, page_size=P,
                                  max_seqlen_q=w.max_seqlen_q)
    elif mode == "dcp":
        w = workloads.dcp_shard(w, extra["cp"], extra["rank"])
        o, lse = mla.decode_dcp(w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                                return_lse=True, g_kv_indptr=w.g_kv_indptr,
                                cp_world_size=w.cp_size, cp_rank=w.cp_rank,
                                max_seqlen_q=w.max_seqlen_q)
    else:
        pre, sptr, suf = workloads.split_prefix(w, extra["prefix"])
        o, lse = mla.decode_cascade(w.q, w.kv_pool, w.qo_indptr, pre, sptr, suf, w.sm_scale,
                                    w.q_scale, w.kv_scale, return_lse=True,
                                    max_seqlen_q=w.max_seqlen_q)
    torch.cuda.synchronize()
    a = oio.workload_args(w)
    o_ref, lse_ref = oio.call_decode(a)
    toks = a["tokens"]
    m = metrics(o[toks], o_ref, lse[toks], lse_ref)
    say(f"[sweep {seed}] {m}")
    return m, mode, kw


@pytest.mark.parametrize("seed", range(256))
def test_random_call_matches_oracle(seed):
    m, mode, _ = run_case(seed)
    assert_gate(m, f"sweep {seed} ({mode})", abs_tol=bf16_abs_tol(m["ref_absmax"]))
