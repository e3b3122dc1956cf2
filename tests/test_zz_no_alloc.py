"""mla_decode_noalloc: mla_decode without a workspace, on the library's fixed
per-device scratch.  Two calls in a row (the second smaller) must give exactly
mla_decode's results, and a call too large for the scratch is refused."""

import pytest
import torch

import workloads
from oracle import io as oio
from tests.parity import assert_gate, metrics

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU machines too
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_attention_amd as mla  # noqa: E402
from mla_latent_attention_amd import _lib  # noqa: E402

DEV = torch.device("cuda:0")


def _args(w):
    return (w.q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
            w.sm_scale, w.q_scale, w.kv_scale)


def _both(w):
    """(o, lse) from mla_decode_noalloc and from mla_decode on w's inputs."""
    T, H = w.num_tokens, w.num_heads
    o_n = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse_n = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    mla.decode_noalloc(*_args(w), return_lse=True, o=o_n, lse=lse_n, max_seqlen_q=w.max_seqlen_q)
    o_r, lse_r = mla.decode(*_args(w), return_lse=True, max_seqlen_q=w.max_seqlen_q)
    torch.cuda.synchronize()
    return o_n, lse_n, o_r, lse_r


def test_scratch_size_is_stated():
    assert _lib.lib().mla_decode_noalloc_scratch_bytes() == 20 << 20


def test_two_calls_in_a_row_match_mla_decode():
    """The headline batch-16 call, then a much smaller one on the same scratch:
    both bitwise equal to mla_decode (same kernels, same split), and the first
    within the gate of the oracle on sampled requests."""
    big = workloads.c16(DEV, "shared", return_lse=True)
    o_n, lse_n, o_r, lse_r = _both(big)
    assert torch.equal(o_n, o_r) and torch.equal(lse_n, lse_r)
    a = oio.workload_args(big, [0, 15])
    o_ref, lse_ref = oio.call_decode(a)
    toks = a["tokens"]
    assert_gate(metrics(o_n[toks], o_ref, lse_n[toks], lse_ref), "noalloc c16")
    del big

    small = workloads.build("noalloc-small", [64, 1, 100, 3000], num_heads=16, real_heads=12,
                            qlens=[1, 1, 3, 2], pool_entries=1 << 13, kv_std=0.5,
                            scale_range=(0.5, 2.0), seed=4242, device=DEV)
    o_n, lse_n, o_r, lse_r = _both(small)
    assert torch.equal(o_n, o_r) and torch.equal(lse_n, lse_r)
    o_ref, lse_ref = oio.call_decode(oio.workload_args(small))
    assert_gate(metrics(o_n, o_ref, lse_n, lse_ref), "noalloc small")


def test_bf16_cache():
    w = workloads.build("noalloc-bf16", [700, 2500], num_heads=16, real_heads=12,
                        pool_entries=1 << 13, dtype="bf16", seed=4243, device=DEV)
    o_n, lse_n, o_r, lse_r = _both(w)
    assert torch.equal(o_n, o_r) and torch.equal(lse_n, lse_r)


def test_call_larger_than_the_scratch_is_refused():
    """A group-mode call (64 heads) needs far more than the scratch holds."""
    w = workloads.build("noalloc-big", [300], num_heads=64, real_heads=64, pool_entries=1024,
                        seed=4244, device=DEV)
    o = torch.empty((1, 64, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.decode_noalloc(*_args(w), o=o, max_seqlen_q=1)
    assert e.value.status == 7
