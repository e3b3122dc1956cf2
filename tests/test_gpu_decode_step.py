"""GPU parity of the fused layer step mla_decode_step (through the C ABI).

The call folds mla_rope_quant_cache into the decode (each worker builds its
units' fp8 q rows and writes the new cache entries its pieces read) and
mla_latent_to_v into the split combine.  Where the three-call chain runs the
standard decode kernel, every output of the fused call must equal the chain's
bit for bit: the new cache rows, o_latent, lse and out.  Where the chain picks
the group-mode kernel (more head groups x query tokens), the fused call is
checked against the oracle's chain instead: its cache rows bit for bit, o and
lse within the parity gate, out within 2^-7 of each row's largest |out|.
"""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import io as oio
from oracle import surround as osur
from tests.parity import assert_gate, metrics

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_latent_attention_amd as mla  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _u16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _new_entry_slots(w):
    """Token j of request b writes its entry at position n_b - qlen_b + j of the
    request's list: that list entry is its slot."""
    kvp = w.kv_indptr.cpu().tolist()
    slots = []
    for b, ql in enumerate(w.qlens):
        for j in range(ql):
            slots.append(int(w.kv_indices[kvp[b + 1] - ql + j]))
    return torch.tensor(slots, dtype=torch.int32, device=DEV)


def _chain(w, s, slots, pool, H, Hp, style):
    q = mla.rope_quant_cache(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin,
                             pool, slots, rope_style=style, num_heads_pad=Hp,
                             q_scale=w.q_scale, kv_scale=w.kv_scale)
    o, lse = mla.decode(q, pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_lens,
                        w.sm_scale, w.q_scale, w.kv_scale, return_lse=True,
                        max_seqlen_q=w.max_seqlen_q)
    v = mla.latent_to_v(o, s.w_uv)
    return q, o, lse, v


def _step(w, s, slots, pool, Hp, style):
    return mla.decode_step(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin, slots,
                           pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.sm_scale, s.w_uv,
                           num_heads_pad=Hp, rope_style=style, q_scale=w.q_scale,
                           kv_scale=w.kv_scale, return_lse=True, max_seqlen_q=w.max_seqlen_q)


CASES = [
    # name, lengths, qlens, real heads, padded heads, rope style
    ("c8-qlen1", [900, 1300, 700, 2000, 333, 1500, 64, 1024], None, 12, 16, 0),
    ("drafts-style1", [1800, 41, 977, 3000], [2, 1, 3, 1], 12, 16, 1),
    ("long-split", [40000, 300, 5000, 1], None, 12, 16, 0),
    ("two-groups", [2500, 700, 1200], None, 20, 32, 1),
]


@pytest.mark.parametrize("name,lengths,qlens,H,Hp,style", CASES, ids=[c[0] for c in CASES])
def test_decode_step_equals_the_three_call_chain(name, lengths, qlens, H, Hp, style):
    say(f"[step] {name}: lengths={lengths} qlens={qlens} H={H}/{Hp} style={style}")
    w = workloads.build(name, lengths, num_heads=Hp, real_heads=H, qlens=qlens,
                        pool_entries=1 << 16, kv_std=0.5, scale_range=(0.5, 2.0), seed=130,
                        device=DEV)
    T = w.num_tokens
    assert (Hp // 16) * w.max_seqlen_q < 4, "the chain must run the standard kernel"
    s = workloads.surround(T, H, 4096, 1 << 16, seed=131, device=DEV)
    slots = _new_entry_slots(w)
    if T > 2:
        slots[1] = -1  # token 1 writes nothing: both sides read the pool's old row
    pool_a, pool_b = w.kv_pool.clone(), w.kv_pool.clone()
    _, o_a, lse_a, v_a = _chain(w, s, slots, pool_a, H, Hp, style)
    v_b, o_b, lse_b = _step(w, s, slots, pool_b, Hp, style)
    torch.cuda.synchronize()
    assert torch.equal(pool_a.view(torch.uint8), pool_b.view(torch.uint8)), "cache"
    assert torch.equal(o_a, o_b), "o_latent"
    assert torch.equal(lse_a, lse_b), "lse"
    assert torch.equal(v_a, v_b), "out"


def test_decode_step_matches_the_oracle_where_the_chain_uses_group_mode():
    """96 heads: the chain's decode runs the group-mode kernel, the fused call
    the standard one; both are held to the oracle."""
    H = Hp = 96
    w = workloads.build("step-96", [1500, 260, 3100], num_heads=Hp, real_heads=H, qlens=[2, 1, 1],
                        pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0), seed=140,
                        device=DEV)
    T = w.num_tokens
    s = workloads.surround(T, H, 4096, 1 << 14, seed=141, device=DEV)
    slots = _new_entry_slots(w)
    pool = w.kv_pool.clone()
    v, o, lse = _step(w, s, slots, pool, Hp, 0)
    torch.cuda.synchronize()
    q_ref, k_ref = osur.rope_quant_cache(
        _u16(s.q_latent), _u16(s.q_pe), _u16(s.k_latent), _u16(s.k_pe),
        s.positions.cpu().numpy(), s.cos_sin.cpu().numpy(), 0, Hp, float(w.q_scale.item()),
        float(w.kv_scale.item()))
    got_pool = pool.view(torch.uint8).cpu().numpy()
    for t, sl in enumerate(slots.cpu().tolist()):
        assert np.array_equal(got_pool[sl], k_ref[t]), f"cache row of token {t}"
    q = torch.from_numpy(q_ref).to(DEV).view(torch.float8_e4m3fn)
    chained = workloads.Workload(**{**w.__dict__, "q": q, "kv_pool": pool})
    toks, o_ref, lse_ref = (lambda a: (a["tokens"], *oio.call_decode(a)))(
        oio.workload_args(chained))
    assert_gate(metrics(o, o_ref, lse, lse_ref), "decode_step (96 heads)")
    v_ref = osur.latent_to_v(o_ref[:, :H], s.w_uv.float().cpu().numpy().astype(np.float64))
    got = v.float().cpu().numpy().astype(np.float64)
    rel = float((np.abs(got - v_ref).max(axis=-1) / np.abs(v_ref).max(axis=-1)).max())
    say(f"[step-96] out row rel {rel:.3e}")
    assert rel <= 2.0 ** -7


def test_decode_step_full_size_c16_equals_the_chain():
    """The batch-16, ~68K-entry call with 12 heads padded to 16 (the layer
    step the bench times): fused and chained results bit for bit."""
    w = workloads.c16(DEV, "shared", return_lse=True)
    T, Hp, H = w.num_tokens, w.num_heads, w.real_heads
    s = workloads.surround(T, H, 73_728, w.kv_pool.shape[0], seed=8000, device=DEV)
    slots = _new_entry_slots(w)
    say(f"[step-c16] T={T} pool={w.kv_pool.shape[0]}")
    pool_a = w.kv_pool
    bytes_a = pool_a.view(torch.uint8)
    rows = slots.long()
    before = bytes_a[rows].clone()
    _, o_a, lse_a, v_a = _chain(w, s, slots, pool_a, H, Hp, 0)
    torch.cuda.synchronize()
    written = bytes_a[rows].clone()
    assert not torch.equal(written, before)
    bytes_a[rows] = before  # the same starting pool for the fused call
    v_b, o_b, lse_b = _step(w, s, slots, pool_a, Hp, 0)
    torch.cuda.synchronize()
    assert torch.equal(bytes_a[rows], written), "cache rows"
    assert torch.equal(o_a, o_b), "o_latent"
    assert torch.equal(lse_a, lse_b), "lse"
    assert torch.equal(v_a, v_b), "out"


def test_decode_step_graph_replay_matches_eager_bitwise():
    T, H, Hp = 4, 12, 16
    w = workloads.build("step-graph", [700, 900, 300, 1200], num_heads=Hp, real_heads=H,
                        pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0), seed=150,
                        device=DEV)
    s = workloads.surround(T, H, 4096, 1 << 14, seed=151, device=DEV)
    slots = _new_entry_slots(w)
    o = torch.empty((T, Hp, 512), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, Hp), dtype=torch.float32, device=DEV)
    ws = mla.new_workspace(mla._lib.lib().mla_decode_step_workspace_bytes(T, T, Hp, 1), DEV)

    def step():
        mla.decode_step(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin, slots,
                        w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices, w.sm_scale, s.w_uv,
                        num_heads_pad=Hp, q_scale=w.q_scale, kv_scale=w.kv_scale,
                        return_lse=True, o_latent=o, out=v, lse=lse, max_seqlen_q=1,
                        workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, v, lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o, v, lse):
            t.zero_()
        mla.latent_to_v(torch.randn((8, 16, 512), device=DEV).to(torch.bfloat16), s.w_uv)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, v, lse), eager):
            assert torch.equal(a, b), rep
