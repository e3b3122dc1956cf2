"""GPU parity of the steps either side of the decode (through the C ABI).

mla_rope_quant_cache writes fp8 codes: they must equal the oracle's bit for
bit (both sides round in binary32 with the same operation order, reading 1 of
oracle.surround).  mla_latent_to_v is compared with the float64 product:
fp32 accumulation plus one bf16 rounding stays within 2^-8 of each row's
largest |out|.  The chain rope -> decode -> latent_to_v is checked against
the oracle's chain on the codes it produced.
"""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import io as oio
from oracle import mla as omla
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


def _oracle_rope(s, style, H_pad):
    return osur.rope_quant_cache(_u16(s.q_latent), _u16(s.q_pe), _u16(s.k_latent), _u16(s.k_pe),
                                 s.positions.cpu().numpy(), s.cos_sin.cpu().numpy(), style, H_pad,
                                 float(s.q_scale.item()), float(s.kv_scale.item()))


@pytest.mark.parametrize("style,T,H,H_pad", [(0, 16, 12, 16), (1, 16, 12, 16), (0, 37, 96, 96),
                                             (1, 1, 1, 16)])
def test_rope_quant_cache_is_bit_exact(style, T, H, H_pad):
    say(f"[rope] style={style} T={T} H={H}/{H_pad}")
    s = workloads.surround(T, H, 4096, 1 << 14, seed=90 + T, device=DEV)
    pool = workloads._fill_values((1 << 14, 576), 0.5, "fp8", 91, DEV)
    before = pool.clone()
    slots = s.slot_mapping.clone()
    if T > 2:
        slots[1] = -1  # no cache write for token 1
    q_out = mla.rope_quant_cache(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin,
                                 pool, slots, rope_style=style, num_heads_pad=H_pad,
                                 q_scale=s.q_scale, kv_scale=s.kv_scale)
    torch.cuda.synchronize()
    q_ref, k_ref = _oracle_rope(s, style, H_pad)
    q_gpu = q_out.view(torch.uint8).cpu().numpy()
    bad = int((q_gpu != q_ref).sum())
    assert bad == 0, f"{bad} q codes differ"
    p = pool.view(torch.uint8).cpu().numpy()
    b = before.view(torch.uint8).cpu().numpy()
    sl = slots.cpu().numpy()
    for t in range(T):
        if sl[t] >= 0:
            assert np.array_equal(p[sl[t]], k_ref[t]), f"cache row of token {t}"
    written = set(int(x) for x in sl if x >= 0)
    untouched = np.array([r for r in range(0, p.shape[0], 97) if r not in written])
    assert np.array_equal(p[untouched], b[untouched])


@pytest.mark.parametrize("T,H,H_pad", [(16, 12, 16), (33, 96, 96), (1, 1, 16)])
def test_latent_to_v_matches_the_float64_product(T, H, H_pad):
    s = workloads.surround(T, H, 16, 64, seed=95 + T, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(96)
    o = torch.randn((T, H_pad, 512), generator=g, device=DEV).to(torch.bfloat16)
    out = mla.latent_to_v(o, s.w_uv)
    torch.cuda.synchronize()
    ref = osur.latent_to_v(o.float().cpu().numpy().astype(np.float64),
                           s.w_uv.float().cpu().numpy().astype(np.float64))
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max(axis=-1)
    rowmax = np.abs(ref).max(axis=-1)
    worst = float((err / rowmax).max())
    say(f"[latent_to_v] T={T} H={H}: worst row rel {worst:.3e}")
    assert worst <= 2.0 ** -8


def test_layer_chain_matches_the_oracle_chain():
    """rope -> decode over a cache holding the new entries -> latent_to_v."""
    T, H, H_pad = 8, 12, 16
    w = workloads.build("chain", [900, 1300, 700, 2000, 333, 1500, 64, 1024], num_heads=H_pad,
                        real_heads=H, pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0),
                        seed=97, device=DEV)
    s = workloads.surround(T, H, 4096, 1 << 14, seed=98, device=DEV)
    # each token's new entry goes to the last slot of its request's list
    kvp = w.kv_indptr.cpu().tolist()
    slots = torch.stack([w.kv_indices[kvp[b + 1] - 1] for b in range(T)]).to(torch.int32)
    q = mla.rope_quant_cache(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin,
                             w.kv_pool, slots, num_heads_pad=H_pad, q_scale=w.q_scale,
                             kv_scale=w.kv_scale)
    o, lse = mla.decode(q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                        w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale, return_lse=True,
                        max_seqlen_q=1)
    v = mla.latent_to_v(o, s.w_uv)
    torch.cuda.synchronize()
    chained = workloads.Workload(**{**w.__dict__, "q": q})
    toks, o_ref, lse_ref = (lambda a: (a["tokens"], *oio.call_decode(a)))(oio.workload_args(chained))
    assert_gate(metrics(o, o_ref, lse, lse_ref), "chain: decode on the fused step's q and cache")
    v_ref = osur.latent_to_v(o_ref, s.w_uv.float().cpu().numpy().astype(np.float64))
    got = v.float().cpu().numpy().astype(np.float64)
    rel = float((np.abs(got - v_ref).max(axis=-1) / np.abs(v_ref).max(axis=-1)).max())
    say(f"[chain] latent_to_v row rel {rel:.3e}")
    assert rel <= 2.0 ** -7


def test_layer_step_graph_replay_matches_eager_bitwise():
    """rope -> paged decode -> latent_to_v, and a DCP-shard decode, captured in
    one HIP graph and replayed (with eager work in between): every replay
    gives the eager results bit for bit."""
    T, H, Hp = 4, 12, 16
    w = workloads.build("graph-paged", [700, 900, 300, 1200], num_heads=Hp, real_heads=H,
                        pool_entries=1 << 14, kv_std=0.5, scale_range=(0.5, 2.0), seed=120,
                        device=DEV, page_size=128)
    s = workloads.surround(T, H, 4096, 1 << 14, seed=121, device=DEV)
    kvp = w.kv_indptr.cpu().tolist()
    last = w.kv_last_page_lens.cpu().tolist()
    # each request's new entry is the last slot of its last page
    slots = torch.tensor([int(w.kv_indices[kvp[b + 1] - 1]) * 128 + last[b] - 1 for b in range(T)],
                         dtype=torch.int32, device=DEV)
    full = workloads.build("graph-dcp", [801, 77], num_heads=16, real_heads=12, qlens=[3, 1],
                           pool_entries=4096, kv_std=0.5, seed=122, device=DEV)
    sh = workloads.dcp_shard(full, 4, 2)
    q = torch.empty((T, Hp, 576), dtype=torch.float8_e4m3fn, device=DEV)
    o = torch.empty((T, Hp, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, Hp), dtype=torch.float32, device=DEV)
    v = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty((sh.num_tokens, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse2 = torch.empty((sh.num_tokens, 16), dtype=torch.float32, device=DEV)
    ws = mla.new_workspace(mla.workspace_bytes(T, T, Hp, 1), DEV)
    ws2 = mla.new_workspace(mla.workspace_bytes(2, sh.num_tokens, 16, 3), DEV)

    def step():
        mla.rope_quant_cache(s.q_latent, s.q_pe, s.k_latent, s.k_pe, s.positions, s.cos_sin,
                             w.kv_pool, slots, num_heads_pad=Hp, q_scale=w.q_scale,
                             kv_scale=w.kv_scale, q_out=q)
        mla.decode_paged(q, w.kv_pool, w.qo_indptr, w.kv_indptr, w.kv_indices,
                         w.kv_last_page_lens, w.sm_scale, w.q_scale, w.kv_scale,
                         return_lse=True, page_size=128, o=o, lse=lse, max_seqlen_q=1,
                         workspace=ws)
        mla.latent_to_v(o, s.w_uv, out=v)
        mla.decode_dcp(sh.q, sh.kv_pool, sh.qo_indptr, sh.kv_indptr, sh.kv_indices, None,
                       sh.sm_scale, sh.q_scale, sh.kv_scale, return_lse=True,
                       g_kv_indptr=sh.g_kv_indptr, cp_world_size=4, cp_rank=2, o=o2, lse=lse2,
                       max_seqlen_q=3, workspace=ws2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (q, o, lse, v, o2, lse2)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (q, o, lse, v, o2, lse2):
            t.zero_()
        mla.latent_to_v(torch.randn((8, 16, 512), device=DEV).to(torch.bfloat16), s.w_uv)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((q, o, lse, v, o2, lse2), eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float8_e4m3fn else a,
                               b.view(torch.uint8) if b.dtype == torch.float8_e4m3fn else b), rep
