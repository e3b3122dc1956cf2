"""Seeded synthetic inputs shaped like the captured MLA decode calls.

This module only draws and lays out inputs: lengths, index lists, pool rows,
queries and scales.  It holds none of the attention arithmetic, and it is the
one module that both the HIP path's tests / benchmark and the oracle's tests
use.  Inputs are drawn with a seeded ``torch.Generator`` on the requested
device; a CPU oracle reads back exactly the bytes the device path consumes.

Shapes follow "[Kimi-K3 MLA TP8] MLA performance" (ROCm/aiter issue 4541),
Sec. 4.1 / 4.2 "Arguments" (q (B, 16, 576) e4m3fn, a 5,283,840-entry token-major
pool, a 4,718,592-entry index buffer, per-request lengths ~68,43x with a
63,911-token shared prefix) and Sec. 5.4 (prefix slots shared by every request).
Value distributions, seeds and the other workloads are this project's choices,
stated in the design notes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

ROW_DIM = 576
LATENT_DIM = 512
E4M3FN_MAX = 448.0
POOL_ENTRIES = 5_283_840  # [Issue] Sec. 4.1, kv_buffer (5283840, 1, 1, 576)
INDEX_BUFFER = 4_718_592  # [Issue] Sec. 4.1, kv_indices (4718592,)
SHARED_PREFIX = 63_911  # [Issue] Sec. 1, workload row
UNIQUE_INPUT = 4_089  # [Issue] Sec. 1, workload row
SM_SCALE_F64 = 192.0 ** -0.5  # [Issue] Sec. 2, sm_scale = 1/sqrt(192)


def fp32(x: float) -> float:
    """Round a Python float to the nearest binary32 value (returned as float)."""
    return float(torch.tensor(x, dtype=torch.float32).item())


SM_SCALE = fp32(SM_SCALE_F64)


@dataclass
class Workload:
    """One decode call's inputs (device tensors) plus the recipe that made them."""

    name: str
    dtype: str  # 'fp8' or 'bf16' storage of q and the pool
    q: torch.Tensor  # (T, H, 576)
    kv_pool: torch.Tensor  # (N, 576)
    qo_indptr: torch.Tensor  # (B+1,) int32
    kv_indptr: torch.Tensor  # (B+1,) int32
    kv_indices: torch.Tensor  # (>= kv_indptr[B],) int32
    kv_last_page_lens: torch.Tensor  # (B,) int32, all ones
    q_scale: torch.Tensor  # 0-d fp32
    kv_scale: torch.Tensor  # 0-d fp32
    sm_scale: float
    num_heads: int
    real_heads: int
    max_seqlen_q: int
    return_lse: bool
    lengths: list[int]
    qlens: list[int]
    recipe: dict = field(default_factory=dict)
    # One DCP shard of a larger call (dcp_shard): offsets of the full lists,
    # the number of shards the positions are dealt over, and this shard.
    g_kv_indptr: torch.Tensor | None = None
    cp_size: int = 1
    cp_rank: int = 0
    # Paged cache (page_size > 1): kv_indptr counts pages, kv_indices holds page
    # numbers and kv_last_page_lens the slots used in each last page.
    page_size: int = 1

    @property
    def batch(self) -> int:
        return len(self.lengths)

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def total_kv(self) -> int:
        return int(sum(self.lengths))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _fill_values(shape, std: float, dtype: str, seed: int, device, chunk_rows: int = 1 << 17):
    """N(0, std) values, clamped to the e4m3fn range, stored as ``dtype``.

    Drawn in row chunks so a multi-GB pool never needs a full fp32 copy.
    """
    tdtype = torch.float8_e4m3fn if dtype == "fp8" else torch.bfloat16
    out = torch.empty(shape, dtype=tdtype, device=device)
    g = _gen(seed, device)
    rows = shape[0]
    flat = out.view(rows, -1)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        x.mul_(std).clamp_(-E4M3FN_MAX, E4M3FN_MAX)
        flat[r0:r1] = x.to(tdtype)
    return out


def _scale(lo_hi, seed: int, device) -> torch.Tensor:
    if lo_hi is None:
        return torch.ones((), dtype=torch.float32, device=device)
    lo, hi = lo_hi
    g = _gen(seed, device)
    return (torch.rand((), generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo)


def make_indices(lengths, shared_prefix, pool_entries, layout, seed, device, index_buffer=None):
    """kv_indices for `lengths`: a seeded permutation (or 128-slot block
    permutation) of the pool; the first `shared_prefix` entries of every request
    are the same slots, the rest are disjoint.  Buffer length >= the sum."""
    gi = _gen(seed, device)
    if layout == "random":
        perm = torch.randperm(pool_entries, generator=gi, device=device, dtype=torch.int64)
    elif layout == "blocked":
        nblk = pool_entries // 128
        bperm = torch.randperm(nblk, generator=gi, device=device, dtype=torch.int64)
        perm = (bperm[:, None] * 128 + torch.arange(128, device=device)[None, :]).reshape(-1)
    else:
        raise ValueError(layout)
    prefix = perm[:shared_prefix]
    parts = []
    off = shared_prefix
    for n in lengths:
        u = max(0, n - shared_prefix)
        parts.append(prefix[: min(n, shared_prefix)])
        parts.append(perm[off : off + u])
        off += u
    used = torch.cat(parts) if parts else torch.empty(0, dtype=torch.int64, device=device)
    total = int(used.numel())
    buf_len = max(total, index_buffer or 0, 1)
    kv_indices = torch.zeros(buf_len, dtype=torch.int32, device=device)
    kv_indices[:total] = used.to(torch.int32)
    return kv_indices


def make_paged_indices(lengths, page_size, shared_prefix, pool_entries, seed, device):
    """Page tables for `lengths` over a pool of pool_entries / page_size pages,
    handed out in a seeded random order.  The first shared_prefix // page_size
    pages of every request are the same pages (only whole pages are shared, as
    in prefix caching); the rest are disjoint.  Returns (kv_indptr in pages,
    kv_indices = page numbers, kv_last_page_lens), int32 on `device`."""
    P = page_size
    npages = pool_entries // P
    gi = _gen(seed, device)
    perm = torch.randperm(npages, generator=gi, device=device, dtype=torch.int64)
    shared = shared_prefix // P
    off = shared
    parts, counts, last = [], [], []
    for n in lengths:
        pages = -(-n // P)
        s = min(pages, shared) if n >= shared * P else 0
        parts.append(perm[:s])
        parts.append(perm[off: off + pages - s])
        off += pages - s
        counts.append(pages)
        last.append(n - (pages - 1) * P if pages else 1)
    if off > npages:
        raise ValueError(f"paged workload needs {off} pages, pool has {npages}")
    kv_indptr = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.cumsum(torch.tensor(counts, dtype=torch.int64), 0).to(torch.int32)
    used = torch.cat(parts) if parts else torch.empty(0, dtype=torch.int64, device=device)
    idx = torch.zeros(max(int(used.numel()), 1), dtype=torch.int32, device=device)
    idx[: used.numel()] = used.to(torch.int32)
    return (kv_indptr.to(device), idx, torch.tensor(last, dtype=torch.int32, device=device))


def build(
    name: str,
    lengths: list[int],
    *,
    num_heads: int = 16,
    real_heads: int | None = None,
    qlens: list[int] | None = None,
    pool_entries: int = 4096,
    dtype: str = "fp8",
    kv_std: float = 1.0,
    q_std: float = 1.0,
    scale_range=None,
    shared_prefix: int = 0,
    layout: str = "random",
    index_buffer: int | None = None,
    return_lse: bool = True,
    seed: int = 0,
    device="cpu",
    page_size: int = 1,
) -> Workload:
    """Assemble a decode call.

    lengths:       KV length (tokens) of each request.
    qlens:         query tokens per request (default all 1).
    shared_prefix: the first ``shared_prefix`` entries of every request use the
                   same pool slots (prefix caching); the rest are disjoint.
    layout:        'random' scatters slots by a seeded permutation of the pool;
                   'blocked' hands out runs of 128 consecutive slots (the
                   allocator's block size) in a seeded random block order.
    page_size:     > 1 builds a paged call (make_paged_indices; layout and
                   index_buffer do not apply).
    Seeds: lengths are the caller's; KV uses seed+1, q seed+2, indices seed+3,
    scales seed+4 (q_scale) and seed+5 (kv_scale).
    """
    B = len(lengths)
    lengths = [int(n) for n in lengths]
    qlens = [1] * B if qlens is None else [int(x) for x in qlens]
    real_heads = num_heads if real_heads is None else real_heads
    T = sum(qlens)
    uniq = [max(0, n - shared_prefix) for n in lengths]
    need = shared_prefix + sum(uniq)
    if need > pool_entries:
        raise ValueError(f"workload needs {need} distinct slots, pool has {pool_entries}")

    if page_size > 1:
        kv_indptr, kv_indices, last_page_lens = make_paged_indices(
            lengths, page_size, shared_prefix, pool_entries, seed + 3, device)
    else:
        kv_indices = make_indices(lengths, shared_prefix, pool_entries, layout, seed + 3, device,
                                  index_buffer)
        kv_indptr = torch.zeros(B + 1, dtype=torch.int32)
        kv_indptr[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        last_page_lens = torch.ones(B, dtype=torch.int32, device=device)
    buf_len = int(kv_indices.numel())
    qo_indptr = torch.zeros(B + 1, dtype=torch.int32)
    qo_indptr[1:] = torch.cumsum(torch.tensor(qlens, dtype=torch.int64), 0).to(torch.int32)

    kv_pool = _fill_values((pool_entries, ROW_DIM), kv_std, dtype, seed + 1, device)
    q = _fill_values((T, num_heads, ROW_DIM), q_std, dtype, seed + 2, device, chunk_rows=1 << 12)
    if real_heads < num_heads:
        q[:, real_heads:, :] = torch.zeros((), dtype=q.dtype, device=device)

    return Workload(
        name=name,
        dtype=dtype,
        q=q,
        kv_pool=kv_pool,
        qo_indptr=qo_indptr.to(device),
        kv_indptr=kv_indptr.to(device),
        kv_indices=kv_indices,
        kv_last_page_lens=last_page_lens,
        q_scale=_scale(scale_range, seed + 4, device),
        kv_scale=_scale(scale_range, seed + 5, device),
        sm_scale=SM_SCALE,
        num_heads=num_heads,
        real_heads=real_heads,
        max_seqlen_q=max(qlens) if qlens else 1,
        return_lse=return_lse,
        lengths=lengths,
        qlens=qlens,
        recipe=dict(
            seed=seed, pool_entries=pool_entries, kv_std=kv_std, q_std=q_std,
            scale_range=scale_range, shared_prefix=shared_prefix, layout=layout,
            index_buffer=buf_len, dtype=dtype, page_size=page_size,
        ),
        page_size=page_size,
    )


# ---------------------------------------------------------------------------
# The five workloads at full size.  Config k draws lengths from seed 1000*k.
# ---------------------------------------------------------------------------


def tiny(device="cpu") -> Workload:
    """B=2, 16 heads (12 real + 4 zero), kv 64 and 100, pool 256 entries, N(0,1)."""
    return build(
        "tiny", [64, 100], num_heads=16, real_heads=12, pool_entries=256, dtype="fp8",
        kv_std=1.0, q_std=1.0, scale_range=None, seed=1000, device=device,
    )


def c16_lengths() -> list[int]:
    """63,911 shared + 4,089 unique + 430 + (b mod 5) decoded, b = 0..15."""
    return [SHARED_PREFIX + UNIQUE_INPUT + 430 + (b % 5) for b in range(16)]


def c16(device="cpu", variant: str = "shared", return_lse: bool = False) -> Workload:
    """Batch 16 at kv ~68,430 (the headline decode call), fp8, N(0,0.5) KV.

    variant: 'shared' (prefix slots shared by all requests, as captured),
             'unshared' (every request's prefix uses its own slots),
             'blocked' (shared prefix, slots handed out in 128-slot runs),
             'paged128' (a page table of 128-slot pages: the 499 whole pages
             of the prefix shared, the rest of each request in its own pages).
    """
    lengths = c16_lengths()
    shared = 0 if variant == "unshared" else SHARED_PREFIX
    layout = "blocked" if variant == "blocked" else "random"
    return build(
        f"c16-{variant}", lengths, num_heads=16, real_heads=12, pool_entries=POOL_ENTRIES,
        dtype="fp8", kv_std=0.5, q_std=1.0, scale_range=(0.5, 2.0), shared_prefix=shared,
        layout=layout, index_buffer=INDEX_BUFFER, return_lse=return_lse, seed=2000,
        device=device, page_size=128 if variant == "paged128" else 1,
    )


def c32(device="cpu") -> Workload:
    """The batch-16 call's request shape at batch 32 (shared 63,911-entry
    prefix + 4,089 unique + 430 + (b mod 5) decoded), fp8, 16 heads (12 real +
    4 zero): a batch whose 12-head query rows fill fewer group-mode units than
    its padded ones (384 rows: 3 units of 128 against 4)."""
    lengths = [SHARED_PREFIX + UNIQUE_INPUT + 430 + (b % 5) for b in range(32)]
    return build(
        "c32", lengths, num_heads=16, real_heads=12, pool_entries=POOL_ENTRIES, dtype="fp8",
        kv_std=0.5, q_std=1.0, scale_range=(0.5, 2.0), shared_prefix=SHARED_PREFIX,
        index_buffer=INDEX_BUFFER, return_lse=False, seed=2500, device=device,
    )


def c24_lengths() -> list[int]:
    g = _gen(3000, "cpu")
    dec = torch.randint(0, 351, (24,), generator=g).tolist()
    return [SHARED_PREFIX + UNIQUE_INPUT + int(d) for d in dec]


def c24(device="cpu", return_lse: bool = False) -> Workload:
    """Batch 24, shared 63,911 prefix + 4,089 unique + U{0..350} decoded, fp8."""
    return build(
        "c24", c24_lengths(), num_heads=16, real_heads=12, pool_entries=POOL_ENTRIES,
        dtype="fp8", kv_std=0.5, q_std=1.0, scale_range=(0.5, 2.0),
        shared_prefix=SHARED_PREFIX, index_buffer=INDEX_BUFFER, return_lse=return_lse,
        seed=3000, device=device,
    )


def mixed_lengths() -> list[int]:
    g = _gen(4000, "cpu")
    u = torch.rand(64, generator=g, dtype=torch.float64)
    lo, hi = math.log(1024.0), math.log(142_000.0)
    return [int(math.floor(math.exp(lo + (hi - lo) * float(x)))) for x in u]


def mixed(device="cpu", dtype: str = "fp8", return_lse: bool = False) -> Workload:
    """Batch 64, kv log-uniform in [1,024, 142,000], disjoint slots, N(0,1)."""
    return build(
        f"mixed-{dtype}", mixed_lengths(), num_heads=16, real_heads=12,
        pool_entries=POOL_ENTRIES, dtype=dtype, kv_std=1.0, q_std=1.0, scale_range=None,
        return_lse=return_lse, seed=4000, device=device,
    )


DCP_LOCAL = 142_000 // 8  # 17,750 positions per request on one DCP8 rank


def dcp_shard(w: Workload, cp_size: int, cp_rank: int) -> Workload:
    """Shard `cp_rank` of call `w` under DCP with positions dealt round-robin over
    `cp_size` shards: the shard's list for request b holds positions cp_rank,
    cp_rank + cp_size, ... of b's list in `w`.  Everything else (q, pool,
    scales) is shared.  The result carries g_kv_indptr = w.kv_indptr."""
    kvp = w.kv_indptr.cpu().tolist()
    parts = [w.kv_indices[kvp[b] + cp_rank: kvp[b + 1]: cp_size] for b in range(w.batch)]
    lens = [int(t.numel()) for t in parts]
    dev = w.kv_indices.device
    kv_indptr = torch.zeros(w.batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    idx = torch.cat(parts) if sum(lens) else torch.zeros(1, dtype=torch.int32, device=dev)
    return Workload(**{
        **w.__dict__,
        "name": f"{w.name}-cp{cp_rank}of{cp_size}",
        "kv_indptr": kv_indptr.to(dev),
        "kv_indices": idx.contiguous(),
        "lengths": lens,
        "recipe": {**w.recipe, "cp_size": cp_size, "cp_rank": cp_rank},
        "g_kv_indptr": w.kv_indptr,
        "cp_size": cp_size,
        "cp_rank": cp_rank,
    })


DCP_FULL = 142_000  # [Blog] Sec. 1: a 142,000-token conversation
DCP_SIZE = 8


def dcp_share(device="cpu", cp_rank: int = DCP_SIZE - 1) -> Workload:
    """One DCP8 rank's share: batch 8, 96 heads (12 per GPU x 8 after the query
    exchange), 4 draft tokens (causal over full-list positions), each request's
    142,000 positions dealt round-robin over 8 shards (17,750 here).  Rank 7
    holds the last position of every request, so its draft tokens mask
    entries."""
    full = build(
        "dcp-full", [DCP_FULL] * 8, num_heads=96, real_heads=96, qlens=[4] * 8,
        pool_entries=POOL_ENTRIES, dtype="fp8", kv_std=0.5, q_std=1.0,
        scale_range=(0.5, 2.0), return_lse=True, seed=5000, device=device,
    )
    w = dcp_shard(full, DCP_SIZE, cp_rank)
    w.name = "dcp-share"
    return w


def dcp_local(device="cpu") -> Workload:
    """One GPU's DCP8-shaped share with the mask taken on the local list: batch 8,
    96 heads, 4 query tokens per request (multi-token verification, causal among
    the draft tokens, bottom-right on the shard's own 17,750 entries = 142,000 / 8),
    fp8 KV N(0,0.5) in the 5,283,840-entry pool, q N(0,1), scales U[0.5,2],
    return_lse on.  This is the plain mla_decode call on the shard's list."""
    return build(
        "dcp-local", [DCP_LOCAL] * 8, num_heads=96, real_heads=96, qlens=[4] * 8,
        pool_entries=POOL_ENTRIES, dtype="fp8", kv_std=0.5, q_std=1.0,
        scale_range=(0.5, 2.0), return_lse=True, seed=5500, device=device,
    )


def redo_case(sign: float = 1.0, num_heads: int = 64, device="cpu") -> Workload:
    """A stress case for the score-range handling: two requests (6,000 and 700
    entries, one query token, 16 * k heads, N(0,0.5) KV, N(0,1) q).  Every q row's
    64 rope dims are set to 8.0, and the rope dims of request 0's entries at
    positions >= 4,500 to 8.0 * sign, so those entries score about
    64 * 64 * sm_scale * log2(e) ~ 426 base-2 units above the first 4,500 (for a
    positive sm_scale and sign = 1; use sign = -1 with a negative sm_scale)."""
    w = build(
        f"redo-h{num_heads}-{'pos' if sign > 0 else 'neg'}", [6000, 700], num_heads=num_heads,
        real_heads=num_heads, pool_entries=1 << 14, dtype="fp8", kv_std=0.5, q_std=1.0,
        scale_range=None, seed=9100, device=device,
    )
    kvp = w.kv_indptr.cpu().tolist()
    big = w.kv_indices[kvp[0] + 4500: kvp[1]].to(torch.int64)
    code = int(torch.tensor(8.0 * sign).to(torch.float8_e4m3fn).view(torch.uint8).item())
    w.kv_pool.view(torch.uint8)[big, LATENT_DIM:] = code  # byte writes: no fp8 index_put needed
    w.q[:, :, LATENT_DIM:] = torch.tensor(8.0, device=device).to(w.q.dtype)
    return w


def merge_shards(
    num_parts: int = 8, num_tokens: int = 32, num_heads: int = 96, parts_dtype: str = "fp32",
    seed: int = 5100, device="cpu", kv_local: int = DCP_LOCAL,
):
    """Synthetic DCP partial answers: o ~ N(0,1), lse ~ N(ln kv_local, 1).

    One (shard, token, head) row per shard is forced to -inf (an empty shard),
    and one (token, head) row is -inf in every shard.
    Returns (o_parts (S,T,H,512), lse_parts (S,T,H) fp32).
    """
    g = _gen(seed, device)
    tdtype = torch.float32 if parts_dtype == "fp32" else torch.bfloat16
    o = torch.randn((num_parts, num_tokens, num_heads, LATENT_DIM), generator=g, device=device)
    lse = torch.randn((num_parts, num_tokens, num_heads), generator=g, device=device)
    lse = lse + math.log(kv_local)
    for s in range(num_parts):
        lse[s, s % num_tokens, (7 * s) % num_heads] = -math.inf
    lse[:, num_tokens - 1, num_heads - 1] = -math.inf
    return o.to(tdtype), lse.to(torch.float32)

def split_prefix(w: Workload, prefix: int):
    """The same call as a shared prefix plus per-request suffixes (the layout
    decode_cascade takes): the first `prefix` entries of every request must be
    the same pool slots (build(..., shared_prefix >= prefix) makes them so).
    Returns (prefix_indices, suffix_indptr, suffix_indices) on w's device."""
    kvp = w.kv_indptr.cpu().tolist()
    idx = w.kv_indices
    pre = idx[kvp[0]: kvp[0] + prefix].clone()
    for b in range(w.batch):
        if kvp[b + 1] - kvp[b] < prefix or not torch.equal(idx[kvp[b]: kvp[b] + prefix], pre):
            raise ValueError(f"request {b} does not start with the shared prefix")
    parts = [idx[kvp[b] + prefix: kvp[b + 1]] for b in range(w.batch)]
    lens = [int(t.numel()) for t in parts]
    suf_indptr = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32,
                              device=idx.device)
    suf = torch.cat(parts) if sum(lens) else torch.zeros(1, dtype=torch.int32, device=idx.device)
    return pre, suf_indptr, suf


# ---------------------------------------------------------------------------
# Inputs of the steps either side of the decode: the fused rope / fp8 /
# cache-write step before it and the latent -> v_head_dim GEMM after it.
# ---------------------------------------------------------------------------

V_HEAD_DIM = 128  # [Issue] Sec. 2
ROPE_DIM = 64  # [Issue] Sec. 2


@dataclass
class SurroundInputs:
    q_latent: torch.Tensor  # (T, H, 512) bf16
    q_pe: torch.Tensor  # (T, H, 64) bf16
    k_latent: torch.Tensor  # (T, 512) bf16
    k_pe: torch.Tensor  # (T, 64) bf16
    positions: torch.Tensor  # (T,) int32
    cos_sin: torch.Tensor  # (max_pos, 64) fp32: cos of 32 angles, then sin
    slot_mapping: torch.Tensor  # (T,) int32, distinct pool slots
    w_uv: torch.Tensor  # (H, 128, 512) bf16
    q_scale: torch.Tensor  # 0-d fp32
    kv_scale: torch.Tensor  # 0-d fp32


def rope_table(max_pos: int, base: float = 10000.0, device="cpu") -> torch.Tensor:
    """cos / sin table of the usual rotary frequencies base^(-2j/64), j < 32,
    at positions 0 .. max_pos-1: (max_pos, 64) fp32 (angles in float64)."""
    j = torch.arange(ROPE_DIM // 2, dtype=torch.float64)
    inv = base ** (-2.0 * j / ROPE_DIM)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32).to(device)


def surround(num_tokens: int, num_heads: int, max_pos: int, pool_entries: int, seed: int,
             device="cpu", scale_range=(0.5, 2.0)) -> SurroundInputs:
    """Seeded inputs: q parts N(0,1), new cache entries N(0,0.5), positions
    U{0..max_pos-1}, distinct random slots, W N(0, 1/512) (bf16)."""
    g = _gen(seed, device)
    T, H = num_tokens, num_heads

    def randn(*shape, std=1.0):
        return (torch.randn(shape, generator=g, device=device) * std).to(torch.bfloat16)

    q_latent = randn(T, H, LATENT_DIM)
    q_pe = randn(T, H, ROPE_DIM)
    k_latent = randn(T, LATENT_DIM, std=0.5)
    k_pe = randn(T, ROPE_DIM, std=0.5)
    positions = torch.randint(0, max_pos, (T,), generator=g, device=device, dtype=torch.int32)
    slots = torch.randperm(pool_entries, generator=g, device=device)[:T].to(torch.int32)
    w_uv = randn(H, V_HEAD_DIM, LATENT_DIM, std=LATENT_DIM ** -0.5)
    return SurroundInputs(q_latent, q_pe, k_latent, k_pe, positions,
                          rope_table(max_pos, device=device), slots, w_uv,
                          _scale(scale_range, seed + 4, device), _scale(scale_range, seed + 5, device))
