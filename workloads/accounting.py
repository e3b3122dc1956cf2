"""Algorithmic bytes and FLOPs of one decode call (benchmark bookkeeping).

The accounting follows "[Kimi-K3 MLA TP8] MLA performance" (ROCm/aiter issue
4541), Sec. 5.3 "Strongly memory-bound": every gathered token slot costs one
576-wide pool row plus one int32 index; q is read once and o written once;
FLOPs count 2 * rows * (576 + 512) per (query row, visible entry), padded heads
included.  Shared-prefix reuse is not subtracted: the method gathers per
request.
"""

from __future__ import annotations

ROW_DIM = 576
LATENT_DIM = 512
INDEX_BYTES = 4

_ELEM = {"fp8": 1, "bf16": 2, "fp32": 4}


def row_bytes(dtype: str) -> int:
    return ROW_DIM * _ELEM[dtype]


def visible(n: int, qlen: int, j: int) -> int:
    return max(0, n - (qlen - 1 - j))


def decode_bytes(lengths, qlens, num_heads, dtype="fp8", return_lse=False, page_size=1) -> int:
    """HBM bytes the method must move for one call.  A paged cache reads one
    index per page plus each request's last-page length instead of one index
    per entry."""
    T = sum(qlens)
    if page_size == 1:
        kv = sum(lengths) * (row_bytes(dtype) + INDEX_BYTES)
    else:
        pages = sum(-(-n // page_size) for n in lengths)
        kv = sum(lengths) * row_bytes(dtype) + (pages + len(lengths)) * INDEX_BYTES
    q = T * num_heads * ROW_DIM * _ELEM[dtype]
    o = T * num_heads * LATENT_DIM * 2
    lse = T * num_heads * 4 if return_lse else 0
    return kv + q + o + lse


def shard_visible(n: int, full: int, qlen: int, j: int, cp_size: int, cp_rank: int) -> int:
    """Visible entries of draft token j on a DCP shard whose i-th entry is
    full-list position cp_rank + i * cp_size (token j sees positions <= full - qlen + j)."""
    last = full - qlen + j
    return 0 if last < cp_rank else min(n, (last - cp_rank) // cp_size + 1)


def decode_flops(lengths, qlens, num_heads, shard=None) -> int:
    """2 * heads * sum over query tokens of visible entries * (576 + 512).
    shard = (full_lengths, cp_size, cp_rank) for one DCP shard's call."""
    if shard is None:
        vis = sum(visible(n, ql, j) for n, ql in zip(lengths, qlens) for j in range(ql))
    else:
        full, cs, cr = shard
        vis = sum(shard_visible(n, N, ql, j, cs, cr)
                  for n, N, ql in zip(lengths, full, qlens) for j in range(ql))
    return 2 * num_heads * vis * (ROW_DIM + LATENT_DIM)


def merge_bytes(num_parts, num_tokens, num_heads, parts_dtype="fp32", with_lse_out=True) -> int:
    rows = num_tokens * num_heads
    return rows * (num_parts * (LATENT_DIM * _ELEM[parts_dtype] + 4) + LATENT_DIM * 2 + (4 if with_lse_out else 0))


def workload_bytes(w) -> int:
    return decode_bytes(w.lengths, w.qlens, w.num_heads, w.dtype, w.return_lse,
                        getattr(w, "page_size", 1))


def workload_flops(w) -> int:
    shard = None
    if getattr(w, "g_kv_indptr", None) is not None:
        g = [int(x) for x in w.g_kv_indptr.cpu().tolist()]
        shard = ([g[b + 1] - g[b] for b in range(len(g) - 1)], w.cp_size, w.cp_rank)
    return decode_flops(w.lengths, w.qlens, w.num_heads, shard)


def cascade_bytes(w, prefix: int) -> int:
    """Bytes a shared-prefix (cascade) call must move: the prefix rows and
    indices once, each request's own rows and indices, q read and o written."""
    rows = prefix + sum(max(0, n - prefix) for n in w.lengths)
    T = sum(w.qlens)
    return (rows * (row_bytes(w.dtype) + INDEX_BYTES) + T * w.num_heads * ROW_DIM * _ELEM[w.dtype]
            + T * w.num_heads * LATENT_DIM * 2 + (T * w.num_heads * 4 if w.return_lse else 0))
