"""The plain definition of absorbed (latent) MLA decode, in float64 (oracle side).

What is computed, and where the pages fix it:

* [Issue] Sec. 2 "K3 MLA geometry": MLA runs in absorbed form, so every cached
  token is one 576-wide latent row (512 latent + 64 rope) shared by all query
  heads (a single latent KV head).  Scores use all 576 dims; the output is the
  softmax-weighted sum of the first 512 dims (the latent part).  The softmax
  scale is 1/sqrt(qk_head_dim) with qk_head_dim = 192.
* [Issue] Sec. 3 "Entry point" and Sec. 4.1 "Arguments": the call takes q
  (tokens, heads, 576), a token-major pool (entries, 576), qo_indptr /
  kv_indptr / kv_indices in CSR form and per-tensor fp32 q_scale / kv_scale.
* [Issue] Sec. 5.2 "The kernel runs with page_size = 1": kv_indptr deltas are
  each request's KV length in tokens and kv_indices holds one pool entry per
  cached token; kv_last_page_lens are all ones and carry no information.
* [Blog] Sec. 4 "MLA: faster long-context decoding with AMD AITER assembly":
  each head attends independently, so added (padding) heads do not change the
  softmax of the original heads.
* [Blog] Sec. 1 "Cache: keep conversation state available for reuse": partial
  answers carry normalisation information and are merged with softmax weights
  (``merge_partials``).

Readings taken where the pages are silent (each is listed in the design notes):

1. Dequantisation is real = stored * scale for both q and the cache; kv_scale
   multiplies K inside the score and V inside the output.
2. The score is s = sm_scale * q_scale * kv_scale * sum_{d<576} q_d k_d.
3. lse is the natural log of sum_i exp(s_i) per (query token, head).
4. Several query tokens per request (multi-token verification) see the
   request's list causally, bottom-right aligned: token j of qlen sees the
   first n - (qlen - 1 - j) entries.
5. A query row that sees no entry gets o = 0 and lse = -inf; a shard with
   lse = -inf has weight 0 in the merge, and an all -inf merge gives o = 0,
   lse = -inf.
6. Under decode context parallelism ([Blog] Sec. 1: each of the GPUs keeps an
   eighth of the cached positions; multi-token verification under DCP; the
   entry point's g_kv_indptr / cp_world_size / cp_rank arguments, [Issue]
   Sec. 3) a request's positions are dealt round-robin: shard r of W holds
   full-list positions r, r + W, r + 2W, ... in that order, and reading 4
   applies to full-list positions (``dcp_visible_length``).
7. Paged caches ([Issue] Sec. 3: the entry point's page_size and
   kv_last_page_lens arguments; Sec. 5.2: the capture uses page_size 1 while
   the allocator's blocks hold 128 slots): kv_indptr counts pages, kv_indices
   holds page numbers, page k holds pool rows k*P .. k*P + P - 1, and a
   request's last page holds kv_last_page_lens[b] of its P slots
   (``paged_entry_rows``).
"""

from __future__ import annotations

import numpy as np

from . import codecs

LATENT_DIM = 512  # kv_lora_rank, [Issue] Sec. 2
ROPE_DIM = 64  # qk_rope_head_dim, [Issue] Sec. 2
ROW_DIM = LATENT_DIM + ROPE_DIM  # 576-wide cache entry, [Issue] Sec. 2
QK_HEAD_DIM = 192  # qk_nope 128 + qk_rope 64, [Issue] Sec. 2


def visible_length(n: int, qlen: int, j: int) -> int:
    """Entries of a length-``n`` list visible to query token ``j`` of ``qlen``.

    Reading 4 above: the last query token sees the whole list, each earlier
    draft token sees one entry fewer.  Equals ``n`` when qlen = 1.
    """
    return max(0, n - (qlen - 1 - j))


def paged_entry_rows(kv_indptr, kv_indices, last_page_lens, page_size: int):
    """Per-entry pool rows of a paged call (reading 7).

    Request b owns pages kv_indices[kv_indptr[b]:kv_indptr[b+1]]; its entry i
    lives in its page number i // P at slot i % P, i.e. pool row
    page * P + i % P, and it has (pages - 1) * P + last_page_lens[b] entries
    (none without pages).  Returns (entry_indptr, rows) in the one-row-per-
    entry form ``mla_decode`` takes.
    """
    P = int(page_size)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    last = np.asarray(last_page_lens, dtype=np.int64)
    rows, counts = [], []
    for b in range(len(kv_indptr) - 1):
        pages = kv_indices[kv_indptr[b]: kv_indptr[b + 1]]
        n = 0 if len(pages) == 0 else (len(pages) - 1) * P + int(last[b])
        i = np.arange(n, dtype=np.int64)
        rows.append(pages[i // P] * P + i % P)
        counts.append(n)
    entry_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return entry_indptr, (np.concatenate(rows) if rows else np.zeros(0, np.int64))


def dcp_visible_length(n_full: int, n_local: int, qlen: int, j: int, cp_size: int,
                      cp_rank: int) -> int:
    """Entries of one DCP shard's list visible to query token ``j`` of ``qlen``.

    Reading 6: local entry i is position cp_rank + i * cp_size of the request's
    full list of ``n_full`` positions, and token j sees the full-list positions
    0 .. n_full - qlen + j (reading 4).  The visible entries are a prefix of
    the local list because positions grow with i.
    """
    last = n_full - qlen + j
    positions = cp_rank + cp_size * np.arange(n_local, dtype=np.int64)
    return int(np.count_nonzero(positions <= last))


def mla_decode(
    q: np.ndarray,
    kv_pool: np.ndarray,
    qo_indptr: np.ndarray,
    kv_indptr: np.ndarray,
    kv_indices: np.ndarray,
    sm_scale: float,
    q_scale: float = 1.0,
    kv_scale: float = 1.0,
    dtype: str = "fp8",
    g_kv_indptr: np.ndarray | None = None,
    cp_size: int = 1,
    cp_rank: int = 0,
) -> tuple[np.ndarray, np.ndarray]:
    """Reference MLA decode.

    Args:
      q:          (T, H, 576) raw codes (uint8 e4m3fn or uint16 bf16).
      kv_pool:    (N, 576) raw codes of the same storage type.
      qo_indptr:  (B+1,) token offsets of each request; qo_indptr[B] == T.
      kv_indptr:  (B+1,) offsets into kv_indices; deltas are KV lengths.
      kv_indices: pool entry of every cached token, request by request.
      sm_scale, q_scale, kv_scale: the scalars exactly as the device sees them.
      dtype:      'fp8' or 'bf16' storage type of q and kv_pool.
      g_kv_indptr, cp_size, cp_rank: one DCP shard (reading 6): kv_indptr /
                  kv_indices are the shard's lists and g_kv_indptr's deltas the
                  full lists' lengths.  None: no DCP.

    Returns (o, lse): o (T, H, 512) float64 and lse (T, H) float64.
    """
    q = np.asarray(q)
    kv_pool = np.asarray(kv_pool)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    if q.ndim != 3 or q.shape[2] != ROW_DIM:
        raise ValueError(f"q must be (T, H, {ROW_DIM}), got {q.shape}")
    if kv_pool.ndim != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError(f"kv_pool must be (N, {ROW_DIM}), got {kv_pool.shape}")
    T, H, _ = q.shape
    B = len(qo_indptr) - 1
    if len(kv_indptr) != B + 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length")
    if qo_indptr[0] != 0 or qo_indptr[B] != T:
        raise ValueError("qo_indptr must start at 0 and end at the token count")

    o = np.zeros((T, H, LATENT_DIM), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    for b in range(B):
        t0, t1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        qlen = t1 - t0
        rows = kv_indices[kv_indptr[b] : kv_indptr[b + 1]]
        n = len(rows)
        # Step 1: one latent row per cached token serves as both K (576) and V (512).
        K = kv_scale * codecs.decode(kv_pool[rows], dtype)  # (n, 576)
        V = K[:, :LATENT_DIM]  # (n, 512)
        for j in range(qlen):
            t = t0 + j
            if g_kv_indptr is None:
                vis = visible_length(n, qlen, j)
            else:
                n_full = int(g_kv_indptr[b + 1] - g_kv_indptr[b])
                vis = dcp_visible_length(n_full, n, qlen, j, cp_size, cp_rank)
            if vis == 0:
                continue  # reading 5: o = 0, lse = -inf
            Q = q_scale * codecs.decode(q[t], dtype)  # (H, 576)
            # Step 2: scores over all 576 dims.
            s = sm_scale * (Q @ K[:vis].T)  # (H, vis)
            # Step 3: softmax and lse, shifted by the row maximum.
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            denom = e.sum(axis=1, keepdims=True)
            # Step 4: weight the latent part.
            o[t] = (e @ V[:vis]) / denom
            lse[t] = m[:, 0] + np.log(denom[:, 0])
    return o, lse


def merge_partials(
    o_parts: np.ndarray, lse_parts: np.ndarray
) -> tuple[np.ndarray, np.ndarray]:
    """LSE-weighted merge of S partial answers over disjoint KV shards.

    Args:
      o_parts:   (S, ..., D) float64, each shard's normalised output.
      lse_parts: (S, ...) float64, each shard's natural-log sum of exp scores;
                 -inf marks an empty shard.

    Returns (o, lse) with the leading S axis merged:
      M = max_s lse_s; L = M + ln sum_s exp(lse_s - M);
      o = sum_s exp(lse_s - L) o_s; lse = L.  All -inf gives o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts must be lse_parts' shape plus a feature axis")
    M = lse_parts.max(axis=0)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_parts - M_safe)  # exp(-inf) = 0 for empty shards
    w = np.where(np.isneginf(lse_parts), 0.0, w)
    total = w.sum(axis=0)
    L = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, total)))
    weights = np.where(empty, 0.0, w / np.where(empty, 1.0, total))
    # Empty shards contribute nothing, whatever their o holds.
    o_used = np.where(np.isneginf(lse_parts)[..., None], 0.0, o_parts)
    o = (weights[..., None] * o_used).sum(axis=0)
    return o, L
