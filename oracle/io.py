"""Marshal a generated workload into the oracle's plain numpy inputs.

Only reshapes and copies bytes: device tensors are copied to the host, storage
codes are reinterpreted as unsigned integers, and the pool is compacted to the
rows the call references (indices remapped accordingly), which leaves the
gather semantics unchanged.  Test infrastructure, like the rest of ``oracle``.
"""

from __future__ import annotations

import numpy as np
import torch


def codes(t: torch.Tensor) -> np.ndarray:
    """Raw storage codes of a float8_e4m3fn / bfloat16 / float32 tensor."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def workload_args(w, requests=None) -> dict:
    """Keyword arguments for ``oracle.mla.mla_decode`` for (a subset of) ``w``.

    requests: indices of the requests to keep (default: all).  The returned
    dict also carries 'tokens', the global token rows the result covers.
    """
    qo = w.qo_indptr.cpu().numpy().astype(np.int64)
    kvp = w.kv_indptr.cpu().numpy().astype(np.int64)
    B = len(qo) - 1
    reqs = list(range(B)) if requests is None else [int(b) for b in requests]
    dev = w.kv_indices.device
    page_size = int(getattr(w, "page_size", 1))
    toks, req_rows = [], []
    for b in reqs:
        toks.extend(range(qo[b], qo[b + 1]))
        if page_size == 1:
            req_rows.append(w.kv_indices[kvp[b]: kvp[b + 1]].to(torch.int64))
        else:  # expand the request's page list to one pool row per entry
            from .mla import paged_entry_rows

            pages = w.kv_indices[kvp[b]: kvp[b + 1]].cpu().numpy()
            last = w.kv_last_page_lens[b: b + 1].cpu().numpy()
            _, rows = paged_entry_rows(np.array([0, len(pages)]), pages, last, page_size)
            req_rows.append(torch.from_numpy(rows).to(dev))
    idx_dev = torch.cat(req_rows or [torch.empty(0, dtype=torch.int64, device=dev)])
    uniq, inverse = torch.unique(idx_dev, return_inverse=True)
    pool_rows = w.kv_pool.index_select(0, uniq) if uniq.numel() else w.kv_pool[:1]
    lens = np.array([int(r.numel()) for r in req_rows], dtype=np.int64)
    qlens = np.array([qo[b + 1] - qo[b] for b in reqs], dtype=np.int64)
    tok_t = torch.tensor(toks, dtype=torch.int64, device=w.q.device)
    dcp = {}
    if getattr(w, "g_kv_indptr", None) is not None:
        g = w.g_kv_indptr.cpu().numpy().astype(np.int64)
        glens = np.array([g[b + 1] - g[b] for b in reqs], dtype=np.int64)
        dcp = dict(g_kv_indptr=np.concatenate([[0], np.cumsum(glens)]), cp_size=int(w.cp_size),
                   cp_rank=int(w.cp_rank))
    return dict(
        q=codes(w.q.index_select(0, tok_t)) if toks else codes(w.q[:0]),
        kv_pool=codes(pool_rows),
        qo_indptr=np.concatenate([[0], np.cumsum(qlens)]),
        kv_indptr=np.concatenate([[0], np.cumsum(lens)]),
        kv_indices=inverse.cpu().numpy().astype(np.int64),
        sm_scale=float(w.sm_scale),
        q_scale=float(w.q_scale.item()),
        kv_scale=float(w.kv_scale.item()),
        dtype=w.dtype,
        tokens=np.array(toks, dtype=np.int64),
        **dcp,
    )


def call_decode(args: dict):
    """Run ``oracle.mla.mla_decode`` on ``workload_args`` output."""
    from .mla import mla_decode

    kw = {k: v for k, v in args.items() if k != "tokens"}
    return mla_decode(**kw)
