"""MI355X-native latent MLA decode: a thin binding over libmla.so (include/mla.h).

This module only marshals arguments: it checks devices, dtypes and contiguity,
allocates a workspace when the caller passes none, and hands raw device
pointers plus the current HIP stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_FP8, DTYPE_FP32, MLAError

__all__ = [
    "decode",
    "merge_partials",
    "workspace_bytes",
    "plan_host",
    "plan_groups_host",
    "decode_cascade",
    "decode_dcp",
    "decode_paged",
    "decode_noalloc",
    "rope_quant_cache",
    "latent_to_v",
    "decode_step",
    "check_inputs",
    "cascade_workspace_bytes",
    "new_workspace",
    "MLAError",
    "library_path",
]

ROW_DIM = 576
LATENT_DIM = 512


def library_path() -> str:
    return _lib.LIB_PATH


def _storage_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float8_e4m3fn:
        return DTYPE_FP8
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(batch: int, num_q_tokens: int, num_heads: int, max_seqlen_q: int = 1,
                    num_workers: int = 0) -> int:
    L = _lib.lib()
    if num_workers:
        n = L.mla_decode_workspace_bytes_ex(batch, num_q_tokens, num_heads, max_seqlen_q, num_workers)
    else:
        n = L.mla_decode_workspace_bytes(batch, num_q_tokens, num_heads, max_seqlen_q)
    if n == 0:
        raise ValueError("invalid shape for the decode workspace (or no HIP device)")
    return int(n)


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A decode workspace (its contents on entry do not matter)."""
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode(
    q: torch.Tensor,
    kv_pool: torch.Tensor,
    qo_indptr: torch.Tensor,
    kv_indptr: torch.Tensor,
    kv_indices: torch.Tensor,
    kv_last_page_lens: torch.Tensor | None,
    sm_scale: float,
    q_scale: torch.Tensor | None = None,
    kv_scale: torch.Tensor | None = None,
    return_lse: bool = False,
    *,
    o: torch.Tensor | None = None,
    lse: torch.Tensor | None = None,
    max_seqlen_q: int | None = None,
    workspace: torch.Tensor | None = None,
    num_workers: int = 0,
    _dcp=None,
    _page_size: int = 1,
):
    """Latent MLA decode; returns o (T, H, 512) bf16, or (o, lse) if return_lse.

    q: (T, H, 576) float8_e4m3fn or bfloat16; kv_pool: (N, 576) or (N, 1, 1, 576)
    of the same dtype; indptr / indices int32; q_scale / kv_scale 0-d fp32
    device tensors (None = 1.0).  max_seqlen_q defaults to the largest
    qo_indptr delta, which costs a device-to-host copy: pass it to avoid that.
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a device tensor")
    if q.dim() != 3 or q.shape[2] != ROW_DIM:
        raise ValueError(f"q must be (T, H, {ROW_DIM})")
    T, H, _ = q.shape
    if kv_pool.dim() == 4:
        if tuple(kv_pool.shape[1:]) not in ((1, 1, ROW_DIM), (_page_size, 1, ROW_DIM)):
            raise ValueError("a 4-d kv_pool must be (N, 1, 1, 576) or (pages, page_size, 1, 576)")
        kv_pool = kv_pool.view(-1, ROW_DIM)
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError(f"kv_pool must be (N, {ROW_DIM})")
    _need(q, "q", dev)
    _need(kv_pool, "kv_pool", dev)
    B = qo_indptr.numel() - 1
    _need(qo_indptr, "qo_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indptr, "kv_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indices, "kv_indices", dev, torch.int32)
    if kv_last_page_lens is not None:
        _need(kv_last_page_lens, "kv_last_page_lens", dev, torch.int32, (B,))
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None:
            _need(s, name, dev, torch.float32)
            if s.numel() != 1:
                raise ValueError(f"{name} must hold one value")
    o_dtype = torch.bfloat16 if _dcp is None else _dcp[3]
    if o is None:
        o = torch.empty((T, H, LATENT_DIM), dtype=o_dtype, device=dev)
    _need(o, "o", dev, o_dtype, (T, H, LATENT_DIM))
    if return_lse:
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        _need(lse, "lse", dev, torch.float32, (T, H))
    if max_seqlen_q is None:
        max_seqlen_q = int((qo_indptr[1:] - qo_indptr[:-1]).max().item()) if B > 0 else 1
    ws_need = workspace_bytes(B, T, H, max_seqlen_q, num_workers)
    if workspace is None:
        workspace = new_workspace(ws_need, dev)
    _need(workspace, "workspace", dev)
    ws_len = workspace.numel() * workspace.element_size()
    L = _lib.lib()
    qdt, kdt = _storage_dtype(q), _storage_dtype(kv_pool)
    head = (
        _ptr(q), qdt, _ptr(kv_pool), kdt, kv_pool.shape[0], _ptr(o), _ptr(qo_indptr),
        _ptr(kv_indptr), _ptr(kv_indices), kv_indices.numel(), _ptr(kv_last_page_lens),
        B, T, H, max_seqlen_q, float(sm_scale), _ptr(q_scale), _ptr(kv_scale),
        1 if return_lse else 0, _ptr(lse) if return_lse else None,
    )
    if _page_size != 1:
        if kv_last_page_lens is None:
            raise ValueError("a paged call needs kv_last_page_lens")
        status = L.mla_decode_paged(*head[:11], int(_page_size), *head[11:], _ptr(workspace),
                                    ws_len, _stream(dev))
        _lib.check(status, "mla_decode_paged")
    elif _dcp is None:
        status = L.mla_decode_ex(*head, _ptr(workspace), ws_len, int(num_workers), _stream(dev))
        _lib.check(status, "mla_decode")
    else:
        g_kv_indptr, cp_world_size, cp_rank, _ = _dcp
        _need(g_kv_indptr, "g_kv_indptr", dev, torch.int32, (B + 1,))
        status = L.mla_decode_dcp(*head, _ptr(g_kv_indptr), int(cp_world_size), int(cp_rank),
                                  _storage_dtype(o), _ptr(workspace), ws_len, _stream(dev))
        _lib.check(status, "mla_decode_dcp")
    return (o, lse) if return_lse else o


def decode_noalloc(
    q: torch.Tensor,
    kv_pool: torch.Tensor,
    qo_indptr: torch.Tensor,
    kv_indptr: torch.Tensor,
    kv_indices: torch.Tensor,
    kv_last_page_lens: torch.Tensor | None,
    sm_scale: float,
    q_scale: torch.Tensor | None = None,
    kv_scale: torch.Tensor | None = None,
    return_lse: bool = False,
    *,
    o: torch.Tensor,
    lse: torch.Tensor | None = None,
    max_seqlen_q: int,
):
    """decode() through mla_decode_noalloc: no workspace, nothing allocated.
    The caller passes o (and lse with return_lse) and max_seqlen_q; the call
    uses the library's fixed per-device scratch.  Returns what decode() returns."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a device tensor")
    if q.dim() != 3 or q.shape[2] != ROW_DIM:
        raise ValueError(f"q must be (T, H, {ROW_DIM})")
    T, H, _ = q.shape
    if kv_pool.dim() == 4:
        kv_pool = kv_pool.view(-1, ROW_DIM)
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError(f"kv_pool must be (N, {ROW_DIM})")
    _need(q, "q", dev)
    _need(kv_pool, "kv_pool", dev)
    B = qo_indptr.numel() - 1
    _need(qo_indptr, "qo_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indptr, "kv_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indices, "kv_indices", dev, torch.int32)
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None:
            _need(s, name, dev, torch.float32)
    _need(o, "o", dev, torch.bfloat16, (T, H, LATENT_DIM))
    if return_lse:
        if lse is None:
            raise ValueError("return_lse needs the caller's lse")
        _need(lse, "lse", dev, torch.float32, (T, H))
    status = _lib.lib().mla_decode_noalloc(
        _ptr(q), _storage_dtype(q), _ptr(kv_pool), _storage_dtype(kv_pool), kv_pool.shape[0],
        _ptr(o), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices), kv_indices.numel(), None,
        B, T, H, int(max_seqlen_q), float(sm_scale), _ptr(q_scale), _ptr(kv_scale),
        1 if return_lse else 0, _ptr(lse) if return_lse else None, _stream(dev))
    _lib.check(status, "mla_decode_noalloc")
    return (o, lse) if return_lse else o


def decode_paged(
    q: torch.Tensor,
    kv_pool: torch.Tensor,
    qo_indptr: torch.Tensor,
    kv_indptr: torch.Tensor,
    kv_indices: torch.Tensor,
    kv_last_page_lens: torch.Tensor,
    sm_scale: float,
    q_scale: torch.Tensor | None = None,
    kv_scale: torch.Tensor | None = None,
    return_lse: bool = False,
    *,
    page_size: int,
    o: torch.Tensor | None = None,
    lse: torch.Tensor | None = None,
    max_seqlen_q: int | None = None,
    workspace: torch.Tensor | None = None,
):
    """decode() over a paged cache (mla_decode_paged): kv_pool (rows, 576) or
    (pages, page_size, 1, 576); kv_indptr counts pages, kv_indices holds page
    numbers and kv_last_page_lens (B,) int32 the slots used in each request's
    last page.  Returns what decode() returns."""
    if page_size == 1:
        raise ValueError("page_size 1 is decode()")
    return decode(q, kv_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_lens, sm_scale,
                  q_scale, kv_scale, return_lse, o=o, lse=lse, max_seqlen_q=max_seqlen_q,
                  workspace=workspace, _page_size=page_size)


def decode_dcp(
    q: torch.Tensor,
    kv_pool: torch.Tensor,
    qo_indptr: torch.Tensor,
    kv_indptr: torch.Tensor,
    kv_indices: torch.Tensor,
    kv_last_page_lens: torch.Tensor | None,
    sm_scale: float,
    q_scale: torch.Tensor | None = None,
    kv_scale: torch.Tensor | None = None,
    return_lse: bool = False,
    *,
    g_kv_indptr: torch.Tensor,
    cp_world_size: int,
    cp_rank: int,
    o_dtype: torch.dtype = torch.bfloat16,
    o: torch.Tensor | None = None,
    lse: torch.Tensor | None = None,
    max_seqlen_q: int | None = None,
    workspace: torch.Tensor | None = None,
):
    """One DCP shard's decode (mla_decode_dcp): kv_indptr / kv_indices hold this
    shard's entries, the full-list positions cp_rank, cp_rank + cp_world_size, ...
    of each request; g_kv_indptr (B+1) int32 on the device gives the full lists'
    offsets.  o_dtype torch.float32 returns the shard's o in fp32 (for
    merge_partials with fp32 parts).  Returns what decode() returns."""
    if o_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("o_dtype must be torch.bfloat16 or torch.float32")
    return decode(q, kv_pool, qo_indptr, kv_indptr, kv_indices, kv_last_page_lens, sm_scale,
                  q_scale, kv_scale, return_lse, o=o, lse=lse, max_seqlen_q=max_seqlen_q,
                  workspace=workspace, _dcp=(g_kv_indptr, cp_world_size, cp_rank, o_dtype))


def cascade_workspace_bytes(batch: int, num_q_tokens: int, num_heads: int,
                            max_seqlen_q: int = 1) -> int:
    n = _lib.lib().mla_decode_cascade_workspace_bytes(batch, num_q_tokens, num_heads, max_seqlen_q)
    if n == 0:
        raise ValueError("invalid shape for the cascade workspace (or no HIP device)")
    return int(n)


def decode_cascade(
    q: torch.Tensor,
    kv_pool: torch.Tensor,
    qo_indptr: torch.Tensor,
    prefix_indices: torch.Tensor,
    suffix_indptr: torch.Tensor,
    suffix_indices: torch.Tensor,
    sm_scale: float,
    q_scale: torch.Tensor | None = None,
    kv_scale: torch.Tensor | None = None,
    return_lse: bool = False,
    *,
    o: torch.Tensor | None = None,
    lse: torch.Tensor | None = None,
    max_seqlen_q: int | None = None,
    workspace: torch.Tensor | None = None,
):
    """Shared-prefix decode: the result of decode() when request b's entries
    are prefix_indices followed by suffix_indices[suffix_indptr[b]:
    suffix_indptr[b+1]].  fp8 only; every request's suffix must hold at least
    qlen_b - 1 entries."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a device tensor")
    if q.dim() != 3 or q.shape[2] != ROW_DIM:
        raise ValueError(f"q must be (T, H, {ROW_DIM})")
    T, H, _ = q.shape
    if kv_pool.dim() == 4:
        kv_pool = kv_pool.view(kv_pool.shape[0], ROW_DIM)
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError(f"kv_pool must be (N, {ROW_DIM})")
    _need(q, "q", dev)
    _need(kv_pool, "kv_pool", dev)
    B = qo_indptr.numel() - 1
    _need(qo_indptr, "qo_indptr", dev, torch.int32, (B + 1,))
    _need(suffix_indptr, "suffix_indptr", dev, torch.int32, (B + 1,))
    _need(prefix_indices, "prefix_indices", dev, torch.int32)
    _need(suffix_indices, "suffix_indices", dev, torch.int32)
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None:
            _need(s, name, dev, torch.float32)
    if o is None:
        o = torch.empty((T, H, LATENT_DIM), dtype=torch.bfloat16, device=dev)
    _need(o, "o", dev, torch.bfloat16, (T, H, LATENT_DIM))
    if return_lse:
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        _need(lse, "lse", dev, torch.float32, (T, H))
    if max_seqlen_q is None:
        max_seqlen_q = int((qo_indptr[1:] - qo_indptr[:-1]).max().item()) if B > 0 else 1
    need = cascade_workspace_bytes(B, T, H, max_seqlen_q)
    if workspace is None:
        workspace = new_workspace(need, dev)
    _need(workspace, "workspace", dev)
    status = _lib.lib().mla_decode_cascade(
        _ptr(q), _storage_dtype(q), _ptr(kv_pool), _storage_dtype(kv_pool), kv_pool.shape[0],
        _ptr(o), _ptr(qo_indptr), _ptr(prefix_indices), prefix_indices.numel(),
        _ptr(suffix_indptr), _ptr(suffix_indices), suffix_indices.numel(), B, T, H, max_seqlen_q,
        float(sm_scale), _ptr(q_scale), _ptr(kv_scale), 1 if return_lse else 0,
        _ptr(lse) if return_lse else None, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev),
    )
    _lib.check(status, "mla_decode_cascade")
    return (o, lse) if return_lse else o


def merge_partials(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, o=None, lse=None,
                   return_lse: bool = True):
    """LSE merge of S shards: o_parts (S, T, H, 512) bf16|fp32, lse_parts (S, T, H) fp32."""
    dev = o_parts.device
    if o_parts.dim() != 4 or o_parts.shape[3] != LATENT_DIM:
        raise ValueError("o_parts must be (S, T, H, 512)")
    S, T, H, _ = o_parts.shape
    _need(o_parts, "o_parts", dev)
    _need(lse_parts, "lse_parts", dev, torch.float32, (S, T, H))
    if o is None:
        o = torch.empty((T, H, LATENT_DIM), dtype=torch.bfloat16, device=dev)
    _need(o, "o", dev, torch.bfloat16, (T, H, LATENT_DIM))
    if return_lse:
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        _need(lse, "lse", dev, torch.float32, (T, H))
    status = _lib.lib().mla_merge_partials(
        _ptr(o_parts), _storage_dtype(o_parts), _ptr(lse_parts), S, T, H, _ptr(o),
        _ptr(lse) if return_lse else None, _stream(dev),
    )
    _lib.check(status, "mla_merge_partials")
    return (o, lse) if return_lse else o


PLAN_FIELDS = ("worker", "token", "head_group", "kv_begin", "kv_end", "unit_len", "slot", "complete")


GROUP_PLAN_FIELDS = ("worker", "request", "unit", "kv_begin", "kv_end", "unit_len", "slot_base",
                     "complete")


def check_inputs(qo_indptr, kv_indptr, kv_indices, pool_entries: int, *, max_seqlen_q: int,
                 num_q_tokens: int | None = None, kv_last_page_lens=None, page_size: int = 1,
                 g_kv_indptr=None, cp_world_size: int = 1, cp_rank: int = 0,
                 status: torch.Tensor | None = None):
    """Device-side check of a decode call's index arguments (mla_check_inputs).

    Enqueues the check on the current stream; with status=None it allocates a
    one-int device word, waits for the check and returns the set of violated
    contracts (names such as "MLA_CHECK_KV_INDEX"; empty if none).  With a
    caller-provided status (1 int32 on the device) it only enqueues the check
    and returns None: the word holds the bits once the stream reaches it."""
    dev = qo_indptr.device
    B = qo_indptr.numel() - 1
    _need(qo_indptr, "qo_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indptr, "kv_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indices, "kv_indices", dev, torch.int32)
    if kv_last_page_lens is not None:
        _need(kv_last_page_lens, "kv_last_page_lens", dev, torch.int32, (B,))
    if g_kv_indptr is not None:
        _need(g_kv_indptr, "g_kv_indptr", dev, torch.int32, (B + 1,))
    if num_q_tokens is None:
        num_q_tokens = int(qo_indptr[-1].item())
    wait = status is None
    if wait:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _need(status, "status", dev, torch.int32, (1,))
    rc = _lib.lib().mla_check_inputs(
        _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices), kv_indices.numel(),
        _ptr(kv_last_page_lens), int(page_size), int(pool_entries), B, int(num_q_tokens),
        int(max_seqlen_q), _ptr(g_kv_indptr), int(cp_world_size), int(cp_rank), _ptr(status),
        _stream(dev))
    _lib.check(rc, "mla_check_inputs")
    if not wait:
        return None
    bits = int(status.item())
    return {name for bit, name in _lib.CHECK_BITS.items() if bits & bit}


def _plan(fn, qo_indptr, kv_indptr, num_heads, num_workers, g_kv_indptr=None):
    qo = np.ascontiguousarray(np.asarray(qo_indptr, dtype=np.int32))
    kv = np.ascontiguousarray(np.asarray(kv_indptr, dtype=np.int32))
    gkv = None if g_kv_indptr is None else np.ascontiguousarray(np.asarray(g_kv_indptr, np.int32))
    gp = None if gkv is None else gkv.ctypes.data
    B = len(qo) - 1
    n = fn(qo.ctypes.data, kv.ctypes.data, gp, B, num_heads, num_workers, None, 0)
    if n < 0:
        raise ValueError("invalid planner input")
    out = np.zeros((max(n, 1), 8), dtype=np.int64)
    n2 = fn(qo.ctypes.data, kv.ctypes.data, gp, B, num_heads, num_workers, out.ctypes.data, n)
    assert n2 == n
    return out[:n]


def plan_host(qo_indptr, kv_indptr, num_heads: int, num_workers: int, *, g_kv_indptr=None,
              cp_world_size: int = 1, cp_rank: int = 0) -> np.ndarray:
    """The planner's pieces for host indptr arrays: int64 array (pieces, 8), columns
    PLAN_FIELDS.  g_kv_indptr / cp_world_size / cp_rank: a DCP shard (mla_decode_dcp)."""
    fn = _lib.lib().mla_plan_host
    return _plan(lambda q, k, g, B, H, nw, out, cap: fn(q, k, g, B, H, nw, cp_world_size, cp_rank,
                                                         out, cap),
                 qo_indptr, kv_indptr, num_heads, num_workers, g_kv_indptr)


def plan_groups_host(qo_indptr, kv_indptr, num_heads: int, num_workers: int,
                     causal: bool = True, *, g_kv_indptr=None, cp_world_size: int = 1,
                     cp_rank: int = 0) -> np.ndarray:
    """The group-mode planner's pieces: int64 array (pieces, 8), columns GROUP_PLAN_FIELDS.
    causal=False: every token sees all of its request's entries.  DCP arguments as for
    plan_host."""
    fn = _lib.lib().mla_plan_groups_host
    c = 1 if causal else 0
    return _plan(lambda q, k, g, B, H, nw, out, cap: fn(q, k, g, B, H, nw, c, cp_world_size,
                                                         cp_rank, out, cap),
                 qo_indptr, kv_indptr, num_heads, num_workers, g_kv_indptr)


def rope_quant_cache(q_latent, q_pe, k_latent, k_pe, positions, cos_sin, kv_pool, slot_mapping,
                     *, rope_style: int = 0, num_heads_pad: int | None = None, q_scale=None,
                     kv_scale=None, q_out=None):
    """The step before the decode (mla_rope_quant_cache): returns q_out
    (T, num_heads_pad, 576) float8_e4m3fn and writes each token's new entry
    to kv_pool[slot_mapping[t]] (negative slots are skipped).

    q_latent (T, H, 512), q_pe (T, H, 64), k_latent (T, 512), k_pe (T, 64)
    bf16; positions / slot_mapping (T,) int32; cos_sin (max_pos, 64) fp32;
    kv_pool (N, 576) float8_e4m3fn; scales 0-d fp32 device tensors or None."""
    dev = q_latent.device
    if q_latent.dim() != 3 or q_latent.shape[2] != LATENT_DIM:
        raise ValueError("q_latent must be (T, H, 512)")
    T, H, _ = q_latent.shape
    Hp = H if num_heads_pad is None else int(num_heads_pad)
    _need(q_latent, "q_latent", dev, torch.bfloat16)
    _need(q_pe, "q_pe", dev, torch.bfloat16, (T, H, 64))
    _need(k_latent, "k_latent", dev, torch.bfloat16, (T, LATENT_DIM))
    _need(k_pe, "k_pe", dev, torch.bfloat16, (T, 64))
    _need(positions, "positions", dev, torch.int32, (T,))
    _need(slot_mapping, "slot_mapping", dev, torch.int32, (T,))
    _need(cos_sin, "cos_sin", dev, torch.float32)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin must be (max_pos, 64)")
    if kv_pool.dim() == 4:
        kv_pool = kv_pool.view(-1, ROW_DIM)
    _need(kv_pool, "kv_pool", dev, torch.float8_e4m3fn)
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError("kv_pool must be (N, 576)")
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None:
            _need(s, name, dev, torch.float32)
    if q_out is None:
        q_out = torch.empty((T, Hp, ROW_DIM), dtype=torch.float8_e4m3fn, device=dev)
    _need(q_out, "q_out", dev, torch.float8_e4m3fn, (T, Hp, ROW_DIM))
    status = _lib.lib().mla_rope_quant_cache(
        _ptr(q_latent), _ptr(q_pe), _ptr(k_latent), _ptr(k_pe), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], int(rope_style), _ptr(q_out), T, H, Hp, _ptr(kv_pool), kv_pool.shape[0],
        _ptr(slot_mapping), _ptr(q_scale), _ptr(kv_scale), _stream(dev))
    _lib.check(status, "mla_rope_quant_cache")
    return q_out


def latent_to_v(o_latent, w_uv, *, out=None):
    """The step after the decode (mla_latent_to_v): out (T, H, 128) bf16 with
    out[t, h] = o_latent[t, h] . w_uv[h]^T; o_latent (T, H_pad, 512) bf16 (the
    decode's o, pad heads unread), w_uv (H, 128, 512) bf16."""
    dev = o_latent.device
    if o_latent.dim() != 3 or o_latent.shape[2] != LATENT_DIM:
        raise ValueError("o_latent must be (T, H_pad, 512)")
    T, Hp, _ = o_latent.shape
    if w_uv.dim() != 3 or tuple(w_uv.shape[1:]) != (128, LATENT_DIM):
        raise ValueError("w_uv must be (H, 128, 512)")
    H = w_uv.shape[0]
    _need(o_latent, "o_latent", dev, torch.bfloat16)
    _need(w_uv, "w_uv", dev, torch.bfloat16)
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16, (T, H, 128))
    status = _lib.lib().mla_latent_to_v(_ptr(o_latent), _ptr(w_uv), _ptr(out), T, H, Hp,
                                        _stream(dev))
    _lib.check(status, "mla_latent_to_v")
    return out


def decode_step(q_latent, q_pe, k_latent, k_pe, positions, cos_sin, slot_mapping, kv_pool,
                qo_indptr, kv_indptr, kv_indices, sm_scale, w_uv, *, num_heads_pad: int,
                rope_style: int = 0, q_scale=None, kv_scale=None, return_lse: bool = False,
                o_latent=None, out=None, lse=None, max_seqlen_q: int | None = None,
                workspace=None):
    """One decode step of an MLA layer (mla_decode_step): the rope / fp8 /
    cache-write step, the decode and the latent -> v map in two launches.
    Returns out (T, H, 128) bf16, and o_latent (T, num_heads_pad, 512) bf16
    (and lse (T, num_heads_pad) if return_lse); kv_pool's new entries are
    written.  Arguments as for rope_quant_cache, decode (fp8 pool, page size 1)
    and latent_to_v; w_uv (H, 128, 512) bf16 gives the real head count."""
    dev = q_latent.device
    if q_latent.dim() != 3 or q_latent.shape[2] != LATENT_DIM:
        raise ValueError("q_latent must be (T, H, 512)")
    T, H, _ = q_latent.shape
    Hp = int(num_heads_pad)
    _need(q_latent, "q_latent", dev, torch.bfloat16)
    _need(q_pe, "q_pe", dev, torch.bfloat16, (T, H, 64))
    _need(k_latent, "k_latent", dev, torch.bfloat16, (T, LATENT_DIM))
    _need(k_pe, "k_pe", dev, torch.bfloat16, (T, 64))
    _need(positions, "positions", dev, torch.int32, (T,))
    _need(slot_mapping, "slot_mapping", dev, torch.int32, (T,))
    _need(cos_sin, "cos_sin", dev, torch.float32)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64:
        raise ValueError("cos_sin must be (max_pos, 64)")
    if kv_pool.dim() == 4:
        kv_pool = kv_pool.view(-1, ROW_DIM)
    _need(kv_pool, "kv_pool", dev, torch.float8_e4m3fn)
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_DIM:
        raise ValueError("kv_pool must be (N, 576)")
    B = qo_indptr.numel() - 1
    _need(qo_indptr, "qo_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indptr, "kv_indptr", dev, torch.int32, (B + 1,))
    _need(kv_indices, "kv_indices", dev, torch.int32)
    _need(w_uv, "w_uv", dev, torch.bfloat16, (H, 128, LATENT_DIM))
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None:
            _need(s, name, dev, torch.float32)
            if s.numel() != 1:
                raise ValueError(f"{name} must hold one value")
    if o_latent is None:
        o_latent = torch.empty((T, Hp, LATENT_DIM), dtype=torch.bfloat16, device=dev)
    _need(o_latent, "o_latent", dev, torch.bfloat16, (T, Hp, LATENT_DIM))
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16, (T, H, 128))
    if return_lse:
        if lse is None:
            lse = torch.empty((T, Hp), dtype=torch.float32, device=dev)
        _need(lse, "lse", dev, torch.float32, (T, Hp))
    if max_seqlen_q is None:
        max_seqlen_q = int((qo_indptr[1:] - qo_indptr[:-1]).max().item()) if B > 0 else 1
    if workspace is None:
        need = _lib.lib().mla_decode_step_workspace_bytes(B, T, Hp, int(max_seqlen_q))
        if need == 0:
            raise ValueError("unsupported decode_step shape")
        workspace = new_workspace(need, dev)
    _need(workspace, "workspace", dev)
    ws_len = workspace.numel() * workspace.element_size()
    status = _lib.lib().mla_decode_step(
        _ptr(q_latent), _ptr(q_pe), _ptr(k_latent), _ptr(k_pe), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], int(rope_style), _ptr(slot_mapping), _ptr(kv_pool), kv_pool.shape[0],
        _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices), kv_indices.numel(), B, T, H, Hp,
        int(max_seqlen_q), float(sm_scale), _ptr(q_scale), _ptr(kv_scale), _ptr(w_uv),
        _ptr(o_latent), _ptr(out), 1 if return_lse else 0, _ptr(lse) if return_lse else None,
        _ptr(workspace), ws_len, _stream(dev))
    _lib.check(status, "mla_decode_step")
    if return_lse:
        return out, o_latent, lse
    return out, o_latent
