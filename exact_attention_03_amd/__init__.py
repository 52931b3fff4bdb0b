"""Exact attention (FlashAttention) forward and backward on AMD MI355X.

Thin binding over the C ABI of ``libfa.so`` (see ``include/fa.h``): it checks
tensors, allocates outputs with torch and passes raw device pointers plus the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; nothing here computes attention.

The operations follow the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV
Pipeline 优化实战" (BiumBiu): §一 for the forward, §二 for the backward.
``forward`` and ``backward`` also take fewer key/value heads than query heads
(grouped-query attention, the page "从算子到 Serving：昇腾推理评测链路实践",
section "GQA Paged Attention"): k and v of shape (Z, Hkv, N, D) with H a whole
multiple of Hkv; query head h uses key/value head h // (H // Hkv).
``forward_varlen`` / ``backward_varlen`` take packed batches of sequences of
different lengths; ``reshape_and_cache`` / ``paged_decode`` work on a paged KV
cache, and ``quest_page_minmax`` / ``quest_select`` / ``paged_decode_sparse``
decode over query-selected pages (the same page, sections "ReshapeAndCache",
"GQA Paged Attention" and "Quest Sparse Attention"); ``paged_decode_sources``
decodes over one or two KV sources under one softmax (the page "在 4 张 A100 上
部署 DeepSeek-V4-Flash-0731", section 7.5).  ``attention`` is the
forward with its backward registered for torch autograd.
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FAError, check, last_error, lib,  # noqa: F401
                   status_name)

__all__ = ["attention", "forward", "backward", "backward_noalloc", "forward_varlen", "backward_varlen", "reshape_and_cache", "paged_decode",
           "quest_page_minmax", "quest_select", "paged_decode_sparse", "paged_decode_sources",
           "paged_attention_sources",
           "bwd_preprocess", "bwd_dkdv", "bwd_dq", "bwd_dq_and_stats", "bwd_fused", "workspace_bytes",
           "device_info", "dkdv_schedule", "fwd_tile_pairs", "FAError", "lib"]


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    codes = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_F32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkv(*ts, names):
    ref = ts[0]
    for t, n in zip(ts, names):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{n} must be (Z, H, N, D), got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if t.shape != ref.shape:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
        if t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, expected {ref.device}")


def _check_kv_group(q, k, v, names=("k", "v")):
    """k, v: (Z, Hkv, N, D) with the batch, length and head dim of q and H a
    whole multiple of Hkv.  Returns Hkv."""
    for t, n in zip((k, v), names):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{n} must be (Z, Hkv, N, D), got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if t.device != q.device:
            raise ValueError(f"{n} is on {t.device}, expected {q.device}")
    if k.shape != v.shape:
        raise ValueError(f"{names[0]} {tuple(k.shape)} and {names[1]} {tuple(v.shape)} differ")
    Z, H, N, D = q.shape
    Hkv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (Z, N, D) or Hkv == 0 or H % Hkv != 0:
        raise ValueError(f"{names[0]} has shape {tuple(k.shape)}; expected (Z, Hkv, N, D) = ({Z}, Hkv, {N}, {D}) "
                         f"with {H} query heads a whole multiple of Hkv")
    return Hkv


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _scale(scale, D):
    return float(1.0 / math.sqrt(D)) if scale is None else float(scale)


def forward(q, k, v, causal=False, scale=None, out_dtype=None):
    """O, lse = attention(q, k, v).  q: (Z, H, N, D), k, v: (Z, H, N, D) or
    grouped (Z, Hkv, N, D); fp16/bf16 GPU tensors.

    out_dtype: dtype of O, either q.dtype (default) or torch.float32.
    Returns O (Z, H, N, D) and lse (Z, H, N) float32 (natural log).
    """
    torch = _torch()
    _check_qkv(q, names=("q",))
    Hkv = _check_kv_group(q, k, v)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    Z, H, N, D = q.shape
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((Z, H, N, D), dtype=odt, device=q.device)
        lse = torch.empty((Z, H, N), dtype=torch.float32, device=q.device)
        if Hkv == H:
            st = lib().fa_fwd(Z, H, N, D, _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(lse), _scale(scale, D), int(bool(causal)), _stream(q))
        else:
            st = lib().fa_fwd_gqa(Z, H, Hkv, N, D, _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(o), _ptr(lse), _scale(scale, D), int(bool(causal)), _stream(q))
    check(st, "fa_fwd" if Hkv == H else "fa_fwd_gqa")
    return o, lse


def workspace_bytes(Z, H, N, D):
    return int(lib().fa_bwd_workspace_bytes(Z, H, N, D))


def backward(q, k, v, o, do, lse, causal=False, scale=None, workspace=None):
    """dq, dk, dv of attention given dO; o and lse from ``forward``.  k and v
    may be grouped (Z, Hkv, N, D); dk and dv then have that shape.

    workspace: optional float32 GPU tensor of >= 2*Z*H*N elements (the row
    statistics); one is allocated when omitted.
    """
    torch = _torch()
    _check_qkv(q, do, o, names=("q", "do", "o"))
    Hkv = _check_kv_group(q, k, v)
    if k.dtype != q.dtype or v.dtype != q.dtype or do.dtype != q.dtype:
        raise TypeError("q, k, v, do must share one dtype")
    Z, H, N, D = q.shape
    if lse.shape != (Z, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (Z, H, N) tensor")
    with torch.cuda.device(q.device):
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        if workspace is None:
            nbytes = lib().fa_bwd_workspace_bytes(Z, H, N, D)
            workspace = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        if workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous float32 GPU tensor")
        common = (_dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                  _ptr(dq), _ptr(dk), _ptr(dv), _scale(scale, D), int(bool(causal)), _ptr(workspace),
                  workspace.numel() * 4, _stream(q))
        if Hkv == H:
            st = lib().fa_bwd(Z, H, N, D, *common)
        else:
            st = lib().fa_bwd_gqa(Z, H, Hkv, N, D, *common)
    check(st, "fa_bwd" if Hkv == H else "fa_bwd_gqa")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, causal=False, scale=None):
    """``backward`` through fa_bwd_noalloc: the row statistics live in the
    library's fixed device array instead of a workspace (plain heads only;
    Z*H*N <= 2^22).  Only the outputs dq, dk, dv are allocated here."""
    torch = _torch()
    _check_qkv(q, k, v, do, o, names=("q", "k", "v", "do", "o"))
    if k.dtype != q.dtype or v.dtype != q.dtype or do.dtype != q.dtype:
        raise TypeError("q, k, v, do must share one dtype")
    Z, H, N, D = q.shape
    if lse.shape != (Z, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 (Z, H, N) tensor on q's device")
    with torch.cuda.device(q.device):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        st = lib().fa_bwd_noalloc(Z, H, N, D, _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _scale(scale, D),
                                  int(bool(causal)), _stream(q))
    check(st, "fa_bwd_noalloc")
    return dq, dk, dv


def _check_varlen(q, k, v, cu_seqlens, max_seqlen):
    """q: (H, T, D); k, v: (Hkv, T, D); cu_seqlens: int32 GPU tensor (B+1,).
    Returns (B, H, Hkv, T, D, max_seqlen)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 3-d GPU tensor, packed (heads, tokens, D)")
        if t.device != q.device:
            raise ValueError(f"{n} is on {t.device}, expected {q.device}")
    H, T, D = q.shape
    Hkv = k.shape[0]
    if k.shape != v.shape or k.shape[1:] != (T, D) or Hkv == 0 or H % Hkv != 0:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} must be (Hkv, {T}, {D}) with {H} a multiple of Hkv")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if (not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 1 or cu_seqlens.device != q.device):
        raise ValueError("cu_seqlens must be a contiguous int32 GPU tensor of B+1 token offsets")
    B = cu_seqlens.numel() - 1
    if max_seqlen is None:
        # One host read of the offsets (a synchronisation); pass max_seqlen to avoid it.
        lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu()
        max_seqlen = int(lens.max()) if B > 0 else 0
    return B, H, Hkv, T, D, int(max_seqlen)


def forward_varlen(q, k, v, cu_seqlens, max_seqlen=None, causal=False, scale=None, out_dtype=None):
    """Attention over a packed batch of variable-length sequences.

    q: (H, T, D); k, v: (Hkv, T, D) (H a multiple of Hkv); sequence b is
    tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head and attends only
    within itself.  max_seqlen: at least the longest sequence (read from
    cu_seqlens when omitted; a smaller value leaves some tiles of the longer
    sequences uncomputed, with unspecified results).  Returns O (H, T, D) and
    lse (H, T).
    """
    torch = _torch()
    B, H, Hkv, T, D, mx = _check_varlen(q, k, v, cu_seqlens, max_seqlen)
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((H, T, D), dtype=odt, device=q.device)
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
        st = lib().fa_fwd_varlen(B, H, Hkv, T, mx, D, _dtype_code(q), _dtype_code(o), _ptr(cu_seqlens), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _scale(scale, D), int(bool(causal)),
                                 _stream(q))
    check(st, "fa_fwd_varlen")
    return o, lse


def backward_varlen(q, k, v, o, do, lse, cu_seqlens, max_seqlen=None, causal=False, scale=None):
    """dq (H, T, D), dk, dv (Hkv, T, D) of ``forward_varlen`` given dO."""
    torch = _torch()
    B, H, Hkv, T, D, mx = _check_varlen(q, k, v, cu_seqlens, max_seqlen)
    for t, n in ((o, "o"), (do, "do")):
        if not t.is_cuda or t.shape != q.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{n} must be a contiguous GPU tensor of shape {tuple(q.shape)}")
    if do.dtype != q.dtype:
        raise TypeError("do must have q's dtype")
    if lse.shape != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (H, T) tensor")
    with torch.cuda.device(q.device):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nbytes = lib().fa_bwd_workspace_bytes(1, H, T, D)
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        st = lib().fa_bwd_varlen(B, H, Hkv, T, mx, D, _dtype_code(q), _dtype_code(o), _ptr(cu_seqlens), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _scale(scale, D), int(bool(causal)), _ptr(ws), ws.numel() * 4, _stream(q))
    check(st, "fa_bwd_varlen")
    return dq, dk, dv


def reshape_and_cache(key, value, slot_mapping, k_cache, v_cache):
    """Write new tokens into a paged cache, in place.

    key, value: (num_tokens, Hkv, D); slot_mapping: int64 GPU tensor
    (num_tokens,), negative = skip; k_cache: (num_blocks, Hkv, D/8, block_size, 8)
    (keys in chunks of 8 channels, chunk-major), v_cache: (num_blocks, Hkv, D,
    block_size) (values transposed), both of key's dtype.
    """
    torch = _torch()
    T, Hkv, D = key.shape
    nb, bs = k_cache.shape[0], k_cache.shape[3]
    for t, n, shp in ((key, "key", (T, Hkv, D)), (value, "value", (T, Hkv, D)),
                      (k_cache, "k_cache", (nb, Hkv, D // 8, bs, 8)), (v_cache, "v_cache", (nb, Hkv, D, bs))):
        if (not t.is_cuda or tuple(t.shape) != shp or not t.is_contiguous() or t.dtype != key.dtype
                or t.device != key.device):
            raise ValueError(f"{n} must be a contiguous GPU tensor of shape {shp}, dtype {key.dtype} and on "
                             f"{key.device}")
    # The kernel reads slot i at element i: a strided view would map tokens to the wrong slots.
    if (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,) or not slot_mapping.is_cuda
            or not slot_mapping.is_contiguous() or slot_mapping.device != key.device):
        raise ValueError(f"slot_mapping must be a contiguous int64 GPU tensor of shape (num_tokens,) on {key.device}")
    with torch.cuda.device(key.device):
        st = lib().fa_reshape_and_cache(T, Hkv, D, bs, nb, _dtype_code(key), _ptr(key), _ptr(value),
                                        _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _stream(key))
    check(st, "fa_reshape_and_cache")


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len=None, scale=None,
                 out_dtype=None):
    """Decode attention over a paged cache: (O (B, H, D), lse (B, H)).

    q: (B, H, D); caches as for ``reshape_and_cache``; block_tables: int32
    (B, max_blocks); context_lens: int32 (B,).  max_context_len (host int)
    sizes the split of long contexts; read from context_lens when omitted.
    """
    torch = _torch()
    B, H, D = q.shape
    if k_cache.dim() != 5:
        raise ValueError("k_cache must be (num_blocks, Hkv, D/8, block_size, 8)")
    nb, Hkv, _, bs, _ = k_cache.shape
    if k_cache.shape != (nb, Hkv, D // 8, bs, 8) or v_cache.shape != (nb, Hkv, D, bs):
        raise ValueError("caches must be (num_blocks, Hkv, D/8, block_size, 8) and (num_blocks, Hkv, D, block_size)")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{n} must be a contiguous GPU tensor of q's dtype and device")
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be (B, max_blocks) and context_lens (B,)")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B > 0 else 0
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((B, H, D), dtype=odt, device=q.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
        nbytes = lib().fa_paged_decode_workspace_bytes(B, H, Hkv, D, int(max_context_len))
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        st = lib().fa_paged_decode(B, H, Hkv, D, bs, nb, block_tables.shape[1], int(max_context_len), _dtype_code(q),
                                   _dtype_code(o), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(context_lens), _ptr(o), _ptr(lse), _scale(scale, D), _ptr(ws), nbytes,
                                   _stream(q))
    check(st, "fa_paged_decode")
    return o, lse


def _check_paged(q, k_cache, v_cache, block_tables, context_lens, q_view=False):
    """Shapes of a paged call; q_view: q is a (B, H, D) view of a larger query
    tensor whose layout the caller checks (only its device and dtype here)."""
    torch = _torch()
    B, H, D = q.shape
    if k_cache.dim() != 5:
        raise ValueError("k_cache must be (num_blocks, Hkv, D/8, block_size, 8)")
    nb, Hkv, _, bs, _ = k_cache.shape
    if k_cache.shape != (nb, Hkv, D // 8, bs, 8) or (v_cache is not None and v_cache.shape != (nb, Hkv, D, bs)):
        raise ValueError("caches must be (num_blocks, Hkv, D/8, block_size, 8) and (num_blocks, Hkv, D, block_size)")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        contiguous = t is None or t.is_contiguous() or (q_view and t is q)
        if t is not None and (not t.is_cuda or not contiguous or t.dtype != q.dtype or t.device != q.device):
            raise ValueError(f"{n} must be a contiguous GPU tensor of q's dtype and device")
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be (B, max_blocks) and context_lens (B,)")
    return B, H, Hkv, D, bs, nb, block_tables.shape[1]


def quest_page_minmax(k_cache, block_tables, context_lens):
    """Page key minimum / maximum (num_blocks, Hkv, 2, D) over each context's valid tokens."""
    torch = _torch()
    nb, Hkv, nc, bs, x = k_cache.shape
    D = nc * x
    B = block_tables.shape[0]
    q_dummy = torch.empty((B, Hkv, D), dtype=k_cache.dtype, device=k_cache.device)
    _check_paged(q_dummy, k_cache, None, block_tables, context_lens)
    with torch.cuda.device(k_cache.device):
        kmeta = torch.zeros((nb, Hkv, 2, D), dtype=k_cache.dtype, device=k_cache.device)
        st = lib().fa_quest_page_minmax(B, Hkv, D, bs, nb, block_tables.shape[1], _dtype_code(k_cache), _ptr(k_cache),
                                        _ptr(block_tables), _ptr(context_lens), _ptr(kmeta), _stream(k_cache))
    check(st, "fa_quest_page_minmax")
    return kmeta


def quest_select(q, kmeta, k_cache, block_tables, context_lens, topk):
    """Kept pages (B, Hkv, topk) int32 (ascending; -1 past the count) and their count (B, Hkv)."""
    torch = _torch()
    B, H, Hkv, D, bs, nb, mxb = _check_paged(q, k_cache, None, block_tables, context_lens)
    if kmeta.shape != (nb, Hkv, 2, D) or kmeta.dtype != q.dtype or not kmeta.is_contiguous():
        raise ValueError("kmeta must be the (num_blocks, Hkv, 2, D) output of quest_page_minmax")
    with torch.cuda.device(q.device):
        sel = torch.full((B, Hkv, topk), -1, dtype=torch.int32, device=q.device)
        nsel = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
        st = lib().fa_quest_select(B, H, Hkv, D, bs, nb, mxb, topk, _dtype_code(q), _ptr(q), _ptr(kmeta),
                                   _ptr(block_tables), _ptr(context_lens), _ptr(sel), _ptr(nsel), _stream(q))
    check(st, "fa_quest_select")
    return sel, nsel


def paged_decode_sparse(q, k_cache, v_cache, block_tables, context_lens, selected, n_selected, scale=None,
                        out_dtype=None):
    """Decode attention over the tokens of the kept pages: (O (B, H, D), lse (B, H))."""
    torch = _torch()
    B, H, Hkv, D, bs, nb, mxb = _check_paged(q, k_cache, v_cache, block_tables, context_lens)
    topk = selected.shape[2]
    if selected.shape != (B, Hkv, topk) or n_selected.shape != (B, Hkv) or selected.dtype != torch.int32 \
            or n_selected.dtype != torch.int32:
        raise ValueError("selected must be int32 (B, Hkv, topk) and n_selected int32 (B, Hkv)")
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((B, H, D), dtype=odt, device=q.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
        nbytes = lib().fa_paged_decode_workspace_bytes(B, H, Hkv, D, topk * bs)
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        st = lib().fa_paged_decode_sparse(B, H, Hkv, D, bs, nb, mxb, topk, _dtype_code(q), _dtype_code(o), _ptr(q),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                                          _ptr(selected), _ptr(n_selected), _ptr(o), _ptr(lse), _scale(scale, D),
                                          _ptr(ws), nbytes, _stream(q))
    check(st, "fa_paged_decode_sparse")
    return o, lse


def _source_records(q3, sources, Tq=1):
    """fa_kv_source records of one or two source dicts for a query of shape
    (B, H, D) (one row per sequence) with Tq rows per sequence; returns
    (ctypes array, Hkv)."""
    from . import _lib

    torch = _torch()
    if not 1 <= len(sources) <= 2:
        raise ValueError("one or two sources")
    B = q3.shape[0]
    recs, Hkv0 = [], None
    for src in sources:
        kc, vc, bt, cl = src["k_cache"], src["v_cache"], src["block_tables"], src["context_lens"]
        _, _, Hkv, _, bs, nb, mxb = _check_paged(q3, kc, vc, bt, cl, q_view=Tq != 1)
        if Hkv0 is not None and Hkv != Hkv0:
            raise ValueError("every source must have the same number of key/value heads")
        Hkv0 = Hkv
        sel, nsel, rows = src.get("selected"), src.get("n_selected"), src.get("row_lens")
        topk = 0
        if nsel is not None:
            if sel is None or sel.dim() != 3:
                raise ValueError("a sparse source needs selected (B, Hkv, topk) with n_selected")
            topk = sel.shape[2]
            if sel.shape != (B, Hkv, topk) or nsel.shape != (B, Hkv) or sel.dtype != torch.int32 \
                    or nsel.dtype != torch.int32 or not sel.is_cuda or not nsel.is_cuda \
                    or not sel.is_contiguous() or not nsel.is_contiguous():
                raise ValueError("selected must be int32 (B, Hkv, topk) and n_selected int32 (B, Hkv), on the GPU")
        elif sel is not None:
            raise ValueError("selected given without n_selected")
        if rows is not None and (rows.shape != (B, Tq) or rows.dtype != torch.int32 or not rows.is_cuda
                                 or not rows.is_contiguous()):
            raise ValueError("row_lens must be a contiguous int32 (B, Tq) GPU tensor")
        mcl = src.get("max_context_len")
        if mcl is None:
            mcl = int(cl.max().item()) if (B > 0 and nsel is None) else 0
        recs.append(_lib.KvSource(_ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl), bs, nb, mxb, int(mcl),
                                  _ptr(sel) if (nsel is not None and topk > 0) else None,
                                  _ptr(nsel) if nsel is not None else None, topk,
                                  _ptr(rows) if rows is not None else None))
    return (_lib.KvSource * len(recs))(*recs), Hkv0


def paged_decode_sources(q, sources, scale=None, out_dtype=None):
    """Decode attention over one or two KV sources under one softmax:
    (O (B, H, D), lse (B, H)).

    Each source is a dict with k_cache, v_cache (layouts as for
    ``reshape_and_cache``), block_tables (int32 (B, max_blocks)),
    context_lens (int32 (B,)) and optionally selected / n_selected (int32
    (B, Hkv, topk) / (B, Hkv), as from ``quest_select``: only the kept pages
    take part) and max_context_len (host int sizing a dense source's split;
    read from context_lens when omitted).  The sources' tokens form one set:
    one maximum and one denominator per query head.
    """
    torch = _torch()
    B, H, D = q.shape
    arr, Hkv = _source_records(q, sources)
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((B, H, D), dtype=odt, device=q.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
        nbytes = lib().fa_paged_decode_sources_workspace_bytes(B, H, Hkv, D, len(arr), arr)
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        st = lib().fa_paged_decode_sources(B, H, Hkv, D, _dtype_code(q), _dtype_code(o), _ptr(q), len(arr), arr,
                                           _ptr(o), _ptr(lse), _scale(scale, D), _ptr(ws), nbytes, _stream(q))
    check(st, "fa_paged_decode_sources")
    return o, lse


def paged_attention_sources(q, sources, scale=None, out_dtype=None):
    """Attention of Tq query tokens per sequence over one or two KV sources
    under one softmax: (O (B, Tq, H, D), lse (B, Tq, H)).

    q: (B, Tq, H, D).  Sources as for ``paged_decode_sources``, each with an
    optional row_lens (int32 (B, Tq)): how many of the source's tokens query
    token t sees (n - Tq + t + 1 for a causal chunk at the end of a context of
    n cached tokens); all of them when omitted.
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be (B, Tq, H, D)")
    B, Tq, H, D = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    arr, Hkv = _source_records(q[:, 0], sources, Tq)
    odt = q.dtype if out_dtype is None else out_dtype
    with torch.cuda.device(q.device):
        o = torch.empty((B, Tq, H, D), dtype=odt, device=q.device)
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
        nbytes = lib().fa_paged_attention_sources_workspace_bytes(B, Tq, H, Hkv, D, len(arr), arr)
        ws = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        st = lib().fa_paged_attention_sources(B, Tq, H, Hkv, D, _dtype_code(q), _dtype_code(o), _ptr(q), len(arr),
                                              arr, _ptr(o), _ptr(lse), _scale(scale, D), _ptr(ws), nbytes,
                                              _stream(q))
    check(st, "fa_paged_attention_sources")
    return o, lse


def bwd_preprocess(o, do, lse):
    """Backward row statistics, float32 (2, Z, H, N): [0] = Delta = rowsum(O * dO),
    [1] = lse * log2(e)."""
    torch = _torch()
    _check_qkv(do, o, names=("do", "o"))
    Z, H, N, D = do.shape
    if lse.shape != (Z, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (Z, H, N) tensor")
    with torch.cuda.device(do.device):
        stats = torch.empty((2, Z, H, N), dtype=torch.float32, device=do.device)
        st = lib().fa_bwd_preprocess(Z, H, N, D, _dtype_code(do), _dtype_code(o), _ptr(o), _ptr(do),
                                     _ptr(lse), _ptr(stats), _stream(do))
    check(st, "fa_bwd_preprocess")
    return stats


def bwd_dkdv(q, k, v, do, stats, causal=False, scale=None, num_programs=0):
    """dK, dV from the persistent key-tile pass (num_programs 0 = device default)."""
    torch = _torch()
    _check_qkv(q, k, v, do, names=("q", "k", "v", "do"))
    Z, H, N, D = q.shape
    with torch.cuda.device(q.device):
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        _check_stats(stats, Z, H, N)
        st = lib().fa_bwd_dkdv(Z, H, N, D, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(stats),
                               _ptr(dk), _ptr(dv), _scale(scale, D), int(bool(causal)), int(num_programs),
                               _stream(q))
    check(st, "fa_bwd_dkdv")
    return dk, dv


def bwd_fused(q, k, v, do, stats, causal=False, scale=None, num_programs=0, workspace=None):
    """dQ, dK, dV from the fused per-head pass (fa_bwd_fused); stats from
    ``bwd_preprocess``.  workspace: optional float32 GPU tensor of at least
    fa_bwd_fused_workspace_bytes / 4 elements (the heads' dQ partials)."""
    torch = _torch()
    _check_qkv(q, k, v, do, names=("q", "k", "v", "do"))
    Z, H, N, D = q.shape
    with torch.cuda.device(q.device):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        _check_stats(stats, Z, H, N)
        nbytes = int(lib().fa_bwd_fused_workspace_bytes(Z, H, N, D))
        if workspace is None:
            workspace = torch.empty((max(1, nbytes // 4),), dtype=torch.float32, device=q.device)
        if (workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous()
                or workspace.device != q.device):
            raise ValueError("workspace must be a contiguous float32 GPU tensor on q's device")
        st = lib().fa_bwd_fused(Z, H, N, D, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(stats),
                                _ptr(dq), _ptr(dk), _ptr(dv), _scale(scale, D), int(bool(causal)), int(num_programs),
                                _ptr(workspace), workspace.numel() * 4, _stream(q))
    check(st, "fa_bwd_fused")
    return dq, dk, dv


def bwd_dq(q, k, v, do, stats, causal=False, scale=None):
    """dQ from the query-tile pass."""
    torch = _torch()
    _check_qkv(q, k, v, do, names=("q", "k", "v", "do"))
    Z, H, N, D = q.shape
    with torch.cuda.device(q.device):
        dq = torch.empty_like(q)
        _check_stats(stats, Z, H, N)
        st = lib().fa_bwd_dq(Z, H, N, D, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(stats),
                             _ptr(dq), _scale(scale, D), int(bool(causal)), _stream(q))
    check(st, "fa_bwd_dq")
    return dq


def bwd_dq_and_stats(q, k, v, o, do, lse, causal=False, scale=None):
    """dQ and the backward row statistics from one pass: (dq, stats)."""
    torch = _torch()
    _check_qkv(q, k, v, do, names=("q", "k", "v", "do"))
    Z, H, N, D = q.shape
    if lse.shape != (Z, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (Z, H, N) tensor")
    with torch.cuda.device(q.device):
        dq = torch.empty_like(q)
        stats = torch.empty((2, Z, H, N), dtype=torch.float32, device=q.device)
        st = lib().fa_bwd_dq_and_stats(Z, H, N, D, _dtype_code(q), _dtype_code(o), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(o), _ptr(do), _ptr(lse), _ptr(stats), _ptr(dq), _scale(scale, D),
                                       int(bool(causal)), _stream(q))
    check(st, "fa_bwd_dq_and_stats")
    return dq, stats


def _check_stats(stats, Z, H, N):
    torch = _torch()
    if stats.shape != (2, Z, H, N) or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be the contiguous float32 (2, Z, H, N) output of bwd_preprocess")


def device_info(D=128, dtype_code=FA_DTYPE_F16):
    """(compute units, default dK/dV persistent grid) of the current device."""
    cus, progs = ctypes.c_int(0), ctypes.c_int(0)
    check(lib().fa_device_info(D, dtype_code, ctypes.byref(cus), ctypes.byref(progs)), "fa_device_info")
    return cus.value, progs.value


def dkdv_schedule(Z, H, N, D, causal, num_programs):
    """Host-only replay of the dK/dV schedule: (units per program, query tiles per program, unit count)."""
    units = (ctypes.c_int64 * num_programs)()
    work = (ctypes.c_int64 * num_programs)()
    n = ctypes.c_int64(0)
    check(lib().fa_dkdv_schedule(Z, H, N, D, int(bool(causal)), num_programs, units, work, ctypes.byref(n)),
          "fa_dkdv_schedule")
    return list(units), list(work), n.value


def fwd_tile_pairs(N, D, causal):
    """Host-only: (query tile, key tile) pairs the forward visits, and the total."""
    vis, tot = ctypes.c_int64(0), ctypes.c_int64(0)
    check(lib().fa_fwd_tile_pairs(N, D, int(bool(causal)), ctypes.byref(vis), ctypes.byref(tot)),
          "fa_fwd_tile_pairs")
    return vis.value, tot.value


class _Attention:
    """torch.autograd.Function for ``attention`` (built on first use, so that
    importing the package does not import torch)."""

    fn = None

    @classmethod
    def get(cls):
        if cls.fn is None:
            torch = _torch()

            class AttentionFunction(torch.autograd.Function):
                @staticmethod
                def forward(ctx, q, k, v, causal, scale):
                    o, lse = forward(q, k, v, causal=causal, scale=scale)
                    ctx.save_for_backward(q, k, v, o, lse)
                    ctx.causal, ctx.scale = causal, scale
                    return o

                @staticmethod
                def backward(ctx, do):
                    q, k, v, o, lse = ctx.saved_tensors
                    dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, causal=ctx.causal, scale=ctx.scale)
                    return dq, dk, dv, None, None

            cls.fn = AttentionFunction
        return cls.fn


def attention(q, k, v, causal=False, scale=None):
    """O = softmax(Q K^T * scale) V with autograd: the forward here, the
    backward (dq, dk, dv) in the library's backward kernels.  Shapes and dtypes
    as for ``forward`` (grouped key/value heads included)."""
    return _Attention.get().apply(q, k, v, bool(causal), scale)
