"""Plain fp64 attention, written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [FA-Ascend] is the page
"把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline 优化实战" (BiumBiu).

The method on that page (tiles, online softmax, recomputation) reaches exactly
this result up to rounding order, so the oracle is the definition itself: it
materialises the full N x N score and probability matrices, which is precisely
what the tiled method avoids.  The only library primitives used are matrix
products, exp, log and reductions.

Readings of points the page leaves open:

* layout: q, k, v, do are (..., N, D) arrays; leading axes are independent heads;
* self-attention with one key/value head per query head, N_q = N_k = N;
* causal means key j is visible to query i iff j <= i (the lower triangle
  including the diagonal, [FA-Ascend] §八);
* the saved row statistic is the natural-log log-sum-exp lse = m + ln(l)
  (the page's backward "recomputes" the softmax, [FA-Ascend] §二, which needs a
  saved row statistic; the page never names it);
* Delta uses the oracle's own fp64 O.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_forward", "attention_forward_full", "attention_backward", "loss_sum_o_do",
           "gqa_kv_head", "attention_forward_gqa", "attention_backward_gqa", "attention_forward_varlen",
           "attention_backward_varlen"]


def _as_f64(x):
    x = np.asarray(x)
    if x.dtype != np.float64:
        x = x.astype(np.float64)
    return x


def _scores(q, k, scale, causal):
    """S = Q @ K^T * scale, with the causal upper triangle set to -inf.

    [FA-Ascend] §一 (first forward equation) and §八 (causal: the upper
    triangle takes no part).
    """
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    if causal:
        n_q, n_k = s.shape[-2], s.shape[-1]
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        s = np.where(j <= i, s, -np.inf)
    return s


def attention_forward_full(q, k, v, scale, causal=False):
    """Forward pass returning every intermediate: dict(S, P, O, lse, m, l).

    [FA-Ascend] §一: S = Q @ K^T * scale; P = softmax(S) row-wise; O = P @ V.
    The softmax is the textbook one: subtract the row max m, exponentiate,
    divide by the row sum l.  lse = m + ln(l).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    scale = float(scale)
    S = _scores(q, k, scale, causal)
    m = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = np.sum(E, axis=-1, keepdims=True)
    P = E / l
    O = np.matmul(P, v)
    lse = (m + np.log(l))[..., 0]
    return {"S": S, "P": P, "O": O, "lse": lse, "m": m[..., 0], "l": l[..., 0]}


def attention_forward(q, k, v, scale, causal=False):
    """(O, lse) of the forward pass; see ``attention_forward_full``."""
    r = attention_forward_full(q, k, v, scale, causal)
    return r["O"], r["lse"]


def attention_backward(q, k, v, do, scale, causal=False):
    """Backward pass, taken literally from [FA-Ascend] §二:

        Delta = rowsum(O * dO)
        P     = softmax(Q @ K^T * scale)          (recomputed)
        dP    = dO @ V^T
        dS    = scale * P * (dP - Delta)
        dQ    = dS @ K
        dK    = dS^T @ Q
        dV    = P^T @ dO

    The page writes the three gradients as accumulations ("+=") over tiles;
    over the whole matrix they are the plain products above.  Returns a dict
    with dq, dk, dv and the intermediates O, lse, P, dP, dS, Delta.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    scale = float(scale)
    fwd = attention_forward_full(q, k, v, scale, causal)
    O, P = fwd["O"], fwd["P"]
    Delta = np.sum(O * do, axis=-1)
    dP = np.matmul(do, np.swapaxes(v, -1, -2))
    dS = scale * P * (dP - Delta[..., None])
    dq = np.matmul(dS, k)
    dk = np.matmul(np.swapaxes(dS, -1, -2), q)
    dv = np.matmul(np.swapaxes(P, -1, -2), do)
    return {"dq": dq, "dk": dk, "dv": dv, "O": O, "lse": fwd["lse"], "P": P,
            "dP": dP, "dS": dS, "Delta": Delta}


def loss_sum_o_do(q, k, v, do, scale, causal=False):
    """L = sum(O * dO) with dO held fixed: its gradient w.r.t. (Q, K, V) is the
    backward pass above, which the finite-difference pin uses."""
    O, _ = attention_forward(q, k, v, scale, causal)
    return float(np.sum(O * _as_f64(do)))


# ---------------------------------------------------------------- grouped KV heads
# [Serving-Ascend] = the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu),
# section "GQA Paged Attention": the number of query heads is an integer
# multiple of the number of key/value heads, and consecutive query heads share
# one key/value head (grouped-query attention; one KV head for all query
# heads is the multi-query case).  Reading of the grouping: with
# G = Hq / Hkv, query head h uses key/value head h // G, the usual contiguous
# grouping.


def gqa_kv_head(h, n_q_heads, n_kv_heads):
    """Key/value head used by query head h: h // (Hq / Hkv)."""
    if n_kv_heads <= 0 or n_q_heads % n_kv_heads != 0:
        raise ValueError("query heads must be a whole multiple of key/value heads")
    return h // (n_q_heads // n_kv_heads)


def attention_forward_gqa(q, k, v, scale, causal=False):
    """(O, lse) with grouped key/value heads.

    q: (Z, Hq, N, D); k, v: (Z, Hkv, N, D).  Each query head is the plain
    forward pass of [FA-Ascend] §一 against the key/value head it shares
    ([Serving-Ascend], "GQA Paged Attention"); O is (Z, Hq, N, D), lse
    (Z, Hq, N).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Z, Hq, N, D = q.shape
    Hkv = k.shape[1]
    O = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    for z in range(Z):
        for h in range(Hq):
            g = gqa_kv_head(h, Hq, Hkv)
            O[z, h], lse[z, h] = attention_forward(q[z, h], k[z, g], v[z, g], scale, causal)
    return O, lse


def attention_backward_gqa(q, k, v, do, scale, causal=False):
    """Backward pass with grouped key/value heads: (dq, dk, dv).

    Each query head's gradients are those of [FA-Ascend] §二 against its
    key/value head; a key/value head's dK and dV are the sums of the
    contributions of all query heads that share it (the shared K and V enter
    each of those heads' scores and outputs).  dq is (Z, Hq, N, D); dk, dv are
    (Z, Hkv, N, D).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    Z, Hq, N, D = q.shape
    Hkv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for z in range(Z):
        for h in range(Hq):
            g = gqa_kv_head(h, Hq, Hkv)
            r = attention_backward(q[z, h], k[z, g], v[z, g], do[z, h], scale, causal)
            dq[z, h] = r["dq"]
            dk[z, g] += r["dk"]
            dv[z, g] += r["dv"]
    return dq, dk, dv


# ---------------------------------------------------------------- variable-length batches
# [Serving-Ascend], sections "GQA Paged Attention" and the integration
# discussion before it: a batch holds sequences of different real lengths
# (context_lens), and tokens past a sequence's length take no part.  Reading:
# the sequences of a batch are packed one after the
# other along the token axis, sequence b occupying tokens cu_seqlens[b] ..
# cu_seqlens[b+1]-1 of every head (head-major packed layout: q is (H, T, D),
# k and v are (Hkv, T, D), T = cu_seqlens[-1]); each sequence is an
# independent self-attention problem of its own length, causal within itself
# when causal is set, and query heads share key/value heads as above.


def _check_cu_seqlens(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at the token count")
    return cu


def attention_forward_varlen(q, k, v, cu_seqlens, scale, causal=False):
    """(O, lse) of a packed variable-length batch.

    q: (H, T, D); k, v: (Hkv, T, D); cu_seqlens: (B+1,) token offsets.  Each
    sequence's tokens attend only to that sequence's tokens
    ([Serving-Ascend], context_lens); per sequence this is the grouped forward
    above.  O is (H, T, D), lse (H, T).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cu = _check_cu_seqlens(cu_seqlens, q.shape[1])
    O = np.zeros_like(q)
    lse = np.zeros(q.shape[:2])
    for b in range(cu.size - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        Ob, lb = attention_forward_gqa(q[None, :, s:e], k[None, :, s:e], v[None, :, s:e], scale, causal)
        O[:, s:e] = Ob[0]
        lse[:, s:e] = lb[0]
    return O, lse


def attention_backward_varlen(q, k, v, do, cu_seqlens, scale, causal=False):
    """(dq, dk, dv) of a packed variable-length batch: per sequence the
    grouped backward above; a token's gradients come only from its own
    sequence.  dq is (H, T, D); dk, dv are (Hkv, T, D)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    cu = _check_cu_seqlens(cu_seqlens, q.shape[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(cu.size - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        g = attention_backward_gqa(q[None, :, s:e], k[None, :, s:e], v[None, :, s:e], do[None, :, s:e], scale, causal)
        dq[:, s:e], dk[:, s:e], dv[:, s:e] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv
