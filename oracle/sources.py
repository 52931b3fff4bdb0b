"""Decode attention over one or two KV sources under a single softmax, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [V4-A100] is the page
"在 4 张 A100 上部署 DeepSeek-V4-Flash-0731" (BiumBiu).  Its section 7.3 keeps
separate paged KV pools (a sliding-window pool and compressed pools); its
section 7.5 describes one sparse attention kernel (gather the listed pages,
Q K^T, online softmax, P V) that serves either a single source (the
sliding-window pool) or two sources, whose pages together form one logical
sparse set normalised by one softmax denominator.

Readings of what the page leaves open:

* a source is a paged cache in the layouts of ``paged.py`` with its own block
  table and context lengths; it contributes every valid token of the
  sequence's context, or, when it carries a page selection (as made by
  ``quest.py``), the valid tokens of the kept logical pages only;
* the attended set of a query head is the concatenation of its sources'
  token sets (entries of different sources are different entries, even when
  they hold the same key), and the output is the plain softmax of
  [FA-Ascend] section 一 over that set: one maximum, one denominator;
* a query head with no token in any source gets O = 0 and lse = -inf;
* several query rows per sequence (section 7.5: prefill and decode share the
  kernel because the causal constraint is expanded into per-row lengths): row
  t of sequence b sees, in each source, the first row_lens[b][t] tokens of
  that source's token set (all of them when the source gives no row lengths).
"""
from __future__ import annotations

import numpy as np

from .paged import gather_context

__all__ = ["source_tokens", "decode_over_sources", "attention_over_sources"]


def source_tokens(src, b, kv_head):
    """(K, V) of the tokens one source contributes to sequence b and
    key/value head kv_head, as fp64 (n, D) arrays in context order.

    src: dict with k_cache (num_blocks, Hkv, D/8, bs, 8), v_cache
    (num_blocks, Hkv, D, bs), block_tables (B, max_blocks), context_lens (B)
    and optionally selected: selected[b][kv_head] lists kept logical pages."""
    k_cache, v_cache = src["k_cache"], src["v_cache"]
    bs = k_cache.shape[3]
    D = k_cache.shape[2] * k_cache.shape[4]
    n = int(src["context_lens"][b])
    K, V = gather_context(k_cache, v_cache, src["block_tables"][b], n, kv_head)
    K, V = np.asarray(K, np.float64), np.asarray(V, np.float64)
    sel = src.get("selected")
    if sel is None:
        return K, V
    tokens = [t for p in sel[b][kv_head] for t in range(p * bs, min((p + 1) * bs, n))]
    if not tokens:
        return np.zeros((0, D)), np.zeros((0, D))
    return K[tokens], V[tokens]


def decode_over_sources(q, sources, scale):
    """(O, lse) of decode attention of q (B, H, D) over the union of the
    sources' token sets: for query head h of sequence b (key/value head
    h // (H / Hkv) in every source), s = scale * q . k over the concatenated
    keys, O = softmax(s) V, lse = ln sum exp(s)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    n_kv = sources[0]["k_cache"].shape[1]
    if any(s["k_cache"].shape[1] != n_kv for s in sources) or n_kv <= 0 or H % n_kv != 0:
        raise ValueError("every source must have the same key/value heads, dividing the query heads")
    G = H // n_kv
    O = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        for hk in range(n_kv):
            parts = [source_tokens(s, b, hk) for s in sources]
            K = np.concatenate([p[0] for p in parts], axis=0)
            V = np.concatenate([p[1] for p in parts], axis=0)
            if K.shape[0] == 0:
                continue
            for h in range(hk * G, (hk + 1) * G):
                s = (K @ q[b, h]) * scale
                m = np.max(s)
                e = np.exp(s - m)
                l = np.sum(e)
                O[b, h] = (e @ V) / l
                lse[b, h] = m + np.log(l)
    return O, lse


def attention_over_sources(q, sources, scale):
    """(O, lse) of attention of several query rows per sequence over the
    sources: q (B, T, H, D); a source may carry row_lens (B, T), the number of
    its tokens (in the order ``source_tokens`` lists them) that each row sees.
    O is (B, T, H, D) and lse (B, T, H); a row with no visible token gets
    O = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    B, T, H, D = q.shape
    n_kv = sources[0]["k_cache"].shape[1]
    if any(s["k_cache"].shape[1] != n_kv for s in sources) or n_kv <= 0 or H % n_kv != 0:
        raise ValueError("every source must have the same key/value heads, dividing the query heads")
    G = H // n_kv
    O = np.zeros((B, T, H, D))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        for hk in range(n_kv):
            parts = [source_tokens(s, b, hk) for s in sources]
            for t in range(T):
                Ks, Vs = [], []
                for s, (K, V) in zip(sources, parts):
                    n = K.shape[0]
                    if s.get("row_lens") is not None:
                        n = max(0, min(n, int(s["row_lens"][b][t])))
                    Ks.append(K[:n])
                    Vs.append(V[:n])
                K, V = np.concatenate(Ks, axis=0), np.concatenate(Vs, axis=0)
                if K.shape[0] == 0:
                    continue
                for h in range(hk * G, (hk + 1) * G):
                    sc = (K @ q[b, t, h]) * scale
                    m = np.max(sc)
                    e = np.exp(sc - m)
                    l = np.sum(e)
                    O[b, t, h] = (e @ V) / l
                    lse[b, t, h] = m + np.log(l)
    return O, lse
