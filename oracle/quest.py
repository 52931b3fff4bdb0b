"""Query-aware page selection (Quest) and attention over the selected pages, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [Serving-Ascend] is
the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu), section "Quest
Sparse Attention": score the logical blocks of a long context cheaply, keep
the Top-K blocks, and run exact attention over the tokens of those blocks
only; it must support grouped heads, per-sequence context lengths, the block
table, and skip blocks and tokens past the context.  The page names the
method (Quest) without its scoring rule; we take the published one (Tang et
al., "Quest: Query-Aware Sparsity for Efficient Long-Context LLM Inference",
2024): each page keeps the channel-wise minimum and maximum of its keys, and
the page's score for a query q is sum_d max(q_d * min_d, q_d * max_d), an
upper bound of q . k over the page's keys.

Readings of what the page leaves open:

* the min / max run over the page's valid tokens (those inside the context);
* a key/value head selects one set of pages for all G query heads sharing
  it: the page score is the sum of the G heads' Quest scores;
* Top-K keeps the topk highest-scoring pages of the context (all of them if
  there are fewer); ties go to the lower page index; the kept pages are
  listed in ascending page order;
* attention then runs over every valid token of the kept pages (the last
  page's tokens past the context stay masked), with the plain softmax.
"""
from __future__ import annotations

import numpy as np

from .paged import gather_context

__all__ = ["quest_page_minmax", "quest_scores", "quest_select", "quest_sparse_decode"]


def quest_page_minmax(k_cache, table_row, context_len, kv_head):
    """(min, max) over the valid keys of each logical page of one sequence
    and key/value head: two (n_pages, D) arrays."""
    bs = k_cache.shape[3]
    K = _keys(k_cache, table_row, context_len, kv_head)
    n_pages = -(-context_len // bs)
    D = K.shape[1]
    mn = np.zeros((n_pages, D))
    mx = np.zeros((n_pages, D))
    for p in range(n_pages):
        page = K[p * bs:(p + 1) * bs]  # the valid tokens of page p
        mn[p] = page.min(axis=0)
        mx[p] = page.max(axis=0)
    return mn, mx


def _keys(k_cache, table_row, context_len, kv_head):
    """The context's keys for one key/value head, token by token."""
    num_blocks, _, n_chunks, bs, x = k_cache.shape
    K = np.empty((context_len, n_chunks * x), dtype=np.float64)
    for t in range(context_len):
        block = int(table_row[t // bs])
        if not 0 <= block < num_blocks:
            raise ValueError(f"block table entry {block} out of range")
        K[t] = k_cache[block, kv_head, :, t % bs, :].reshape(-1)
    return K


def quest_scores(q_group, mn, mx):
    """Page scores for the G query heads of a key/value head:
    score_p = sum_h sum_d max(q_hd * min_pd, q_hd * max_pd)."""
    q_group = np.asarray(q_group, dtype=np.float64)
    s = np.zeros(mn.shape[0])
    for h in range(q_group.shape[0]):
        s += np.sum(np.maximum(q_group[h] * mn, q_group[h] * mx), axis=1)
    return s


def quest_select(scores, topk):
    """Indices of the topk highest scores (ties: lower index first), returned
    in ascending order."""
    order = sorted(range(len(scores)), key=lambda p: (-scores[p], p))
    return sorted(order[:topk])


def quest_sparse_decode(q, k_cache, v_cache, block_tables, context_lens, selected, scale):
    """(O, lse) of decode attention over the tokens of the selected logical
    pages.  selected[b][hk] lists the kept pages of sequence b for key/value
    head hk (ascending); the pages' valid tokens take part, nothing else."""
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    n_kv = k_cache.shape[1]
    G = H // n_kv
    bs = k_cache.shape[3]
    O = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        for hk in range(n_kv):
            K, V = gather_context(k_cache, v_cache, block_tables[b], n, hk)
            tokens = [t for p in selected[b][hk] for t in range(p * bs, min((p + 1) * bs, n))]
            if not tokens:
                continue
            Ks, Vs = np.asarray(K, np.float64)[tokens], np.asarray(V, np.float64)[tokens]
            for h in range(hk * G, (hk + 1) * G):
                s = (Ks @ q[b, h]) * scale
                m = np.max(s)
                e = np.exp(s - m)
                O[b, h] = (e @ Vs) / np.sum(e)
                lse[b, h] = m + np.log(np.sum(e))
    return O, lse
