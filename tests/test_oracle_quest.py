"""Pins of the Quest oracle (page min/max, scores, Top-K, attention over the
kept pages).  [Serving-Ascend] is the page "从算子到 Serving：昇腾推理评测链路
实践" (BiumBiu), section "Quest Sparse Attention"; the scoring rule is the
published Quest one (an upper bound of q . k over a page).
"""
import numpy as np
import pytest

from oracle import paged_decode, quest_page_minmax, quest_scores, quest_select, quest_sparse_decode


def _cache(rng, lens, n_kv, D, bs, extra=3):
    """Random caches in the documented layouts and block tables dealing random
    distinct blocks (test-side, plain indexing)."""
    pages = [-(-n // bs) for n in lens]
    nb = sum(pages) + extra
    kc = rng.standard_normal((nb, n_kv, D // 8, bs, 8))
    vc = rng.standard_normal((nb, n_kv, D, bs))
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(pages) + 1), -1, dtype=np.int32)
    i = 0
    for b, p in enumerate(pages):
        tables[b, :p] = perm[i:i + p]
        i += p
    return kc, vc, tables


def _keys(kc, row, n, hk):
    bs = kc.shape[3]
    return np.stack([kc[row[t // bs], hk, :, t % bs, :].reshape(-1) for t in range(n)])


def test_page_minmax_and_score_bound():
    """min / max over the valid keys only (a partial last page included); the
    score bounds q . k of every token of the page, with equality for a page
    of one token; a slip that scores with the max alone is no bound."""
    rng = np.random.default_rng(91)
    bs, D = 16, 16
    lens = [37, 16, 1]
    kc, vc, tables = _cache(rng, lens, 2, D, bs)
    for b, n in enumerate(lens):
        for hk in range(2):
            mn, mx = quest_page_minmax(kc, tables[b], n, hk)
            K = _keys(kc, tables[b], n, hk)
            assert mn.shape == (-(-n // bs), D)
            for p in range(mn.shape[0]):
                page = K[p * bs:min((p + 1) * bs, n)]
                assert np.array_equal(mn[p], page.min(0)) and np.array_equal(mx[p], page.max(0))
                q = rng.standard_normal(D)
                s = quest_scores(q[None], mn[p:p + 1], mx[p:p + 1])[0]
                assert np.all(page @ q <= s + 1e-12)
                if len(page) == 1:
                    assert abs(s - page[0] @ q) <= 1e-12


def test_planted_max_only_score_is_no_bound():
    """A plausible slip, scoring with q . max alone, is not an upper bound:
    keys (-1, 0) and (1, 0), query (-1, 0).  The Quest score is."""
    mn, mx = np.array([[-1.0, 0.0]]), np.array([[1.0, 0.0]])
    q = np.array([[-1.0, 0.0]])
    keys = np.array([[-1.0, 0.0], [1.0, 0.0]])
    assert float(np.max(keys @ q[0])) == 1.0
    assert float(q[0] @ mx[0]) < 1.0
    assert quest_scores(q, mn, mx)[0] == 1.0


def test_group_score_is_sum_over_heads():
    rng = np.random.default_rng(93)
    mn, mx = rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    mn, mx = np.minimum(mn, mx), np.maximum(mn, mx)
    q = rng.standard_normal((3, 8))
    want = sum(quest_scores(q[h:h + 1], mn, mx) for h in range(3))
    assert np.allclose(quest_scores(q, mn, mx), want, rtol=0, atol=1e-12)


def test_select_brute_force_and_ties():
    rng = np.random.default_rng(95)
    for n, k in ((10, 3), (7, 7), (5, 9), (1, 1)):
        s = rng.integers(0, 4, size=n).astype(float)  # many ties
        kept = quest_select(s, k)
        assert kept == sorted(kept) and len(kept) == min(n, k)
        dropped = [p for p in range(n) if p not in kept]
        for a in kept:
            for d in dropped:
                assert s[a] > s[d] or (s[a] == s[d] and a < d)


def test_all_pages_kept_equals_dense_decode_and_sdpa():
    """topk >= pages: the sparse result is the dense paged decode, bit for bit;
    a real selection against torch SDPA over the tokens the test gathers."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(97)
    bs, D, H, Hkv = 16, 16, 4, 2
    lens = [50, 16, 33]
    kc, vc, tables = _cache(rng, lens, Hkv, D, bs)
    q = rng.standard_normal((3, H, D))
    allp = [[list(range(-(-n // bs)))] * Hkv for n in lens]
    O, lse = quest_sparse_decode(q, kc, vc, tables, lens, allp, 0.25)
    Od, lsed = paged_decode(q, kc, vc, tables, np.array(lens), 0.25)
    assert np.array_equal(O, Od) and np.array_equal(lse, lsed)
    sel = [[[0, 3], [1]], [[0], [0]], [[2], [0, 1]]]  # pages 3 of 50 tokens is the partial one
    O, lse = quest_sparse_decode(q, kc, vc, tables, lens, sel, 0.25)
    for b, n in enumerate(lens):
        for hk in range(Hkv):
            toks = [t for p in sel[b][hk] for t in range(p * bs, min((p + 1) * bs, n))]
            K = _keys(kc, tables[b], n, hk)[toks]
            V = np.stack([vc[tables[b][t // bs], hk, :, t % bs] for t in toks])
            for h in range(hk * 2, hk * 2 + 2):
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.tensor(q[b, h][None, None]), torch.tensor(K[None]), torch.tensor(V[None]), scale=0.25)
                assert np.max(np.abs(o.numpy()[0, 0] - O[b, h])) <= 1e-12
