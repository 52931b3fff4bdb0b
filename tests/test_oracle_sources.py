"""Pins of the two-source decode oracle.  [V4-A100] is the page "在 4 张 A100
上部署 DeepSeek-V4-Flash-0731" (BiumBiu), section 7.5: the pages of one or two
sources form one logical sparse set under a single softmax denominator.
"""
import numpy as np

import oracle
from oracle import decode_over_sources, paged_decode


def _cache(rng, lens, n_kv, D, bs, extra=2):
    """A random cache in the documented layouts with block tables that deal
    random distinct blocks (test-side, plain indexing)."""
    pages = [-(-n // bs) for n in lens]
    nb = sum(pages) + extra
    kc = rng.standard_normal((nb, n_kv, D // 8, bs, 8))
    vc = rng.standard_normal((nb, n_kv, D, bs))
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(max(pages), 1) + 1), -1, dtype=np.int32)
    i = 0
    for b, p in enumerate(pages):
        tables[b, :p] = perm[i:i + p]
        i += p
    return {"k_cache": kc, "v_cache": vc, "block_tables": tables, "context_lens": np.array(lens, np.int32)}


def test_page_partition_equals_whole_context():
    """Splitting a context's pages between two sources (even pages in one,
    odd pages in the other) gives attention over the whole context: this pins
    the single denominator (normalising each source on its own, or dropping
    one, fails it)."""
    rng = np.random.default_rng(201)
    bs, D, n_kv, H = 16, 16, 2, 6
    lens = [70, 16, 33, 1]
    src = _cache(rng, lens, n_kv, D, bs)
    q = rng.standard_normal((len(lens), H, D))
    even = [[[p for p in range(-(-n // bs)) if p % 2 == 0] for _ in range(n_kv)] for n in lens]
    odd = [[[p for p in range(-(-n // bs)) if p % 2 == 1] for _ in range(n_kv)] for n in lens]
    O, lse = decode_over_sources(q, [dict(src, selected=even), dict(src, selected=odd)], 0.3)
    O_ref, lse_ref = paged_decode(q, src["k_cache"], src["v_cache"], src["block_tables"], src["context_lens"], 0.3)
    assert np.allclose(O, O_ref, rtol=0, atol=1e-13)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_planted_per_source_normalisation_fails_the_partition_pin():
    """The slip the pin above guards against: softmax per source, then the two
    outputs averaged, differs from attention over the whole context."""
    rng = np.random.default_rng(203)
    bs, D = 16, 8
    src = _cache(rng, [64], 1, D, bs)
    q = rng.standard_normal((1, 1, D)) * 2
    halves = ([[[0, 1]]], [[[2, 3]]])
    parts = [decode_over_sources(q, [dict(src, selected=s)], 1.0)[0] for s in halves]
    O_ref, _ = paged_decode(q, src["k_cache"], src["v_cache"], src["block_tables"], src["context_lens"], 1.0)
    assert np.max(np.abs(0.5 * (parts[0] + parts[1]) - O_ref)) > 1e-3


def test_single_source_and_empty_second_source():
    """One dense source is plain paged decode; a second source with nothing to
    contribute (context length 0, or no kept page) changes nothing; a query
    with no token anywhere gets O = 0 and lse = -inf."""
    rng = np.random.default_rng(205)
    bs, D, n_kv, H = 32, 16, 1, 2
    a = _cache(rng, [40, 0, 96], n_kv, D, bs)
    b = _cache(rng, [0, 0, 0], n_kv, D, 16)
    q = rng.standard_normal((3, H, D))
    O_ref, lse_ref = paged_decode(q, a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.25)
    for srcs in ([a], [a, b], [b, a], [a, dict(a, selected=[[[]], [[]], [[]]])]):
        O, lse = decode_over_sources(q, srcs, 0.25)
        assert np.array_equal(O, O_ref) and np.array_equal(lse, lse_ref)
    assert np.all(O[1] == 0) and np.all(lse[1] == -np.inf)


def test_zero_keys_give_the_mean_of_both_sources():
    """With all keys zero every score is 0: O is the mean of the value rows of
    both sources (different block sizes and a partial last page included) and
    lse = ln(n_a + n_b)."""
    rng = np.random.default_rng(207)
    D = 16
    a = _cache(rng, [21], 1, D, 16)
    b = _cache(rng, [50], 1, D, 32)
    a["k_cache"][:] = 0.0
    b["k_cache"][:] = 0.0
    b_sel = dict(b, selected=[[[1]]])  # tokens 32 .. 49 of b
    q = rng.standard_normal((1, 3, D))
    O, lse = decode_over_sources(q, [a, b_sel], 0.7)
    rows = [a["v_cache"][a["block_tables"][0, t // 16], 0, :, t % 16] for t in range(21)]
    rows += [b["v_cache"][b["block_tables"][0, t // 32], 0, :, t % 32] for t in range(32, 50)]
    want = np.mean(np.stack(rows), axis=0)
    for h in range(3):
        assert np.allclose(O[0, h], want, rtol=0, atol=1e-14)
        assert abs(lse[0, h] - np.log(39)) <= 1e-14


def test_source_order_and_grouped_heads():
    """The set is unordered: swapping the sources gives the same O and lse
    (up to summation order); query heads h use key/value head h // G in every
    source."""
    rng = np.random.default_rng(209)
    D, n_kv, H = 16, 2, 4
    a = _cache(rng, [48, 17], n_kv, D, 16)
    b = _cache(rng, [64, 80], n_kv, D, 32)
    b["selected"] = [[[0], [1]], [[2], [0, 1]]]
    q = rng.standard_normal((2, H, D))
    O1, l1 = decode_over_sources(q, [a, b], 0.5)
    O2, l2 = decode_over_sources(q, [b, a], 0.5)
    assert np.allclose(O1, O2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)
    # query head 3 of sequence 1 reads key/value head 1: its answer depends
    # only on that head's tokens
    a2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    a2["k_cache"][:, 0] += 5.0
    O3, _ = decode_over_sources(q, [a2, b], 0.5)
    assert np.array_equal(O3[:, 2:], O1[:, 2:]) and not np.allclose(O3[:, :2], O1[:, :2])


def test_exported():
    assert oracle.decode_over_sources is decode_over_sources


def test_several_rows_one_row_is_decode():
    """One query row per sequence without row lengths is the decode above."""
    rng = np.random.default_rng(211)
    a = _cache(rng, [40, 0, 70], 2, 16, 16)
    b = _cache(rng, [33, 5, 64], 2, 16, 32)
    b["selected"] = [[[0, 1], [1]], [[0], []], [[1], [0, 1]]]
    q = rng.standard_normal((3, 4, 16))
    O1, l1 = decode_over_sources(q, [a, b], 0.4)
    O2, l2 = oracle.attention_over_sources(q[:, None], [a, b], 0.4)
    assert np.array_equal(O2[:, 0], O1) and np.array_equal(l2[:, 0], l1)


def test_causal_prefill_chunk_is_causal_attention():
    """A chunk of the last T tokens of each sequence, each row seeing the
    cached tokens up to its own position (row lengths n - T + t + 1), is the
    last T rows of causal attention over the whole sequence
    (oracle.attention_forward, pinned by finite differences and closed forms)."""
    rng = np.random.default_rng(213)
    D, n_kv, H, T = 16, 2, 4, 5
    lens = [37, 5, 64]
    src = _cache(rng, lens, n_kv, D, 16)
    q = rng.standard_normal((3, T, H, D))
    src["row_lens"] = [[n - T + t + 1 for t in range(T)] for n in lens]
    O, lse = oracle.attention_over_sources(q, [src], 0.35)
    G = H // n_kv
    for b, n in enumerate(lens):
        for h in range(H):
            K, V = oracle.gather_context(src["k_cache"], src["v_cache"], src["block_tables"][b], n, h // G)
            Q = np.zeros((n, D))
            Q[n - T:] = q[b, :, h]  # the chunk's rows at their positions (earlier rows unused)
            Of, lf = oracle.attention_forward(Q, K, V, 0.35, causal=True)
            assert np.allclose(O[b, :, h], Of[n - T:], rtol=0, atol=1e-13)
            assert np.allclose(lse[b, :, h], lf[n - T:], rtol=0, atol=1e-13)


def test_row_lengths_clamp_and_empty_rows():
    """Row lengths beyond a source's set are clamped to it; a row that sees
    nothing in any source gets O = 0, lse = -inf; per-source lengths apply to
    each source's own token order (a sparse source's kept tokens)."""
    rng = np.random.default_rng(215)
    a = _cache(rng, [20], 1, 8, 16)
    b = _cache(rng, [48], 1, 8, 16)
    b["selected"] = [[[0, 2]]]  # kept pages (ascending): tokens 0..15, then 32..47
    q = rng.standard_normal((1, 3, 2, 8))
    a["row_lens"] = [[0, 100, 3]]
    b["row_lens"] = [[0, 0, 20]]
    O, lse = oracle.attention_over_sources(q, [a, b], 1.0)
    assert np.all(O[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    a2, b2 = dict(a, row_lens=None), dict(b, row_lens=None)
    O1, _ = oracle.attention_over_sources(q[:, 1:2], [a2], 1.0)
    assert np.array_equal(O[0, 1], O1[0, 0])  # 100 clamps to the 20 tokens of a; b sees nothing
    Kb, Vb = oracle.source_tokens(b2, 0, 0)
    Ka, Va = oracle.source_tokens(a2, 0, 0)
    K = np.concatenate([Ka[:3], Kb[:20]])
    V = np.concatenate([Va[:3], Vb[:20]])
    for h in range(2):
        s = K @ q[0, 2, h]
        e = np.exp(s - s.max())
        assert np.allclose(O[0, 2, h], e @ V / e.sum(), rtol=0, atol=1e-13)
