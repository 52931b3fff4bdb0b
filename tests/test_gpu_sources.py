"""GPU parity of decode attention over two KV sources under one softmax (the
page "在 4 张 A100 上部署 DeepSeek-V4-Flash-0731", section 7.5: the pages of a
sliding-window pool and of a second pool form one sparse set with a single
softmax denominator), against the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import LSE_MAX_ABS, O_MAX_ABS, has_gpu, log, max_abs, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _random_selection(rng, lens, Hkv, bs, topk, empty=()):
    """Ascending random page subsets of at most topk pages per (sequence,
    head); the (b, hk) pairs in `empty` keep nothing."""
    B = len(lens)
    sel = np.full((B, Hkv, max(topk, 1)), -1, dtype=np.int32)
    nsel = np.zeros((B, Hkv), dtype=np.int32)
    lists = []
    for b in range(B):
        npg = -(-int(lens[b]) // bs)
        row = []
        for hk in range(Hkv):
            k = 0 if (b, hk) in empty else min(topk, npg)
            pages = sorted(rng.choice(npg, size=k, replace=False).tolist()) if k else []
            sel[b, hk, :k] = pages
            nsel[b, hk] = k
            row.append(pages)
        lists.append(row)
    return sel[:, :, :topk], nsel, lists


def _oracle_src(cpu, selected=None):
    _, kc, vc, tables, lens = cpu
    d = {"k_cache": to_f64(kc), "v_cache": to_f64(vc), "block_tables": tables.numpy(), "context_lens": lens.numpy()}
    if selected is not None:
        d["selected"] = selected
    return d


def _gpu_src(cpu, sel=None, nsel=None):
    import torch

    _, kc, vc, tables, lens = (t.cuda() for t in cpu)
    d = {"k_cache": kc, "v_cache": vc, "block_tables": tables, "context_lens": lens}
    if nsel is not None:
        d["selected"] = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
        d["n_selected"] = torch.from_numpy(nsel).cuda()
    return d


CASES = [
    # B, H, Hkv, D, dtype, (window bs, lo, hi), (pool bs, lo, hi), topk (0 = dense second source)
    (4, 8, 2, 128, "bf16", (16, 1, 300), (16, 100, 3000), 12),
    (3, 4, 4, 64, "f16", (32, 0, 200), (64, 1, 900), 5),
    (2, 16, 1, 256, "bf16", (16, 64, 64), (32, 500, 2500), 20),
    (3, 6, 3, 128, "f16", (64, 1, 700), (16, 1, 5000), 0),      # two dense sources
    (2, 32, 2, 128, "bf16", (16, 300, 1200), (16, 2000, 6000), 64),  # 16 query heads per key/value head
]


@pytest.mark.parametrize("B,H,Hkv,D,dtype,win,pool,topk", CASES, ids=lambda x: str(x))
def test_two_sources_against_oracle(B, H, Hkv, D, dtype, win, pool, topk):
    """A dense window source and a sparse (given pages) or dense second pool
    of another block size: O (fp32 and stored), lse against the oracle over
    the concatenated sets; the stored O is RNE of the fp32 O."""
    import torch

    fa = _fa()
    wa = workloads.DecodeWorkload("sources_window", 700 + D + B, B, H, Hkv, D, win[0], win[1], win[2], dtype)
    wb = workloads.DecodeWorkload("sources_pool", 800 + D + B, B, H, Hkv, D, pool[0], pool[1], pool[2], dtype)
    log(f"case two sources {wa} {wb} topk={topk}")
    ca, cb = workloads.make_decode_inputs(wa), workloads.make_decode_inputs(wb)
    rng = np.random.default_rng(B * 31 + D)
    if topk:
        sel, nsel, lists = _random_selection(rng, cb[4].numpy(), Hkv, pool[0], topk, empty={(0, Hkv - 1)})
        gb, ob = _gpu_src(cb, sel, nsel), _oracle_src(cb, lists)
    else:
        gb, ob = _gpu_src(cb), _oracle_src(cb)
    q = ca[0].cuda()
    srcs = [_gpu_src(ca), gb]
    o32, lse = fa.paged_decode_sources(q, srcs, scale=wa.scale, out_dtype=torch.float32)
    o16, _ = fa.paged_decode_sources(q, srcs, scale=wa.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), "O16 != RNE(O32)"
    O, L = oracle.decode_over_sources(to_f64(ca[0]), [_oracle_src(ca), ob], wa.scale)
    eo = max_abs(to_f64(o32), O)
    fin = np.isfinite(L)
    el = max_abs(to_f64(lse)[fin], L[fin]) if fin.any() else 0.0
    assert np.array_equal(np.isfinite(to_f64(lse)), fin)
    log(f"  O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS


def test_page_partition_equals_dense_decode():
    """One cache split into two sparse sources (even and odd pages) is the
    dense decode of the whole context, to rounding.  The two runs split the
    tokens differently, so each rounds P to fp16 against other running
    maxima: O may differ by up to 2^-11 max|v| per side; lse sums fp32 P."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("sources_partition", 901, 3, 8, 2, 128, 16, 50, 4000, "f16")
    cpu = workloads.make_decode_inputs(w)
    lens = cpu[4].numpy()
    npg = -(-lens // 16)
    top = int(npg.max())
    parts = []
    for parity in (0, 1):
        sel = np.full((3, 2, top), -1, dtype=np.int32)
        nsel = np.zeros((3, 2), dtype=np.int32)
        for b in range(3):
            pages = [p for p in range(int(npg[b])) if p % 2 == parity]
            sel[b, :, :len(pages)] = pages
            nsel[b, :] = len(pages)
        parts.append(_gpu_src(cpu, sel, nsel))
    g = [t.cuda() for t in cpu]
    o, lse = fa.paged_decode_sources(g[0], parts, scale=w.scale, out_dtype=torch.float32)
    od, lsed = fa.paged_decode(*g, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bound = 2 * 2.0 ** -11 * float(cpu[2].abs().max())
    eo, el = (o - od).abs().max().item(), (lse - lsed).abs().max().item()
    log(f"partition vs dense: O {eo:.3e} (bound {bound:.3e}) | lse {el:.3e}")
    assert eo <= bound and el <= 1e-5
    O, L = oracle.paged_decode(to_f64(cpu[0]), to_f64(cpu[1]), to_f64(cpu[2]), cpu[3].numpy(), lens, w.scale)
    assert max_abs(to_f64(o), O) <= O_MAX_ABS and max_abs(to_f64(lse), L) <= LSE_MAX_ABS


def test_one_source_is_the_existing_call_bit_for_bit():
    """A single dense or sparse source runs the same kernels with the same
    split as fa_paged_decode / fa_paged_decode_sparse."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("sources_one", 903, 4, 8, 2, 128, 16, 1, 6000, "bf16")
    cpu = workloads.make_decode_inputs(w)
    g = [t.cuda() for t in cpu]
    rng = np.random.default_rng(5)
    sel, nsel, _ = _random_selection(rng, cpu[4].numpy(), 2, 16, 30)
    o1, l1 = fa.paged_decode_sources(g[0], [_gpu_src(cpu)], scale=w.scale, out_dtype=torch.float32)
    o2, l2 = fa.paged_decode(*g, scale=w.scale, out_dtype=torch.float32)
    s = _gpu_src(cpu, sel, nsel)
    o3, l3 = fa.paged_decode_sources(g[0], [s], scale=w.scale, out_dtype=torch.float32)
    o4, l4 = fa.paged_decode_sparse(*g, s["selected"], s["n_selected"], scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_empty_sources():
    """A second source with no tokens leaves the first source's answer (to
    rounding: the combine runs); sequences with no token anywhere give O = 0
    and lse = -inf."""
    import torch

    fa = _fa()
    wa = workloads.DecodeWorkload("sources_empty_a", 905, 3, 4, 2, 64, 16, 0, 400, "f16")
    ca = workloads.make_decode_inputs(wa)
    lens = ca[4].clone()
    lens[1] = 0  # sequence 1 has nothing in the first source
    ca = (ca[0], ca[1], ca[2], ca[3], lens)
    wb = workloads.DecodeWorkload("sources_empty_b", 906, 3, 4, 2, 64, 32, 0, 0, "f16")
    cb = workloads.make_decode_inputs(wb)  # every context empty
    q = ca[0].cuda()
    o, lse = fa.paged_decode_sources(q, [_gpu_src(ca), _gpu_src(cb)], scale=wa.scale, out_dtype=torch.float32)
    o1, l1 = fa.paged_decode_sources(q, [_gpu_src(ca)], scale=wa.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o - o1).abs().max().item() <= 1e-6
    fin = torch.isfinite(l1)
    assert torch.equal(torch.isfinite(lse), fin) and (lse[fin] - l1[fin]).abs().max().item() <= 1e-6
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))


def test_window_and_quest_selection_end_to_end():
    """The intended use: a sliding-window pool attended whole plus the pages
    the query-aware selection keeps from the long-context pool, one softmax;
    checked against the oracle given the GPU's selection."""
    import torch

    fa = _fa()
    wp = workloads.DecodeWorkload("sources_pool_q", 907, 3, 16, 4, 128, 16, 1000, 5000, "bf16")
    ww = workloads.DecodeWorkload("sources_win_q", 908, 3, 16, 4, 128, 16, 256, 256, "bf16")
    cp, cw = workloads.make_decode_inputs(wp), workloads.make_decode_inputs(ww)
    gp = [t.cuda() for t in cp]
    kmeta = fa.quest_page_minmax(gp[1], gp[3], gp[4])
    sel, nsel = fa.quest_select(gp[0], kmeta, gp[1], gp[3], gp[4], 32)
    pool = {"k_cache": gp[1], "v_cache": gp[2], "block_tables": gp[3], "context_lens": gp[4], "selected": sel,
            "n_selected": nsel}
    o, lse = fa.paged_decode_sources(gp[0], [_gpu_src(cw), pool], scale=wp.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    s, n = sel.cpu().numpy(), nsel.cpu().numpy()
    lists = [[list(s[b, hk, :n[b, hk]]) for hk in range(4)] for b in range(3)]
    O, L = oracle.decode_over_sources(to_f64(cp[0]), [_oracle_src(cw), _oracle_src(cp, lists)], wp.scale)
    eo, el = max_abs(to_f64(o), O), max_abs(to_f64(lse), L)
    log(f"window + selection: O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS


def _rows_tensor(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


@pytest.mark.parametrize("B,Tq,H,Hkv,D,dtype,bs", [
    (3, 7, 8, 2, 128, "bf16", 16),    # 28 query rows per key/value head: two column blocks
    (2, 33, 4, 4, 64, "f16", 32),     # a longer chunk, one query head per key/value head
    (2, 5, 16, 1, 256, "bf16", 16),   # 80 rows on one key/value head
])
def test_causal_prefill_chunk_over_paged_cache(B, Tq, H, Hkv, D, dtype, bs):
    """The last Tq tokens of each context as queries, each seeing the cache up
    to its own position (row lengths n - Tq + t + 1): against the oracle, and
    the stored O is RNE of the fp32 O."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("prefill", 950 + Tq + D, B, H, Hkv, D, bs, Tq, 3000, dtype)
    log(f"case prefill chunk {w} Tq={Tq}")
    cpu = workloads.make_decode_inputs(w)
    lens = cpu[4].numpy()
    rng = np.random.default_rng(Tq)
    qd = torch.from_numpy((rng.integers(-32, 32, size=(B, Tq, H, D)) / 16).astype(np.float32)).to(cpu[0].dtype)
    rows = [[int(n) - Tq + t + 1 for t in range(Tq)] for n in lens]
    src = _gpu_src(cpu)
    src["row_lens"] = _rows_tensor(rows)
    q = qd.cuda()
    o32, lse = fa.paged_attention_sources(q, [src], scale=w.scale, out_dtype=torch.float32)
    o16, _ = fa.paged_attention_sources(q, [src], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), "O16 != RNE(O32)"
    O, L = oracle.attention_over_sources(to_f64(qd), [dict(_oracle_src(cpu), row_lens=rows)], w.scale)
    eo, el = max_abs(to_f64(o32), O), max_abs(to_f64(lse), L)
    log(f"  O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS


def test_two_sources_with_row_lengths():
    """A window pool and a sparse pool, each with its own per-row lengths
    (zero, partial, past the end), rows that see nothing anywhere included."""
    import torch

    fa = _fa()
    B, Tq, H, Hkv, D = 3, 6, 8, 2, 128
    wa = workloads.DecodeWorkload("rows_a", 960, B, H, Hkv, D, 16, 1, 200, "bf16")
    wb = workloads.DecodeWorkload("rows_b", 961, B, H, Hkv, D, 32, 100, 2000, "bf16")
    ca, cb = workloads.make_decode_inputs(wa), workloads.make_decode_inputs(wb)
    rng = np.random.default_rng(962)
    sel, nsel, lists = _random_selection(rng, cb[4].numpy(), Hkv, 32, 9)
    ra = rng.integers(-3, 260, size=(B, Tq)).astype(np.int32)
    rb = rng.integers(0, 400, size=(B, Tq)).astype(np.int32)
    ra[0, 0] = 0
    rb[0, 0] = 0  # row 0 of sequence 0 sees nothing
    qd = torch.from_numpy((rng.integers(-32, 32, size=(B, Tq, H, D)) / 16).astype(np.float32)).to(torch.bfloat16)
    ga, gb = _gpu_src(ca), _gpu_src(cb, sel, nsel)
    ga["row_lens"], gb["row_lens"] = _rows_tensor(ra), _rows_tensor(rb)
    o, lse = fa.paged_attention_sources(qd.cuda(), [ga, gb], scale=wa.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oa = dict(_oracle_src(ca), row_lens=ra.tolist())
    ob = dict(_oracle_src(cb, lists), row_lens=rb.tolist())
    O, L = oracle.attention_over_sources(to_f64(qd), [oa, ob], wa.scale)
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(to_f64(lse)), fin) and not fin[0, 0].any()
    assert np.all(to_f64(o)[0, 0] == 0)
    eo, el = max_abs(to_f64(o), O), max_abs(to_f64(lse)[fin], L[fin])
    log(f"two sources with row lengths: O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS


def test_one_query_row_is_the_decode_call():
    """Tq = 1 without row lengths runs what fa_paged_decode_sources runs, bit for bit."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("rows_one", 963, 4, 8, 2, 128, 16, 1, 5000, "f16")
    cpu = workloads.make_decode_inputs(w)
    rng = np.random.default_rng(7)
    sel, nsel, _ = _random_selection(rng, cpu[4].numpy(), 2, 16, 20)
    srcs = [_gpu_src(cpu), _gpu_src(cpu, sel, nsel)]
    q = cpu[0].cuda()
    o1, l1 = fa.paged_decode_sources(q, srcs, scale=w.scale, out_dtype=torch.float32)
    o2, l2 = fa.paged_attention_sources(q[:, None].contiguous(), srcs, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


def test_verify_workload():
    """The causal-chunk workload (64 sequences of 512..16000
    tokens, 4 causal query tokens each) on its shortest, longest and one
    middle sequence."""
    import torch

    fa = _fa()
    w = workloads.DECODE_WORKLOADS["verify_gqa_bf16"]
    cpu = workloads.make_decode_inputs(w)
    q, kc, vc, tables, lens = cpu
    n = lens.numpy()
    T = w.q_len
    rows = np.array([[int(x) - T + t + 1 for t in range(T)] for x in n], dtype=np.int32)
    src = _gpu_src(cpu)
    src["row_lens"] = _rows_tensor(rows)
    o, lse = fa.paged_attention_sources(q.cuda(), [src], scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    seqs = sorted({int(np.argmin(n)), int(np.argmax(n)), 7})
    t = tables[seqs].numpy()
    used = sorted({int(x) for x in t.flatten() if x >= 0})
    remap = np.full(kc.shape[0], -1, dtype=np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    sub = {"k_cache": to_f64(kc[used]), "v_cache": to_f64(vc[used]),
           "block_tables": np.where(t >= 0, remap[np.clip(t, 0, None)], -1), "context_lens": n[seqs],
           "row_lens": rows[seqs].tolist()}
    O, L = oracle.attention_over_sources(to_f64(q[seqs]), [sub], w.scale)
    eo, el = max_abs(to_f64(o[seqs]), O), max_abs(to_f64(lse[seqs]), L)
    log(f"verify_gqa_bf16 sequences {seqs}: O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS
