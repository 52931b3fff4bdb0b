"""GPU parity of the query-aware page selection (Quest) and of attention over
the kept pages, against the fp64 oracle (the page "从算子到 Serving：昇腾推理
评测链路实践", section "Quest Sparse Attention").

The page asks that the selection be fixed before the attention is compared.
So: page min / max are compared bit for bit; the selection, decided by fp32
scores on the GPU, is checked for validity against the oracle's fp64 scores
(every kept page scores at least as high as every dropped one, up to the fp32
rounding bound) and must equal the oracle's choice wherever the fp64 scores
are not within that bound of the cut; attention over the kept pages is then
compared with the oracle given the same pages, to the attention tolerances.
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


def _subset(cpu, seqs):
    """The sampled sequences' inputs with only their physical blocks, renumbered
    (the oracle then converts a few MB instead of the whole cache)."""
    q, kc, vc, tables, lens = cpu
    t = tables[seqs].numpy()
    used = sorted({int(x) for x in t.flatten() if x >= 0})
    remap = np.full(kc.shape[0], -1, dtype=np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    t2 = np.where(t >= 0, remap[np.clip(t, 0, None)], -1).astype(np.int32)
    return to_f64(q[seqs]), to_f64(kc[used]), to_f64(vc[used]), t2, lens[seqs].numpy()


def _check(w, cpu, topk, label, seqs=None):
    import torch

    fa = _fa()
    q, kc, vc, tables, lens = cpu
    g = [t.cuda() for t in cpu]
    kmeta = fa.quest_page_minmax(g[1], g[3], g[4])
    sel, nsel = fa.quest_select(g[0], kmeta, g[1], g[3], g[4], topk)
    o32, lse32 = fa.paged_decode_sparse(g[0], g[1], g[2], g[3], g[4], sel, nsel, scale=w.scale,
                                        out_dtype=torch.float32)
    o16, _ = fa.paged_decode_sparse(g[0], g[1], g[2], g[3], g[4], sel, nsel, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), f"{label}: O16 != RNE(O32)"
    kmeta, sel, nsel = kmeta.cpu(), sel.cpu().numpy(), nsel.cpu().numpy()
    seqs = list(range(w.B)) if seqs is None else seqs
    q_s, kc_s, vc_s, tab_s, lens_s = _subset(cpu, seqs)
    G = w.H // w.Hkv
    exact_sets = near = 0
    for i, b in enumerate(seqs):
        n = int(lens[b])
        for hk in range(w.Hkv):
            mn, mx = oracle.quest_page_minmax(kc_s, tab_s[i], n, hk)
            npg = mn.shape[0]
            blocks = tables[b, :npg].numpy()
            got = to_f64(kmeta[blocks, hk])
            assert np.array_equal(got[:, 0], mn) and np.array_equal(got[:, 1], mx), f"{label}: min/max b={b} hk={hk}"
            qg = q_s[i, hk * G:(hk + 1) * G]
            s = oracle.quest_scores(qg, mn, mx)
            bound = np.sum(np.abs(qg) @ np.maximum(np.abs(mn), np.abs(mx)).T, axis=0) * 1e-5 + 1e-6
            k = int(nsel[b, hk])
            kept = list(sel[b, hk, :k])
            assert k == min(topk, npg) and kept == sorted(kept) and len(set(kept)) == k
            dropped = sorted(set(range(npg)) - set(kept))
            if kept and dropped:
                assert min(s[kept] + bound[kept]) >= max(s[dropped] - bound[dropped]), f"{label}: invalid selection"
            want = oracle.quest_select(s, topk)
            if kept == want:
                exact_sets += 1
            else:  # only pages within the rounding bound of the cut may differ
                cut = np.sort(s)[::-1][k - 1]
                for p in set(kept) ^ set(want):
                    assert abs(s[p] - cut) <= 2 * bound[p], f"{label}: page {p} differs away from the cut"
                near += 1
    selected = [[list(sel[b, hk, :nsel[b, hk]]) for hk in range(w.Hkv)] for b in seqs]
    sub = np.asarray(seqs)
    O, lse = oracle.quest_sparse_decode(q_s, kc_s, vc_s, tab_s, lens_s, selected, w.scale)
    eo = max_abs(to_f64(o32[sub]), O)
    fin = np.isfinite(lse)
    el = max_abs(to_f64(lse32[sub])[fin], lse[fin]) if fin.any() else 0.0
    log(f"{label}: topk={topk} (sequence, head) sets equal to the oracle's {exact_sets}, near-tie differences "
        f"{near} | O32 max-abs {eo:.3e} | lse {el:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS
    return sel, nsel


SMALL = [
    # B, H, Hkv, D, block_size, lo, hi, dtype, topk
    (4, 8, 2, 128, 16, 0, 1000, "bf16", 8),
    (3, 4, 4, 64, 32, 1, 300, "f16", 3),
    (2, 16, 1, 128, 16, 200, 3000, "f16", 40),
    (3, 6, 3, 256, 64, 17, 900, "bf16", 5),
    (5, 4, 2, 64, 16, 1, 60, "f16", 16),     # topk above the page count: every page kept
    (2, 4, 2, 128, 16, 100, 200, "f16", 0),  # nothing kept
    (2, 32, 1, 128, 16, 200, 1500, "f16", 10),  # 32 query heads on one key/value head
]


@pytest.mark.parametrize("B,H,Hkv,D,bs,lo,hi,dtype,topk", SMALL, ids=lambda x: str(x))
def test_quest_small(B, H, Hkv, D, bs, lo, hi, dtype, topk):
    w = workloads.DecodeWorkload("quest_small", 400 + B + D + bs, B, H, Hkv, D, bs, lo, hi, dtype)
    log(f"case {w} topk={topk}")
    _check(w, workloads.make_decode_inputs(w), topk, f"B={B} H={H}/{Hkv} D={D} bs={bs} {dtype}")


def test_quest_full_budget_equals_dense_decode():
    """With every page kept the sparse decode attends to the whole context:
    it matches the dense decode to rounding (the split sizes differ)."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("quest_full", 411, 3, 8, 2, 128, 16, 50, 700, "f16")
    g = [t.cuda() for t in workloads.make_decode_inputs(w)]
    mxb = g[3].shape[1]
    kmeta = fa.quest_page_minmax(g[1], g[3], g[4])
    sel, nsel = fa.quest_select(g[0], kmeta, g[1], g[3], g[4], mxb)
    o, lse = fa.paged_decode_sparse(*g, sel, nsel, scale=w.scale, out_dtype=torch.float32)
    od, lsed = fa.paged_decode(*g, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o - od).abs().max().item() <= 1e-5 and (lse - lsed).abs().max().item() <= 1e-5


def test_quest_given_selection():
    """Attention over test-chosen pages (random ascending subsets, a count of
    zero, the last partial page) against the oracle given the same pages."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("quest_given", 413, 3, 4, 2, 64, 16, 40, 300, "bf16")
    cpu = workloads.make_decode_inputs(w)
    q, kc, vc, tables, lens = cpu
    rng = np.random.default_rng(3)
    topk = 5
    sel = np.full((3, 2, topk), -1, dtype=np.int32)
    nsel = np.zeros((3, 2), dtype=np.int32)
    chosen = []
    for b in range(3):
        npg = -(-int(lens[b]) // 16)
        row = []
        for hk in range(2):
            k = 0 if (b, hk) == (1, 0) else min(topk, npg)
            pages = sorted(rng.choice(npg, size=k, replace=False).tolist())
            if (b, hk) == (2, 1):
                pages = sorted(set(pages[1:] + [npg - 1]))  # the partial last page
            sel[b, hk, :len(pages)] = pages
            nsel[b, hk] = len(pages)
            row.append(pages)
        chosen.append(row)
    g = [t.cuda() for t in cpu]
    o, lse = fa.paged_decode_sparse(*g, torch.from_numpy(sel).cuda(), torch.from_numpy(nsel).cuda(), scale=w.scale,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.quest_sparse_decode(to_f64(q), to_f64(kc), to_f64(vc), tables.numpy(), lens.numpy(), chosen, w.scale)
    assert max_abs(to_f64(o), O) <= O_MAX_ABS
    assert np.all(np.isneginf(to_f64(lse[1, :2]))) and np.all(to_f64(o[1, :2]) == 0)
    fin = np.isfinite(L)
    assert max_abs(to_f64(lse)[fin], L[fin]) <= LSE_MAX_ABS


def test_quest_ties_go_to_the_lower_page():
    """Pages with equal scores (identical metadata): the kept ones are the
    lowest pages of the tie, as in the oracle."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("quest_ties", 417, 2, 4, 2, 64, 16, 300, 600, "bf16")
    q, kc, vc, tables, lens = workloads.make_decode_inputs(w)
    g = [t.cuda() for t in (q, kc, vc, tables, lens)]
    kmeta = fa.quest_page_minmax(g[1], g[3], g[4])
    # make every page of sequence 0 / head 1 score the same: copy one page's metadata to all
    blocks = tables[0, : -(-int(lens[0]) // 16)].long().cuda()
    kmeta[blocks, 1] = kmeta[blocks[3], 1].clone()
    sel, nsel = fa.quest_select(g[0], kmeta, g[1], g[3], g[4], 5)
    torch.cuda.synchronize()
    assert sel[0, 1, :5].tolist() == [0, 1, 2, 3, 4] and int(nsel[0, 1]) == 5


def test_quest_workload():
    """The 64-sequence decode workload with 64 of its ~580 pages kept per
    context, on 3 sampled sequences."""
    w = workloads.DECODE_WORKLOADS["decode_gqa_bf16"]
    cpu = workloads.make_decode_inputs(w)
    lens = cpu[4].numpy()
    _check(w, cpu, 64, w.name, sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7}))
