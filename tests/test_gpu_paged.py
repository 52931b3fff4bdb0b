"""GPU parity of the paged KV cache: fa_reshape_and_cache (bit for bit) and
fa_paged_decode against the fp64 oracle (the page "从算子到 Serving：昇腾推理
评测链路实践", sections "ReshapeAndCache" and "GQA Paged Attention").
Decode tolerances as for attention: O max-abs <= 1e-2 on the fp32 O, lse
max-abs <= 1e-3; the 16-bit O is the RNE cast of the fp32 O bit for bit.
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


def _tdt(dtype):
    import torch

    return {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def test_reshape_and_cache_bit_exact():
    import torch

    fa = _fa()
    rng = np.random.default_rng(101)
    for (nb, Hkv, bs, D, T, dt) in ((9, 2, 16, 64, 40, "f16"), (5, 3, 32, 128, 70, "bf16"), (4, 1, 64, 256, 33, "f16")):
        kc0 = torch.from_numpy(rng.standard_normal((nb, Hkv, D // 8, bs, 8), dtype=np.float32)).to(_tdt(dt))
        vc0 = torch.from_numpy(rng.standard_normal((nb, Hkv, D, bs), dtype=np.float32)).to(_tdt(dt))
        key = torch.from_numpy(rng.standard_normal((T, Hkv, D), dtype=np.float32)).to(_tdt(dt))
        val = torch.from_numpy(rng.standard_normal((T, Hkv, D), dtype=np.float32)).to(_tdt(dt))
        slots = rng.permutation(nb * bs)[:T].astype(np.int64)
        slots[::7] = -1
        slots[5] = nb * bs + 3  # past the cache: skipped
        want_k, want_v = oracle.reshape_and_cache(key.view(torch.int16).numpy(), val.view(torch.int16).numpy(),
                                                  np.where(slots >= nb * bs, -1, slots),
                                                  kc0.view(torch.int16).numpy(), vc0.view(torch.int16).numpy())
        kc, vc = kc0.cuda(), vc0.cuda()
        fa.reshape_and_cache(key.cuda(), val.cuda(), torch.from_numpy(slots).cuda(), kc, vc)
        torch.cuda.synchronize()
        assert np.array_equal(kc.cpu().view(torch.int16).numpy(), want_k), (nb, Hkv, bs, D)
        assert np.array_equal(vc.cpu().view(torch.int16).numpy(), want_v), (nb, Hkv, bs, D)
        log(f"reshape_and_cache nb={nb} Hkv={Hkv} bs={bs} D={D} T={T} {dt}: bit-exact")


def _decode_check(w, cpu, label, seqs=None):
    import torch

    fa = _fa()
    q, kc, vc, tables, lens = cpu
    g = [t.cuda() for t in cpu]
    o32, lse32 = fa.paged_decode(*g, max_context_len=w.hi, scale=w.scale, out_dtype=torch.float32)
    o16, lse16 = fa.paged_decode(*g, max_context_len=w.hi, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), f"{label}: O16 != RNE(O32)"
    assert torch.equal(lse16, lse32), f"{label}: lse differs between O dtypes"
    seqs = list(range(w.B)) if seqs is None else seqs
    sub = np.asarray(seqs)
    O, lse = oracle.paged_decode(to_f64(q[sub]), to_f64(kc), to_f64(vc), tables.numpy()[sub], lens.numpy()[sub],
                                 w.scale)
    eo = max_abs(to_f64(o32[sub]), O)
    finite = np.isfinite(lse)
    el = max_abs(to_f64(lse32[sub])[finite], lse[finite]) if finite.any() else 0.0
    assert np.array_equal(np.isneginf(to_f64(lse32[sub])), ~finite), f"{label}: empty contexts"
    ws = fa.lib().fa_paged_decode_workspace_bytes(w.B, w.H, w.Hkv, w.D, w.hi)
    log(f"{label}: sequences={len(seqs)} O32 max-abs {eo:.3e} | lse {el:.3e} | "
        f"splits {max(1, ws // (4 * w.B * w.H * (w.D + 1)))}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS
    return o16, lse16


SMALL = [
    # B, H, Hkv, D, block_size, lo, hi, dtype
    (4, 8, 2, 128, 16, 0, 1000, "bf16"),     # several splits; an empty context possible
    (3, 4, 4, 64, 32, 1, 70, "f16"),
    (2, 16, 1, 128, 16, 200, 3000, "f16"),   # MQA, 16 query heads
    (5, 6, 3, 256, 64, 17, 520, "bf16"),
    (64, 16, 16, 64, 16, 1, 40, "f16"),      # one split
    (1, 2, 1, 128, 48, 1, 1, "bf16"),        # one token
    (2, 32, 1, 128, 16, 100, 900, "bf16"),   # 32 query heads on one key/value head: two blocks of 16
    (2, 40, 2, 64, 32, 1, 300, "f16"),       # 20 per key/value head: a full and a partial block
]


@pytest.mark.parametrize("B,H,Hkv,D,bs,lo,hi,dtype", SMALL, ids=lambda x: str(x))
def test_paged_decode_small(B, H, Hkv, D, bs, lo, hi, dtype):
    w = workloads.DecodeWorkload("decode_small", 200 + B + D + bs, B, H, Hkv, D, bs, lo, hi, dtype)
    log(f"case {w}")
    _decode_check(w, workloads.make_decode_inputs(w), f"B={B} H={H}/{Hkv} D={D} bs={bs} len {lo}..{hi} {dtype}")


def test_paged_decode_workload_and_determinism():
    """The 64-sequence workload (contexts of 512..16000 tokens) on 4 sampled
    sequences, and a repeated call is bitwise identical."""
    import torch

    fa = _fa()
    w = workloads.DECODE_WORKLOADS["decode_gqa_bf16"]
    cpu = workloads.make_decode_inputs(w)
    lens = cpu[4].numpy()
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 1, w.B - 1})
    o16, lse16 = _decode_check(w, cpu, w.name, seqs)
    o2, lse2 = fa.paged_decode(*[t.cuda() for t in cpu], max_context_len=w.hi, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o16.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse16, lse2)


def test_paged_decode_skips_invalid_blocks_and_appends_tokens():
    """A block-table entry of -1 inside a context drops that page's tokens
    (checked against the oracle on the context without that page); a token
    appended with fa_reshape_and_cache is seen by the next decode."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("decode_edit", 301, 3, 8, 2, 128, 16, 100, 400, "f16")
    q, kc, vc, tables, lens = workloads.make_decode_inputs(w)
    t2 = tables.clone()
    t2[1, 2] = -1                      # page 2 of sequence 1 (its tokens 32..47) is invalid
    o, lse = fa.paged_decode(q.cuda(), kc.cuda(), vc.cuda(), t2.cuda(), lens.cuda(), scale=w.scale,
                             out_dtype=torch.float32)
    kept = torch.cat([tables[1, :2], tables[1, 3:]])  # the same pages without page 2
    want, _ = oracle.paged_decode(to_f64(q[1:2]), to_f64(kc), to_f64(vc), kept[None].numpy(),
                                  np.array([int(lens[1]) - 16]), w.scale)
    assert max_abs(to_f64(o[1]), want[0]) <= O_MAX_ABS
    # append one token to every sequence and decode again
    kcg, vcg = kc.cuda(), vc.cuda()
    rng = np.random.default_rng(7)
    new_k = torch.from_numpy(rng.standard_normal((3, 2, 128), dtype=np.float32)).half()
    new_v = torch.from_numpy(rng.standard_normal((3, 2, 128), dtype=np.float32)).half()
    n = lens.numpy().astype(np.int64)
    # the new token's page: the last page, or a block no sequence uses when the last page is full
    tables = torch.cat([tables, torch.full((3, 1), -1, dtype=torch.int32)], dim=1)
    spare = sorted(set(range(kc.shape[0])) - set(tables.flatten().tolist()))
    for b in range(3):
        if n[b] % 16 == 0:
            tables[b, n[b] // 16] = spare.pop()
    slots = np.array([int(tables[b, n[b] // 16]) * 16 + n[b] % 16 for b in range(3)], dtype=np.int64)
    fa.reshape_and_cache(new_k.cuda(), new_v.cuda(), torch.from_numpy(slots).cuda(), kcg, vcg)
    lens2 = lens + 1
    o2, _ = fa.paged_decode(q.cuda(), kcg, vcg, tables.cuda(), lens2.cuda(), scale=w.scale, out_dtype=torch.float32)
    kc2, vc2 = oracle.reshape_and_cache(new_k.float().numpy(), new_v.float().numpy(), slots, kc.float().numpy(),
                                        vc.float().numpy())
    want2, _ = oracle.paged_decode(to_f64(q), kc2, vc2, tables.numpy(), lens2.numpy(), w.scale)
    assert max_abs(to_f64(o2), want2) <= O_MAX_ABS
    log("invalid page skipped and appended token seen")
