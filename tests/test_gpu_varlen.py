"""GPU parity of packed variable-length batches (fa_fwd_varlen /
fa_bwd_varlen) against the fp64 oracle's variable-length functions (the page
"从算子到 Serving：昇腾推理评测链路实践": sequences of different real lengths in
one batch, tokens past a sequence's end taking no part).  Layout (H, T, D) /
(Hkv, T, D), sequences at cu_seqlens offsets.  Tolerances as for plain
attention; sequences are compared one by one over all their heads.
"""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import (GRAD_NORMWISE, LSE_MAX_ABS, O_MAX_ABS, ZERO_REF_MAX_ABS, NormAccumulator, has_gpu, log, max_abs,
                      oracle_varlen_group, to_f64, varlen_device_inputs)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _run(w, gpu, cu):
    import torch

    fa = _fa()
    q, k, v, do = gpu
    mx = max(w.lengths) if w.lengths else 0
    o32, lse32 = fa.forward_varlen(q, k, v, cu, mx, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    o16, lse16 = fa.forward_varlen(q, k, v, cu, mx, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward_varlen(q, k, v, o16, do, lse16, cu, mx, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o32, lse32, o16, lse16, dq, dk, dv


def _compare(w, cpu, outs, seqs, label):
    import torch

    o32, lse32, o16, lse16, dq, dk, dv = outs
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), f"{label}: O16 != RNE(O32)"
    assert torch.equal(lse16, lse32), f"{label}: lse differs between O dtypes"
    cu = w.cu_seqlens
    err_o = err_lse = 0.0
    acc = {n: NormAccumulator() for n in ("dq", "dk", "dv")}
    for b in seqs:
        if cu[b + 1] == cu[b]:
            continue
        for kvh in range(w.kv_heads):
            r = oracle_varlen_group(cpu, cu, b, kvh, w.scale, w.causal)
            rows = r["rows"]
            for i, h in enumerate(r["heads"]):
                err_o = max(err_o, max_abs(to_f64(o32[h, rows]), r["O"][i]))
                err_lse = max(err_lse, max_abs(to_f64(lse32[h, rows]), r["lse"][i]))
                acc["dq"].add(to_f64(dq[h, rows]), r["dq"][i])
            acc["dk"].add(to_f64(dk[kvh, rows]), r["dk"])
            acc["dv"].add(to_f64(dv[kvh, rows]), r["dv"])
    log(f"{label}: sequences={len(seqs)} O32 max-abs {err_o:.3e} | lse {err_lse:.3e} | dq {acc['dq'].value:.3e} "
        f"dk {acc['dk'].value:.3e} dv {acc['dv'].value:.3e}")
    assert err_o <= O_MAX_ABS, f"{label}: O max-abs {err_o}"
    assert err_lse <= LSE_MAX_ABS, f"{label}: lse max-abs {err_lse}"
    for name in ("dq", "dk", "dv"):
        if acc[name].exact_zero:
            assert acc[name].max_abs <= ZERO_REF_MAX_ABS, f"{label}: {name} max-abs {acc[name].max_abs}"
        else:
            assert acc[name].value <= GRAD_NORMWISE, f"{label}: {name} normwise {acc[name].value}"


SMALL = [
    # lengths, H, Hkv, D, dtype, causal
    ((1, 0, 17, 128, 300), 4, 2, 64, "f16", True),
    ((1, 0, 17, 128, 300), 4, 4, 64, "bf16", False),
    ((129, 33, 256, 5), 2, 1, 128, "f16", True),
    ((200, 7, 64), 3, 3, 128, "bf16", False),
    ((160, 1, 40), 2, 2, 256, "f16", True),
    ((97, 250), 4, 1, 256, "bf16", False),
    ((513, 2, 1000, 31, 64, 400), 8, 2, 128, "bf16", True),
]


@pytest.mark.parametrize("lengths,H,Hkv,D,dtype,causal", SMALL, ids=lambda x: str(x))
def test_varlen_small_batches_all_sequences(lengths, H, Hkv, D, dtype, causal):
    seed = 500 + sum(lengths) % 97 + D + H
    w = workloads.Workload("varlen_small", seed, len(lengths), H, max(lengths), D, dtype, causal, 1.0, Hkv,
                           tuple(lengths))
    log(f"case lengths={lengths} H={H} Hkv={Hkv} D={D} dtype={dtype} causal={causal} seed={seed}")
    cpu, gpu, cu = varlen_device_inputs(w)
    outs = _run(w, gpu, cu)
    _compare(w, cpu, outs, list(range(len(lengths))), f"{lengths} H={H}/{Hkv} D={D} {dtype} causal={causal}")


def test_varlen_workload_parity_and_determinism():
    """The 32-sequence workload at full size: the shortest, the longest and
    one middle sequence against the oracle; a second backward is bitwise
    identical."""
    import torch

    fa = _fa()
    w = workloads.by_name("varlen_causal_bf16")
    log(f"workload {w.name}: B={w.Z} H={w.H} T={w.T} max={w.N} D={w.D} {w.dtype} causal={w.causal}")
    cpu, gpu, cu = varlen_device_inputs(w)
    outs = _run(w, gpu, cu)
    L = np.asarray(w.lengths)
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), len(L) // 2})
    o32, lse32, o16, lse16, dq, dk, dv = outs
    err_o = 0.0
    acc = {n: NormAccumulator() for n in ("dq", "dk", "dv")}
    # one key/value head (first and last by turns) per sampled sequence keeps the oracle to seconds
    for i, b in enumerate(seqs):
        kvh = 0 if i % 2 == 0 else w.kv_heads - 1
        r = oracle_varlen_group(cpu, w.cu_seqlens, b, kvh, w.scale, w.causal)
        rows = r["rows"]
        for i, h in enumerate(r["heads"]):
            err_o = max(err_o, max_abs(to_f64(o32[h, rows]), r["O"][i]))
            acc["dq"].add(to_f64(dq[h, rows]), r["dq"][i])
        acc["dk"].add(to_f64(dk[kvh, rows]), r["dk"])
        acc["dv"].add(to_f64(dv[kvh, rows]), r["dv"])
    log(f"{w.name}: sequences {seqs} (lengths {[int(L[b]) for b in seqs]}) O32 max-abs {err_o:.3e} | "
        f"dq {acc['dq'].value:.3e} dk {acc['dk'].value:.3e} dv {acc['dv'].value:.3e}")
    assert err_o <= O_MAX_ABS
    for name in ("dq", "dk", "dv"):
        assert acc[name].value <= GRAD_NORMWISE, (name, acc[name].value)
    q, k, v, do = gpu
    from invariants import backward_ratios_varlen

    ratios = backward_ratios_varlen(q, k, o16, do, dq, dk, dv, w.cu_seqlens, w.scale, w.dtype)
    log(f"{w.name}: identities over every sequence at {ratios} of their bounds")
    assert max(ratios.values()) <= 1.0, ratios
    dq2, dk2, dv2 = fa.backward_varlen(q, k, v, o16, do, lse16, cu, w.N, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b_, n in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), f"{n} not deterministic"


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_equal_dense_batch(causal):
    """Equal lengths: the packed batch is the dense (Z, H, N, D) batch with
    its axes reordered, and every output is bit for bit the dense one."""
    import torch

    fa = _fa()
    Z, H, Hkv, N, D = 3, 4, 2, 200, 128
    w = workloads.Workload("varlen_eq", 29, Z, H, N, D, "f16", causal, 1.0, Hkv, (N,) * Z)
    cpu, gpu, cu = varlen_device_inputs(w)
    q, k, v, do = gpu
    o, lse = fa.forward_varlen(q, k, v, cu, N, causal=causal, scale=w.scale)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, N, causal=causal, scale=w.scale)

    def dense(t):  # (heads, Z*N, D) -> (Z, heads, N, D)
        return t.reshape(t.shape[0], Z, N, D).permute(1, 0, 2, 3).contiguous()

    qd, kd, vd, dod = (dense(t) for t in (q, k, v, do))
    od, lsed = fa.forward(qd, kd, vd, causal=causal, scale=w.scale)
    dqd, dkd, dvd = fa.backward(qd, kd, vd, od, dod, lsed, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in ((o, od, "o"), (dq, dqd, "dq"), (dk, dkd, "dk"), (dv, dvd, "dv")):
        assert torch.equal(dense(a).view(torch.int16), b.view(torch.int16)), n
    assert torch.equal(lse.reshape(H, Z, N).permute(1, 0, 2), lsed)


def test_varlen_rows_of_other_sequences_are_untouched():
    """Outputs are written only inside each sequence's rows: a batch whose
    offsets leave a gap of tokens (cu_seqlens[-1] < T) keeps the gap's
    prefilled values in O, lse, dQ, dK and dV."""
    import torch

    fa = _fa()
    H, Hkv, D, T = 2, 1, 64, 300
    gen = torch.Generator().manual_seed(5)
    q, do = (torch.randn((H, T, D), generator=gen).half().cuda() for _ in range(2))
    k, v = (torch.randn((Hkv, T, D), generator=gen).half().cuda() for _ in range(2))
    cu = torch.tensor([0, 100, 250], dtype=torch.int32, device="cuda")  # tokens 250..299 belong to no sequence
    lib = fa.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    o = torch.full((H, T, D), 7.0, dtype=torch.float16, device="cuda")
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device="cuda")
    assert lib.fa_fwd_varlen(2, H, Hkv, T, 150, D, 0, 0, p(cu), p(q), p(k), p(v), p(o), p(lse), 0.125, 1, None) == 0
    grads = [torch.full_like(t, 7.0) for t in (q, k, v)]
    ws = torch.empty((fa.workspace_bytes(1, H, T, D) // 4,), dtype=torch.float32, device="cuda")
    st = lib.fa_bwd_varlen(2, H, Hkv, T, 150, D, 0, 0, p(cu), p(q), p(k), p(v), p(o), p(do), p(lse),
                           *(p(g) for g in grads), 0.125, 1, p(ws), ws.numel() * 4, None)
    assert st == 0, fa.last_error()
    torch.cuda.synchronize()
    for t, n in ((o, "o"), (lse, "lse"), (grads[0], "dq"), (grads[1], "dk"), (grads[2], "dv")):
        assert bool((t[:, 250:] == 7.0).all()), f"{n} written past the last sequence"
        assert not bool((t[:, :250] == 7.0).all()), f"{n} not written"


def test_varlen_stage_forms_equal_fused_backward():
    """fa_bwd_dq_and_stats_varlen then fa_bwd_dkdv_varlen give fa_bwd_varlen's bits."""
    import torch

    fa = _fa()
    lib = fa.lib()
    lengths = (77, 0, 300, 129)
    H, Hkv, D = 4, 2, 64
    w = workloads.Workload("varlen_stages", 37, len(lengths), H, max(lengths), D, "f16", True, 1.0, Hkv, lengths)
    cpu, gpu, cu = varlen_device_inputs(w)
    q, k, v, do = gpu
    T, mx = w.T, max(lengths)
    o, lse = fa.forward_varlen(q, k, v, cu, mx, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, mx, causal=True, scale=w.scale)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stats = torch.empty((2, H, T), dtype=torch.float32, device="cuda")
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    assert lib.fa_bwd_dq_and_stats_varlen(len(lengths), H, Hkv, T, mx, D, 0, 0, p(cu), p(q), p(k), p(v), p(o), p(do),
                                          p(lse), p(stats), p(dq2), w.scale, 1, None) == 0, fa.last_error()
    assert lib.fa_bwd_dkdv_varlen(len(lengths), H, Hkv, T, mx, D, 0, p(cu), p(q), p(k), p(v), p(do), p(stats), p(dk2),
                                  p(dv2), w.scale, 1, 0, None) == 0, fa.last_error()
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
