"""GPU parity of grouped key/value heads (GQA, and MQA with one key/value
head): fa_fwd_gqa / fa_bwd_gqa against the fp64 oracle's grouped functions
(the page "从算子到 Serving：昇腾推理评测链路实践", section "GQA Paged
Attention": query head h uses key/value head h // G, G = H / Hkv, and a shared
head's dK, dV sum over its G query heads).  Tolerances as for plain attention.
"""
import ctypes

import pytest

import workloads
from gpu_util import (GRAD_NORMWISE, LSE_MAX_ABS, O_MAX_ABS, NormAccumulator, device_inputs, has_gpu, log, max_abs,
                      oracle_group, to_f64)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _run(w, gpu):
    import torch

    fa = _fa()
    q, k, v, do = gpu
    o32, lse32 = fa.forward(q, k, v, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    o16, lse16 = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o16, do, lse16, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o32, lse32, o16, lse16, dq, dk, dv


def _compare(w, cpu, outs, groups, label):
    """Compare the key/value heads `groups` ((z, kvh) pairs) and all their query heads."""
    import torch

    o32, lse32, o16, lse16, dq, dk, dv = outs
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), f"{label}: O16 != RNE(O32)"
    assert torch.equal(lse16, lse32), f"{label}: lse differs between O dtypes"
    err_o = err_lse = 0.0
    acc = {n: NormAccumulator() for n in ("dq", "dk", "dv")}
    for z, kvh in groups:
        r = oracle_group(cpu, z, kvh, w.scale, w.causal)
        for i, h in enumerate(r["heads"]):
            err_o = max(err_o, max_abs(to_f64(o32[z, h]), r["O"][i]))
            err_lse = max(err_lse, max_abs(to_f64(lse32[z, h]), r["lse"][i]))
            acc["dq"].add(to_f64(dq[z, h]), r["dq"][i])
        acc["dk"].add(to_f64(dk[z, kvh]), r["dk"])
        acc["dv"].add(to_f64(dv[z, kvh]), r["dv"])
    log(f"{label}: kv heads={len(groups)} O32 max-abs {err_o:.3e} | lse {err_lse:.3e} | dq {acc['dq'].value:.3e} "
        f"dk {acc['dk'].value:.3e} dv {acc['dv'].value:.3e}")
    assert err_o <= O_MAX_ABS, f"{label}: O max-abs {err_o}"
    assert err_lse <= LSE_MAX_ABS, f"{label}: lse max-abs {err_lse}"
    for name in ("dq", "dk", "dv"):
        assert acc[name].value <= GRAD_NORMWISE, f"{label}: {name} normwise {acc[name].value}"


SMALL = [
    # (Z, H, Hkv, N, D), dtype, causal
    ((2, 4, 2, 300, 64), "f16", False),
    ((2, 4, 2, 300, 64), "bf16", True),
    ((2, 4, 1, 300, 128), "bf16", True),     # MQA
    ((1, 8, 2, 129, 128), "f16", False),
    ((1, 6, 3, 257, 128), "f16", True),
    ((1, 4, 2, 160, 256), "bf16", True),
    ((1, 4, 1, 33, 256), "f16", False),
    ((3, 3, 1, 17, 64), "bf16", True),
    ((1, 16, 1, 1000, 128), "f16", True),    # MQA, 16 query heads on one key/value head
]


@pytest.mark.parametrize("shape,dtype,causal", SMALL, ids=lambda x: str(x))
def test_gqa_small_shapes_all_heads(shape, dtype, causal):
    Z, H, Hkv, N, D = shape
    seed = 300 + N + D + H + Hkv + (7 if causal else 0)
    w = workloads.Workload("gqa_small", seed, Z, H, N, D, dtype, causal, 1.0, Hkv)
    log(f"case shape={shape} dtype={dtype} causal={causal} seed={seed}")
    cpu, gpu = device_inputs(w)
    outs = _run(w, gpu)
    _compare(w, cpu, outs, [(z, g) for z in range(Z) for g in range(Hkv)], f"{shape} {dtype} causal={causal}")


def test_gqa_workload_parity_and_determinism():
    """The grouped workload at full size, compared on sampled key/value heads
    (each with its 4 query heads); a second backward is bitwise identical."""
    import torch

    fa = _fa()
    w = workloads.by_name("gqa_causal_bf16")
    log(f"workload {w.name}: shape={w.shape} kv_heads={w.kv_heads} dtype={w.dtype} causal={w.causal}")
    cpu, gpu = device_inputs(w)
    outs = _run(w, gpu)
    _compare(w, cpu, outs, [(0, 0), (w.Z - 1, w.kv_heads - 1)], w.name)
    q, k, v, do = gpu
    from invariants import backward_ratios

    ratios = backward_ratios(q, k, outs[2], do, outs[4], outs[5], outs[6], w.scale, w.dtype)
    log(f"{w.name}: full-size identities at {ratios} of their bounds")
    assert max(ratios.values()) <= 1.0, ratios
    dq2, dk2, dv2 = fa.backward(q, k, v, outs[2], do, outs[3], causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in ((outs[4], dq2, "dq"), (outs[5], dk2, "dk"), (outs[6], dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n} not deterministic"


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_heads(causal):
    """Forward and dQ of the grouped call equal, bit for bit, plain attention
    on K and V repeated per query head (the same per-head arithmetic); dK and
    dV equal the group sums of the plain call's per-head gradients to fp32
    summation order."""
    import torch

    fa = _fa()
    Z, H, Hkv, N, D = 2, 8, 2, 333, 128
    w = workloads.Workload("gqa_rep", 17, Z, H, N, D, "f16", causal, 1.0, Hkv)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    G = H // Hkv
    kr, vr = (t.repeat_interleave(G, dim=1).contiguous() for t in (k, v))
    o, lse = fa.forward(q, k, v, causal=causal, scale=w.scale)
    o_r, lse_r = fa.forward(q, kr, vr, causal=causal, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=w.scale)
    dq_r, dk_r, dv_r = fa.backward(q, kr, vr, o_r, do, lse_r, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_r.view(torch.int16))
    assert torch.equal(lse, lse_r)
    assert torch.equal(dq.view(torch.int16), dq_r.view(torch.int16))
    for a, b, n in ((dk, dk_r, "dk"), (dv, dv_r, "dv")):
        want = b.float().reshape(Z, Hkv, G, N, D).sum(2)
        err = ((a.float() - want).norm() / want.norm()).item()
        log(f"causal={causal} {n}: grouped vs summed repeated heads normwise {err:.3e}")
        assert err <= 2e-3, (n, err)


def test_gqa_entry_points_with_one_group_are_plain_attention():
    """fa_fwd_gqa / fa_bwd_gqa with Hkv = H are fa_fwd / fa_bwd bit for bit."""
    import torch

    fa = _fa()
    lib = fa.lib()
    Z, H, N, D = 1, 4, 250, 64
    w = workloads.Workload("gqa_one", 23, Z, H, N, D, "bf16", True)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, scale=w.scale)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.fa_fwd_gqa(Z, H, H, N, D, 1, 1, p(q), p(k), p(v), p(o2), p(lse2), w.scale, 1, None)
    assert st == 0, fa.last_error()
    ws = torch.empty((fa.workspace_bytes(Z, H, N, D) // 4,), dtype=torch.float32, device="cuda")
    st = lib.fa_bwd_gqa(Z, H, H, N, D, 1, 1, p(q), p(k), p(v), p(o), p(do), p(lse), p(dq2), p(dk2), p(dv2),
                        w.scale, 1, p(ws), ws.numel() * 4, None)
    assert st == 0, fa.last_error()
    torch.cuda.synchronize()
    for a, b in ((o, o2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse, lse2)


def test_gqa_shape_errors():
    import torch

    fa = _fa()
    q = torch.zeros((1, 6, 64, 64), dtype=torch.float16, device="cuda")
    k = torch.zeros((1, 4, 64, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        fa.forward(q, k, k)  # 6 query heads over 4 key/value heads
    with pytest.raises(ValueError):
        fa.forward(q, k[:, :2], k[:, :3].contiguous())  # k and v differ


def test_gqa_stage_forms_equal_fused_backward():
    """fa_bwd_dq_and_stats_gqa then fa_bwd_dkdv_gqa (what a caller timing or
    scheduling the stages runs) give fa_bwd_gqa's bits."""
    import torch

    fa = _fa()
    lib = fa.lib()
    Z, H, Hkv, N, D = 2, 6, 2, 300, 128
    w = workloads.Workload("gqa_stages", 31, Z, H, N, D, "bf16", True, 1.0, Hkv)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, scale=w.scale)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stats = torch.empty((2, Z, H, N), dtype=torch.float32, device="cuda")
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    assert lib.fa_bwd_dq_and_stats_gqa(Z, H, Hkv, N, D, 1, 1, p(q), p(k), p(v), p(o), p(do), p(lse), p(stats),
                                       p(dq2), w.scale, 1, None) == 0, fa.last_error()
    assert lib.fa_bwd_dkdv_gqa(Z, H, Hkv, N, D, 1, p(q), p(k), p(v), p(do), p(stats), p(dk2), p(dv2), w.scale, 1, 0,
                               None) == 0, fa.last_error()
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
