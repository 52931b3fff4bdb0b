"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small shapes are compared on every head; the four full-size workloads are run
whole on the GPU and compared with the oracle on sampled heads.  Tolerances:
O max-abs <= 1e-2 (on the fp32 O), dQ/dK/dV normwise relative <= 2e-2, lse
max-abs <= 1e-3.  The 16-bit O must be the round-to-nearest-even cast of the
fp32 O bit for bit, and repeated runs must be bitwise identical.
"""
import numpy as np
import pytest

import workloads
from gpu_util import (GRAD_NORMWISE, LSE_MAX_ABS, O_MAX_ABS, ZERO_REF_MAX_ABS, NormAccumulator, device_inputs, has_gpu, log,
                      max_abs, oracle_head, sample_heads, to_f64)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _run(w, gpu):
    """fwd with fp32 O, fwd with 16-bit O, bwd from the 16-bit O."""
    import torch

    fa = _fa()
    q, k, v, do = gpu
    o32, lse32 = fa.forward(q, k, v, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    o16, lse16 = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward(q, k, v, o16, do, lse16, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o32, lse32, o16, lse16, dq, dk, dv


def _compare(w, cpu, outs, heads, label):
    import torch

    o32, lse32, o16, lse16, dq, dk, dv = outs
    # bitwise: the 16-bit O is RNE(fp32 O) and both calls give the same lse
    assert torch.equal(o16.view(torch.int16), o32.to(o16.dtype).view(torch.int16)), f"{label}: O16 != RNE(O32)"
    assert torch.equal(lse16, lse32), f"{label}: lse differs between O dtypes"
    err_o = err_o16 = err_lse = floor = 0.0
    acc = {n: NormAccumulator() for n in ("dq", "dk", "dv")}
    for z, h in heads:
        r = oracle_head(cpu, z, h, w.scale, w.causal)
        err_o = max(err_o, max_abs(to_f64(o32[z, h]), r["O"]))
        err_o16 = max(err_o16, max_abs(to_f64(o16[z, h]), r["O"]))
        floor = max(floor, max_abs(to_f64(torch.from_numpy(r["O"]).to(o16.dtype)), r["O"]))
        err_lse = max(err_lse, max_abs(to_f64(lse32[z, h]), r["lse"]))
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            acc[name].add(to_f64(t[z, h]), r[name])
    log(f"{label}: heads={len(heads)} O32 max-abs {err_o:.3e} | O{o16.dtype} max-abs {err_o16:.3e} "
        f"(rounding floor {floor:.3e}) | lse {err_lse:.3e} | dq {acc['dq'].value:.3e} dk {acc['dk'].value:.3e} "
        f"dv {acc['dv'].value:.3e}")
    assert err_o <= O_MAX_ABS, f"{label}: O max-abs {err_o}"
    assert err_lse <= LSE_MAX_ABS, f"{label}: lse max-abs {err_lse}"
    for name in ("dq", "dk", "dv"):
        if acc[name].exact_zero:
            assert acc[name].max_abs <= ZERO_REF_MAX_ABS, f"{label}: {name} max-abs {acc[name].max_abs}"
        else:
            assert acc[name].value <= GRAD_NORMWISE, f"{label}: {name} normwise {acc[name].value}"
    return err_o, {n: a.value for n, a in acc.items()}


SMALL = [
    ((2, 2, 300, D), dt, causal) for D in (64, 128, 256) for dt in ("f16", "bf16") for causal in (False, True)
] + [
    ((1, 2, n, 128), "f16", causal) for n in (1, 17, 64, 129, 257) for causal in (False, True)
] + [
    ((1, 1, n, 64), "bf16", True) for n in (2, 200)
] + [
    ((1, 1, n, 256), "f16", causal) for n in (33, 160) for causal in (False, True)
] + [
    # D = 256 with the mask over eight key tiles: every dK/dV unit and dQ item
    # crosses the diagonal, where at this width the waves run their wholly
    # masked tiles instead of skipping them.
    ((2, 4, 1024, 256), "bf16", True),
]


@pytest.mark.parametrize("shape,dtype,causal", SMALL, ids=lambda x: str(x))
def test_small_shapes_all_heads(shape, dtype, causal):
    Z, H, N, D = shape
    seed = 100 + N + D + (7 if causal else 0) + (3 if dtype == "bf16" else 0)
    w = workloads.Workload("small", seed, Z, H, N, D, dtype, causal)
    log(f"case shape={shape} dtype={dtype} causal={causal} seed={seed}")
    cpu, gpu = device_inputs(w)
    outs = _run(w, gpu)
    heads = [(z, h) for z in range(Z) for h in range(H)]
    _compare(w, cpu, outs, heads, f"{shape} {dtype} causal={causal}")


# Error levels these workloads reach (fp32 O max-abs, worst of the dQ / dK / dV
# normwise errors, on the sampled heads).  A result inside the tolerances but
# ten times worse than these points to a lost precision (a dropped fp32
# accumulation, a wrong rounding), so the check below also holds it to
# 10 x these levels.
EXPECTED = {
    "tiny": (1.6e-4, 3.0e-4),
    "d64": (8.0e-5, 3.0e-4),
    "d128_causal": (2.9e-4, 3.3e-4),
    "d256_bf16": (4.1e-4, 2.4e-3),
    "d256_causal_bf16": (3.7e-3, 2.4e-3),
    "long_causal_bf16": (3.3e-3, 3.2e-3),
}


def _full_size_invariants(w, gpu, outs, label):
    """Checks over every head, without the oracle, with bounds from the
    arithmetic (see tests/invariants.py; u = unit roundoff of the input type):

    * sum_j dV_j = sum_i dO_i, sum_j dK_j = 0 (per channel) and
      Q^T dQ = dK^T K (per head, a D x D matrix), each within twice its
      rounding bound;
    * every O row is a convex combination of the value rows it sees (all of
      them, or rows 0..i when causal): per channel between their minimum and
      maximum, up to 2 u max|v| (the rounded P's weights sum to 1 + O(u)).
    A skipped key unit, query tile or head breaks one of them."""
    import torch

    from invariants import backward_ratios, unit_roundoff

    q, k, v, do = gpu
    o32, _, o16, _, dq, dk, dv = outs
    ratios = backward_ratios(q, k, o16, do, dq, dk, dv, w.scale, w.dtype)
    torch.cuda.empty_cache()
    u = unit_roundoff(w.dtype)
    vf = v.float()
    if w.causal:
        hi, lo = torch.cummax(vf, dim=2).values, torch.cummin(vf, dim=2).values
    else:
        hi, lo = vf.amax(dim=2, keepdim=True), vf.amin(dim=2, keepdim=True)
    slack = 2 * u * vf.abs().amax(dim=(2, 3), keepdim=True)
    outside = float(torch.clamp(torch.maximum(o32 - hi, lo - o32) - slack, min=0).max())
    log(f"{label}: full-size identities at " + ", ".join(f"{n} {r:.3f}" for n, r in ratios.items()) +
        f" of their bounds | O outside the V hull by {outside:.2e}")
    for n, r in ratios.items():
        assert r <= 1.0, f"{label}: {n} identity broken beyond its rounding bound ({r})"
    assert outside == 0.0, f"{label}: an O row leaves the convex hull of its value rows"
    assert bool(torch.isfinite(o32).all()), f"{label}: non-finite O"


@pytest.mark.parametrize("name", ["tiny", "d64", "d128_causal", "d256_bf16", "d256_causal_bf16", "long_causal_bf16"])
def test_workload_parity(name):
    import torch

    w = workloads.by_name(name)
    log(f"workload {name}: shape={w.shape} dtype={w.dtype} causal={w.causal} seed={w.seed}")
    cpu, gpu = device_inputs(w)
    outs = _run(w, gpu)
    heads = sample_heads(w, 2 if w.N > 4096 else 3)
    err_o, grads = _compare(w, cpu, outs, heads, name)
    lvl_o, lvl_g = EXPECTED[name]
    assert err_o <= 10 * lvl_o, f"{name}: O error {err_o:.2e} is over 10x its usual {lvl_o:.1e}"
    assert max(grads.values()) <= 10 * lvl_g, f"{name}: gradient error {grads} over 10x its usual {lvl_g:.1e}"
    _full_size_invariants(w, gpu, outs, name)
    # determinism: a second backward is bitwise identical
    fa = _fa()
    q, k, v, do = gpu
    dq2, dk2, dv2 = fa.backward(q, k, v, outs[2], do, outs[3], causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in ((outs[4], dq2, "dq"), (outs[5], dk2, "dk"), (outs[6], dv2, "dv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: {n} not deterministic"


@pytest.mark.parametrize("Z,H,N,D,dtype", [(2, 4, 1000, 128, "f16"), (1, 4, 600, 256, "bf16")])
def test_dkdv_bitwise_independent_of_grid_size(Z, H, N, D, dtype):
    """No atomics and a fixed accumulation order: any persistent grid size gives the same bits."""
    import torch

    fa = _fa()
    w = workloads.Workload("grid", 77, Z, H, N, D, dtype, True)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    stats = fa.bwd_preprocess(o, do, lse)
    cus, default = fa.device_info(D, fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F16)
    log(f"device: {cus} CUs, default dK/dV grid {default}")
    ref = fa.bwd_dkdv(q, k, v, do, stats, causal=True, scale=w.scale, num_programs=0)
    for P in (1, 7, cus, 3 * cus + 1):
        dk, dv = fa.bwd_dkdv(q, k, v, do, stats, causal=True, scale=w.scale, num_programs=P)
        torch.cuda.synchronize()
        assert torch.equal(dk.view(torch.int16), ref[0].view(torch.int16)), f"dk differs at P={P}"
        assert torch.equal(dv.view(torch.int16), ref[1].view(torch.int16)), f"dv differs at P={P}"


@pytest.mark.parametrize("shape,dtype,causal,o32", [
    ((1, 3, 333, 64), "bf16", False, False),
    ((2, 2, 300, 128), "f16", True, True),
    ((1, 2, 200, 256), "bf16", True, False),
])
def test_stages_match_fused_backward(shape, dtype, causal, o32):
    """fa_bwd (dQ with the row statistics, then dK/dV) == preprocess + dK/dV +
    dQ called one by one, bit for bit; the statistics the dQ pass computes
    equal the preprocess pass's bit for bit (Delta is checked in fp64 against
    the stored O and dO, lse * log2 e against lse)."""
    import torch

    fa = _fa()
    Z, H, N, D = shape
    w = workloads.Workload("stages", 91 + D, Z, H, N, D, dtype, causal)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    log(f"case shape={shape} dtype={dtype} causal={causal} o32={o32}")
    o, lse = fa.forward(q, k, v, causal=causal, scale=w.scale, out_dtype=torch.float32 if o32 else None)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=w.scale)
    stats = fa.bwd_preprocess(o, do, lse)
    dk2, dv2 = fa.bwd_dkdv(q, k, v, do, stats, causal=causal, scale=w.scale)
    dq2 = fa.bwd_dq(q, k, v, do, stats, causal=causal, scale=w.scale)
    dq3, stats3 = fa.bwd_dq_and_stats(q, k, v, o, do, lse, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv"), (dq3, dq2, "dq (fused stats)")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
    assert torch.equal(stats3.view(torch.int32), stats.view(torch.int32)), "statistics differ"
    # Delta from the stored O, in fp64 on the host
    want = np.sum(to_f64(o) * to_f64(do), axis=-1)
    assert max_abs(to_f64(stats[0]), want) <= 1e-4 * max(1.0, float(np.max(np.abs(want))))
    lse2 = to_f64(lse) * np.log2(np.e)
    assert max_abs(to_f64(stats[1]), lse2) <= 1e-6 * max(1.0, float(np.max(np.abs(lse2))))


def test_negative_controls_fail_the_check():
    """The comparison must turn red on a wrong answer: swapped K/V, flipped
    causal flag, one perturbed input element."""
    import torch

    fa = _fa()
    w = workloads.Workload("neg", 5, 1, 1, 256, 64, "f16", True)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    r = oracle_head(cpu, 0, 0, w.scale, True)
    o, _ = fa.forward(v.contiguous(), k, q.contiguous(), causal=True, scale=w.scale, out_dtype=torch.float32)
    assert max_abs(to_f64(o[0, 0]), r["O"]) > O_MAX_ABS
    o, _ = fa.forward(q, k, v, causal=False, scale=w.scale, out_dtype=torch.float32)
    assert max_abs(to_f64(o[0, 0]), r["O"]) > O_MAX_ABS
    v2 = v.clone()
    v2[0, 0, 0, 0] += 4.0
    o, _ = fa.forward(q, k, v2, causal=True, scale=w.scale, out_dtype=torch.float32)
    assert max_abs(to_f64(o[0, 0]), r["O"]) > O_MAX_ABS


def test_empty_problem_and_errors():
    import torch

    fa = _fa()
    q = torch.empty((0, 2, 16, 64), dtype=torch.float16, device="cuda")
    o, lse = fa.forward(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    bad = torch.zeros((1, 1, 16, 96), dtype=torch.float16, device="cuda")
    with pytest.raises(fa.FAError) as ei:
        fa.forward(bad, bad, bad)
    assert ei.value.status == 2  # FA_ERR_UNSUPPORTED


def test_autograd_attention_matches_explicit_calls():
    """fa.attention under torch autograd gives the explicit forward / backward
    results bit for bit (plain and grouped heads)."""
    import torch

    fa = _fa()
    for (Z, H, Hkv, N, D, causal) in ((1, 4, 4, 200, 64, True), (2, 8, 2, 129, 128, False)):
        w = workloads.Workload("autograd", 41 + H, Z, H, N, D, "f16", causal, 1.0, Hkv)
        cpu, gpu = device_inputs(w)
        q, k, v, do = (t.clone().requires_grad_(i < 3) for i, t in enumerate(gpu))
        o = fa.attention(q, k, v, causal=causal, scale=w.scale)
        o.backward(do)
        o2, lse2 = fa.forward(gpu[0], gpu[1], gpu[2], causal=causal, scale=w.scale)
        dq2, dk2, dv2 = fa.backward(gpu[0], gpu[1], gpu[2], o2, gpu[3], lse2, causal=causal, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.detach().view(torch.int16), o2.view(torch.int16))
        for a, b in ((q.grad, dq2), (k.grad, dk2), (v.grad, dv2)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
