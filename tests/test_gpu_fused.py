"""GPU parity of the fused per-head backward (fa_bwd_fused: dQ, dK, dV of a
head from one persistent workgroup) against the fp64 oracle, through the C
ABI: small shapes on every head, the five workloads on sampled heads plus the
oracle-free identities on every head, bitwise independence of the program
count, repeatability, and agreement with the two-pass backward."""
import pytest

import workloads
from gpu_util import (GRAD_NORMWISE, ZERO_REF_MAX_ABS, NormAccumulator, device_inputs, has_gpu, log, oracle_head,
                      sample_heads, to_f64)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _fused(w, gpu, num_programs=0):
    """forward (16-bit O), the statistics pass, then the fused backward."""
    import torch

    fa = _fa()
    q, k, v, do = gpu
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    stats = fa.bwd_preprocess(o, do, lse)
    dq, dk, dv = fa.bwd_fused(q, k, v, do, stats, causal=w.causal, scale=w.scale, num_programs=num_programs)
    torch.cuda.synchronize()
    return o, lse, stats, (dq, dk, dv)


def _compare_grads(w, cpu, grads, heads, label):
    dq, dk, dv = grads
    acc = {n: NormAccumulator() for n in ("dq", "dk", "dv")}
    for z, h in heads:
        r = oracle_head(cpu, z, h, w.scale, w.causal)
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            acc[name].add(to_f64(t[z, h]), r[name])
    log(f"{label}: heads={len(heads)} fused dq {acc['dq'].value:.3e} dk {acc['dk'].value:.3e} "
        f"dv {acc['dv'].value:.3e}")
    for name in ("dq", "dk", "dv"):
        if acc[name].exact_zero:
            assert acc[name].max_abs <= ZERO_REF_MAX_ABS, f"{label}: {name} max-abs {acc[name].max_abs}"
        else:
            assert acc[name].value <= GRAD_NORMWISE, f"{label}: {name} normwise {acc[name].value}"
    return {n: a.value for n, a in acc.items()}


SMALL = [
    ((2, 2, 300, D), dt, causal) for D in (64, 128, 256) for dt in ("f16", "bf16") for causal in (False, True)
] + [
    ((1, 2, n, 128), "f16", causal) for n in (1, 17, 64, 129, 257, 513) for causal in (False, True)
] + [
    ((1, 3, n, 64), "bf16", True) for n in (2, 200)
] + [
    ((1, 1, n, 256), "f16", causal) for n in (33, 160) for causal in (False, True)
]


@pytest.mark.parametrize("shape,dtype,causal", SMALL, ids=lambda x: str(x))
def test_fused_small_shapes_all_heads(shape, dtype, causal):
    Z, H, N, D = shape
    seed = 300 + N + D + (7 if causal else 0) + (3 if dtype == "bf16" else 0)
    w = workloads.Workload("fused_small", seed, Z, H, N, D, dtype, causal)
    log(f"case shape={shape} dtype={dtype} causal={causal} seed={seed}")
    cpu, gpu = device_inputs(w)
    _, _, _, grads = _fused(w, gpu)
    _compare_grads(w, cpu, grads, [(z, h) for z in range(Z) for h in range(H)], f"{shape} {dtype} causal={causal}")


# Gradient error levels of the two-pass backward on these workloads (worst of
# dQ / dK / dV on the sampled heads); the fused pass rounds the same products
# and must stay within 10x of them.
EXPECTED_GRAD = {"tiny": 3.0e-4, "d64": 3.0e-4, "d128_causal": 3.3e-4, "d256_bf16": 2.4e-3,
                 "long_causal_bf16": 3.2e-3}


@pytest.mark.parametrize("name", ["tiny", "d64", "d128_causal", "d256_bf16", "long_causal_bf16"])
def test_fused_workload_parity(name):
    import torch

    from invariants import backward_ratios

    fa = _fa()
    w = workloads.by_name(name)
    log(f"workload {name}: shape={w.shape} dtype={w.dtype} causal={w.causal} seed={w.seed}")
    cpu, gpu = device_inputs(w)
    o, lse, stats, grads = _fused(w, gpu)
    errs = _compare_grads(w, cpu, grads, sample_heads(w, 2 if w.N > 4096 else 3), name)
    assert max(errs.values()) <= 10 * EXPECTED_GRAD[name], (name, errs)
    q, k, v, do = gpu
    ratios = backward_ratios(q, k, o, do, *grads, w.scale, w.dtype)
    log(f"{name}: fused full-size identities at {ratios} of their bounds")
    assert max(ratios.values()) <= 1.0, ratios
    # repeatable bit for bit
    again = fa.bwd_fused(q, k, v, do, stats, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in zip(grads, again, ("dq", "dk", "dv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: {n} not deterministic"
    # the two-pass backward computes the same gradients (summation orders differ)
    split = fa.backward(q, k, v, o, do, lse, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for a, b, n in zip(grads, split, ("dq", "dk", "dv")):
        rel = float((a.double() - b.double()).norm() / b.double().norm())
        log(f"{name}: fused vs two-pass {n} normwise {rel:.2e}")
        assert rel <= 2 * EXPECTED_GRAD[name], (name, n, rel)


def test_fused_bitwise_independent_of_program_count():
    """Every head is computed by one program in a fixed order, so any grid
    size gives the same bits."""
    import torch

    fa = _fa()
    w = workloads.Workload("fused_grid", 78, 2, 5, 700, 128, "f16", True)
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    o, lse, stats, ref = _fused(w, gpu)
    cus, _ = fa.device_info(128, fa.FA_DTYPE_F16)
    for P in (1, 3, 7, cus, 3 * cus + 1):
        got = fa.bwd_fused(q, k, v, do, stats, causal=True, scale=w.scale, num_programs=P)
        torch.cuda.synchronize()
        for a, b, n in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n} differs at P={P}"
        log(f"program count {P}: bitwise equal")


def test_fused_argument_errors():
    import torch

    fa = _fa()
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda")
    o, lse = fa.forward(q, q, q)
    stats = fa.bwd_preprocess(o, q, lse)
    small = torch.empty((8,), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as ei:
        fa.bwd_fused(q, q, q, q, stats, workspace=small)
    assert ei.value.status == 1 and "workspace" in ei.value.detail
