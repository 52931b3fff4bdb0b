"""The oracle-free full-size checks (tests/invariants.py) pass on correct
gradients rounded to the input type and fail on planted one-head mistakes.
CPU only: the correct gradients come from the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from invariants import backward_ratios, backward_ratios_varlen


def _exact(w):
    """Inputs and oracle results of a dense (possibly grouped) workload, the
    outputs rounded to its dtype as the kernels store them."""
    q, k, v, do = workloads.make_inputs(w)
    dt = q.dtype
    f = lambda t: t.double().numpy()  # noqa: E731
    O, _ = oracle.attention_forward_gqa(f(q), f(k), f(v), w.scale, w.causal)
    dq, dk, dv = oracle.attention_backward_gqa(f(q), f(k), f(v), f(do), w.scale, w.causal)
    r = lambda a: torch.from_numpy(a).to(dt)  # noqa: E731  (RNE cast)
    return q, k, v, do, r(O), r(dq), r(dk), r(dv)


CASES = [
    workloads.Workload("inv", 31, 2, 4, 192, 64, "f16", False),
    workloads.Workload("inv", 32, 2, 4, 160, 128, "f16", True),
    workloads.Workload("inv", 33, 1, 4, 256, 64, "bf16", True, 2.0),
    workloads.Workload("inv", 34, 2, 4, 128, 64, "bf16", False, 1.0, 2),  # grouped: Hkv = 2
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"H{w.H}kv{w.kv_heads}N{w.N}D{w.D}{w.dtype}c{int(w.causal)}")
def test_invariants_hold_on_rounded_exact_gradients(w):
    q, k, v, do, o, dq, dk, dv = _exact(w)
    r = backward_ratios(q, k, o, do, dq, dk, dv, w.scale, w.dtype)
    assert max(r.values()) <= 1.0, r


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"H{w.H}kv{w.kv_heads}N{w.N}D{w.D}{w.dtype}c{int(w.causal)}")
def test_planted_one_head_mistakes_fail(w):
    """Each plausible mistake confined to one head (a swapped head, a skipped
    key tile, a missing scale, dS without the Delta term) breaks an identity."""
    q, k, v, do, o, dq, dk, dv = _exact(w)
    Hkv = k.shape[1]
    name = lambda **kw: max(backward_ratios(**{**dict(q=q, k=k, o=o, do=do, dq=dq, dk=dk, dv=dv),  # noqa: E731
                                               **kw}, scale=w.scale, dtype=w.dtype).values())

    other = (w.Z - 1, Hkv - 1) if (w.Z, Hkv) != (1, 1) else None
    if other is not None and other != (0, 0):
        dk2 = dk.clone()
        dk2[0, 0] = dk[other]
        assert name(dk=dk2) > 1.0, "dK of another head not caught"
        dv2 = dv.clone()
        dv2[0, 0] = dv[other]
        assert name(dv=dv2) > 1.0, "dV of another head not caught"
        dq2 = dq.clone()
        dq2[0, 0] = dq[w.Z - 1, w.H - 1]
        assert name(dq=dq2) > 1.0, "dQ of another head not caught"
    dk2 = dk.clone()
    dk2[0, 0, 32:64] = 0
    assert name(dk=dk2) > 1.0, "skipped key tile not caught"
    dq2 = dq.clone()
    dq2[0, 0] *= 1.25
    assert name(dq=dq2) > 1.0, "wrong dQ scale on one head not caught"
    # dS = scale * P * dP (the Delta term dropped) on the first key/value head
    f = lambda t: t.double().numpy()  # noqa: E731
    G = w.H // Hkv
    dk2 = dk.clone()
    acc = 0.0
    for m in range(G):
        fw = oracle.attention_forward_full(f(q[0, m]), f(k[0, 0]), f(v[0, 0]), w.scale, w.causal)
        dP = f(do[0, m]) @ f(v[0, 0]).T
        acc = acc + w.scale * (fw["P"] * dP).T @ f(q[0, m])
    dk2[0, 0] = torch.from_numpy(acc).to(dk.dtype)
    assert name(dk=dk2) > 1.0, "dS without Delta not caught"


def test_varlen_invariants_and_planted_sequence():
    lengths = (40, 1, 130, 0, 77)
    w = workloads.Workload("inv_var", 35, len(lengths), 4, max(lengths), 64, "f16", True, 1.0, 2, lengths)
    q, k, v, do = workloads.make_inputs(w)
    cu = w.cu_seqlens
    f = lambda t: t.double().numpy()  # noqa: E731
    O, _ = oracle.attention_forward_varlen(f(q), f(k), f(v), cu, w.scale, True)
    dq, dk, dv = oracle.attention_backward_varlen(f(q), f(k), f(v), f(do), cu, w.scale, True)
    r = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(q.dtype)  # noqa: E731
    o, dq, dk, dv = r(O), r(dq), r(dk), r(dv)
    ok = backward_ratios_varlen(q, k, o, do, dq, dk, dv, cu, w.scale, w.dtype)
    assert max(ok.values()) <= 1.0, ok
    dk2 = dk.clone()
    dk2[:, cu[2]:cu[2] + 32] = 0  # a skipped key tile of the third sequence
    bad = backward_ratios_varlen(q, k, o, do, dq, dk2, dv, cu, w.scale, w.dtype)
    assert max(bad.values()) > 1.0, bad
