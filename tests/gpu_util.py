"""Helpers shared by the GPU parity tests: device inputs, oracle on sampled
heads, error metrics.  Test infrastructure only."""
from __future__ import annotations

import os

import numpy as np

import oracle
import workloads


def has_gpu() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def log(msg: str) -> None:
    print(msg, flush=True)


def to_f64(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def device_inputs(w: workloads.Workload):
    """(cpu tensors, gpu tensors) of q, k, v, do for a workload."""
    cpu = workloads.make_inputs(w)
    gpu = tuple(t.cuda() for t in cpu)
    return cpu, gpu


def sample_heads(w: workloads.Workload, count: int):
    """Deterministic spread of (z, h) pairs: first, last and evenly between."""
    n = w.Z * w.H
    if n <= count:
        idx = list(range(n))
    else:
        idx = sorted(set(int(round(x)) for x in np.linspace(0, n - 1, count)))
    return [(i // w.H, i % w.H) for i in idx]


def oracle_head(cpu, z, h, scale, causal):
    q, k, v, do = (to_f64(t[z, h]) for t in cpu)
    return oracle.attention_backward(q, k, v, do, scale, causal)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def rel_fro(a, b_ref) -> float:
    a = np.asarray(a, np.float64)
    b_ref = np.asarray(b_ref, np.float64)
    return float(np.linalg.norm(a - b_ref) / max(np.linalg.norm(b_ref), 1e-300))


class NormAccumulator:
    """Accumulates ||x - ref||^2 and ||ref||^2 over heads for a normwise relative error."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.count = 0
        self.max_abs = 0.0
        self.worst_head = 0.0

    def add(self, x, ref):
        x = np.asarray(x, np.float64)
        ref = np.asarray(ref, np.float64)
        n = float(np.sum((x - ref) ** 2))
        d = float(np.sum(ref ** 2))
        self.num += n
        self.den += d
        self.count += ref.size
        self.max_abs = max(self.max_abs, float(np.max(np.abs(x - ref))) if ref.size else 0.0)
        self.worst_head = max(self.worst_head, (n / max(d, 1e-300)) ** 0.5)

    @property
    def exact_zero(self) -> bool:
        """True when the reference is zero up to fp64 rounding (e.g. N = 1, where
        dS is identically 0): a relative norm is meaningless there."""
        return self.den <= 1e-24 * max(self.count, 1)

    @property
    def value(self) -> float:
        return (self.num / max(self.den, 1e-300)) ** 0.5


# Tolerances fixed for floating point results.
ZERO_REF_MAX_ABS = 1e-3  # max-abs bound used when the exact gradient is zero
O_MAX_ABS = 1e-2      # max-abs error of the fp32 O
GRAD_NORMWISE = 2e-2  # normwise relative error of dQ, dK, dV
LSE_MAX_ABS = 1e-3    # max-abs error of lse (natural log)


def oracle_group(cpu, z, kvh, scale, causal):
    """Oracle for key/value head (z, kvh) of a grouped-head input and every
    query head that shares it: {"heads": [query heads], "O", "lse", "dq"
    (stacked over those heads), "dk", "dv" (of the key/value head)}."""
    q, k, v, do = cpu
    H, Hkv = q.shape[1], k.shape[1]
    G = H // Hkv
    heads = list(range(kvh * G, (kvh + 1) * G))
    sl = slice(heads[0], heads[-1] + 1)
    qq, dd = to_f64(q[z:z + 1, sl]), to_f64(do[z:z + 1, sl])
    kk, vv = to_f64(k[z:z + 1, kvh:kvh + 1]), to_f64(v[z:z + 1, kvh:kvh + 1])
    O, lse = oracle.attention_forward_gqa(qq, kk, vv, scale, causal)
    dq, dk, dv = oracle.attention_backward_gqa(qq, kk, vv, dd, scale, causal)
    return {"heads": heads, "O": O[0], "lse": lse[0], "dq": dq[0], "dk": dk[0, 0], "dv": dv[0, 0]}


def varlen_device_inputs(w: workloads.Workload):
    """(cpu tensors, gpu tensors, gpu int32 offsets) of a variable-length workload."""
    import torch

    cpu, gpu = device_inputs(w)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    return cpu, gpu, cu


def oracle_varlen_group(cpu, cu_seqlens, b, kvh, scale, causal):
    """Oracle for sequence b and key/value head kvh (with its G query heads)
    of a packed variable-length input: {"heads", "rows" (slice), "O", "lse",
    "dq", "dk", "dv"} over that sequence's rows only."""
    q, k, v, do = cpu
    H, Hkv = q.shape[0], k.shape[0]
    G = H // Hkv
    s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
    hs = slice(kvh * G, (kvh + 1) * G)
    qq, dd = to_f64(q[hs, s:e]), to_f64(do[hs, s:e])
    kk, vv = to_f64(k[kvh:kvh + 1, s:e]), to_f64(v[kvh:kvh + 1, s:e])
    one = [0, e - s]
    O, lse = oracle.attention_forward_varlen(qq, kk, vv, one, scale, causal)
    dq, dk, dv = oracle.attention_backward_varlen(qq, kk, vv, dd, one, scale, causal)
    return {"heads": list(range(kvh * G, (kvh + 1) * G)), "rows": slice(s, e), "O": O, "lse": lse, "dq": dq,
            "dk": dk[0], "dv": dv[0]}
