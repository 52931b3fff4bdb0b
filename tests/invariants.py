"""Oracle-free checks of full-size backward results (test infrastructure).

Every identity below holds exactly for the true gradients of one attention
problem ([FA-Ascend] §二: dS = scale * P * (dP - Delta), dQ = dS K,
dK = dS^T Q, dV = P^T dO), so it can be checked on every head of a workload
far too large for the oracle.  The bounds come from the rounding the kernels
do (u = unit roundoff of the input type: 2^-11 fp16, 2^-8 bf16); each check
allows twice its bound.

* sum_j dV_j = sum_i dO_i per channel (every row of P sums to 1).  Rounding:
  P and dV are cast to the input type, so |sum dV - sum dO| <=
  u (sum |dO| + sum |dV|).
* sum_j dK_j = 0 per channel: sum_j dK_j = scale sum_i (sum_j dS_ij) q_i and
  sum_j dS_ij = sum_j P_ij dP_ij - Delta_i = 0.  Rounding: dK is cast
  (u sum_j |dK_j|), and Delta is formed from the stored O, which is off by at
  most u |O| per element, so sum_j dS_ij = -delta_i with
  |delta_i| <= u sum_d |O_id dO_id|, contributing scale sum_i |delta_i| |q_i|.
* Q^T dQ = dK^T K per problem (a D x D matrix; entry (a, b) of both is
  scale sum_ij dS_ij q_ia k_jb for any dS; its trace is <Q, dQ> = <K, dK>).
  Rounding: the casts of dQ and dK, u (|Q|^T |dQ| + |dK|^T |K|) per entry.
A skipped or misplaced key tile, query tile or head breaks one of them.

Tensors may live on any torch device; each function returns the worst ratio
of an identity's defect to its allowed bound (<= 1 passes) and is used both
on GPU results and, with planted mistakes, on CPU copies.
"""
from __future__ import annotations


def unit_roundoff(dtype: str) -> float:
    return 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11


def _groups(q, kv_heads):
    """(Z, H, N, D) -> (Z, Hkv, G, N, D): the G query heads of each key/value head."""
    Z, H, N, D = q.shape
    return q.reshape(Z, kv_heads, H // kv_heads, N, D)


def dv_sum_ratio(do, dv, u):
    """sum_j dV_j against sum_i dO_i over the query heads of each key/value head."""
    Hkv = dv.shape[1]
    g = _groups(do.double(), Hkv)
    s_do = g.sum(dim=(2, 3))
    a_do = g.abs().sum(dim=(2, 3))
    dv64 = dv.double()
    defect = (dv64.sum(dim=2) - s_do).abs()
    bound = 2 * u * (a_do + dv64.abs().sum(dim=2)) + 1e-6
    return float((defect / bound).max())


def dk_sum_ratio(q, o, do, dk, scale, u):
    """sum_j dK_j = 0 per (batch, key/value head, channel)."""
    Hkv = dk.shape[1]
    dk64 = dk.double()
    defect = dk64.sum(dim=2).abs()
    # |delta_i| <= u sum_d |O_id dO_id|, one per query row
    delta = u * (o.double().abs() * do.double().abs()).sum(dim=-1, keepdim=True)
    dterm = scale * _groups(delta * q.double().abs(), Hkv).sum(dim=(2, 3))
    bound = 2 * (u * dk64.abs().sum(dim=2) + dterm) + 1e-6
    return float((defect / bound).max())


def qdq_kdk_ratio(q, k, dq, dk, u):
    """Q^T dQ = dK^T K per (batch, key/value head): entry (a, b) of both is
    scale sum_ij dS_ij q_ia k_jb (its trace is <Q, dQ> = <K, dK>).  Checked
    as a D x D matrix, so that a gradient of the wrong head, which may keep
    the trace by chance, still fails."""
    Z, H, N, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    q64 = q.double().reshape(Z, Hkv, G * N, D)
    dq64 = dq.double().reshape(Z, Hkv, G * N, D)
    k64, dk64 = k.double(), dk.double()
    lhs = q64.transpose(-1, -2) @ dq64
    rhs = dk64.transpose(-1, -2) @ k64
    mag = q64.abs().transpose(-1, -2) @ dq64.abs() + dk64.abs().transpose(-1, -2) @ k64.abs()
    bound = 2 * u * mag + 1e-6
    return float(((lhs - rhs).abs() / bound).max())


def backward_ratios(q, k, o, do, dq, dk, dv, scale, dtype):
    """All three identities on a dense (Z, H, N, D) batch (k, dk, dv may be
    grouped (Z, Hkv, N, D)).  Returns {name: worst ratio}."""
    u = unit_roundoff(dtype)
    return {"sum_dV": dv_sum_ratio(do, dv, u), "sum_dK": dk_sum_ratio(q, o, do, dk, scale, u),
            "QdQ_KdK": qdq_kdk_ratio(q, k, dq, dk, u)}


def backward_ratios_varlen(q, k, o, do, dq, dk, dv, cu_seqlens, scale, dtype):
    """The same on a packed variable-length batch (q (H, T, D), k (Hkv, T, D)):
    each sequence is its own problem."""
    out = {"sum_dV": 0.0, "sum_dK": 0.0, "QdQ_KdK": 0.0}
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        one = lambda t: t[:, s:e].unsqueeze(0)  # noqa: E731  (1, heads, n, D)
        r = backward_ratios(one(q), one(k), one(o), one(do), one(dq), one(dk), one(dv), scale, dtype)
        out = {n: max(out[n], r[n]) for n in out}
    return out
