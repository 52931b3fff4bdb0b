"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the oracle.

[FA-Ascend] is the page "把 FlashAttention 搬上昇腾：Triton-Ascend CV Pipeline
优化实战" (BiumBiu).  Each test names the part of the oracle it pins.  The last
group plants mistakes in copies of the oracle and checks that a pin fails.
"""
import math

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_gqa, attention_forward, attention_forward_full,
                    attention_forward_gqa, gqa_kv_head, loss_sum_o_do, attention_forward_varlen,
                    attention_backward_varlen)

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _tiny(n=16, d=8, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(4)]


def _fd_grad(fn, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = fn()
        x[idx] = old - h
        fm = fn()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def _fd_check(bwd_fn, causal, seed=0, scale=0.37):
    q, k, v, do = _tiny(seed=seed)
    g = bwd_fn(q, k, v, do, scale, causal)
    errs = []
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _fd_grad(lambda: loss_sum_o_do(q, k, v, do, scale, causal), x)
        errs.append(np.max(np.abs(fd - g[name])) / np.max(np.abs(g[name])))
    return max(errs)


# ---------------------------------------------------------------- backward formulas
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_finite_differences(causal):
    """dQ, dK, dV of [FA-Ascend] §二 are the gradient of L = sum(O * dO):
    central differences (h = 1e-6) over every element of Q, K and V, N=16, D=8."""
    assert _fd_check(attention_backward, causal) <= 1e-6


# ---------------------------------------------------------------- softmax and stats
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, v, _ = _tiny(n=33, d=5, seed=3)
    P = attention_forward_full(q, k, v, 0.5, causal)["P"]
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-15 * 33
    assert np.all(P >= 0)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_library_logsumexp(causal):
    from scipy.special import logsumexp

    q, k, v, _ = _tiny(n=40, d=7, seed=5)
    scale = 0.3
    _, lse = attention_forward(q, k, v, scale, causal)
    S = (q @ k.T) * scale
    if causal:
        S = np.where(np.tril(np.ones_like(S)) > 0, S, -np.inf)
    assert np.max(np.abs(lse - logsumexp(S, axis=-1))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_delta_equals_rowsum_p_dp(causal):
    """Delta = rowsum(O * dO) ([FA-Ascend] §二) equals rowsum(P * dP), because
    O = P V and dP = dO V^T."""
    q, k, v, do = _tiny(n=24, d=6, seed=7)
    r = attention_backward(q, k, v, do, 0.4, causal)
    assert np.max(np.abs(r["Delta"] - np.sum(r["P"] * r["dP"], -1))) <= 1e-14


def test_causal_row_zero_attends_only_to_key_zero():
    """Causal ([FA-Ascend] §八): query 0 sees only key 0, so P00 = 1, O0 = V0,
    lse0 = S00; and the last key is seen only by the last query, so
    dK_{N-1} = scale * P_{N-1,N-1} (dP_{N-1,N-1} - Delta_{N-1}) q_{N-1}."""
    q, k, v, do = _tiny(n=12, d=4, seed=11)
    scale = 0.6
    f = attention_forward_full(q, k, v, scale, True)
    assert f["P"][0, 0] == 1.0
    assert np.array_equal(f["O"][0], v[0])
    assert f["lse"][0] == pytest.approx(scale * float(q[0] @ k[0]), abs=1e-15)
    r = attention_backward(q, k, v, do, scale, True)
    n = q.shape[0] - 1
    want = scale * r["P"][n, n] * (r["dP"][n, n] - r["Delta"][n]) * q[n]
    assert np.max(np.abs(r["dk"][n] - want)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0 makes every score 0: O is the mean of the visible values and
    lse = ln(#visible keys)."""
    n, d = 37, 6
    rng = np.random.default_rng(13)
    q = np.zeros((n, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    O, lse = attention_forward(q, k, v, 0.9, causal)
    if causal:
        cnt = np.arange(1, n + 1)
        want = np.cumsum(v, axis=0) / cnt[:, None]
        assert np.max(np.abs(lse - np.log(cnt))) <= 1e-15 * 4
    else:
        want = np.broadcast_to(v.mean(0), (n, d))
        assert np.max(np.abs(lse - math.log(n))) <= 1e-15 * 4
    assert np.max(np.abs(O - want)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """Adding one vector u to every key adds scale*q_i.u to row i of S: the
    softmax, O and all three gradients are unchanged and lse shifts by it."""
    q, k, v, do = _tiny(n=20, d=5, seed=17)
    u = np.random.default_rng(19).standard_normal(5)
    scale = 0.45
    a = attention_backward(q, k, v, do, scale, causal)
    b = attention_backward(q, k + u, v, do, scale, causal)
    for name in ("O", "dq", "dk", "dv"):
        assert np.max(np.abs(a[name] - b[name])) <= 1e-13, name
    assert np.max(np.abs(b["lse"] - a["lse"] - scale * q @ u)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """sum_j dK_j = 0; <Q,dQ> = <K,dK>; sum_j dV_j = sum_i dO_i; <V,dV> = sum_i Delta_i."""
    q, k, v, do = _tiny(n=29, d=7, seed=23)
    r = attention_backward(q, k, v, do, 0.33, causal)
    assert np.max(np.abs(r["dk"].sum(0))) <= 1e-13
    assert abs(np.sum(q * r["dq"]) - np.sum(k * r["dk"])) <= 1e-13
    assert np.max(np.abs(r["dv"].sum(0) - do.sum(0))) <= 1e-13
    assert abs(np.sum(v * r["dv"]) - r["Delta"].sum()) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(causal):
    """An independent library routine: torch's CPU scaled_dot_product_attention
    in float64 with autograd, on a batch of heads."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(29)
    shp = (2, 3, 50, 16)
    q, k, v, do = (rng.standard_normal(shp) for _ in range(4))
    scale = 0.21
    r = attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do))
    assert np.max(np.abs(o.detach().numpy() - r["O"])) <= 1e-12
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.max(np.abs(t.grad.numpy() - r[name])) <= 1e-12, name


def test_brute_force_tiny():
    """Pure-Python loops over the definition on N=5, D=3 (no numpy linear algebra)."""
    rng = np.random.default_rng(31)
    n, d, scale = 5, 3, 0.7
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        O, lse = attention_forward(q, k, v, scale, causal)
        for i in range(n):
            js = [j for j in range(n) if (j <= i or not causal)]
            s = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in js]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            for t in range(d):
                want = sum(e[a] * v[js[a]][t] for a in range(len(js))) / tot
                assert abs(O[i][t] - want) <= 1e-14
            assert abs(lse[i] - (mx + math.log(tot))) <= 1e-14


def test_batched_heads_are_independent():
    """Leading axes are independent heads: a (2,3,N,D) call equals per-head calls."""
    rng = np.random.default_rng(37)
    q, k, v, do = (rng.standard_normal((2, 3, 16, 4)) for _ in range(4))
    r = attention_backward(q, k, v, do, 0.5, True)
    for z in range(2):
        for h in range(3):
            s = attention_backward(q[z, h], k[z, h], v[z, h], do[z, h], 0.5, True)
            for name in ("O", "lse", "dq", "dk", "dv"):
                assert np.array_equal(r[name][z, h], s[name])


# ---------------------------------------------------------------- planted mistakes
def _bwd_mutant(kind):
    """A copy of the backward with one planted mistake, to show the pins bite."""

    def bwd(q, k, v, do, scale, causal):
        f = attention_forward_full(q, k, v, scale, causal)
        O, P = f["O"], f["P"]
        Delta = np.sum(O * do, -1)
        dP = do @ v.T
        if kind == "no_scale_in_ds":
            dS = P * (dP - Delta[:, None])
        elif kind == "delta_sign":
            dS = scale * P * (dP + Delta[:, None])
        else:
            dS = scale * P * (dP - Delta[:, None])
        dq = dS @ k
        dk = dS.T @ q
        dv = P.T @ do
        if kind == "dv_untransposed":
            dv = P @ do
        if kind == "dk_uses_k":
            dk = dS.T @ k
        if kind == "dq_transposed_ds":
            dq = dS.T @ k
        return {"dq": dq, "dk": dk, "dv": dv}

    return bwd


@pytest.mark.parametrize("kind", ["no_scale_in_ds", "delta_sign", "dv_untransposed", "dk_uses_k",
                                  "dq_transposed_ds"])
def test_finite_differences_catch_planted_backward_mistakes(kind):
    assert _fd_check(_bwd_mutant(kind), causal=True) > 1e-3


def test_closed_form_catches_wrong_causal_diagonal():
    """A mask that hides the diagonal (j < i instead of j <= i) breaks the
    causal closed form; the pin must see it."""
    n, d = 9, 3
    rng = np.random.default_rng(41)
    v = rng.standard_normal((n, d))
    S = np.zeros((n, n))
    i, j = np.arange(n)[:, None], np.arange(n)[None, :]
    S = np.where(j < i, S, -np.inf)
    S[0, 0] = 0.0  # keep row 0 finite
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    wrong = P @ v
    want = np.cumsum(v, 0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(wrong - want)) > 1e-3


# ---------------------------------------------------------------- grouped key/value heads
# [Serving-Ascend] is the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu),
# section "GQA Paged Attention": query heads a whole multiple of key/value
# heads, consecutive query heads sharing one.


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_gradient_matches_finite_differences(causal):
    """dK and dV of a shared key/value head are the gradient of
    L = sum(O * dO) over all the query heads that use it: central differences
    over every element of Q, K and V (Z=1, Hq=4, Hkv=2, N=6, D=4)."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 4, 6, 4))
    k, v = (rng.standard_normal((1, 2, 6, 4)) for _ in range(2))
    do = rng.standard_normal((1, 4, 6, 4))
    scale = 0.41

    def loss():
        O, _ = attention_forward_gqa(q, k, v, scale, causal)
        return float(np.sum(O * do))

    dq, dk, dv = attention_backward_gqa(q, k, v, do, scale, causal)
    for g, x in ((dq, q), (dk, k), (dv, v)):
        fd = _fd_grad(loss, x)
        assert np.max(np.abs(fd - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 1), (3, 3)])
def test_gqa_against_torch_sdpa(causal, hq, hkv):
    """An independent library routine: torch's CPU scaled_dot_product_attention
    with enable_gqa in float64, forward and autograd backward."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(47 + hq + hkv)
    q = rng.standard_normal((2, hq, 20, 8))
    k, v = (rng.standard_normal((2, hkv, 20, 8)) for _ in range(2))
    do = rng.standard_normal((2, hq, 20, 8))
    scale = 0.3
    O, lse = attention_forward_gqa(q, k, v, scale, causal)
    dq, dk, dv = attention_backward_gqa(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                         enable_gqa=True)
    o.backward(torch.tensor(do))
    assert np.max(np.abs(o.detach().numpy() - O)) <= 1e-12
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(t.grad.numpy() - g)) <= 1e-12


def test_gqa_one_group_is_plain_attention():
    """Hkv == Hq: every query head has its own key/value head, so the grouped
    oracle equals the per-head oracle exactly."""
    rng = np.random.default_rng(53)
    q, k, v, do = (rng.standard_normal((1, 3, 12, 4)) for _ in range(4))
    O, lse = attention_forward_gqa(q, k, v, 0.5, True)
    dq, dk, dv = attention_backward_gqa(q, k, v, do, 0.5, True)
    r = attention_backward(q, k, v, do, 0.5, True)
    for a, b in ((O, r["O"]), (lse, r["lse"]), (dq, r["dq"]), (dk, r["dk"]), (dv, r["dv"])):
        assert np.array_equal(a, b)


def test_gqa_head_map_and_planted_interleaving():
    """Consecutive query heads share a key/value head (h // G); an interleaved
    map (h % Hkv), a plausible slip, disagrees with torch's grouping."""
    assert [gqa_kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        gqa_kv_head(0, 6, 4)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(59)
    q = rng.standard_normal((1, 4, 10, 4))
    k, v = (rng.standard_normal((1, 2, 10, 4)) for _ in range(2))
    o = torch.nn.functional.scaled_dot_product_attention(*(torch.tensor(x) for x in (q, k, v)), scale=0.5,
                                                         enable_gqa=True).numpy()
    wrong = np.stack([attention_forward(q[0, h], k[0, h % 2], v[0, h % 2], 0.5)[0] for h in range(4)])
    assert np.max(np.abs(wrong - o[0])) > 1e-3


# ---------------------------------------------------------------- variable-length batches
# [Serving-Ascend]: sequences of different real lengths in one batch, tokens
# past a sequence's end taking no part.  Packed head-major layout (H, T, D)
# with cu_seqlens token offsets.


def _varlen_inputs(rng, H, Hkv, cu, D):
    T = int(cu[-1])
    q = rng.standard_normal((H, T, D))
    k, v = (rng.standard_normal((Hkv, T, D)) for _ in range(2))
    do = rng.standard_normal((H, T, D))
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_against_torch_sdpa_block_mask(causal):
    """An independent library routine: torch's CPU SDPA in float64 over the
    whole packed token axis with a block-diagonal (and causal) boolean mask,
    enable_gqa, forward and autograd backward."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(61)
    cu = np.array([0, 5, 5, 17, 18, 30])  # includes an empty and a one-token sequence
    H, Hkv, D = 4, 2, 8
    q, k, v, do = _varlen_inputs(rng, H, Hkv, cu, D)
    T = int(cu[-1])
    seg = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seg]
    mask = seg[:, None] == seg[None, :]
    if causal:
        mask &= pos[None, :] <= pos[:, None]
    scale = 0.37
    O, lse = attention_forward_varlen(q, k, v, cu, scale, causal)
    dq, dk, dv = attention_backward_varlen(q, k, v, do, cu, scale, causal)
    tq, tk, tv = (torch.tensor(x[None], requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(mask), scale=scale,
                                                         enable_gqa=True)
    o.backward(torch.tensor(do[None]))
    assert np.max(np.abs(o.detach().numpy()[0] - O)) <= 1e-12
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(t.grad.numpy()[0] - g)) <= 1e-12
    # lse against a direct log-sum-exp over each token's visible keys (head 0)
    G = H // Hkv
    for h in range(H):
        S = (q[h] @ k[h // G].T) * scale
        want = np.log(np.sum(np.where(mask, np.exp(S), 0.0), axis=1))
        assert np.max(np.abs(lse[h] - want)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_gradient_matches_finite_differences(causal):
    rng = np.random.default_rng(67)
    cu = np.array([0, 3, 7])
    q, k, v, do = _varlen_inputs(rng, 2, 1, cu, 3)
    scale = 0.53

    def loss():
        O, _ = attention_forward_varlen(q, k, v, cu, scale, causal)
        return float(np.sum(O * do))

    dq, dk, dv = attention_backward_varlen(q, k, v, do, cu, scale, causal)
    for g, x in ((dq, q), (dk, k), (dv, v)):
        fd = _fd_grad(loss, x)
        assert np.max(np.abs(fd - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))


def test_varlen_sequences_are_independent_and_planted_merge_fails():
    """Changing one sequence's tokens leaves every other sequence's outputs
    bit for bit; one-token sequences give O = v (closed form) and
    lse = scale * q.k; treating the batch as one sequence (a plausible slip)
    changes the result."""
    rng = np.random.default_rng(71)
    cu = np.array([0, 6, 7, 15])
    q, k, v, do = _varlen_inputs(rng, 2, 2, cu, 4)
    O, lse = attention_forward_varlen(q, k, v, cu, 0.5, True)
    k2 = k.copy()
    k2[:, 8:12] += 3.0  # inside the third sequence
    O2, lse2 = attention_forward_varlen(q, k2, v, cu, 0.5, True)
    assert np.array_equal(O[:, :7], O2[:, :7]) and np.array_equal(lse[:, :7], lse2[:, :7])
    assert not np.array_equal(O[:, 7:], O2[:, 7:])
    assert np.max(np.abs(O[:, 6] - v[:, 6])) <= 1e-15
    assert np.max(np.abs(lse[:, 6] - 0.5 * np.sum(q[:, 6] * k[:, 6], axis=-1))) <= 1e-14
    merged, _ = attention_forward_varlen(q, k, v, np.array([0, 15]), 0.5, True)
    assert np.max(np.abs(merged[:, 7:] - O[:, 7:])) > 1e-3
    with pytest.raises(ValueError):
        attention_forward_varlen(q, k, v, np.array([0, 8, 7, 15]), 0.5, True)
