"""Pins of the paged-cache oracle (cache writes and decode attention).

[Serving-Ascend] is the page "从算子到 Serving：昇腾推理评测链路实践"
(BiumBiu), sections "ReshapeAndCache" and "GQA Paged Attention".  Each pin
checks the oracle against something other than itself: a library routine
(torch SDPA over a contiguous context built by the test), exact round trips,
invariances, closed forms, and planted slips that must fail.
"""
import numpy as np
import pytest

from oracle import gather_context, paged_decode, reshape_and_cache


def _scatter_pages(rng, K, V, num_blocks, block_size):
    """Test-side page layout: put the contiguous per-sequence contexts
    K, V (list of (Hkv, n_b, D)) into random distinct physical blocks, by
    plain indexing.  Returns caches and block tables; unused cache entries
    hold NaN so that any stray read shows."""
    n_kv, D = K[0].shape[0], K[0].shape[2]
    kc = np.full((num_blocks, n_kv, D // 8, block_size, 8), np.nan)
    vc = np.full((num_blocks, n_kv, D, block_size), np.nan)
    need = [-(-k.shape[1] // block_size) for k in K]
    perm = rng.permutation(num_blocks)[: sum(need)]
    tables = np.full((len(K), max(need) + 1), -7, dtype=np.int32)  # spare entries hold garbage
    i = 0
    for b, (k, v) in enumerate(zip(K, V)):
        for p in range(need[b]):
            blk = int(perm[i]); i += 1
            tables[b, p] = blk
            t0, t1 = p * block_size, min((p + 1) * block_size, k.shape[1])
            kc[blk, :, :, : t1 - t0, :] = k[:, t0:t1, :].reshape(n_kv, t1 - t0, D // 8, 8).transpose(0, 2, 1, 3)
            vc[blk, :, :, : t1 - t0] = np.swapaxes(v[:, t0:t1, :], 1, 2)
    return kc, vc, tables


@pytest.mark.parametrize("H,Hkv,block_size", [(8, 2, 16), (4, 4, 32), (6, 1, 16)])
def test_paged_decode_against_torch_sdpa(H, Hkv, block_size):
    """torch's CPU SDPA (float64, enable_gqa) on the contiguous contexts the
    test scattered into pages; unused slots are NaN, so the last-block mask
    and the block-table walk are both checked."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(81 + H + block_size)
    D, lens = 16, [1, 37, 64, 100]
    K = [rng.standard_normal((Hkv, n, D)) for n in lens]
    V = [rng.standard_normal((Hkv, n, D)) for n in lens]
    kc, vc, tables = _scatter_pages(rng, K, V, 40, block_size)
    q = rng.standard_normal((len(lens), H, D))
    O, lse = paged_decode(q, kc, vc, tables, np.array(lens), 0.3)
    for b, n in enumerate(lens):
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b][None, :, None, :]), torch.tensor(K[b][None]), torch.tensor(V[b][None]), scale=0.3,
            enable_gqa=True)
        assert np.max(np.abs(o.numpy()[0, :, 0, :] - O[b])) <= 1e-12
        G = H // Hkv
        for h in range(H):
            s = 0.3 * (K[b][h // G] @ q[b, h])
            assert abs(lse[b, h] - (np.max(s) + np.log(np.sum(np.exp(s - np.max(s)))))) <= 1e-12


def test_paged_decode_invariances_and_closed_forms():
    rng = np.random.default_rng(83)
    H, Hkv, D, bs = 4, 2, 8, 16
    lens = [1, 30, 0]
    K = [rng.standard_normal((Hkv, max(n, 1), D))[:, :n] for n in lens]
    V = [rng.standard_normal((Hkv, max(n, 1), D))[:, :n] for n in lens]
    kc, vc, tables = _scatter_pages(rng, K, V, 12, bs)
    q = rng.standard_normal((3, H, D))
    O, lse = paged_decode(q, kc, vc, tables, np.array(lens), 0.5)
    # one token: O = v_0, lse = scale q.k_0 (query head h uses key/value head h // 2)
    for h in range(H):
        assert np.max(np.abs(O[0, h] - V[0][h // 2, 0])) <= 1e-15
        assert abs(lse[0, h] - 0.5 * q[0, h] @ K[0][h // 2, 0]) <= 1e-14
    # empty context: no keys
    assert np.all(O[2] == 0) and np.all(np.isneginf(lse[2]))
    # relabelling the physical blocks (cache and table together) changes nothing, bit for bit
    perm = rng.permutation(12)
    inv = np.argsort(perm)
    kc2, vc2 = kc[inv], vc[inv]  # block b moves to position perm[b]
    t2 = np.where(tables >= 0, perm[np.clip(tables, 0, None)], tables).astype(np.int32)
    O2, lse2 = paged_decode(q, kc2, vc2, t2, np.array(lens), 0.5)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    # garbage past the context in the last block does not leak (it is NaN already); a wrong
    # in-block offset (t+1) % bs, a plausible slip, reads a NaN or another token
    Kg, Vg = gather_context(kc, vc, tables[1], 30, 1)
    assert np.array_equal(Kg, K[1][1]) and np.array_equal(Vg, V[1][1])
    slipped = np.array([kc[tables[1][t // bs], 1, :, (t + 1) % bs, :].reshape(D) for t in range(30)])
    assert not np.allclose(slipped[:29], K[1][1][:29])


def test_reshape_and_cache_round_trip_and_skips():
    rng = np.random.default_rng(89)
    nb, Hkv, bs, D, T = 6, 2, 16, 8, 20
    kc0 = rng.standard_normal((nb, Hkv, D // 8, bs, 8)).astype(np.float16)
    vc0 = rng.standard_normal((nb, Hkv, D, bs)).astype(np.float16)
    key = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    val = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[[3, 11]] = -1
    kc, vc = reshape_and_cache(key, val, slots, kc0, vc0)
    touched_k = np.zeros(kc.shape, bool)
    touched_v = np.zeros(vc.shape, bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = s // bs, s % bs
        assert np.array_equal(kc[b, :, :, o, :].reshape(Hkv, D), key[i]) and np.array_equal(vc[b, :, :, o], val[i])
        touched_k[b, :, :, o, :] = True
        touched_v[b, :, :, o] = True
    assert np.array_equal(kc[~touched_k], kc0[~touched_k]) and np.array_equal(vc[~touched_v], vc0[~touched_v])
    assert touched_k.sum() == (T - 2) * Hkv * D
    # a plausible slip: block and offset swapped
    b, o = slots[0] % bs, slots[0] // bs
    if b < nb and o < bs and (b, o) != (slots[0] // bs, slots[0] % bs):
        assert not np.array_equal(kc[b, :, :, o, :].reshape(Hkv, D), key[0])
    with pytest.raises(ValueError):
        reshape_and_cache(key, val, np.full(T, nb * bs, dtype=np.int64), kc0, vc0)
