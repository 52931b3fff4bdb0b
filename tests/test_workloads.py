"""Host checks of the seeded input generators (no GPU): the same seed gives the
same bits, the recipes hold what their documentation states, and the paged
layouts are valid (every page of every context has its own physical block)."""
import math

import numpy as np
import torch

import workloads


def test_dense_draws_are_seeded_and_gain_is_exact():
    a = workloads.random_inputs((1, 2, 33, 64), "bf16", 5)
    b = workloads.random_inputs((1, 2, 33, 64), "bf16", 5)
    c = workloads.random_inputs((1, 2, 33, 64), "bf16", 6)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)) and not torch.equal(x, z)
    # q and k of a gain-2 draw are exactly twice the gain-1 draw (a power of two)
    w1 = workloads.Workload("g", 9, 1, 1, 40, 64, "f16", True)
    q1, k1, v1, d1 = workloads.draw_f32(w1)
    q2, k2, v2, d2 = workloads.draw_f32(w1.with_(qk_gain=2.0))
    assert np.array_equal(q2, 2 * q1) and np.array_equal(k2, 2 * k1)
    assert np.array_equal(v2, v1) and np.array_equal(d2, d1)


def test_grouped_and_variable_length_shapes():
    w = workloads.WORKLOADS["gqa_causal_bf16"]
    assert w.q_shape == (4, 32, 4096, 128) and w.kv_draw_shape == (4, 8, 4096, 128)
    v = workloads.WORKLOADS["varlen_causal_bf16"]
    cu = v.cu_seqlens
    assert cu[0] == 0 and list(np.diff(cu)) == list(v.lengths) and cu[-1] == v.T == sum(v.lengths)
    assert all(64 <= n <= 4096 for n in v.lengths) and v.N == max(v.lengths)
    assert v.q_shape == (16, v.T, 128)


def test_scale_is_the_float32_value():
    for D in (64, 128, 256):
        s = workloads.f32_scale(D)
        assert s == float(np.float32(1 / math.sqrt(D))) and np.float32(s) == s


def test_decode_draws_are_exact_and_layout_valid():
    w = workloads.DecodeWorkload("t", 21, 5, 8, 2, 64, 16, 0, 300, "f16")
    lens, tables, nb = w.layout()
    assert list(lens) == list(w.lengths()) and all(0 <= n <= 300 for n in lens)
    pages = [-(-int(n) // 16) for n in lens]
    used = sum(pages)
    assert nb == used + used // 8 + 1
    blocks = [int(b) for r, p in zip(tables, pages) for b in r[:p]]
    assert len(set(blocks)) == used and all(0 <= b < nb for b in blocks)  # one block per page
    assert all((r[p:] == -1).all() for r, p in zip(tables, pages))
    x = workloads.make_decode_inputs(w)
    y = workloads.make_decode_inputs(w)
    for a, b in zip(x, y):
        assert torch.equal(a, b)
    for t in x[:3]:  # integers in [-32, 32) / 16: exact in the 16-bit type
        s = t.double() * 16
        assert torch.equal(s, s.round()) and float(s.min()) >= -32 and float(s.max()) < 32
    bf = workloads.make_decode_inputs(w.__class__(**{**w.__dict__, "dtype": "bf16"}))
    assert torch.equal(bf[1].double(), x[1].double())  # the same values in either type


def test_window_pool_recipe():
    w = workloads.DECODE_WORKLOADS["window_quest_gqa_bf16"]
    p = w.window_pool()
    assert (p.lo, p.hi, p.seed, p.B, p.Hkv, p.D, p.block_size) == (1024, 1024, w.seed + 1, w.B, w.Hkv, w.D,
                                                                    w.block_size)
    small = workloads.DecodeWorkload("t", 3, 2, 4, 2, 64, 16, 10, 50, "bf16", 4, 64).window_pool()
    lens, tables, _ = small.layout()
    assert list(lens) == [64, 64] and tables.shape == (2, 4)
