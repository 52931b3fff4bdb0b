"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module holds shapes, seeds and random draws only.  It contains none of the
attention arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from here without sharing any of the method.

Recipe (one generator per workload, PCG64 through ``numpy.random.default_rng``):

* seed = the workload's index (1..5);
* draw, in this order, ``q, k, v, do`` as ``standard_normal(shape, float32)``
  with shape (Z, H, N, D) for q and do and (Z, Hkv, N, D) for k and v (Hkv =
  H except for the grouped key/value head workload); a variable-length
  workload draws, in the same order, q and do of shape (H, T, D) and k and v
  of shape (Hkv, T, D), T the sum of its sequence lengths (packed head-major);
* variable-length workloads take their sequence lengths from a generator of
  their own, ``default_rng(1000 + seed).integers(lo, hi + 1, size=B)``;
* for the long-sequence workload only, multiply q and k by 2 in float32 (exact),
  which sharpens the softmax and exercises the running-max rescaling;
* cast to the workload's dtype with round-to-nearest-even.

``scale`` is a float32 value; the oracle receives the same float32 value upcast
to float64, so both sides see the identical number.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "by_name", "draw_f32", "make_inputs", "f32_scale"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    Z: int
    H: int
    N: int
    D: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    qk_gain: float = 1.0  # multiplier applied to q and k in float32
    Hkv: int = 0          # key/value heads (0 = H: one per query head)
    lengths: tuple = ()   # variable-length batch: per-sequence lengths (Z = count, N = longest)

    @property
    def scale(self) -> float:
        return f32_scale(self.D)

    @property
    def shape(self):
        return (self.Z, self.H, self.N, self.D)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def kv_shape(self):
        return (self.Z, self.kv_heads, self.N, self.D)

    @property
    def heads(self) -> int:
        return self.Z * self.H

    @property
    def varlen(self) -> bool:
        return len(self.lengths) > 0

    @property
    def T(self) -> int:
        """Tokens of a variable-length batch (sum of the lengths)."""
        return int(sum(self.lengths))

    @property
    def cu_seqlens(self):
        """Token offsets (B+1,) int32 of a variable-length batch."""
        return np.concatenate([[0], np.cumsum(np.asarray(self.lengths, dtype=np.int64))]).astype(np.int32)

    @property
    def q_shape(self):
        return (self.H, self.T, self.D) if self.varlen else self.shape

    @property
    def kv_draw_shape(self):
        return (self.kv_heads, self.T, self.D) if self.varlen else self.kv_shape

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def f32_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32, returned as a Python float holding that value."""
    return float(np.float32(1.0 / math.sqrt(D)))


# The five workloads: a tiny parity case, three Z=128 x H=8 x N=1024 cases at
# head dims 64/128/256, and a long-sequence causal case with a peaked softmax;
# then the D = 256 case with the causal mask, a grouped key/value head case: Z=4, 32 query heads over 8 key/value
# heads (4 query heads per key/value head), N=4096, D=128, causal.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 64, "f16", False),
    "d64": Workload("d64", 2, 128, 8, 1024, 64, "f16", False),
    "d128_causal": Workload("d128_causal", 3, 128, 8, 1024, 128, "f16", True),
    "d256_bf16": Workload("d256_bf16", 4, 128, 8, 1024, 256, "bf16", False),
    "d256_causal_bf16": Workload("d256_causal_bf16", 8, 128, 8, 1024, 256, "bf16", True),
    "long_causal_bf16": Workload("long_causal_bf16", 5, 16, 16, 8192, 128, "bf16", True, 2.0),
    "gqa_causal_bf16": Workload("gqa_causal_bf16", 6, 4, 32, 4096, 128, "bf16", True, 1.0, 8),
}


def draw_lengths(seed: int, count: int, lo: int, hi: int) -> tuple:
    """Sequence lengths of a variable-length workload: uniform integers in
    [lo, hi] from the workload's own length generator."""
    rng = np.random.default_rng(1000 + seed)
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=count))


_VARLEN_LENGTHS = draw_lengths(7, 32, 64, 4096)
# A variable-length causal batch: 32 sequences of 64..4096 tokens, 16 heads.
WORKLOADS["varlen_causal_bf16"] = Workload("varlen_causal_bf16", 7, len(_VARLEN_LENGTHS), 16, max(_VARLEN_LENGTHS),
                                           128, "bf16", True, 1.0, 0, _VARLEN_LENGTHS)


def by_name(name: str) -> Workload:
    return WORKLOADS[name]


def draw_f32(w: Workload, heads: slice | None = None):
    """Return float32 (q, k, v, do) drawn from the workload's seed: q and do of
    shape (Z, H, N, D), k and v of shape (Z, Hkv, N, D).

    ``heads`` is ignored for the draw itself (the stream must stay identical); it
    exists so that callers can document that they slice afterwards.
    """
    rng = np.random.default_rng(w.seed)
    out = []
    for name in ("q", "k", "v", "do"):
        x = rng.standard_normal(size=w.kv_draw_shape if name in ("k", "v") else w.q_shape, dtype=np.float32)
        if name in ("q", "k") and w.qk_gain != 1.0:
            x *= np.float32(w.qk_gain)
        out.append(x)
    return tuple(out)


def make_inputs(w: Workload):
    """Return torch CPU tensors (q, k, v, do) in the workload's dtype (RNE cast)."""
    import torch

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    return tuple(torch.from_numpy(x).to(tdt) for x in draw_f32(w))


def random_inputs(shape, dtype: str, seed: int, qk_gain: float = 1.0, kv_heads: int = 0):
    """Seeded (q, k, v, do) torch CPU tensors of an arbitrary shape, same recipe."""
    w = Workload("adhoc", seed, *shape, dtype, False, qk_gain, kv_heads)
    return make_inputs(w)


# ---------------------------------------------------------------- paged decode
# Decode over a paged KV cache: B sequences, one query token each, contexts of
# drawn lengths stored in pages (physical blocks) of block_size tokens per
# key/value head.  Recipe: a generator default_rng(seed) draws, in order, the
# context lengths (uniform integers in [lo, hi]), the physical block of every
# page (a random permutation of the blocks, taken sequence by sequence), then
# q (B, H, D), k_cache (num_blocks, Hkv, D/8, block_size, 8) and v_cache
# (num_blocks, Hkv, D, block_size) as integers uniform in [-32, 32) divided by
# 16 (values in [-2, 2) on a 1/16 grid, exact in fp16 and bf16, so that a
# gigabyte-scale cache is drawn in seconds).  Every cache element is random
# (also slots past a context), and num_blocks has a spare block per 8 in use
# that no sequence uses.


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    B: int
    H: int
    Hkv: int
    D: int
    block_size: int
    lo: int            # shortest context
    hi: int            # longest context
    dtype: str
    topk: int = 0      # pages kept per (sequence, key/value head) by the query-aware selection; 0 = all
    window: int = 0    # tokens per sequence of a second, sliding-window pool attended whole; 0 = none
    q_len: int = 1     # query tokens per sequence: the last q_len positions of each context, each causal

    @property
    def scale(self) -> float:
        return f32_scale(self.D)

    def lengths(self):
        rng = np.random.default_rng(self.seed)
        return rng.integers(self.lo, self.hi + 1, size=self.B)

    def window_pool(self) -> "DecodeWorkload":
        """The sliding-window pool: its own cache, every sequence holding
        `window` tokens (drawn from seed + 1)."""
        return DecodeWorkload(self.name + "_window", self.seed + 1, self.B, self.H, self.Hkv, self.D,
                              self.block_size, self.window, self.window, self.dtype)

    def layout(self):
        """(context_lens int32 (B,), block_tables int32 (B, max_blocks), num_blocks)."""
        rng = np.random.default_rng(self.seed)
        lens = rng.integers(self.lo, self.hi + 1, size=self.B)
        pages = -(-lens // self.block_size)
        used = int(pages.sum())
        num_blocks = used + used // 8 + 1
        perm = rng.permutation(num_blocks)
        max_blocks = int(pages.max()) if self.B else 0
        tables = np.full((self.B, max(max_blocks, 1)), -1, dtype=np.int32)
        i = 0
        for b in range(self.B):
            tables[b, : pages[b]] = perm[i:i + pages[b]]
            i += int(pages[b])
        return lens.astype(np.int32), tables, num_blocks


DECODE_WORKLOADS = {
    # 64 sequences of 512..16000 tokens (about 8K on average), 32 query heads over 8
    # key/value heads, D = 128, pages of 16 tokens
    "decode_gqa_bf16": DecodeWorkload("decode_gqa_bf16", 11, 64, 32, 8, 128, 16, 512, 16000, "bf16"),
    # a causal chunk on the same batch and cache: the last 4 tokens of every context
    # are written to the cache and attend, each causally, to the context up to themselves
    "verify_gqa_bf16": DecodeWorkload("verify_gqa_bf16", 11, 64, 32, 8, 128, 16, 512, 16000, "bf16", 0, 0, 4),
    # the same batch and cache with 64 pages (1024 tokens) kept per context by the query-aware selection
    "quest_gqa_bf16": DecodeWorkload("quest_gqa_bf16", 11, 64, 32, 8, 128, 16, 512, 16000, "bf16", 64),
    # two sources under one softmax: the same 64 kept pages plus a sliding-window pool of the
    # last 1024 tokens of every sequence, held in a cache of its own
    "window_quest_gqa_bf16": DecodeWorkload("window_quest_gqa_bf16", 11, 64, 32, 8, 128, 16, 512, 16000, "bf16",
                                            64, 1024),
}


def make_decode_inputs(w: DecodeWorkload):
    """torch CPU tensors (q, k_cache, v_cache, block_tables, context_lens) of a decode workload."""
    import torch

    lens, tables, num_blocks = w.layout()
    rng = np.random.default_rng(w.seed)
    rng.integers(w.lo, w.hi + 1, size=w.B)  # the lengths drawn by layout()
    rng.permutation(num_blocks)             # the page placement drawn by layout()
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def draw(shape):
        x = torch.from_numpy(rng.integers(-32, 32, size=shape, dtype=np.int8))
        return x.to(tdt) * 0.0625  # exact: a power-of-two scale of small integers

    q = draw((w.B, w.H, w.D) if w.q_len == 1 else (w.B, w.q_len, w.H, w.D))
    kc = draw((num_blocks, w.Hkv, w.D // 8, w.block_size, 8))
    vc = draw((num_blocks, w.Hkv, w.D, w.block_size))
    return q, kc, vc, torch.from_numpy(tables), torch.from_numpy(lens)
