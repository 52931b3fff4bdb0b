"""Paged KV cache: cache writes and decode attention over pages, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  [Serving-Ascend] is
the page "从算子到 Serving：昇腾推理评测链路实践" (BiumBiu), sections
"ReshapeAndCache" and "GQA Paged Attention".

What the page fixes: a new token's key and value go to the physical block
slot // block_size at offset slot % block_size, and tokens with a negative
slot are skipped; attention reads the pages of a sequence through its block
table, uses the sequence's context length, masks the invalid tokens of the
last block, and lets several query heads share one key/value head.

Readings of what it leaves open:

* cache layouts: k_cache is (num_blocks, Hkv, D/8, block_size, 8), one page
  of a key/value head holding its keys in chunks of 8 channels, chunk-major
  (channel d of the token at offset o is at [block, head, d // 8, o, d % 8]);
  v_cache is (num_blocks, Hkv, D, block_size), the page's values stored
  transposed (one row of block_size values per channel d);
* new tokens arrive as key, value (num_tokens, Hkv, D) with an int64
  slot_mapping (num_tokens,); slots of one call are distinct;
* decode: one query token per sequence, q (B, H, D); block_tables
  (B, max_blocks) int32, token t of sequence b lives in physical block
  block_tables[b, t // block_size] at offset t % block_size; context_lens (B,);
  every token of the context is visible (the query is the newest token);
* query head h uses key/value head h // (H / Hkv), as for grouped attention;
* a sequence with context length 0 has no keys: O = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

__all__ = ["reshape_and_cache", "gather_context", "paged_decode"]


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def reshape_and_cache(key, value, slot_mapping, k_cache, v_cache):
    """Return copies of (k_cache, v_cache) with each token written at its slot.

    [Serving-Ascend] "ReshapeAndCache": block = slot // block_size, offset =
    slot % block_size; a negative slot skips the token.  The caches keep
    their dtype (the write is a copy, no arithmetic).
    """
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    num_blocks, n_kv, n_chunks, block_size, x = k_cache.shape
    D = n_chunks * x
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if key.shape != (slots.size, n_kv, D) or value.shape != key.shape:
        raise ValueError("key and value must be (num_tokens, Hkv, D) matching the caches")
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = int(slot) // block_size, int(slot) % block_size
        if block >= num_blocks:
            raise ValueError(f"slot {slot} lies past the last block")
        for hk in range(n_kv):
            k_cache[block, hk, :, offset, :] = key[i, hk, :].reshape(n_chunks, x)
            v_cache[block, hk, :, offset] = value[i, hk, :]
    return k_cache, v_cache


def gather_context(k_cache, v_cache, table_row, context_len, kv_head):
    """The context of one sequence for one key/value head as contiguous
    (context_len, D) K and V, token by token through the block table
    ([Serving-Ascend] "GQA Paged Attention": logical block t // block_size
    maps to a physical block, the token sits at offset t % block_size)."""
    num_blocks, _, n_chunks, block_size, x = k_cache.shape
    D = n_chunks * x
    K = np.empty((context_len, D), dtype=k_cache.dtype)
    V = np.empty((context_len, D), dtype=v_cache.dtype)
    for t in range(context_len):
        block = int(table_row[t // block_size])
        if not 0 <= block < num_blocks:
            raise ValueError(f"block table entry {block} out of range")
        K[t] = k_cache[block, kv_head, :, t % block_size, :].reshape(D)
        V[t] = v_cache[block, kv_head, :, t % block_size]
    return K, V


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale):
    """(O, lse) of decode attention over a paged cache.

    q: (B, H, D).  For sequence b and query head h (key/value head
    h // (H / Hkv)): s_t = scale * q . k_t over the context's tokens
    t < context_lens[b]; O = sum_t softmax(s)_t v_t; lse = ln sum_t exp(s_t)
    (the plain softmax of [FA-Ascend] §一 for one query row; the page's
    online softmax reaches the same values).  Tokens past the context,
    including the rest of the last block, take no part.
    """
    q = _as_f64(q)
    B, H, D = q.shape
    n_kv = k_cache.shape[1]
    if n_kv <= 0 or H % n_kv != 0:
        raise ValueError("query heads must be a whole multiple of key/value heads")
    G = H // n_kv
    O = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        for hk in range(n_kv):
            K, V = gather_context(k_cache, v_cache, block_tables[b], n, hk)
            K, V = _as_f64(K), _as_f64(V)
            for h in range(hk * G, (hk + 1) * G):
                s = (K @ q[b, h]) * scale
                m = np.max(s)
                e = np.exp(s - m)
                l = np.sum(e)
                O[b, h] = (e @ V) / l
                lse[b, h] = m + np.log(l)
    return O, lse
