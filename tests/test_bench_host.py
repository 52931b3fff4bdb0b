"""Host checks of bench.py's bookkeeping: the executed-work ratios and the
decode byte models (no GPU)."""
import numpy as np

import bench
import workloads


def _brute_pairs(n, bq, bk, causal):
    """Blocks of bq queries x bk keys a kernel computes, enumerated: a block
    is skipped only when every key follows every query of the block."""
    total = 0
    for q0 in range(0, n, bq):
        for k0 in range(0, n, bk):
            if causal and k0 > q0 + bq - 1:
                continue
            total += bq * bk
    return total


def test_computed_pairs_against_enumeration():
    for n in (1, 31, 32, 33, 100, 128, 1000):
        for bq, bk in ((32, 32), (32, 64), (64, 32)):
            for causal in (False, True):
                assert bench._computed_pairs(n, bq, bk, causal) == _brute_pairs(n, bq, bk, causal)


def test_executed_ratios():
    r = bench.executed_over_counted(workloads.WORKLOADS["d128_causal"])
    # 1024 tokens in 32-blocks: 32 * 33 / 2 lower-triangle blocks of 1024 pairs over 1024^2 / 2
    assert r["fa_fwd"] == round(528 / 512, 4) and r["fa_bwd_dkdv"] == round(528 / 512, 4)
    assert r["fa_bwd_dq"] == round(3 * 528 / 512, 4)
    r = bench.executed_over_counted(workloads.WORKLOADS["d256_bf16"])
    assert r == {"fa_fwd": 1.5, "fa_bwd_dq": 3.0, "fa_bwd_dkdv": 1.0, "fa_bwd_fused": 1.0}


def test_two_source_bytes_add_the_window():
    w = workloads.DECODE_WORKLOADS["window_quest_gqa_bf16"]
    wq = workloads.DECODE_WORKLOADS["quest_gqa_bf16"]
    lens = np.array([1000, 16000, 17], dtype=np.int64)
    sel_a, dec_a = bench.quest_bytes(w, lens)
    sel_b, dec_b = bench.quest_bytes(wq, lens)
    per_seq = 1024 * w.Hkv * w.D * 2 * 2 + (1024 // 16) * w.Hkv * 4
    assert sel_a == sel_b and dec_a - dec_b == len(lens) * per_seq


def test_source_hash_ignores_comments_only():
    """A stored measurement stays valid across comment edits, not across code edits."""
    a = "int f(int x) {  // twice\n  return 2 * x; /* scaled */\n}\n"
    b = "// a new header line\nint f(int x) {\n  return 2 * x;\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)
