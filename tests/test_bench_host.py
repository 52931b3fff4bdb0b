"""Host checks of bench.py's bookkeeping: the executed-work ratios and the
decode byte models, and a static check of its names (no GPU)."""
import os

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


def test_bench_functions_use_only_defined_names():
    """Every name a top-level function of bench.py reads is bound in that
    function (or a function nested in it), at module level or in builtins:
    a static guard for the paths only a GPU run executes."""
    import ast
    import builtins

    src = open(bench.__file__, encoding="utf-8").read()
    tree = ast.parse(src)
    module_names = set(dir(builtins))
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            module_names.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            module_names.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, (ast.Assign, ast.AnnAssign, ast.AugAssign)):
            for t in (node.targets if isinstance(node, ast.Assign) else [node.target]):
                module_names.update(n.id for n in ast.walk(t) if isinstance(n, ast.Name))
    missing = {}
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef)):
        bound, loads = set(), set()
        for n in ast.walk(fn):
            if isinstance(n, (ast.FunctionDef, ast.Lambda)):
                a = n.args
                bound.update(x.arg for x in a.args + a.kwonlyargs + a.posonlyargs)
                bound.update(x.arg for x in (a.vararg, a.kwarg) if x is not None)
                if isinstance(n, ast.FunctionDef):
                    bound.add(n.name)
            elif isinstance(n, ast.Name):
                (bound if isinstance(n.ctx, (ast.Store, ast.Del)) else loads).add(n.id)
            elif isinstance(n, (ast.Import, ast.ImportFrom)):
                bound.update((a.asname or a.name).split(".")[0] for a in n.names)
            elif isinstance(n, ast.ExceptHandler) and n.name:
                bound.add(n.name)
        undefined = loads - bound - module_names
        if undefined:
            missing[fn.name] = sorted(undefined)
    assert not missing, missing
