"""Host-side checks that need no GPU: the C ABI loads and exports every symbol
its header declares, argument errors come back before any HIP call, and the
schedule/tile logic reproduces the page's worked numbers (tests/golden/)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The argument-check tests hand the library dummy pointers that must fail
# validation before any HIP call; where a GPU is visible a slip in such a test
# would launch a kernel on them, so they run only where none is.
_NO_GPU = pytest.mark.skipif(_gpu_visible(), reason="dummy-pointer argument checks run only without a GPU")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=")
                out[k] = float(v) if "." in v else int(v)
    return out


@pytest.fixture(scope="module")
def fa():
    import exact_attention_03_amd as fa

    fa.lib()  # raises if libfa.so has not been built
    return fa


def test_library_exports_every_declared_symbol(fa):
    from exact_attention_03_amd._lib import SIGNATURES

    header = open(os.path.join(ROOT, "include", "fa.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", header))
    assert declared, "no declarations found"
    lib = fa.lib()
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in fa.h but not exported"
    assert declared == set(SIGNATURES), "binding signatures out of step with fa.h"


def test_status_strings(fa):
    assert fa.status_name(0) == "FA_OK"
    assert fa.status_name(1) == "FA_ERR_INVALID_ARGUMENT"
    assert fa.status_name(2) == "FA_ERR_UNSUPPORTED"
    assert fa.status_name(3) == "FA_ERR_HIP"
    assert fa.lib().fa_version() >= 100


P = ctypes.c_void_p(0x10000)  # aligned dummy; never dereferenced on error paths
MIS = ctypes.c_void_p(0x10008)


def _fwd(fa, Z=1, H=1, N=128, D=64, dtype=0, odt=0, q=P, k=P, v=P, o=P, lse=P, scale=0.125, causal=0):
    return fa.lib().fa_fwd(Z, H, N, D, dtype, odt, q, k, v, o, lse, scale, causal, None)


@_NO_GPU
@pytest.mark.parametrize("kw,status", [
    (dict(D=96), 2), (dict(D=0), 2), (dict(N=-1), 1), (dict(dtype=7), 1), (dict(odt=1), 1),
    (dict(q=None), 1), (dict(o=MIS), 1), (dict(lse=None), 1), (dict(scale=0.0), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1), (dict(causal=2), 1),
    (dict(N=1 << 30, D=256), 2),
])
def test_fwd_argument_errors(fa, kw, status):
    assert _fwd(fa, **kw) == status
    assert fa.last_error() != ""


@_NO_GPU
def test_empty_problem_is_ok_without_pointers(fa):
    assert _fwd(fa, Z=0, q=None, k=None, v=None, o=None, lse=None) == 0
    assert _fwd(fa, N=0, q=None, k=None, v=None, o=None, lse=None) == 0
    lib = fa.lib()
    assert lib.fa_bwd(0, 1, 8, 64, 0, 0, *([None] * 9), 0.125, 0, None, 0, None) == 0


@_NO_GPU
def test_bwd_workspace_rules(fa):
    lib = fa.lib()
    assert lib.fa_bwd_workspace_bytes(128, 8, 1024, 128) == 2 * 128 * 8 * 1024 * 4
    need = lib.fa_bwd_workspace_bytes(1, 2, 100, 64)
    st = lib.fa_bwd(1, 2, 100, 64, 0, 0, *([P] * 9), 0.125, 0, P, need - 4, None)
    assert st == 1 and "workspace" in fa.last_error()
    st = lib.fa_bwd(1, 2, 100, 64, 0, 0, *([P] * 9), 0.125, 0, None, need, None)
    assert st == 1


@_NO_GPU
def test_noalloc_backward_refuses_rows_past_its_array(fa):
    """fa_bwd_noalloc refuses a problem whose row statistics would not fit its
    fixed array before touching the device."""
    lib = fa.lib()
    limit = 1 << 22
    assert lib.fa_bwd_noalloc(1, 1, limit + 1, 64, 0, 0, *([P] * 9), 0.125, 0, None) == 2
    assert "FA_BWD_NOALLOC_MAX_ROWS" in fa.last_error()
    assert lib.fa_bwd_noalloc(4, 1 << 10, 1025, 64, 0, 0, *([P] * 9), 0.125, 0, None) == 2


@_NO_GPU
def test_stage_argument_errors(fa):
    lib = fa.lib()
    assert lib.fa_bwd_preprocess(1, 1, 64, 64, 0, 1, P, P, P, P, None) == 1    # o_dtype bf16 with f16
    assert lib.fa_bwd_preprocess(1, 1, 64, 64, 0, 0, P, P, None, P, None) == 1  # no lse
    assert lib.fa_bwd_dkdv(1, 1, 64, 64, 0, *([P] * 7), 0.125, 0, -1, None) == 1  # negative grid
    assert lib.fa_bwd_dkdv(1, 1, 64, 64, 0, *([P] * 4), None, P, P, 0.125, 0, 0, None) == 1  # no stats
    assert lib.fa_bwd_dq(1, 1, 64, 32, 0, *([P] * 6), 0.125, 0, None) == 2      # D = 32
    assert lib.fa_bwd_dq(1, 1, 64, 64, 0, *([P] * 5), MIS, 0.125, 0, None) == 1  # misaligned dq
    assert lib.fa_bwd_dq_and_stats(1, 1, 64, 64, 0, 1, *([P] * 8), 0.125, 0, None) == 1  # o bf16 with f16
    assert lib.fa_bwd_dq_and_stats(1, 1, 64, 64, 0, 0, *([P] * 5), None, P, P, 0.125, 0, None) == 1  # no lse
    assert lib.fa_bwd_dq_and_stats(1, 1, 64, 64, 0, 0, *([P] * 7), MIS, 0.125, 0, None) == 1  # misaligned dq
    assert lib.fa_bwd_dq_and_stats(1, 1, 64, 48, 0, 0, *([P] * 8), 0.125, 0, None) == 2  # D = 48
    assert lib.fa_bwd_dq_and_stats(0, 1, 64, 64, 0, 0, *([None] * 8), 0.125, 0, None) == 0  # empty


def test_causal_tile_count_matches_page(fa):
    g = _golden("causal_tile_count.txt")
    # The forward's query tiles are 128 rows, so N = 8 * 128 is the page's grid
    # of 8 query tiles.  Its key tiles are narrower (128 / r keys), so every
    # cell of the page's 8 x 8 grid is r key tiles: the visited count is the
    # page's 36 of 64, scaled by r, for every head dim.
    for D in (64, 128, 256):
        vis, tot = fa.fwd_tile_pairs(8 * 128, D, True)
        r = tot // g["full_tiles"]
        assert r * g["full_tiles"] == tot
        assert (vis, tot) == (r * g["causal_tiles"], r * g["full_tiles"])
        assert 100.0 * (1 - vis / tot) == pytest.approx(g["saved_percent"])
        assert fa.fwd_tile_pairs(8 * 128, D, False) == (tot, tot)


def test_persistent_dealing_matches_page(fa):
    """One key tile per head (N = 128) and no mask: the schedule deals heads to
    20 programs exactly as the page's fixed stride does: 51 or 52 each."""
    g = _golden("persistent_programs.txt")
    units, work, n = fa.dkdv_schedule(g["Z"], g["H"], 128, 64, False, g["programs"])
    assert n == g["heads"] == sum(units)
    assert min(units) == g["min_heads_per_program"] and max(units) == g["max_heads_per_program"]
    assert units.count(52) == g["heads"] - 51 * g["programs"]


@pytest.mark.parametrize("Z,H,N,D,causal,Pn", [
    (128, 8, 1024, 128, True, 256), (16, 16, 8192, 128, True, 256), (128, 8, 1024, 64, False, 256),
    (3, 5, 1000, 64, True, 97), (1, 1, 130, 256, True, 7), (2, 2, 300, 128, False, 1000),
])
def test_schedule_covers_units_and_balances(fa, Z, H, N, D, causal, Pn):
    units, work, n = fa.dkdv_schedule(Z, H, N, D, causal, Pn)
    bk = 128  # keys per unit: 32 per wave, 4 waves
    assert sum(units) == n == Z * H * ((N + bk - 1) // bk)
    bq = 32
    nq = (N + bq - 1) // bq
    total = sum(nq - ((kt * bk) // bq if causal else 0) for kt in range((N + bk - 1) // bk)) * Z * H
    assert sum(work) == total
    if n >= 4 * Pn:
        mean = total / Pn
        assert max(work) <= 1.10 * mean, (max(work), mean)


def test_workspace_versus_page_full_scratch(fa):
    g = _golden("full_scratch.txt")
    full = g["Z"] * g["H"] * g["N"] * g["N"] * g["bytes_per_element"]
    assert full == g["one_copy_bytes"]
    ours = fa.workspace_bytes(g["Z"], g["H"], g["N"], 128)
    assert ours == 2 * g["Z"] * g["H"] * g["N"] * 4 and ours * 256 == full


@_NO_GPU
def test_grouped_head_argument_errors(fa):
    lib = fa.lib()

    def fwd(H, Hkv, N=128, D=64):
        return lib.fa_fwd_gqa(1, H, Hkv, N, D, 0, 0, P, P, P, P, P, 0.125, 0, None)

    def bwd(H, Hkv, N=128, D=64):
        return lib.fa_bwd_gqa(1, H, Hkv, N, D, 0, 0, *([P] * 9), 0.125, 0, P, 1 << 30, None)

    for f in (fwd, bwd):
        assert f(6, 4) == 1 and "multiple" in fa.last_error()  # 6 query heads over 4
        assert f(4, 0) == 1
        assert f(4, -1) == 1
        assert f(4, 8) == 1                                  # more key/value heads than query heads
        assert f(1 << 14, 1, N=1 << 16, D=128) == 2          # one group beyond 32-bit offsets
        assert "group" in fa.last_error()
    assert lib.fa_fwd_gqa(1, 0, 0, 128, 64, 0, 0, *([None] * 5), 0.125, 0, None) == 0  # no heads: empty
    assert lib.fa_bwd_gqa(0, 4, 2, 128, 64, 0, 0, *([None] * 9), 0.125, 0, None, 0, None) == 0


@_NO_GPU
def test_varlen_argument_errors(fa):
    lib = fa.lib()
    CU = ctypes.c_void_p(0x20000)

    def fwd(B=2, H=4, Hkv=2, T=100, mx=60, D=64, cu=CU):
        return lib.fa_fwd_varlen(B, H, Hkv, T, mx, D, 0, 0, cu, P, P, P, P, P, 0.125, 1, None)

    def bwd(B=2, H=4, Hkv=2, T=100, mx=60, D=64, cu=CU, ws=1 << 30):
        return lib.fa_bwd_varlen(B, H, Hkv, T, mx, D, 0, 0, cu, *([P] * 9), 0.125, 1, P, ws, None)

    for f in (fwd, bwd):
        assert f(cu=None) == 1 and "cu_seqlens" in fa.last_error()
        assert f(cu=ctypes.c_void_p(0x20002)) == 1                 # misaligned offsets
        assert f(T=-1) == 1
        assert f(H=6, Hkv=4) == 1                                   # grouping
        assert f(D=96) == 2
        assert f(T=1 << 26, D=128) == 2 and "packed" in fa.last_error()
        assert f(B=0, cu=None) == 0 and f(T=0) == 0 and f(mx=0, cu=None) == 0  # empty problems
    assert bwd(ws=2 * 4 * 100 * 4 - 4) == 1 and "workspace" in fa.last_error()
    assert lib.fa_bwd_dkdv_varlen(2, 4, 2, 100, 60, 64, 0, CU, *([P] * 4), None, P, P, 0.125, 1, 0, None) == 1
    assert lib.fa_bwd_dq_and_stats_varlen(2, 4, 2, 100, 60, 64, 0, 1, CU, *([P] * 8), 0.125, 1, None) == 1


@_NO_GPU
def test_paged_and_quest_argument_errors(fa):
    """Every call here must fail validation (or be empty) before any HIP call:
    the pointers are dummies that no kernel may ever see."""
    lib = fa.lib()
    I4 = ctypes.c_void_p(0x30000)   # 4-byte aligned index array
    I8 = ctypes.c_void_p(0x30008)

    def dec(B=2, H=8, Hkv=2, D=128, bs=16, nb=10, mxb=4, mctx=64, ws=None, wsb=0, bt=I4):
        return lib.fa_paged_decode(B, H, Hkv, D, bs, nb, mxb, mctx, 0, 0, P, P, P, bt, I4, P, P, 0.1, ws, wsb, None)

    assert dec(Hkv=0) == 1 and dec(H=6, Hkv=4) == 1
    assert dec(D=96) == 2 and dec(bs=8) == 2 and dec(bs=24) == 2
    assert dec(bt=ctypes.c_void_p(0x30002)) == 1
    need = lib.fa_paged_decode_workspace_bytes(1, 8, 1, 128, 10000)
    assert need > 0 and lib.fa_paged_decode_workspace_bytes(64, 32, 8, 128, 200) == 0  # one split
    assert dec(B=1, Hkv=1, mctx=10000, mxb=700) == 1 and "workspace" in fa.last_error()
    assert dec(B=1, Hkv=1, mctx=10000, mxb=700, ws=P, wsb=need - 4) == 1
    assert dec(B=0, bt=None) == 0                                   # empty batch
    # cache writes
    rc = lambda T=4, Hkv=2, D=128, bs=16, nb=4, sl=I8: lib.fa_reshape_and_cache(  # noqa: E731
        T, Hkv, D, bs, nb, 0, P, P, sl, P, P, None)
    assert rc(sl=ctypes.c_void_p(0x30004)) == 1                     # slots not 8-byte aligned
    assert rc(sl=None) == 1 and rc(bs=8) == 2 and rc(D=32) == 2 and rc(T=-1) == 1
    assert rc(T=0, sl=None) == 0
    # page selection
    sel = lambda B=2, H=8, Hkv=2, mxb=100, topk=8, s=I4, ns=I4: lib.fa_quest_select(  # noqa: E731
        B, H, Hkv, 128, 16, 1000, mxb, topk, 0, P, P, I4, I4, s, ns, None)
    assert sel(mxb=4097) == 2 and "4096" in fa.last_error()
    assert sel(topk=-1) == 1 and sel(s=None) == 1 and sel(ns=None) == 1 and sel(H=40, Hkv=3) == 1
    assert lib.fa_quest_page_minmax(2, 2, 128, 16, 100, 5, 0, P, I4, I4, None, None) == 1
    assert lib.fa_quest_page_minmax(2, 2, 96, 16, 100, 5, 0, P, I4, I4, P, None) == 2
    sp = lambda topk=8, s=I4: lib.fa_paged_decode_sparse(  # noqa: E731
        2, 8, 2, 128, 16, 100, 50, topk, 0, 0, P, P, P, I4, I4, s, I4, P, P, 0.1, None, 0, None)
    assert sp(topk=-1) == 1 and sp(s=None) == 1


@_NO_GPU
def test_two_source_decode_argument_errors(fa):
    """Argument rules of fa_paged_decode_sources; every call fails validation
    (or is empty) before any HIP call."""
    from exact_attention_03_amd._lib import KvSource

    lib = fa.lib()
    I4 = ctypes.c_void_p(0x30000)

    def src(bs=16, nb=100, mxb=50, mctx=800, sel=None, nsel=None, topk=0, kc=P, bt=I4):
        return KvSource(kc, P, bt, I4, bs, nb, mxb, mctx, sel, nsel, topk)

    def call(srcs, n=None, B=2, H=8, Hkv=2, ws=None, wsb=0):
        arr = (KvSource * max(1, len(srcs)))(*srcs)
        n = len(srcs) if n is None else n
        return lib.fa_paged_decode_sources(B, H, Hkv, 128, 0, 0, P, n, arr, P, P, 0.1, ws, wsb, None)

    dense, sparse = src(), src(sel=I4, nsel=I4, topk=8)
    assert call([dense], n=0) == 1 and call([dense, sparse], n=3) == 1
    assert lib.fa_paged_decode_sources(2, 8, 2, 128, 0, 0, P, 1, None, P, P, 0.1, None, 0, None) == 1
    assert call([dense, src(bs=8)]) == 2 and "source 1" in fa.last_error()
    assert call([src(sel=I4)]) == 1                                  # selected without n_selected
    assert call([src(sel=None, nsel=I4, topk=4)]) == 1               # topk > 0 needs selected
    assert call([dense, src(kc=None)]) == 1 and call([src(bt=ctypes.c_void_p(0x30002))]) == 1
    assert call([src(mxb=-1)]) == 1
    assert call([dense, sparse], B=0) == 0                           # empty batch
    assert call([dense, src(kc=None)], B=0) == 0                     # pointers unread when empty
    # workspace: the splits of both sources together
    one = lib.fa_paged_decode_sources_workspace_bytes(1, 8, 1, 128, 1, (KvSource * 1)(src(mctx=10000)))
    assert one == lib.fa_paged_decode_workspace_bytes(1, 8, 1, 128, 10000) > 0
    two = lib.fa_paged_decode_sources_workspace_bytes(1, 8, 1, 128, 2, (KvSource * 2)(src(mctx=10000),
                                                                                      src(mctx=5000)))
    assert two > one
    # two one-split sources still need a combine: workspace for 2 splits
    small = (KvSource * 2)(src(mctx=64), src(sel=I4, nsel=I4, topk=2))
    assert lib.fa_paged_decode_sources_workspace_bytes(1, 8, 1, 128, 2, small) == 8 * 2 * 129 * 4
    assert call([src(mctx=64), src(sel=I4, nsel=I4, topk=2)], B=1, Hkv=1) == 1 and "workspace" in fa.last_error()


@_NO_GPU
def test_several_query_rows_argument_errors(fa):
    """fa_paged_attention_sources: Tq rules, row_lens alignment, workspace for
    Tq rows; every call fails validation (or is empty) before any HIP call."""
    from exact_attention_03_amd._lib import KvSource

    lib = fa.lib()
    I4 = ctypes.c_void_p(0x30000)

    def src(rows=None, mctx=800):
        return KvSource(P, P, I4, I4, 16, 100, 50, mctx, None, None, 0, rows)

    def call(srcs, Tq=3, B=2, ws=None, wsb=0):
        arr = (KvSource * len(srcs))(*srcs)
        return lib.fa_paged_attention_sources(B, Tq, 8, 2, 128, 0, 0, P, len(srcs), arr, P, P, 0.1, ws, wsb, None)

    assert call([src()], Tq=-1) == 1
    assert call([src()], Tq=0) == 0                                      # empty
    assert call([src(rows=ctypes.c_void_p(0x30002))]) == 1 and "row_lens" in fa.last_error()
    one = lib.fa_paged_attention_sources_workspace_bytes(1, 1, 8, 2, 128, 1, (KvSource * 1)(src(mctx=10000)))
    five = lib.fa_paged_attention_sources_workspace_bytes(1, 5, 8, 2, 128, 1, (KvSource * 1)(src(mctx=10000)))
    assert one > 0 and five == 5 * one
    assert one == lib.fa_paged_decode_sources_workspace_bytes(1, 8, 2, 128, 1, (KvSource * 1)(src(mctx=10000)))
    assert call([src(mctx=10000)], Tq=5, B=1, ws=P, wsb=five - 4) == 1 and "workspace" in fa.last_error()
