"""fa_bwd_noalloc (the backward whose row statistics live in the library's
fixed device array) against fa_bwd with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller problem, each equal to fa_bwd bit
for bit (the same kernels in the same order) and therefore within the
gradient tolerance of the oracle comparison; sizes past the array are
refused before any work."""
import ctypes

import pytest

import workloads
from gpu_util import GRAD_NORMWISE, device_inputs, has_gpu, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _bwd_both(fa, w):
    import torch

    lib = fa.lib()
    cpu, gpu = device_inputs(w)
    q, k, v, do = gpu
    Z, H, N, D = w.shape
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.scale)
    code = fa._dtype_code(q)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty((lib.fa_bwd_workspace_bytes(Z, H, N, D) // 4,), dtype=torch.float32, device="cuda")
    st = lib.fa_bwd(Z, H, N, D, code, code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                    *(_ptr(t) for t in ref), w.scale, int(w.causal), _ptr(ws), ws.numel() * 4, stream)
    assert st == 0, fa.last_error()
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = lib.fa_bwd_noalloc(Z, H, N, D, code, code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                            *(_ptr(t) for t in got), w.scale, int(w.causal), stream)
    assert st == 0, fa.last_error()
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_equals_workspace_backward_twice():
    import torch

    import exact_attention_03_amd as fa

    for w in (workloads.Workload("noalloc_a", 61, 2, 4, 700, 128, "f16", True),
              workloads.Workload("noalloc_b", 62, 1, 3, 200, 64, "bf16", False)):
        log(f"case {w.name} shape={w.shape} dtype={w.dtype} causal={w.causal}")
        ref, got = _bwd_both(fa, w)
        for a, b, n in zip(ref, got, ("dq", "dk", "dv")):
            err = float((b.double() - a.double()).norm() / a.double().norm())
            assert err <= GRAD_NORMWISE, (w.name, n, err)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (w.name, n, "not bitwise equal")
        log(f"{w.name}: dq/dk/dv equal fa_bwd bit for bit")


def test_noalloc_refuses_problems_past_its_array():
    import exact_attention_03_amd as fa

    lib = fa.lib()
    rows = 1 << 22
    # One row more than the array holds; the pointers are never dereferenced.
    dummy = ctypes.c_void_p(256)
    st = lib.fa_bwd_noalloc(1, 1, rows + 1, 128, 0, 0, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                            dummy, 0.1, 0, None)
    assert st == fa._lib.FA_ERR_UNSUPPORTED
    assert "FA_BWD_NOALLOC_MAX_ROWS" in fa.last_error()
