"""The library's calls under HIP graph capture (torch.cuda.graph): every call
only enqueues kernels on the caller's stream and allocates nothing, so a
captured forward + backward and a captured split paged decode replay to the
eager results bit for bit (the kernels use no atomics).  Each graph is replayed
several times with other eager work of the library and synchronisations in
between, and every replay is checked.
"""
import numpy as np
import pytest

import workloads
from gpu_util import device_inputs, has_gpu, log

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _fa():
    import exact_attention_03_amd as fa

    return fa


def _bits(t):
    import torch

    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("Hkv", [4, 2])
def test_forward_backward_graph_replays(Hkv):
    import torch

    fa = _fa()
    w = workloads.Workload("graph", 61 + Hkv, 2, 4, 300, 128, "bf16", True, 1.0, Hkv)
    log(f"case graph fwd+bwd {w}")
    _, (q, k, v, do) = device_inputs(w)
    o_e, lse_e = fa.forward(q, k, v, causal=True, scale=w.scale)
    grads_e = fa.backward(q, k, v, o_e, do, lse_e, causal=True, scale=w.scale)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side, as torch recommends
        fa.forward(q, k, v, causal=True, scale=w.scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, lse_g = fa.forward(q, k, v, causal=True, scale=w.scale)
        grads_g = fa.backward(q, k, v, o_g, do, lse_g, causal=True, scale=w.scale)
    other = device_inputs(workloads.Workload("graph_other", 71, 1, 2, 200, 64, "f16", False, 1.0))[1]
    for r in range(3):
        for t in (o_g, lse_g, *grads_g):
            t.zero_()
        g.replay()
        fa.forward(*other[:3], scale=0.125)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(o_g), _bits(o_e)) and torch.equal(lse_g, lse_e), f"replay {r}: forward"
        for a, b in zip(grads_g, grads_e):
            assert torch.equal(_bits(a), _bits(b)), f"replay {r}: gradients"


def test_paged_decode_graph_replays():
    """A decode whose contexts are split over several workgroups (partial
    results in a workspace, then the combine kernel), captured and replayed."""
    import torch

    fa = _fa()
    w = workloads.DecodeWorkload("graph_decode", 73, 3, 8, 2, 128, 16, 2000, 9000, "bf16")
    g_in = [t.cuda() for t in workloads.make_decode_inputs(w)]
    mcl = int(g_in[4].max())
    splits = fa.lib().fa_paged_decode_workspace_bytes(3, 8, 2, 128, mcl)
    assert splits > 0  # the split path (workspace + combine) is what is captured
    o_e, lse_e = fa.paged_decode(*g_in, max_context_len=mcl, scale=w.scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o_g, lse_g = fa.paged_decode(*g_in, max_context_len=mcl, scale=w.scale)
    for r in range(3):
        o_g.zero_()
        lse_g.zero_()
        g.replay()
        fa.paged_decode(*g_in, max_context_len=mcl, scale=w.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o_g), _bits(o_e)) and torch.equal(lse_g, lse_e), f"replay {r}: decode"
    assert np.isfinite(lse_e.cpu().numpy()).all()
