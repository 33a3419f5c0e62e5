"""HIP-graph capture of a whole layer (moe_layer_fwd + moe_layer_bwd).

The library's calls only enqueue kernels on the caller's stream, read every
per-expert size from device memory and never synchronise, so a layer can be
captured once and replayed (the pages run dropless MoE under full CUDA-graph
coverage with sync-free dynamic shapes: German technical summary, section 2 D).
Each replay, with the outputs overwritten by eager work in between, must give
results bit-identical to the eager run.
"""
import pytest
import torch

from moe_workloads import Workload, make_inputs

from gpu_common import announce, need_gpu

pytestmark = pytest.mark.gpu

CASES = [
    (Workload("graph_bf16", T=300, d=256, E=8, k=2, f=384), dict(router_grad=True)),
    (Workload("graph_shared", T=200, d=256, E=16, k=4, f=256, f_shared=256), {}),
    (Workload("graph_e4m3", T=260, d=256, E=16, k=2, f=256, dtype="e4m3", skew=True),
     dict(router_grad=True)),
    (Workload("graph_mx_me", T=260, d=256, E=8, k=3, f=256, dtype="mxfp8"),
     dict(memory_efficient=1)),
]

INPUT_KEYS = ("logits", "x", "W1", "W3", "W2", "Ws1", "Ws3", "Ws2", "dY", "wq", "wmx",
              "aux_alpha", "memory_efficient")


@pytest.mark.parametrize("wl,kw", CASES, ids=lambda c: c.name if isinstance(c, Workload) else "")
def test_layer_graph_replay_equals_eager(wl, kw):
    need_gpu()
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import layer_buffers
    announce(f"graph capture {wl.name} {kw}")
    inp = make_inputs(wl, seed=5, device="cuda")
    sh, b, wsf, wsb = layer_buffers(wl.T, wl.d, wl.E, wl.k, wl.f, wl.f_shared, wl.dtype, "cuda", inp,
                                    **kw)
    outs = {n: t for n, t in b.items()
            if isinstance(t, torch.Tensor) and n not in INPUT_KEYS}
    tre.moe_layer_fwd(sh, b, wsf)
    tre.moe_layer_bwd(sh, b, wsb)
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in outs.items()}

    def poison():
        for t in outs.values():
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-5 if t.dtype != torch.uint8 else 0xAB)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        tre.moe_layer_fwd(sh, b, wsf)
        tre.moe_layer_bwd(sh, b, wsb)
    torch.cuda.synchronize()
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, ref in eager.items():
            got = outs[n]
            same = torch.equal(got.view(torch.uint8), ref.view(torch.uint8)) \
                if got.dtype.itemsize == 1 else torch.equal(
                    got.view({2: torch.int16, 4: torch.int32, 8: torch.int64}[got.dtype.itemsize]),
                    ref.view({2: torch.int16, 4: torch.int32, 8: torch.int64}[ref.dtype.itemsize]))
            assert same, f"replay {rep}: {n} differs from the eager run"
    del g
