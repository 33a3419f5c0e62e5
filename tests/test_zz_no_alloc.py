"""moe_permute_noalloc (the permutation map with its scratch in the library's
own device array) against moe_permute with a caller workspace, through the C
ABI, on the same seeded inputs: counts, offsets, row_of, token_of and the
permuted rows bit-exact, on two calls in a row, the second with a smaller
input (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import announce, bits, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(T, E, k, d, seed):
    g = torch.Generator().manual_seed(seed)
    L = torch.randn(T, E, generator=g)
    L[:, 1] -= 50.0                                          # an expert with no rows
    x = torch.randn(T, d, generator=g).to(torch.bfloat16)
    p = torch.rand(T, k, generator=g)
    return L, x, p


def _outputs(T, E, k, d):
    P = T * k
    return dict(c=torch.full((E,), -3, dtype=torch.int32, device="cuda"),
                o=torch.full((E + 1,), -3, dtype=torch.int32, device="cuda"),
                r=torch.full((T, k), -3, dtype=torch.int32, device="cuda"),
                tk=torch.full((P,), -3, dtype=torch.int32, device="cuda"),
                xp=torch.full((P, d), 7.0, dtype=torch.bfloat16, device="cuda"),
                dO=torch.full((P, d), 7.0, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("second", [(257, 16, 2, 128), (1, 4, 3, 64)])
def test_noalloc_permute_matches_workspace_permute(second):
    need_gpu()
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    for T, E, k, d in [(3000, 256, 8, 256), second]:
        announce(f"moe_permute_noalloc T={T} E={E} k={k} d={d}")
        sh = tre.make_shape(T, d, E, k, 128, 0, "bf16")
        L, x, p = _inputs(T, E, k, d, seed=T + E)
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
        tre.moe_route(L.cuda(), k, idx, prob)
        xc, pc = x.cuda(), p.cuda()
        ref, got = _outputs(T, E, k, d), _outputs(T, E, k, d)
        ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8,
                         device="cuda")
        tre.moe_permute(sh, xc, idx, None, 1, ref["c"], ref["o"], ref["r"], ref["tk"], ref["xp"], ws)
        tre.moe_permute(sh, xc, None, pc, 0, None, None, ref["r"], None, ref["dO"], None)
        tre.moe_permute_noalloc(sh, xc, idx, None, 1, got["c"], got["o"], got["r"], got["tk"],
                                got["xp"])
        tre.moe_permute_noalloc(sh, xc, None, pc, 0, None, None, got["r"], None, got["dO"])
        torch.cuda.synchronize()
        for name in ("c", "o", "r", "tk"):
            assert torch.equal(got[name], ref[name]), name
        assert np.array_equal(bits(got["xp"]), bits(ref["xp"]))
        assert np.array_equal(bits(got["dO"]), bits(ref["dO"]))
        # and both are the oracle's map
        counts, offsets, row_of, token_of = oracle.permute_map(idx.cpu().numpy(), E)
        assert np.array_equal(got["o"].cpu().numpy(), offsets)
        assert np.array_equal(got["r"].cpu().numpy(), row_of)


def test_noalloc_permute_refuses_maps_beyond_its_array():
    """E * ceil(T / 256) int32 counts above 1 MiB: MOE_ERR_WORKSPACE, nothing enqueued."""
    need_gpu()
    import ctypes as C
    from token_routed_expert_amd import _native as N, make_shape
    sh = make_shape(1025 * 256, 64, 256, 2, 128, 0, "bf16")   # 256 * 1025 * 4 B > 1 MiB
    P = C.c_void_p(16)
    # the size check comes before any launch, so the dummy pointers are never used
    assert N.lib().moe_permute_noalloc(C.byref(sh), P, P, None, 1, P, P, P, P, P, None) == \
        N.MOE_ERR_WORKSPACE
