"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
run the oracle on the same stored inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_workloads import Workload, make_inputs, to_f64

TOL = {"f32": 1e-4, "bf16": 2e-2}
PROB_TOL = 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str):
    print(f"\n[gpu-case] {msg}", file=sys.stderr, flush=True)


def gpu_inputs(wl: Workload, seed: int = 0, **logit_overrides):
    inp = make_inputs(wl, seed=seed, device="cuda")
    torch.cuda.synchronize()
    return inp


def run_layer(wl: Workload, inp: dict, **kw):
    """moe_layer_fwd + moe_layer_bwd through the C ABI; returns every buffer.
    kw goes to layer_buffers (router_grad, aux_alpha)."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import layer_buffers
    sh, b, wsf, wsb = layer_buffers(wl.T, wl.d, wl.E, wl.k, wl.f, wl.f_shared, wl.dtype, "cuda", inp,
                                    **kw)
    tre.moe_layer_fwd(sh, b, wsf)
    tre.moe_layer_bwd(sh, b, wsb)
    torch.cuda.synchronize()
    return b


def host_inputs(inp: dict):
    """fp64 numpy copies of the stored inputs (exact up-casts); logits stay fp32."""
    out = {k: to_f64(v) for k, v in inp.items() if k != "logits"}
    out["logits"] = inp["logits"].cpu().numpy()
    return out


def oracle_layer(wl: Workload, h: dict):
    shared = (h["Ws1"], h["Ws3"], h["Ws2"]) if wl.f_shared else None
    st = oracle.layer_fwd(h["logits"], h["x"], h["W1"], h["W3"], h["W2"], wl.k, shared)
    g = oracle.layer_bwd(st, h["dY"], h["W1"], h["W3"], h["W2"], shared)
    return st, g


def np_of(t: torch.Tensor):
    return to_f64(t)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a tensor as an integer numpy array."""
    t = t.detach().cpu().contiguous()
    it = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}[t.dtype]
    return t.view(it).numpy()


def assert_close(name, got, ref, tol):
    err = oracle.row_rel_err(got, ref)
    assert err <= tol, f"{name}: row-relative error {err:.3e} > {tol:.1e}"
    return err


def check_routing_and_map(wl, b, inp, st):
    """Bit-exact routing indices, counts, offsets, row map and permuted rows."""
    assert np.array_equal(b["topk_idx"].cpu().numpy(), st["idx"]), "topk_idx"
    assert np.abs(b["topk_prob"].cpu().numpy().astype(np.float64) - st["p"]).max() <= PROB_TOL
    assert np.array_equal(b["counts"].cpu().numpy(), st["counts"]), "counts"
    assert np.array_equal(b["offsets"].cpu().numpy(), st["offsets"]), "offsets"
    assert np.array_equal(b["row_of"].cpu().numpy(), st["row_of"]), "row_of"
    assert np.array_equal(b["token_of"].cpu().numpy(), st["token_of"]), "token_of"
    if "xp" in b:                     # (the fused permutation writes no xp)
        assert np.array_equal(bits(b["xp"]), oracle.permute_rows(bits(inp["x"]), st["token_of"])), "xp"
