"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the oracle-side tests and by the GPU-side tests and
benchmark. It holds shapes, seeds and random draws only: no routing, no
permutation, no GEMM, no activation and no quantisation.  Every tensor is drawn
in fp32 from a per-tensor torch generator and then stored in the workload's
storage dtype (fp32 or bf16; torch's float->bfloat16 cast rounds to nearest
even).

Workload shapes follow the expert layer of the models the pages measure
(Scalable Training of Mixture-of-Experts Models with Megatron Core, gist.science
summaries, results sections: DeepSeek-V3 and Qwen3-235B), plus a Mixtral-class
shape, a tiny fp32 case and a skewed fp8 stress case.

Notation: T tokens, d hidden size, E experts, k experts per token, f expert FFN
width, f_shared the width of an always-on shared expert (0 = none).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    f_shared: int = 0
    dtype: str = "bf16"          # "f32" | "bf16" | "e4m3" | "mxfp8" (fp8: bf16 x, dY; fp32 weights)
    skew: bool = False           # add a Zipf-rank bias to the logits (hot/cold experts)

    @property
    def P(self) -> int:
        """Routed rows: every token goes to exactly k experts (dropless)."""
        return self.T * self.k

    def flops_fwd_bwd(self) -> float:
        """Algorithmic GEMM flop of one forward+backward pass.

        Each routed (token, expert) pair costs 6*d*f flop forward (three
        d-by-f products at 2 flop per multiply-add), the same for dgrad and
        for wgrad; the shared expert adds the same per token.
        """
        return 18.0 * self.d * self.f * self.P + 18.0 * self.d * self.f_shared * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of this project.  Sizes and distributions are described
# next to each; the skewed case's bias recipe is in skew_bias() below.
WORKLOADS = {
    # tiny fp32 layer, small enough for the oracle in well under a second
    "tiny_f32": Workload("tiny_f32", T=256, d=64, E=8, k=2, f=128, dtype="f32"),
    # Mixtral-class: 8 experts, top-2, wide FFN
    "mixtral_bf16": Workload("mixtral_bf16", T=4096, d=4096, E=8, k=2, f=14336),
    # Qwen3-MoE-class: 128 fine-grained experts, top-8 (about 512 rows per expert)
    "qwen3_bf16": Workload("qwen3_bf16", T=8192, d=4096, E=128, k=8, f=1536),
    # DeepSeek-V3-class: 256 routed experts, top-8, plus one shared expert
    "deepseek_v3_bf16": Workload("deepseek_v3_bf16", T=16384, d=7168, E=256, k=8, f=2048,
                                 f_shared=2048),
    # Qwen3 shape with T off the tile grid, Zipf-skewed routing, fp8 expert GEMMs
    "skewed_fp8": Workload("skewed_fp8", T=8200, d=4096, E=128, k=8, f=1536, dtype="e4m3",
                           skew=True),
}
# The skewed fp8 shape with MXFP8 operands (E8M0 scales per 32 values) in place
# of the blockwise e4m3 recipe.
VARIANTS = {
    "skewed_mxfp8": WORKLOADS["skewed_fp8"].with_(name="skewed_mxfp8", dtype="mxfp8"),
}

# Order in which per-tensor streams are named (each gets its own generator).
TENSOR_NAMES = ("bias_perm", "logits", "x", "W1", "W3", "W2", "Ws1", "Ws3", "Ws2", "dY")


def _stream_seed(seed: int, workload: str, tensor: str) -> int:
    h = hashlib.sha256(f"{seed}/{workload}/{tensor}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, wl: Workload, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, wl.name, tensor))
    return g


def storage_dtype(wl: Workload) -> torch.dtype:
    """dtype of x, dY and (for f32/bf16) the expert weights."""
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def weight_dtype(wl: Workload) -> torch.dtype:
    """The fp8 workload draws fp32 master weights; the path quantises them itself."""
    if wl.dtype in ("e4m3", "mxfp8"):
        return torch.float32
    return storage_dtype(wl)


def skew_bias(wl: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Per-expert logit bias of the skewed workload (fp32 [E]).

    Experts are ranked by a seeded permutation pi; the expert at Zipf rank r
    (1-based) gets bias 3 * r**-1.2 for the E-10 hottest ranks, and the 10
    coldest ranks get -64, so that N(0,1) logits can never put them in any
    token's top k: exactly 10 experts receive no tokens.
    """
    assert wl.E > 10 + wl.k
    g = _gen(seed, wl, "bias_perm", "cpu")
    perm = torch.randperm(wl.E, generator=g)
    bias = torch.empty(wl.E, dtype=torch.float32)
    for r in range(1, wl.E + 1):
        e = int(perm[r - 1])
        bias[e] = 3.0 * r ** -1.2 if r <= wl.E - 10 else -64.0
    return bias.to(device)


def _randn(shape, g, device, std=1.0, dtype=torch.float32, chunk_dim0=False):
    """fp32 N(0, std^2) draw, cast to `dtype`.  With chunk_dim0, draws one
    leading-index slice at a time to bound the fp32 temporary."""
    if not chunk_dim0:
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dtype)
    out = torch.empty(shape, device=device, dtype=dtype)
    for i in range(shape[0]):
        t = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[i].copy_(t)
    return out


def make_inputs(wl: Workload, seed: int = 0, device="cpu", with_grad: bool = True) -> dict:
    """All layer inputs of workload `wl` as torch tensors on `device`.

    logits fp32 [T][E] ~ N(0,1) (+ skew_bias for the skewed workload), given
    directly as the router output; x [T][d] ~ N(0,1); W1, W3 [E][d][f] ~
    N(0, 1/d); W2 [E][f][d] ~ N(0, 1/f); the shared expert (if any) Ws1, Ws3
    [d][f_shared] ~ N(0, 1/d), Ws2 [f_shared][d] ~ N(0, 1/f_shared); upstream
    gradient dY [T][d] ~ N(0,1).  Variance is 1/fan_in (std = fan_in**-0.5).
    """
    dev = torch.device(device)
    sd = storage_dtype(wl)
    wd = weight_dtype(wl)
    big = dev.type != "cpu" or wl.E * wl.d * wl.f > (1 << 26)
    out = {}
    logits = _randn((wl.T, wl.E), _gen(seed, wl, "logits", dev), dev)
    if wl.skew:
        logits += skew_bias(wl, seed, dev)[None, :]
    out["logits"] = logits.contiguous()
    out["x"] = _randn((wl.T, wl.d), _gen(seed, wl, "x", dev), dev, dtype=sd)
    out["W1"] = _randn((wl.E, wl.d, wl.f), _gen(seed, wl, "W1", dev), dev, wl.d ** -0.5, wd, big)
    out["W3"] = _randn((wl.E, wl.d, wl.f), _gen(seed, wl, "W3", dev), dev, wl.d ** -0.5, wd, big)
    out["W2"] = _randn((wl.E, wl.f, wl.d), _gen(seed, wl, "W2", dev), dev, wl.f ** -0.5, wd, big)
    if wl.f_shared:
        fs = wl.f_shared
        out["Ws1"] = _randn((wl.d, fs), _gen(seed, wl, "Ws1", dev), dev, wl.d ** -0.5, wd)
        out["Ws3"] = _randn((wl.d, fs), _gen(seed, wl, "Ws3", dev), dev, wl.d ** -0.5, wd)
        out["Ws2"] = _randn((fs, wl.d), _gen(seed, wl, "Ws2", dev), dev, fs ** -0.5, wd)
    if with_grad:
        out["dY"] = _randn((wl.T, wl.d), _gen(seed, wl, "dY", dev), dev, dtype=sd)
    return out


def tied_logits(T: int, E: int, levels: int = 3, seed: int = 0) -> torch.Tensor:
    """fp32 logits drawn from a few integer levels, so that many ties occur
    (used to exercise lowest-index tie-breaking)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, levels, (T, E), generator=g).to(torch.float32)


def to_f64(t: torch.Tensor):
    """Exact up-cast of a stored tensor (fp32 or bf16) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bytes_per_elem(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "e4m3": 1, "mxfp8": 1}[dtype]


__all__ = ["Workload", "WORKLOADS", "VARIANTS", "make_inputs", "skew_bias", "tied_logits", "to_f64",
           "storage_dtype", "weight_dtype", "bytes_per_elem"]
