"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, and rejects bad arguments before touching the device."""
import ctypes as C
import glob
import os
import re
import subprocess

import pytest

from token_routed_expert_amd import _native as N
from token_routed_expert_amd import make_shape, moe_status_str, moe_workspace_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, re.M))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"moe_route", "moe_permute", "moe_unpermute", "moe_grouped_gemm_fwd",
            "moe_grouped_gemm_bwd", "moe_layer_fwd", "moe_layer_bwd"} <= names
    lib = N.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(N.exported_names()) == names


def test_library_carries_gfx950_code_objects():
    assert b"amdgcn-amd-amdhsa--gfx950" in open(N.LIB_PATH, "rb").read()


def test_status_strings():
    assert moe_status_str(0) == "MOE_OK"
    assert moe_status_str(2) == "MOE_ERR_UNSUPPORTED"
    assert moe_status_str(99) == "MOE_ERR_UNKNOWN"


def test_workspace_sizes():
    sh = make_shape(8192, 4096, 128, 8, 1536)
    assert moe_workspace_bytes(sh, N.MOE_WS_PERMUTE) == 128 * 32 * 4
    assert moe_workspace_bytes(sh, N.MOE_WS_LAYER_FWD) == 128 * 32 * 4 + 256
    assert moe_workspace_bytes(sh, N.MOE_WS_GEMM_FWD) == 0
    bad = make_shape(8192, 4096, 128, 200, 1536)           # k > E
    assert moe_workspace_bytes(bad, N.MOE_WS_PERMUTE) == 0


P = C.c_void_p(16)  # a non-null dummy: the calls below must fail before any use


@pytest.mark.parametrize("T,E,k,expect", [(0, 8, 2, 1), (4, 8, 0, 1), (4, 8, 9, 1), (4, 300, 2, 2)])
def test_route_rejects(T, E, k, expect):
    assert N.lib().moe_route(P, T, E, k, P, P, None) == expect


def test_route_rejects_null():
    assert N.lib().moe_route(None, 4, 8, 2, P, P, None) == N.MOE_ERR_INVALID


@pytest.mark.parametrize("shape,expect", [
    (dict(T=4, d=128, E=8, k=2, f=128, dtype="bf16"), None),
    (dict(T=4, d=100, E=8, k=2, f=128, dtype="bf16"), N.MOE_ERR_UNSUPPORTED),   # 16-byte rows
    (dict(T=4, d=128, E=8, k=9, f=128, dtype="bf16"), N.MOE_ERR_INVALID),
    (dict(T=4, d=128, E=512, k=2, f=128, dtype="bf16"), N.MOE_ERR_UNSUPPORTED),
])
def test_permute_validation(shape, expect):
    sh = make_shape(**shape)
    lib = N.lib()
    st = lib.moe_permute(C.byref(sh), P, P, None, 1, P, P, P, P, P, P, 0, None)
    assert st == (N.MOE_ERR_WORKSPACE if expect is None else expect)
    assert lib.moe_permute(C.byref(sh), None, P, None, 0, None, None, P, None, P, None, 0, None) in (
        N.MOE_ERR_INVALID, expect)


def test_gemm_validation():
    lib = N.lib()
    sh = make_shape(64, 256, 8, 2, 200, 0, "bf16")                 # f not a multiple of 128
    assert lib.moe_grouped_gemm_fwd(C.byref(sh), P, P, P, P, P, P, P, P, None, 0, None) == \
        N.MOE_ERR_UNSUPPORTED
    sh = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    assert lib.moe_grouped_gemm_fwd(C.byref(sh), None, P, P, P, P, P, P, P, None, 0, None) == \
        N.MOE_ERR_INVALID
    assert lib.moe_grouped_gemm_bwd(C.byref(sh), P, P, P, P, P, P, P, P, P, P, P, P, None, None, 0,
                                    None) == N.MOE_ERR_INVALID
    bad = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    bad.reserved = 1
    assert lib.moe_grouped_gemm_fwd(C.byref(bad), P, P, P, P, P, P, P, P, None, 0, None) == \
        N.MOE_ERR_INVALID
    bad = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    bad.dtype = 7
    assert lib.moe_unpermute(C.byref(bad), P, P, None, None, P, None) == N.MOE_ERR_UNSUPPORTED


def test_gemm_32bit_ranges():
    """bf16 expert GEMMs refuse shapes whose per-expert byte ranges reach 2^32
    (P * max(d, 2f) * 2 or d * f * 2) before looking at any pointer."""
    lib = N.lib()
    big_rows = make_shape(1 << 19, 512, 8, 8, 128, 0, "bf16")      # P * d * 2 = 2^32
    ok_rows = make_shape(1 << 19, 256, 8, 8, 128, 0, "bf16")       # P * 2f * 2 = 2^31
    big_ab = make_shape(1 << 19, 128, 8, 8, 256, 0, "bf16")        # P * 2f * 2 = 2^32
    big_w = make_shape(4, 65536, 8, 2, 32768, 0, "bf16")           # d * f * 2 = 2^32
    for sh, expect in ((big_rows, N.MOE_ERR_UNSUPPORTED), (big_ab, N.MOE_ERR_UNSUPPORTED),
                       (big_w, N.MOE_ERR_UNSUPPORTED), (ok_rows, N.MOE_ERR_INVALID)):
        assert lib.moe_grouped_gemm_fwd(C.byref(sh), None, P, P, P, P, P, P, P, None, 0,
                                        None) == expect
        assert lib.moe_grouped_gemm_bwd(C.byref(sh), None, P, P, P, P, P, P, P, P, P, P, P, P, None,
                                        0, None) == expect
        assert lib.moe_grouped_gemm_fwd_rowscaled(C.byref(sh), None, P, P, P, P, P, P, P, P,
                                                  None) == expect
        io = N.moe_layer_io()
        assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 1 << 20, None) == expect
        assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), P, 1 << 20, None) == expect
    # the shared expert runs over all T tokens: T * 2 f_s * 2 = 2^33, while the
    # routed experts' P * max(d, 2f) * 2 = 2^25 is fine
    sh = make_shape(1 << 16, 128, 4, 1, 128, 1 << 15, "bf16")
    io = N.moe_layer_io()
    assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 1 << 20, None) == N.MOE_ERR_UNSUPPORTED
    # fp32 layers address with 64-bit offsets: no such limit
    sh = make_shape(1 << 19, 512, 8, 8, 128, 0, "f32")
    assert lib.moe_grouped_gemm_fwd(C.byref(sh), None, P, P, P, P, P, P, P, None, 0,
                                    None) == N.MOE_ERR_INVALID


def test_permute_noalloc_validation():
    """The allocation-free map refuses maps larger than its 1 MiB array before
    any HIP call, and validates its arguments as moe_permute does."""
    lib = N.lib()
    sh = make_shape(1025 * 256, 64, 256, 2, 128, 0, "bf16")        # 256 * 1025 * 4 B > 1 MiB
    assert lib.moe_permute_noalloc(C.byref(sh), P, P, None, 1, P, P, P, P, P, None) == \
        N.MOE_ERR_WORKSPACE
    sh = make_shape(64, 256, 8, 2, 128, 0, "bf16")
    assert lib.moe_permute_noalloc(C.byref(sh), None, P, None, 1, P, P, P, P, P, None) == \
        N.MOE_ERR_INVALID
    assert lib.moe_permute_noalloc(C.byref(sh), P, None, None, 1, P, P, P, P, P, None) == \
        N.MOE_ERR_INVALID
    sh = make_shape(4, 100, 8, 2, 128, 0, "bf16")                  # 16-byte rows
    assert lib.moe_permute_noalloc(C.byref(sh), P, P, None, 1, P, P, P, P, P, None) == \
        N.MOE_ERR_UNSUPPORTED


def test_layer_validation():
    lib = N.lib()
    sh = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    io = N.moe_layer_io()
    assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 1 << 20, None) == N.MOE_ERR_INVALID
    assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), P, 1 << 20, None) == N.MOE_ERR_INVALID
    for name in N.IO_FIELDS:
        setattr(io, name, 16)
    assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 8, None) == N.MOE_ERR_WORKSPACE
    assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), None, 0, None) == N.MOE_ERR_WORKSPACE


def test_product_path_does_not_use_the_oracle():
    """The package and the oracle share no code and neither imports the other."""
    pkg = os.path.join(ROOT, "token_routed_expert_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".h", ".cpp")):
            assert "oracle" not in open(path).read().replace("oracles", ""), path
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        assert "token_routed_expert_amd" not in open(path).read(), path


def test_router_grad_validation():
    lib = N.lib()
    f = C.c_float
    assert lib.moe_aux_loss(P, 4, 8, 2, P, f(0.01), P, P, 0, None) == N.MOE_ERR_WORKSPACE
    assert lib.moe_aux_loss(P, 0, 8, 2, P, f(0.01), P, P, 1 << 20, None) == N.MOE_ERR_INVALID
    assert lib.moe_aux_loss(P, 4, 8, 9, P, f(0.01), P, P, 1 << 20, None) == N.MOE_ERR_INVALID
    assert lib.moe_aux_loss(None, 4, 8, 2, P, f(0.01), P, P, 1 << 20, None) == N.MOE_ERR_INVALID
    assert lib.moe_aux_loss(P, 4, 300, 2, P, f(0.01), P, P, 1 << 20, None) == \
        N.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_bwd(P, 4, 8, 2, P, P, None, P, f(0.0), f(1.0), P, None) == \
        N.MOE_ERR_INVALID
    assert lib.moe_route_bwd(P, 4, 257, 2, P, P, P, P, f(0.0), f(1.0), P, None) == \
        N.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_bwd(P, 4, 8, 9, P, P, P, P, f(0.0), f(1.0), P, None) == N.MOE_ERR_INVALID
    sh = make_shape(4, 16392, 8, 2, 128, 0, "bf16")          # 32784-byte rows
    assert lib.moe_combine_bwd(C.byref(sh), P, P, P, P, P, P, None) == N.MOE_ERR_UNSUPPORTED
    sh = make_shape(4, 256, 8, 2, 128, 0, "bf16")
    assert lib.moe_combine_bwd(C.byref(sh), P, P, P, P, P, None, None) == N.MOE_ERR_INVALID
    assert moe_workspace_bytes(make_shape(8200, 4096, 128, 8, 1536), N.MOE_WS_AUX_LOSS) == \
        -(-257 * 128 * 4 // 256) * 256


def test_layer_router_grad_validation():
    """The aux loss needs its workspace after the forward's, and dlogits needs
    dprob: both are rejected before any launch."""
    lib = N.lib()
    for dtype in ("bf16", "e4m3"):
        sh = make_shape(64, 256, 8, 2, 256, 0, dtype)
        io = N.moe_layer_io()
        for name in N.IO_FIELDS:
            setattr(io, name, 16)
        if dtype == "e4m3":
            w = N.moe_e4m3_weights(*([16] * 9))         # dummy non-null pointers, never read
            io.wq = C.cast(C.pointer(w), C.c_void_p).value
        base = moe_workspace_bytes(sh, N.MOE_WS_LAYER_FWD)
        assert base > 0
        assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, base, None) == N.MOE_ERR_WORKSPACE
        io.dprob = None
        assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), P, 1 << 30, None) == N.MOE_ERR_INVALID


def test_rowscaled_validation():
    lib = N.lib()
    for dtype, expect in (("f32", N.MOE_ERR_UNSUPPORTED), ("e4m3", N.MOE_ERR_UNSUPPORTED)):
        sh = make_shape(64, 256, 8, 2, 256, 0, dtype)
        assert lib.moe_grouped_gemm_fwd_rowscaled(C.byref(sh), *([P] * 10)) == expect
        assert lib.moe_grouped_gemm_bwd_rowscaled(C.byref(sh), *([P] * 4), 0, *([P] * 13), 1 << 20,
                                                  None) == expect
    sh = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    args = [P] * 10
    args[6] = None                                           # row_prob
    assert lib.moe_grouped_gemm_fwd_rowscaled(C.byref(sh), *args) == N.MOE_ERR_INVALID
    need = moe_workspace_bytes(sh, N.MOE_WS_GEMM_BWD_ROWSCALED)
    assert need == -(-128 * 1 * 4 // 256) * 256
    assert lib.moe_grouped_gemm_bwd_rowscaled(C.byref(sh), *([P] * 4), 1, *([P] * 13), need - 1,
                                              None) == N.MOE_ERR_WORKSPACE
    assert lib.moe_row_probs(C.byref(sh), None, P, P, None) == N.MOE_ERR_INVALID
    assert moe_workspace_bytes(make_shape(64, 256, 8, 2, 256, 0, "f32"),
                               N.MOE_WS_LAYER_BWD_ROWSCALED) == 0


def test_layer_memory_efficient_validation():
    lib = N.lib()
    io = N.moe_layer_io()
    for name in N.IO_FIELDS:
        setattr(io, name, 16)
    io.memory_efficient = 1
    sh = make_shape(64, 256, 8, 2, 256, 0, "bf16")
    need = moe_workspace_bytes(sh, N.MOE_WS_LAYER_BWD_ROWSCALED)
    assert need == 256 + moe_workspace_bytes(sh, N.MOE_WS_GEMM_BWD_ROWSCALED)
    assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), P, need - 1, None) == N.MOE_ERR_WORKSPACE
    io.row_prob = None
    assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 1 << 30, None) == N.MOE_ERR_INVALID
    assert lib.moe_layer_bwd(C.byref(sh), C.byref(io), P, 1 << 30, None) == N.MOE_ERR_INVALID
    sh = make_shape(64, 256, 8, 2, 256, 0, "f32")
    assert lib.moe_layer_fwd(C.byref(sh), C.byref(io), P, 1 << 30, None) == N.MOE_ERR_UNSUPPORTED


def test_fp8_memory_efficient_workspace():
    for dtype in ("e4m3", "mxfp8"):
        sh = make_shape(64, 256, 8, 2, 256, 0, dtype)
        assert moe_workspace_bytes(sh, N.MOE_WS_LAYER_BWD_ROWSCALED) == \
            moe_workspace_bytes(sh, N.MOE_WS_LAYER_BWD) + -(-128 * 1 * 4 // 256) * 256


def test_probe_mfma_validation():
    """The matrix-core probe checks its arguments before it touches the device."""
    f, khz = C.c_int64(0), C.c_int64(0)
    lib = N.lib()
    assert lib.moe_probe_mfma(N.MOE_BF16, 16, None, P, C.byref(f), C.byref(khz), None) == N.MOE_ERR_INVALID
    assert lib.moe_probe_mfma(N.MOE_BF16, 16, P, P, None, C.byref(khz), None) == N.MOE_ERR_INVALID
    assert lib.moe_probe_mfma(N.MOE_BF16, 0, P, P, C.byref(f), C.byref(khz), None) == N.MOE_ERR_INVALID
    assert lib.moe_probe_mfma(N.MOE_BF16, 1 << 25, P, P, C.byref(f), C.byref(khz), None) == N.MOE_ERR_INVALID
    assert lib.moe_probe_mfma(N.MOE_F32, 16, P, P, C.byref(f), C.byref(khz), None) == N.MOE_ERR_UNSUPPORTED
    assert lib.moe_probe_mfma(N.MOE_MXFP8, 16, P, P, C.byref(f), C.byref(khz), None) == N.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["moe_quantize_token_blocks", "moe_quantize_token_blocks_mx",
                                  "moe_quantize_token_blocks_with_rows",
                                  "moe_quantize_token_blocks_with_rows_mx"])
def test_token_block_quantiser_validation(name):
    """The token-block quantisers (with or without the row blocks) check their
    arguments before they touch the device."""
    fn = getattr(N.lib(), name)
    rows = name.endswith("with_rows") or name.endswith("with_rows_mx")
    extra = (P, P) if rows else ()
    assert fn(None, 8, 1024, P, None, 256, P, P, P, *extra, None) == N.MOE_ERR_INVALID
    assert fn(P, 8, 1024, P, None, 256, P, None, P, *extra, None) == N.MOE_ERR_INVALID
    assert fn(P, 0, 1024, P, None, 256, P, P, P, *extra, None) == N.MOE_ERR_INVALID
    assert fn(P, 8, 1024, P, None, 200, P, P, P, *extra, None) == N.MOE_ERR_UNSUPPORTED
    assert fn(P, 300, 1024, P, None, 256, P, P, P, *extra, None) == N.MOE_ERR_UNSUPPORTED
    if rows:
        assert fn(P, 8, 1024, P, None, 256, P, P, P, None, P, None) == N.MOE_ERR_INVALID
        assert fn(P, 8, 1024, P, None, 256, P, P, P, P, None, None) == N.MOE_ERR_INVALID
