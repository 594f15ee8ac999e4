"""The C ABI without a GPU: the library loads, exports every entry point
include/moe.h declares, and rejects bad arguments on the host before any
launch (status codes and messages)."""
import ctypes
import os
import re

import pytest

import routing_permute_grouped_router_amd as moe
from routing_permute_grouped_router_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(b.EXPORTED) == _declared()


def test_library_exports_every_declared_symbol():
    lib = moe.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(T=64, H=128, F=64, E=8, k=2, align=1, score=0, renorm=0, dtype=1, weight_site=0, swiglu_limit=0.0)
    base.update(kw)
    return b.moe_config(*[base[n] for n, _ in b.moe_config._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), b.MOE_ERR_INVALID_ARG),
    (dict(k=0), b.MOE_ERR_INVALID_ARG),
    (dict(E=0), b.MOE_ERR_INVALID_ARG),
    (dict(E=2000), b.MOE_ERR_INVALID_ARG),
    (dict(T=-1), b.MOE_ERR_INVALID_ARG),
    (dict(align=0), b.MOE_ERR_INVALID_ARG),
    (dict(score=5), b.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), b.MOE_ERR_INVALID_ARG),
    (dict(weight_site=3), b.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=-1.0), b.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=float("nan")), b.MOE_ERR_INVALID_ARG),
    (dict(swiglu_limit=float("inf")), b.MOE_ERR_INVALID_ARG),
])
def test_bad_config_rejected_on_host(kw, status):
    lib = moe.load_library()
    c = _cfg(**kw)
    st = lib.moe_route(ctypes.byref(c), 256, None, 256, 256, None)
    assert st == status
    assert lib.moe_last_error()


def test_misaligned_pointers_rejected():
    lib = moe.load_library()
    c = _cfg()
    assert lib.moe_route(ctypes.byref(c), 264, None, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert b"logits" in lib.moe_last_error() and b"aligned" in lib.moe_last_error()
    assert lib.moe_route(ctypes.byref(c), 256, 260, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert b"bias" in lib.moe_last_error()
    assert _forward(lib, c, y=512 + 4) == b.MOE_ERR_INVALID_ARG
    assert b"y" in lib.moe_last_error()


def test_null_pointers_rejected():
    lib = moe.load_library()
    c = _cfg()
    assert lib.moe_route(ctypes.byref(c), None, None, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert b"logits" in lib.moe_last_error()
    assert lib.moe_combine(ctypes.byref(c), 256, None, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, 256, None, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    # routing backward: every input and dlogits required, dw optional
    assert lib.moe_route_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, None, None, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bwd(ctypes.byref(c), 256, None, 256, 256, 256, None, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_route_bwd(None, 256, 256, 256, 256, 256, None, 256, None) == b.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op that touches nothing
    assert lib.moe_route_bwd(ctypes.byref(_cfg(T=0)), None, None, None, None, None, None, None, None) == b.MOE_OK


def test_unsupported_shapes():
    lib = moe.load_library()
    c = _cfg(H=96)
    assert lib.moe_grouped_swiglu_gemm(ctypes.byref(c), 256, None, 256, None, 256, 256, None, None, None, 0, None) == \
        b.MOE_ERR_UNSUPPORTED
    c = _cfg(F=40)
    assert lib.moe_grouped_down_gemm(ctypes.byref(c), 256, None, 256, None, 256, 256, None, 0, None) == b.MOE_ERR_UNSUPPORTED
    c = _cfg(F=192, dtype=b.MOE_MXFP8)  # MXFP8 tiles F by 128
    assert lib.moe_grouped_down_gemm(ctypes.byref(c), 256, 256, 256, 256, 256, 256, None, 0, None) == b.MOE_ERR_UNSUPPORTED
    assert b"128" in lib.moe_last_error()
    c = _cfg(H=32768, F=16384)  # one expert's weights must stay below 2^32 bytes
    assert lib.moe_grouped_down_gemm(ctypes.byref(c), 256, None, 256, None, 256, 256, None, 0, None) == b.MOE_ERR_UNSUPPORTED


def test_workspace_checks():
    lib = moe.load_library()
    c = _cfg(T=5000, E=128, k=8)
    need = lib.moe_workspace_size(ctypes.byref(c))
    assert need > 0
    st = lib.moe_permute(ctypes.byref(c), 256, None, 256, 256, None, 256, 256, 256, 256, None, 256, need - 1, None)
    assert st == b.MOE_ERR_WORKSPACE
    assert lib.moe_rows_capacity(ctypes.byref(c)) == 5000 * 8
    c2 = _cfg(T=5000, E=128, k=8, align=128)
    assert lib.moe_rows_capacity(ctypes.byref(c2)) == 5000 * 8 + 128 * 127
    # the grouped GEMMs take the same workspace
    st = lib.moe_grouped_swiglu_gemm(ctypes.byref(c), 256, None, 256, None, 256, 256, None, None, 256, need - 1, None)
    assert st == b.MOE_ERR_WORKSPACE
    st = lib.moe_grouped_down_gemm(ctypes.byref(c), 256, None, 256, None, 256, 256, None, 0, None)
    assert st == b.MOE_ERR_WORKSPACE


def test_backward_workspace_bounds():
    lib = moe.load_library()
    # the skewed workload: the weight-gradient partial sums stay within about 1 GiB
    c = _cfg(T=16384, H=2048, F=768, E=128, k=8)
    need = lib.moe_backward_workspace_size(ctypes.byref(c))
    assert 0 < need <= (1 << 30) + (1 << 20)
    # the bf16 forward: grouping scratch plus the GEMMs' queue counters and split-tile partial sums
    assert (64 << 20) < lib.moe_workspace_size(ctypes.byref(c)) < (65 << 20)
    assert lib.moe_workspace_size(ctypes.byref(_cfg(T=16384, H=2048, F=768, E=128, k=8, dtype=b.MOE_F32))) < (1 << 20)
    # too few rows to split an expert: only the per-expert table
    c = _cfg(T=64, H=128, F=64, E=8, k=2)
    assert lib.moe_backward_workspace_size(ctypes.byref(c)) < 4096
    # the backward is built for bf16 storage only
    assert lib.moe_backward_workspace_size(ctypes.byref(_cfg(dtype=b.MOE_F32))) == 0
    st = lib.moe_grouped_down_bwd(ctypes.byref(_cfg(T=16384, H=2048, F=768, E=128, k=8)), 256, 256, 256, 256, 256,
                                  256, 256, 256, need - 1, None)
    assert st == b.MOE_ERR_WORKSPACE


def test_quantize_rejects_ragged_cols():
    lib = moe.load_library()
    assert lib.moe_quantize_mxfp8(256, 4, 33, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp4(256, 4, 48, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp4(256, -1, 32, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp4(None, 4, 64, 256, 256, None) == b.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp4(None, 0, 64, None, None, None) == b.MOE_OK  # nothing to do


def test_mxfp4_shapes_and_backward_checked_on_host():
    """MXFP4 needs H and F to be multiples of 512 (a 128-byte GEMM stage holds
    256 values and a 16-byte load brings a row's scales of two stages), and
    the backward is built for bf16 storage only."""
    lib = moe.load_library()
    for H, F in ((256, 512), (512, 256), (640, 512)):
        c = _cfg(dtype=b.MOE_MXFP4, H=H, F=F)
        mx = dict(x_scale=256, w1_scale=256, w2_scale=256, xp_scale=256, h_scale=256)
        assert _forward(lib, c, **mx) == b.MOE_ERR_UNSUPPORTED, (H, F)
        assert b"512" in lib.moe_last_error()
    c = _cfg(dtype=b.MOE_MXFP4, H=512, F=512)
    assert _backward(lib, c, ws_bytes=1 << 20) == b.MOE_ERR_UNSUPPORTED
    # the MX scales are required
    mx = dict(x_scale=256, w1_scale=256, w2_scale=256, xp_scale=256, h_scale=256)
    for name in ("h_scale", "xp_scale", "x_scale", "w1_scale"):
        assert _forward(lib, c, **{**mx, name: None}) == b.MOE_ERR_INVALID_ARG, name


def test_python_layer_type_errors():
    import torch
    cfg = moe.MoEConfig(4, 128, 64, 8, 2)
    with pytest.raises(ValueError):  # CPU tensors are refused before any call
        moe.moe_route(cfg, torch.zeros(4, 8), torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))


def test_device_e4m3_rounding_matches_oracle(tmp_path):
    """The E4M3 rounding the MXFP8 kernels use (compiled for the host) against
    the oracle's encoder on every float in [2^-10, 2^10) of both signs: the
    range the quantiser and the SwiGLU epilogue feed it after the block scale
    (below 2^-10 everything rounds to 0 and is sampled)."""
    import subprocess
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    lib = root / "oracle" / "liboracle.so"
    if not lib.exists():
        pytest.skip("oracle library not built")
    exe = tmp_path / "e4m3_check"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950", "-x", "hip",
                    "-I", str(root / "include"), "-I", str(root / "routing_permute_grouped_router_amd" / "csrc"),
                    str(root / "tests" / "e4m3_check.cpp"), "-x", "none", str(lib), "-Wl,-rpath," + str(lib.parent),
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]


def test_device_e2m1_rounding_matches_the_oracle(tmp_path):
    """The E2M1 rounding of the MXFP4 quantiser and epilogue, compiled for the
    host, against the oracle's encoder on every float in [2^-4, 2^5) of both
    signs (below, everything rounds to 0; above, everything saturates: both
    sampled)."""
    import subprocess
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    lib = root / "oracle" / "liboracle.so"
    if not lib.exists():
        pytest.skip("oracle library not built")
    exe = tmp_path / "e2m1_check"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950", "-x", "hip",
                    "-I", str(root / "include"), "-I", str(root / "routing_permute_grouped_router_amd" / "csrc"),
                    str(root / "tests" / "e2m1_check.cpp"), "-x", "none", str(lib), "-Wl,-rpath," + str(lib.parent),
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]


def test_weighted_gemms_and_placement_checked_on_host():
    lib = moe.load_library()
    c = _cfg(weight_site=b.MOE_WEIGHT_AT_FC2)
    need = lib.moe_workspace_size(ctypes.byref(c))
    # the per-row weights need src_map and w
    st = lib.moe_grouped_down_gemm_weighted(ctypes.byref(c), 256, None, 256, None, 256, None, 256, 256, 256, need, None)
    assert st == b.MOE_ERR_INVALID_ARG and b"src_map" in lib.moe_last_error()
    st = lib.moe_grouped_swiglu_gemm_weighted(ctypes.byref(c), 256, None, 256, None, 256, 256, None, 256, None, 256, need, None)
    assert st == b.MOE_ERR_INVALID_ARG and b"w" in lib.moe_last_error()
    # the workspace holds the per-row weights as well
    c0 = _cfg()
    assert need == lib.moe_workspace_size(ctypes.byref(c0))
    assert need >= 4 * (64 * 2 + 256)
    # the backward is built for the weights applied in the combine
    assert lib.moe_combine_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, 256, None) == b.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, 256, 256, None) == b.MOE_ERR_UNSUPPORTED
    # an unweighted combine takes w = NULL (T = 0: nothing to launch)
    assert lib.moe_combine(ctypes.byref(_cfg(T=0)), None, None, None, None, None) == b.MOE_OK


def test_new_entry_points_host_edge_cases():
    lib = moe.load_library()
    c0 = _cfg(T=0)  # no rows: every GEMM entry point is a no-op, nothing is dereferenced
    n0 = lib.moe_workspace_size(ctypes.byref(c0))
    assert lib.moe_grouped_swiglu_gemm_weighted(ctypes.byref(c0), None, None, None, None, None, None, None, None,
                                                None, None, 0, None) == b.MOE_OK
    assert lib.moe_grouped_down_gemm_weighted(ctypes.byref(c0), None, None, None, None, None, None, None, None,
                                              None, 0, None) == b.MOE_OK
    assert lib.moe_grouped_swiglu_gemm_gather(ctypes.byref(c0), None, None, None, None, None, None, None, None,
                                              None, None, n0, None) == b.MOE_OK
    c = _cfg(weight_site=b.MOE_WEIGHT_AT_FC1)
    need = lib.moe_workspace_size(ctypes.byref(c))
    # a missing output is rejected before anything is launched
    st = lib.moe_grouped_swiglu_gemm_weighted(ctypes.byref(c), 256, None, 256, None, 256, 256, 256, None, None, 256, need, None)
    assert st == b.MOE_ERR_INVALID_ARG and b"h" in lib.moe_last_error()
    st = lib.moe_grouped_down_gemm_weighted(ctypes.byref(c), 256, None, 256, None, 256, 256, 256, None, 256, need, None)
    assert st == b.MOE_ERR_INVALID_ARG and b"yp" in lib.moe_last_error()
    # too small a workspace (the per-row weights live there)
    st = lib.moe_grouped_down_gemm_weighted(ctypes.byref(c), 256, None, 256, None, 256, 256, 256, 256, 256, need - 256, None)
    assert st == b.MOE_ERR_WORKSPACE
    # the gather form needs the routing maps
    st = lib.moe_grouped_swiglu_gemm_gather(ctypes.byref(c), 256, None, None, 256, 256, None, 256, 256, None, 256, need, None)
    assert st == b.MOE_ERR_INVALID_ARG and b"src_map" in lib.moe_last_error()
    # a clamp limit is accepted by every call that takes the config
    cl = _cfg(swiglu_limit=7.0)
    assert lib.moe_workspace_size(ctypes.byref(cl)) == lib.moe_workspace_size(ctypes.byref(_cfg()))


# moe_forward's pointer arguments after cfg, in order (ws_bytes and stream follow)
_FWD = ("logits", "bias", "x", "x_scale", "w1", "w1_scale", "w2", "w2_scale", "y", "idx", "w", "counts", "offsets",
        "row_map", "src_map", "xp", "xp_scale", "h", "h_scale", "yp", "gu_stash", "err", "ws")
_BWD = ("dy", "w", "w1", "w2", "offsets", "row_map", "src_map", "xp", "h", "gu_stash", "dyp", "dgu", "dxp", "dx",
        "dw1", "dw2", "ws")


def _forward(lib, c, ws_bytes=None, **override):
    args = {n: 256 for n in _FWD}
    args.update({"bias": None, "x_scale": None, "w1_scale": None, "w2_scale": None, "xp_scale": None, "h_scale": None,
                 "gu_stash": None, "err": None})
    args.update(override)
    nb = lib.moe_workspace_size(ctypes.byref(c)) if ws_bytes is None else ws_bytes
    return lib.moe_forward(ctypes.byref(c), *[args[n] for n in _FWD], nb, None)


def _backward(lib, c, ws_bytes=None, **override):
    args = {n: 256 for n in _BWD}
    args.update(override)
    nb = lib.moe_backward_workspace_size(ctypes.byref(c)) if ws_bytes is None else ws_bytes
    return lib.moe_backward(ctypes.byref(c), *[args[n] for n in _BWD], nb, None)


def test_fused_calls_check_everything_before_launching():
    """Without a GPU any launch fails with MOE_ERR_HIP, so a call that returns
    the specific status of a later step's argument checked every step before
    its first launch."""
    lib = moe.load_library()
    c = _cfg()
    need = lib.moe_workspace_size(ctypes.byref(c))
    assert _forward(lib, c, ws_bytes=need - 1) == b.MOE_ERR_WORKSPACE
    for name in ("h", "yp", "y", "x", "row_map", "w1", "w2"):
        assert _forward(lib, c, **{name: None}) == b.MOE_ERR_INVALID_ARG, name
        assert name.encode() in lib.moe_last_error(), name
    # MXFP8: the scales of every operand and of h
    cm = _cfg(dtype=b.MOE_MXFP8, F=128)
    mx = dict(x_scale=256, w1_scale=256, w2_scale=256, xp_scale=256, h_scale=256)
    for name in ("h_scale", "xp_scale", "x_scale"):
        assert _forward(lib, cm, **{**mx, name: None}) == b.MOE_ERR_INVALID_ARG, name
    # the gather form (xp NULL) refuses a stash and needs src_map
    assert _forward(lib, c, xp=None, gu_stash=256) == b.MOE_ERR_INVALID_ARG
    assert _forward(lib, c, xp=None, src_map=None) == b.MOE_ERR_INVALID_ARG
    # an epilogue weight site checks the per-row weights' inputs first
    assert _forward(lib, _cfg(weight_site=b.MOE_WEIGHT_AT_FC2), w=None) == b.MOE_ERR_INVALID_ARG
    # backward: a short workspace and a missing last output are found before the first step runs
    cb = _cfg()
    assert _backward(lib, cb, ws_bytes=lib.moe_backward_workspace_size(ctypes.byref(cb)) - 1) == b.MOE_ERR_WORKSPACE
    for name in ("dx", "dxp", "dw1", "gu_stash", "xp"):
        assert _backward(lib, cb, **{name: None}) == b.MOE_ERR_INVALID_ARG, name


def test_backward_takes_bf16_storage_only():
    lib = moe.load_library()
    for dt in (b.MOE_F32, b.MOE_MXFP8):
        c = _cfg(dtype=dt, F=128)
        assert _backward(lib, c, ws_bytes=1 << 20) == b.MOE_ERR_UNSUPPORTED
        assert lib.moe_combine_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, 256, None) == b.MOE_ERR_UNSUPPORTED
        assert lib.moe_permute_bwd(ctypes.byref(c), 256, 256, 256, None) == b.MOE_ERR_UNSUPPORTED
        assert lib.moe_grouped_down_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, 256, 256, 256, 1 << 20, None) == \
            b.MOE_ERR_UNSUPPORTED
        assert lib.moe_grouped_swiglu_bwd(ctypes.byref(c), 256, 256, 256, 256, 256, 256, 256, 1 << 20, None) == \
            b.MOE_ERR_UNSUPPORTED


def test_noalloc_forward_limit_checked_on_host():
    """moe_forward_noalloc refuses a config whose scratch exceeds its static
    array before touching the device, and reports a bad config like moe_forward."""
    lib = moe.load_library()
    big = _cfg(T=400000, H=2048, F=768, E=128, k=8)
    assert lib.moe_workspace_size(ctypes.byref(big)) > 68 << 20
    args = [256] * 22
    assert lib.moe_forward_noalloc(ctypes.byref(big), *args, None) == b.MOE_ERR_WORKSPACE
    assert b"68" in lib.moe_last_error() or b"static" in lib.moe_last_error()
    assert lib.moe_forward_noalloc(ctypes.byref(_cfg(k=0)), *args, None) == b.MOE_ERR_INVALID_ARG
