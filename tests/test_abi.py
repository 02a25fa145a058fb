"""C-ABI library checks that need no GPU: it loads, exports every declared
symbol, and rejects bad arguments on the host before any HIP call."""
import ctypes
import subprocess

import pytest

from blocked_local_self_amd import _native
from blocked_local_self_amd import select_kernel, HaloError


@pytest.fixture(scope="module")
def lib():
    return _native.load()


def test_exports_every_declared_symbol(lib):
    names = _native.declared_functions()
    assert {"halo_attn_fwd", "halo_attn_fwd_kernel", "halo_attn_last_error",
            "halo_attn_select_kernel", "halo_attn_abi_version"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in names:
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version(lib):
    text = open(_native.HEADER).read()
    assert f"#define HALO_ATTN_ABI_VERSION {lib.halo_attn_abi_version()}" in text


def test_library_built_from_these_sources(lib):
    """The identifier compiled into the library is the hash of csrc/ as it is
    now: the library is not older than its sources."""
    from blocked_local_self_amd import build
    assert lib.halo_attn_build_id().decode() == build.source_id()


def test_stale_library_warns(lib, monkeypatch):
    """A library built from other sources than csrc/ holds draws a warning
    when the binding loads it."""
    from blocked_local_self_amd import build
    monkeypatch.setattr(build, "source_id", lambda: "0" * 16)
    with pytest.warns(RuntimeWarning, match="rebuild"):
        _native._check_build_id(lib)


def call(lib, *, q=1, k=1, v=1, rh=1, rw=1, out=1 << 40, B=1, heads=1, H=8, W=8, d=16, block=4,
         halo=1, stride=1, scale=0.25, dtype=1, kernel=0):
    # Fake, non-overlapping pointers: every call below must fail before the
    # library touches the device.
    ptr = lambda x: ctypes.c_void_p(x << 32 if x not in (0, 1 << 40) else x)
    return lib.halo_attn_fwd_kernel(ptr(q), ptr(k), ptr(v), ptr(rh), ptr(rw),
                                    ctypes.c_void_p(out), B, heads, H, W, d, block, halo, stride,
                                    scale, dtype, kernel, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(rw=0), -1), (dict(out=0), -1),
    (dict(dtype=7), -3),
    (dict(d=0), -2), (dict(d=129), -2), (dict(block=0), -2), (dict(halo=-1), -2),
    (dict(stride=0), -2), (dict(stride=3, block=4), -2), (dict(stride=2, H=9), -2),
    (dict(B=-1), -2), (dict(W=-3), -2), (dict(kernel=9), -2),
    (dict(block=200, halo=30), -2), (dict(scale=float("inf")), -2), (dict(scale=float("nan")), -2),
    (dict(kernel=2, dtype=0), -4), (dict(kernel=2, d=48), -4), (dict(kernel=2, block=6), -4),
    (dict(kernel=2, d=64, block=8, halo=13), -4),          # d = 64 takes windows of up to 32 columns
    (dict(kernel=3, d=64), -4),                            # the strip kernel takes d = 16 and 32 only
    (dict(kernel=2, block=8, halo=17), -4), (dict(kernel=2, block=8, halo=17, d=32), -4),
    (dict(kernel=3, block=8, halo=13, d=32), -4),          # the strip kernel holds 32 columns at d = 32
    (dict(B=1 << 30, heads=1 << 30, H=1 << 15, W=1 << 15), -2),
    # 46341^2 >= 2^31 pixels in one image: the kernels' 32-bit pixel indices
    # would wrap (d = 1 keeps every other size check satisfied)
    (dict(H=46341, W=46341, d=1), -2),
])
def test_invalid_arguments_rejected_on_host(lib, kw, status):
    assert call(lib, **kw) == status
    assert _native.last_error() != ""


def test_alias_rejected(lib):
    # out overlapping q
    assert call(lib, out=1 << 32) == -6


def test_empty_is_a_noop(lib):
    for kw in (dict(B=0), dict(heads=0), dict(H=0), dict(W=0)):
        assert call(lib, q=0, k=0, v=0, rh=0, rw=0, out=0, **kw) == 0
    assert _native.last_error() == ""


def test_kernel_selection():
    assert select_kernel(16, 8, 3, 1, "bf16") == "mfma"
    assert select_kernel(32, 8, 3, 1, "bf16") == "mfma"
    assert select_kernel(16, 8, 3, 2, "bf16") == "mfma"
    assert select_kernel(32, 12, 3, 1, "bf16") == "mfma"
    assert select_kernel(16, 4, 1, 1, "fp32") == "generic"
    assert select_kernel(64, 8, 3, 1, "bf16") == "mfma"        # 64 channels: the streaming kernel
    assert select_kernel(64, 8, 13, 1, "bf16") == "generic"    # ... for windows of up to 32 columns
    assert select_kernel(48, 8, 3, 1, "bf16") == "generic"
    assert select_kernel(16, 2, 1, 1, "bf16") == "generic"
    assert select_kernel(16, 8, 13, 1, "bf16") == "mfma"      # r = 34: three column chunks (d = 16)
    assert select_kernel(32, 8, 13, 1, "bf16") == "mfma"      # r = 34 with d = 32: the streaming kernel
    assert select_kernel(32, 8, 17, 1, "bf16") == "generic"   # r = 42
    assert select_kernel(16, 8, 17, 1, "bf16") == "generic"   # r = 42
    with pytest.raises(HaloError):
        select_kernel(16, 4, 1, 3, "bf16")


def test_kernel_name_query_on_the_host():
    # answers that need no device: the generic kernel (fp32), nothing to compute, invalid arguments
    assert _native.fwd_kernel_name(1, 2, 16, 16, 16, 4, 1, 1, _native.HALO_F32) == "generic"
    assert _native.fwd_kernel_name(1, 2, 16, 16, 16, 4, 1, 1, _native.HALO_BF16,
                                   kernel=_native.HALO_KERNEL_GENERIC) == "generic"
    assert _native.fwd_kernel_name(0, 2, 16, 16, 16, 4, 1, 1, _native.HALO_BF16) == "none"
    assert _native.fwd_kernel_name(1, 2, 24, 24, 64, 8, 3, 1, _native.HALO_BF16) == "wide"     # d = 64
    with pytest.raises(ValueError, match="query_stride"):
        _native.fwd_kernel_name(1, 2, 16, 16, 16, 4, 1, 3, _native.HALO_BF16)
    with pytest.raises(ValueError, match="matrix-core"):
        _native.fwd_kernel_name(1, 2, 16, 16, 16, 4, 1, 1, _native.HALO_F32, kernel=_native.HALO_KERNEL_MFMA)
    with pytest.raises(ValueError, match="halo_kernel"):
        _native.fwd_kernel_name(1, 2, 16, 16, 16, 4, 1, 1, _native.HALO_BF16, kernel=9)


def test_backward_kernel_name_query():
    bf, f32 = _native.HALO_BF16, _native.HALO_F32
    name = _native.bwd_kernel_name
    assert name(32, 8, 64, 64, 16, 8, 3, 1, bf) == "strip"          # 14x14 windows, whole blocks
    assert name(8, 8, 128, 128, 32, 12, 3, 1, bf) == "tile"         # 18x18 windows, partial blocks
    assert name(1, 2, 20, 28, 16, 8, 3, 1, bf) == "tile"            # partial blocks
    assert name(8, 8, 64, 64, 16, 32, 3, 1, bf) == "generic"        # 38x38 windows
    assert name(1, 2, 16, 16, 16, 4, 1, 1, f32) == "generic"
    assert name(1, 2, 16, 16, 16, 4, 1, 1, bf, flags=_native.HALO_ZERO_PAD) == "strip"
    assert name(1, 2, 20, 28, 16, 8, 3, 1, bf, flags=_native.HALO_ZERO_PAD) == "generic"
    assert name(1, 2, 20, 28, 16, 8, 3, 1, bf, kernel=_native.HALO_KERNEL_GENERIC) == "generic"
    assert name(0, 2, 20, 28, 16, 8, 3, 1, bf) == "none"
    with pytest.raises(ValueError, match="matrix-core"):
        name(8, 8, 64, 64, 16, 32, 3, 1, bf, kernel=_native.HALO_KERNEL_MFMA)
    with pytest.raises(ValueError, match="query_stride"):
        name(1, 2, 16, 16, 16, 4, 1, 3, bf)


def test_python_wrapper_validates_before_the_library():
    import torch
    from blocked_local_self_amd import halo_attn_fwd
    x = torch.zeros(1, 1, 8, 8, 16)
    t = torch.zeros(11, 16)
    with pytest.raises(ValueError):
        halo_attn_fwd(x, x, x, t, t, 4, 1)   # CPU tensors are refused


# ------------------------------------------------------------------ backward
def bwd_call(lib, *, q=1, k=2, v=3, rh=4, rw=5, out=0, dout=6, lse=0, dq=7, dk=8, dv=9, drh=10, drw=11,
             ws=12, ws_bytes=1 << 40, B=1, heads=1, H=8, W=8, d=16, block=4, halo=1, stride=1, scale=0.25,
             dtype=1, kernel=0):
    # fake, non-overlapping pointers (i << 36): every call below fails before any HIP call
    ptr = lambda x: ctypes.c_void_p(x << 36 if x else None)
    return lib.halo_attn_bwd_kernel(ptr(q), ptr(k), ptr(v), ptr(rh), ptr(rw), ptr(out), ptr(dout), ptr(lse),
                                    ptr(dq), ptr(dk), ptr(dv), ptr(drh), ptr(drw), ptr(ws), ws_bytes,
                                    B, heads, H, W, d, block, halo, stride, scale, dtype, kernel, None)


@pytest.mark.parametrize("kw,status", [
    (dict(drh=0), -1), (dict(q=0), -1), (dict(dq=0), -1), (dict(ws=0), -1), (dict(dout=0), -1),
    (dict(out=13), -1), (dict(lse=13), -1),                  # only one of out / lse
    (dict(dtype=5), -3), (dict(d=0), -2), (dict(stride=3), -2), (dict(kernel=7), -2),
    (dict(scale=float("nan")), -2),
    (dict(ws_bytes=16), -7),                                 # workspace too small
    (dict(kernel=2, dtype=0), -4), (dict(kernel=2, d=24), -4), (dict(kernel=2, block=20, halo=2), -4),
    (dict(dq=1), -6), (dict(dk=7), -6), (dict(ws=1), -6),   # aliasing
])
def test_backward_invalid_arguments_rejected_on_host(lib, kw, status):
    assert bwd_call(lib, **kw) == status, _native.last_error()
    assert _native.last_error() != ""


def test_backward_workspace_query():
    from blocked_local_self_amd import bwd_workspace_bytes
    n = bwd_workspace_bytes(32, 8, 64, 64, 16, 8, 3, 1, "bf16")
    strips, H, r, d = 32 * 8 * 8, 64, 14, 16
    assert n >= strips * H * r * 2 * d * 4           # per-block-column dk/dv shares (fp32)
    assert bwd_workspace_bytes(0, 8, 64, 64, 16, 8, 3, 1, "bf16") == 0
    assert bwd_workspace_bytes(1, 1, 8, 8, 16, 4, 1, 1, "fp32") > 0
    with pytest.raises(HaloError):
        bwd_workspace_bytes(1, 1, 8, 8, 16, 4, 1, 3, "bf16")


# ------------------------------------------------------------------ the layer

def layer_call(lib, *, x=1, wq=2, wkv=3, wo=4, bo=5, rh=6, rw=7, y=8, ws=9, ws_bytes=1 << 40, B=1, H=8, W=8,
               C=32, Co=32, heads=2, d=16, block=4, halo=1, stride=1, scale=0.25, layout=0, dtype=1,
               kernel=_native.HALO_LAYER_KERNEL_SPLIT):
    # fake pointers 2^36 apart: every call below must fail before any launch
    # (the split path, whose checks include the workspace's)
    ptr = lambda v: ctypes.c_void_p(v << 36 if v else None)
    return lib.halo_attn_layer_fwd_ex(ptr(x), ptr(wq), ptr(wkv), ptr(wo), ptr(bo), ptr(rh), ptr(rw), ptr(y),
                                      ptr(ws), ws_bytes, B, H, W, C, Co, heads, d, block, halo, stride, scale,
                                      layout, dtype, kernel, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), -1), (dict(bo=0), -1), (dict(y=0), -1), (dict(ws=0), -1),
    (dict(dtype=4), -3), (dict(layout=2), -2), (dict(C=-1), -2), (dict(heads=300, d=16), -2),
    (dict(stride=3), -2), (dict(stride=2, block=5), -2), (dict(layout=1, block=3), -2),
    (dict(d=0, heads=2, block=0), -2), (dict(scale=float("nan")), -2), (dict(d=200), -2),
    (dict(ws_bytes=1024), -7),
    (dict(y=1), -6), (dict(ws=8), -6),                     # y / workspace overlap
])
def test_layer_invalid_arguments_rejected_on_host(lib, kw, status):
    assert layer_call(lib, **kw) == status, _native.last_error()
    assert _native.last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), -1), (dict(y=1), -6), (dict(stride=2), -4), (dict(dtype=0), -4), (dict(C=48, Co=48), -4),
])
def test_fused_layer_invalid_arguments_rejected_on_host(lib, kw, status):
    """The fused path's own refusals (it takes no workspace: a null one is
    not an error there)."""
    assert layer_call(lib, ws=0, kernel=_native.HALO_LAYER_KERNEL_FUSED, **kw) == status, _native.last_error()


def test_layer_kernel_query_and_choice_on_host(lib):
    bf, f32 = _native.HALO_BF16, _native.HALO_F32
    FUSED = _native.HALO_LAYER_KERNEL_FUSED
    name = lambda *a: _native.layer_kernel_name(*a, kernel=FUSED)
    assert name(32, 64, 64, 128, 128, 8, 16, 8, 3, 1, 0, bf) == "fused"     # the bench's layer shape
    assert name(2, 16, 24, 64, 48, 4, 16, 8, 3, 1, 1, bf) == "fused"        # blocked layout
    assert name(1, 12, 8, 64, 128, 4, 32, 4, 6, 1, 0, bf) == "fused"        # block 4, 16x16 window
    for args in [(1, 12, 8, 64, 256, 4, 32, 4, 6, 1, 0, bf),               # W_o of a head beyond the prefetch
                 (32, 64, 64, 128, 128, 8, 16, 8, 3, 2, 0, bf),             # query stride 2
                 (32, 64, 64, 128, 128, 8, 16, 8, 3, 1, 0, f32),            # fp32
                 (1, 24, 24, 128, 128, 8, 16, 12, 3, 1, 0, bf),             # block 12
                 (1, 16, 16, 128, 128, 4, 32, 8, 5, 1, 0, bf),              # 18x18 window
                 (1, 16, 16, 48, 48, 3, 16, 8, 3, 1, 0, bf),                # C % 32 != 0
                 (1, 16, 16, 64, 512, 4, 16, 8, 3, 1, 0, bf),               # C_out > 256
                 (1, 16, 16, 1024, 64, 4, 16, 8, 4, 1, 0, bf)]:             # window of x beyond the LDS
        with pytest.raises(ValueError, match="fused"):
            name(*args)
        assert _native.layer_kernel_name(*args) == "split"
    # AUTO takes the split path (the faster where both apply)
    assert _native.layer_kernel_name(32, 64, 64, 128, 128, 8, 16, 8, 3, 1, 0, bf) == "split"
    assert name(0, 16, 16, 64, 64, 4, 16, 8, 3, 1, 0, bf) == "none"
    with pytest.raises(ValueError, match="query_stride"):
        name(1, 16, 16, 64, 64, 4, 16, 8, 3, 3, 0, bf)
    with pytest.raises(ValueError, match="kernel"):
        _native.layer_kernel_name(1, 16, 16, 64, 64, 4, 16, 8, 3, 1, 0, bf, kernel=7)
    p = lambda v: ctypes.c_void_p(v << 36 if v else None)
    args = [p(1), p(2), p(3), p(4), p(5), p(6), p(7), p(8), p(9), 1 << 40, 1, 16, 16, 64, 64, 2, 16, 8, 2]
    # an unknown kernel value; the fused kernel asked for a strided layer (refused before any launch)
    assert lib.halo_attn_layer_fwd_ex(*args, 1, 0.25, 0, bf, 3, None) == -2
    assert lib.halo_attn_layer_fwd_ex(*args, 2, 0.25, 0, bf, _native.HALO_LAYER_KERNEL_FUSED, None) == -4
    assert "fused" in _native.last_error()


def test_layer_parts_reject_on_host(lib):
    p = lambda v: ctypes.c_void_p(v << 36 if v else None)
    # proj_in: q overlaps x; unknown layout; blocked layout not dividing H
    assert lib.halo_attn_layer_proj_in(p(1), p(2), p(3), p(1), p(5), p(6), 1, 8, 8, 32, 2, 16, 4, 0, 1, None) == -6
    assert lib.halo_attn_layer_proj_in(p(1), p(2), p(3), p(4), p(5), p(6), 1, 8, 8, 32, 2, 16, 4, 3, 1, None) == -2
    assert lib.halo_attn_layer_proj_in(p(1), p(2), p(3), p(4), p(5), p(6), 1, 9, 8, 32, 2, 16, 4, 1, 1, None) == -2
    assert lib.halo_attn_layer_proj_in(p(1), p(0), p(3), p(4), p(5), p(6), 1, 8, 8, 32, 2, 16, 4, 0, 1, None) == -1
    # proj_out: y overlaps w_o; bad dtype
    assert lib.halo_attn_layer_proj_out(p(1), p(2), p(3), p(2), 1, 8, 8, 32, 2, 16, 4, 0, 1, None) == -6
    assert lib.halo_attn_layer_proj_out(p(1), p(2), p(3), p(4), 1, 8, 8, 32, 2, 16, 4, 0, 9, None) == -3
    # zero sizes are no-ops even with null pointers
    assert lib.halo_attn_layer_proj_in(p(0), p(0), p(0), p(0), p(0), p(0), 0, 8, 8, 32, 2, 16, 4, 0, 1, None) == 0


def test_layer_workspace_query():
    from blocked_local_self_amd import layer_workspace_bytes
    n = layer_workspace_bytes(32, 64, 64, 8, 16)
    assert n == 4 * 32 * 8 * 64 * 64 * 16 * 2          # q, k, v and the attention output, bf16
    assert layer_workspace_bytes(32, 64, 64, 8, 16, 2) == 3 * 32 * 8 * 64 * 64 * 16 * 2 + 32 * 8 * 32 * 32 * 16 * 2
    assert layer_workspace_bytes(0, 64, 64, 8, 16) == 0
    with pytest.raises(HaloError):
        layer_workspace_bytes(1, 8, 8, 2, 16, 3)


def test_noalloc_backward_rejects_oversized_calls_on_host(lib):
    # the early-stage shape needs ~270 MB of workspace, more than the static
    # scratch: refused before any HIP call (fake pointers are never touched)
    fake = [ctypes.c_void_p((i + 1) << 32) for i in range(13)]
    assert lib.halo_attn_noalloc_scratch_bytes() == 64 << 20
    st = lib.halo_attn_bwd_noalloc(*fake, 32, 8, 64, 64, 16, 8, 3, 1, 0.25, 1, None)
    assert st == -7
    assert "static scratch" in _native.last_error()
