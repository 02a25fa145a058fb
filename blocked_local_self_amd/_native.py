"""ctypes loader for libhaloattn.so (the C ABI declared in include/halo_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhaloattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "halo_attn.h")

HALO_F32, HALO_BF16 = 0, 1
HALO_KERNEL_AUTO, HALO_KERNEL_GENERIC, HALO_KERNEL_MFMA, HALO_KERNEL_MFMA_STRIP, HALO_KERNEL_MFMA_RING = 0, 1, 2, 3, 4
HALO_CENTRED_OFFSET, HALO_ZERO_PAD, HALO_CENTRED_MASK, HALO_HALF_SPLIT = 1, 2, 4, 8
HALO_LAYOUT_NHWC, HALO_LAYOUT_BLOCKED = 0, 1
HALO_LAYER_KERNEL_AUTO, HALO_LAYER_KERNEL_FUSED, HALO_LAYER_KERNEL_SPLIT = 0, 1, 2
STATUS = {0: "HALO_OK", -1: "HALO_ERR_NULL", -2: "HALO_ERR_SHAPE", -3: "HALO_ERR_DTYPE",
          -4: "HALO_ERR_UNSUPPORTED", -5: "HALO_ERR_HIP", -6: "HALO_ERR_ALIAS",
          -7: "HALO_ERR_WORKSPACE"}

_lib = None


class HaloError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m blocked_local_self_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.halo_attn_fwd.argtypes = [vp] * 6 + [i] * 8 + [f, i, vp]
    lib.halo_attn_fwd.restype = i
    lib.halo_attn_fwd_kernel.argtypes = [vp] * 6 + [i] * 8 + [f, i, i, vp]
    lib.halo_attn_fwd_kernel.restype = i
    sz = ctypes.c_size_t
    lib.halo_attn_fwd_ex.argtypes = [vp] * 7 + [i] * 8 + [f, i, i, i, vp]
    lib.halo_attn_fwd_ex.restype = i
    lib.halo_attn_fwd_lse.argtypes = [vp] * 7 + [i] * 8 + [f, i, i, vp]
    lib.halo_attn_fwd_lse.restype = i
    lib.halo_attn_bwd_ex.argtypes = [vp] * 14 + [sz] + [i] * 8 + [f, i, i, i, vp]
    lib.halo_attn_bwd_ex.restype = i
    lib.halo_attn_bwd_kernel.argtypes = [vp] * 14 + [sz] + [i] * 8 + [f, i, i, vp]
    lib.halo_attn_bwd_kernel.restype = i
    lib.halo_attn_bwd.argtypes = [vp] * 14 + [sz] + [i] * 8 + [f, i, vp]
    lib.halo_attn_bwd.restype = i
    lib.halo_attn_bwd_noalloc.argtypes = [vp] * 13 + [i] * 8 + [f, i, vp]
    lib.halo_attn_bwd_noalloc.restype = i
    lib.halo_attn_noalloc_scratch_bytes.argtypes = []
    lib.halo_attn_noalloc_scratch_bytes.restype = ctypes.c_longlong
    lib.halo_attn_bwd_workspace_bytes.argtypes = [i] * 9
    lib.halo_attn_bwd_workspace_bytes.restype = ctypes.c_longlong
    lib.halo_attn_layer_proj_in.argtypes = [vp] * 6 + [i] * 9 + [vp]
    lib.halo_attn_layer_proj_in.restype = i
    lib.halo_attn_layer_proj_out.argtypes = [vp] * 4 + [i] * 9 + [vp]
    lib.halo_attn_layer_proj_out.restype = i
    lib.halo_attn_layer_workspace_bytes.argtypes = [i] * 7
    lib.halo_attn_layer_workspace_bytes.restype = ctypes.c_longlong
    lib.halo_attn_layer_fwd.argtypes = [vp] * 9 + [sz] + [i] * 10 + [f, i, i, vp]
    lib.halo_attn_layer_fwd.restype = i
    lib.halo_attn_layer_fwd_ex.argtypes = [vp] * 9 + [sz] + [i] * 10 + [f, i, i, i, vp]
    lib.halo_attn_layer_fwd_ex.restype = i
    lib.halo_attn_layer_kernel_name.argtypes = [i] * 13
    lib.halo_attn_layer_kernel_name.restype = ctypes.c_char_p
    lib.halo_attn_probe_issue.argtypes = [i, i, i, vp, vp]
    lib.halo_attn_probe_issue.restype = i
    lib.halo_attn_fwd_kernel_name.argtypes = [i] * 11
    lib.halo_attn_fwd_kernel_name.restype = ctypes.c_char_p
    lib.halo_attn_bwd_kernel_name.argtypes = [i] * 11
    lib.halo_attn_bwd_kernel_name.restype = ctypes.c_char_p
    lib.halo_attn_select_kernel.argtypes = [i] * 5
    lib.halo_attn_select_kernel.restype = i
    lib.halo_attn_last_error.argtypes = []
    lib.halo_attn_last_error.restype = ctypes.c_char_p
    lib.halo_attn_abi_version.argtypes = []
    lib.halo_attn_abi_version.restype = i
    lib.halo_attn_build_id.argtypes = []
    lib.halo_attn_build_id.restype = ctypes.c_char_p
    _check_build_id(lib)
    _lib = lib
    return lib


def _check_build_id(lib) -> None:
    """Warn when the library was built from other sources than those in csrc/."""
    from . import build
    built, here = lib.halo_attn_build_id().decode(), build.source_id()
    if built != here:
        import warnings
        warnings.warn(f"{LIB_PATH} was built from sources {built}, csrc/ now holds {here}: rebuild "
                      "(__graft_entry__.build())", RuntimeWarning, stacklevel=3)


def fwd_kernel_name(B, heads, H, W, d, block, halo, stride, dtype, flags=0, kernel=HALO_KERNEL_AUTO) -> str:
    """The forward kernel halo_attn_fwd_ex runs for these arguments (queries the device)."""
    name = load().halo_attn_fwd_kernel_name(B, heads, H, W, d, block, halo, stride, dtype, flags, kernel)
    if name is None:
        raise ValueError(f"halo_attn_fwd_kernel_name: {last_error()}")
    return name.decode()


def bwd_kernel_name(B, heads, H, W, d, block, halo, stride, dtype, flags=0, kernel=HALO_KERNEL_AUTO) -> str:
    """The backward kernels halo_attn_bwd_ex runs for these arguments (host only)."""
    name = load().halo_attn_bwd_kernel_name(B, heads, H, W, d, block, halo, stride, dtype, flags, kernel)
    if name is None:
        raise ValueError(f"halo_attn_bwd_kernel_name: {last_error()}")
    return name.decode()


def layer_kernel_name(B, H, W, C, C_out, heads, d, block, halo, stride, layout, dtype,
                      kernel=HALO_LAYER_KERNEL_AUTO) -> str:
    """The path halo_attn_layer_fwd_ex takes for these sizes ("fused" or "split"; host only)."""
    name = load().halo_attn_layer_kernel_name(B, H, W, C, C_out, heads, d, block, halo, stride, layout, dtype,
                                              kernel)
    if name is None:
        raise ValueError(f"halo_attn_layer_kernel_name: {last_error()}")
    return name.decode()


def last_error() -> str:
    return load().halo_attn_last_error().decode()


def check(status: int) -> None:
    if status != 0:
        raise HaloError(status, last_error())


def declared_functions() -> list[str]:
    """Function names declared in include/halo_attn.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s]+?\*?\s*(halo_attn_\w+)\s*\(", text, flags=re.M)))
