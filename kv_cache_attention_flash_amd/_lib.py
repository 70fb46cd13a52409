"""ctypes view of libfdllm.so (the C ABI declared in include/fdllm.h).

Loading never falls back to anything: a missing or unloadable library raises.
torch is imported first so that the library binds to the HIP runtime torch has
already loaded (both carry the soname libamdhip64.so.7).
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before the library)

# FDL_LIB names another build of the same library (the host-sanitised one,
# for instance); by default the in-tree libfdllm.so.
LIB_PATH = os.environ.get("FDL_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libfdllm.so")

FDL_OK, FDL_EINVAL, FDL_EUNSUPPORTED, FDL_EWORKSPACE, FDL_EHIP, FDL_ESCRATCH = 0, 1, 2, 3, 4, 5

c_i32, c_i64, c_f32, c_size, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_size_t, ctypes.c_void_p)


class KVCacheStruct(ctypes.Structure):
    _fields_ = [("num_heads", c_i32), ("head_dim", c_i32), ("block_size", c_i32),
                ("num_blocks", c_i32), ("max_blocks_per_seq", c_i32),
                ("k_cache", c_vp), ("v_cache", c_vp), ("block_table", c_vp)]


EXPORTS = {
    "flash_cache_step": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_vp, c_i32,
                                        c_i32, c_vp, c_vp, c_vp, c_f32, c_vp, c_vp, c_vp, c_size,
                                        c_vp]),
    "fdl_flash_cache_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "flash_cache_step_unfused": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_vp,
                                                c_i32, c_i32, c_vp, c_vp, c_vp, c_f32, c_vp, c_vp,
                                                c_vp, c_size, c_vp]),
    "fdl_flash_cache_unfused_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "scheduled_attention": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_i32, c_vp,
                                           c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp, c_i32,
                                           c_vp, c_size, c_vp]),
    "fdl_attention_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "fdl_attention_path": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "scheduled_attention_static": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_i32,
                                                  c_vp, c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp,
                                                  c_i32, c_vp]),
    "fdl_static_scratch_bytes": (c_size, []),
    "track_topb": (ctypes.c_int, [c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "verify_accept": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_i32, c_f32, c_vp, c_vp]),
    "decode_plan": (ctypes.c_int, [c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp,
                                   c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
    "gather_hidden": (ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                     c_vp, c_vp]),
    "lm_head_confidence": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                          c_size, c_vp]),
    "fdl_lm_head_workspace_bytes": (c_size, [c_i32, c_i32]),
    "flash_cache_attention_step": (ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_vp,
                                                  c_i32, c_i32, c_vp, c_vp, c_vp, c_f32, c_vp,
                                                  c_vp, c_vp, c_i32, c_i32, c_vp, c_f32, c_vp,
                                                  c_vp, c_i32, c_vp, c_size, c_vp]),
    "flash_cache_attention_step_single_launch": (
        ctypes.c_int, [ctypes.POINTER(KVCacheStruct), c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp,
                       c_vp, c_f32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp, c_i32,
                       c_vp, c_size, c_vp]),
    "fdl_fused_step_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "fdl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fdl_last_hip_error": (ctypes.c_int, []),
    "fdl_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the library; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m kv_cache_attention_flash_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FdlError(RuntimeError):
    def __init__(self, call: str, status: int):
        lib = load()
        msg = lib.fdl_status_string(status).decode()
        if status == FDL_EHIP:
            msg += f" (hipError {lib.fdl_last_hip_error()})"
        super().__init__(f"{call}: {msg} [status {status}]")
        self.status = status


def check(call: str, status: int) -> None:
    if status != FDL_OK:
        raise FdlError(call, status)
