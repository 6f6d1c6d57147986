"""ctypes loader for libmoe.so and the C signatures of include/moe.h.

There is no fallback: if the library is not built the import of an op fails
with an error that says how to build it.
"""

import ctypes
import glob
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")


def source_files():
    """Every file the library is built from: the HIP sources and headers, the
    public header and the build script (its flags)."""
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))) + \
        [HEADER, os.path.join(HERE, "build.py")]


def source_hash():
    """First 16 hex digits of a sha256 over the names and contents of
    source_files(); build.py compiles it into the library."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]

MOE_OK, MOE_E_INVAL, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = range(5)
SCORING = {"softmax": 0, "sigmoid": 1, "sqrtsoftplus": 2}
WFORMAT = {"bf16": 0, "fp8": 1, "mxfp4": 2}
STAGE = {"quant": 1, "gemm1": 2, "gemm2": 4, "combine": 8, "all": 15}
NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

SIGNATURES = {
    "moe_status_str": (ctypes.c_char_p, [_i]),
    "moe_source_hash": (ctypes.c_char_p, []),
    "moe_route": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_workspace_size": (_sz, [_i, _i, _i]),
    "moe_route_align": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp, _vp,
                             _vp, _sz, _vp]),
    "moe_route_align_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "moe_align": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_align_workspace_size": (_sz, [_i, _i, _i]),
    "moe_align_max_padded": (_i64, [_i, _i, _i, _i]),
    "moe_align_max_blocks": (_i64, [_i, _i, _i, _i]),
    "moe_expert_ffn": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn_stages": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _sz, _i, _vp]),
    "moe_layer": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _f,
                       _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_layer_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "moe_layer_noalloc": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                               _i, _f, _vp, _vp, _vp, _vp]),
    "moe_layer_block_m": (_i, [_i, _i, _i, _i, _i]),
    "moe_debug_error": (_i32, [_vp, _vp]),
    "moe_probe_empty": (_i, [_vp]),
    "moe_probe_read": (_i, [_vp, _sz, _vp, _vp]),
    "moe_probe_read_sink_len": (_sz, [_sz]),
    "moe_probe_mfma": (_i, [_i, _i, _i, _i, _vp, _vp]),
    "moe_probe_mfma_sink_len": (_sz, [_i]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().moe_status_str(status).decode()
        super().__init__(f"{where}: {msg}")


def lib():
    """The loaded libmoe (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; build it with `python -m mixture_experts_layer_04_amd.build` "
                "(hipcc, gfx950). There is no fallback path.")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        built, now = L.moe_source_hash().decode(), source_hash()
        if built != now:
            raise RuntimeError(
                f"{LIB_PATH} was built from other sources (hash {built}, sources {now}); rebuild it with "
                "`python -m mixture_experts_layer_04_amd.build`.")
        _lib = L
    return _lib


def check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)
