"""ctypes loader for libswattn.so (the C ABI in include/swattn.h).

torch is imported first on purpose: it loads its bundled HIP runtime, whose soname
(libamdhip64.so.7) then satisfies libswattn.so's dependency, so one process holds one HIP runtime.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load, see above)

# SWATTN_LIBRARY names another build of the same library (the CPU ABI tests use it to load the
# host-side AddressSanitizer build); by default the in-tree libswattn.so is loaded.
LIB_PATH = os.environ.get("SWATTN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libswattn.so")

SWATTN_BF16 = 0
SWATTN_F32 = 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small",
          -4: "HIP error"}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

SIGNATURES = {
    "attn_abi_version": (_i, []),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz,
                      _vp]),
    "attn_bwd_dq": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "attn_bwd_dkdv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz,
                           _vp]),
    "attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_kv_append": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "attn_decode_launches": (_i, [_i, _i, _i, _i, _i]),
    "attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "attn_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz,
                              _vp]),
    "attn_decode_step_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                      _vp]),
    "attn_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_bwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                             _i, _vp, _sz, _vp]),
    "attn_fwd_qknorm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                             ctypes.c_float, _vp]),
    "attn_bwd_qknorm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                             _i, _vp, _sz, _vp]),
}

_LIB = None


def load() -> ctypes.CDLL:
    """Load libswattn.so once and attach the C signatures.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (or python causal_sliding_window_attn_amd/build.py); there is no "
                "fallback implementation")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def last_error() -> str:
    return load().attn_last_error().decode(errors="replace")


def check(rc: int, what: str) -> None:
    if rc != 0:
        msg = f"{what} failed with status {rc} ({STATUS.get(rc, '?')}): {last_error()}"
        if rc in (-1, -2, -3):
            raise ValueError(msg)
        raise RuntimeError(msg)
