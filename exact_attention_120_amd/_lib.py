"""ctypes loader for libfa.so and the raw C signatures of include/fa.h."""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build, unless FA_LIBRARY names another build of the same C ABI
# (the host-sanitizer run of the ABI tests loads one built for the host alone).
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(PKG, "libfa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fa.h")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK = 0
FA_MASK_BLOCK = 64

_c = ctypes
_vp, _int, _flt, _sz = _c.c_void_p, _c.c_int, _c.c_float, _c.c_size_t


class FaOptions(_c.Structure):
    """struct fa_options of include/fa.h."""
    _fields_ = [("kv_heads", _int), ("window_left", _int), ("window_right", _int)]


_opt = _c.POINTER(FaOptions)

# name -> (restype, argtypes); must match include/fa.h.
SIGNATURES = {
    "fa_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _int, _vp]),
    "fa_bwd_workspace_size": (_sz, [_int, _int, _int, _int]),
    "fa_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                      _flt, _int, _int, _vp, _sz, _vp]),
    "fa_fwd_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _int,
                         _opt, _vp]),
    "fa_bwd_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                         _flt, _int, _int, _opt, _vp, _sz, _vp]),
    "fa_fwd_keysplit": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _int,
                               _opt, _vp]),
    "fa_fwd_num_splits": (_int, [_int, _int, _int, _int, _int]),
    "fa_fwd_splitkv_workspace_size": (_sz, [_int, _int, _int, _int, _int, _int]),
    "fa_fwd_splitkv": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _int,
                              _opt, _int, _vp, _sz, _vp]),
    "fa_fwd_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _flt, _flt,
                          _flt, _int, _opt, _vp]),
    "fa_fwd_sparse": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _flt, _int, _int,
                             _opt, _vp, _vp]),
    "fa_bwd_sparse": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                             _flt, _int, _int, _opt, _vp, _vp, _sz, _vp]),
    "fa_bwd_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int,
                              _flt, _int, _int, _vp]),
    "fa_strerror": (_c.c_char_p, [_int]),
}

_lib = None


def header_functions() -> list[str]:
    """Names of the functions include/fa.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\**\s*(fa_[a-z_0-9]+)\s*\(",
                      text, flags=re.M)


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                " (there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib
