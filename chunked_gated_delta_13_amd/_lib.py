"""ctypes view of libkda.so (the C ABI declared in include/kda.h).

The library is loaded lazily.  ``torch`` is imported first so that libkda binds
to the HIP runtime torch already loaded (both carry the SONAME
libamdhip64.so.7), giving one runtime, one set of devices and streams per
process.  A missing library is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE = 3
KDA_ERR_DEVICE = 4

KDA_BF16 = 0
KDA_F32 = 1

# bytes of the device array behind kda_chunk_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

# name -> (restype, argtypes); mirrors include/kda.h
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
SIGNATURES = {
    "kda_abi_version": (_i, []),
    "kda_status_string": (ctypes.c_char_p, [_i]),
    "kda_chunk_prefill_plan": (_i, [_i, _i, _i, _i, _i, _i, _i,
                                    ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "kda_chunk_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_chunk_prefill_workspace_bytes_ex": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "kda_chunk_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_prefill_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_prefill_ckpt": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i, _i, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_prefill_gate": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "kda_chunk_prefill_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "kda_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _vp]),
    "kda_spec_verify": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _i, _vp]),
    "kda_spec_commit": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _i, _vp]),
}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status) if _lib is not None else f"status {status}"
        super().__init__(f"{where}: {msg}")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (binds libkda to torch's HIP runtime)

    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "(python chunked_gated_delta_13_amd/build.py)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kda_abi_version() != 1:
        raise RuntimeError("libkda ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != KDA_OK:
        raise KDAError(status, where)
