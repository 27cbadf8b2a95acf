"""ctypes loader for libattn.so and the C ABI's argument/return types."""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"
_lock = threading.Lock()
_lib = None

STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGN",
    5: "ATTN_ERR_WORKSPACE",
    6: "ATTN_ERR_HIP",
    7: "ATTN_ERR_SCRATCH",
}

# ATTN_DECODE_SCRATCH_BYTES: static per-device scratch of attn_decode_noalloc
DECODE_SCRATCH_BYTES = 16 << 20

# exported functions and their ctypes signatures (mirrors include/attn.h)
P, I, D, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_rope": (I, [P, P, I, I, I, I, I, P, I, D, P]),
    "attn_rope_backward": (I, [P, P, I, I, I, I, I, P, I, D, P]),
    "attn_prefill": (I, [P, P, P, P, I, I, I, I, I, I, F, D, P]),
    "attn_prefill_lse": (I, [P, P, P, P, P, I, I, I, I, I, I, F, D, P]),
    "attn_prefill_backward_workspace_size": (SZ, [I, I, I, I, I]),
    "attn_prefill_backward": (I, [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P]),
    "attn_decode_workspace_size": (SZ, [I, I, I, I, I]),
    "attn_decode": (I, [P, P, P, P, I, I, I, I, I, I, P, I, F, D, P, SZ, P]),
    "attn_decode_noalloc": (I, [P, P, P, P, I, I, I, I, I, I, P, I, F, D, P]),
    "attn_decode_paged": (I, [P, P, P, P, I, I, I, I, I, I, I, P, I, P, I, I, F, D, P, SZ, P]),
    "attn_cca_mix": (I, [P, P, P, P, P, P, I, I, I, I, I, I, P, P, I, P, P, P, D, P]),
    "attn_cca_mix_backward_workspace_size": (SZ, [I, I, I, I, I, I]),
    "attn_cca_mix_backward": (I, [P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, I, P, P,
                                  P, D, P, SZ, P]),
    "attn_cca_mix_decode": (I, [P, P, P, P, P, P, I, I, I, I, I, P, P, I, P, P, P, P, P, P, P, D,
                                P]),
    "attn_status_string": (ctypes.c_char_p, [I]),
}


def _dtype_codes():
    import torch
    return {torch.float32: 0, torch.bfloat16: 1}


class _LazyCodes(dict):
    def __missing__(self, key):
        self.update(_dtype_codes())
        return dict.__getitem__(self, key)


DTYPE_CODES = _LazyCodes()


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib():
    """The loaded C ABI library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m compressed_latent_causal_amd.build` "
                    "(there is no fallback implementation)")
            handle = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


class AttnError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int):
        self.status = status
        msg = lib().attn_status_string(status).decode()
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
