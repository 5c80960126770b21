"""ctypes binding of libckks_ks.so (argument marshalling only; every step runs in the HIP library).

The shared object is built in-tree by `python -m rns_ckks_key_amd.build`.  If
it is missing, or was built from other sources than the ones beside it,
importing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libckks_ks.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ckks_ks.h")

STATUS = {0: "CKKS_OK", -1: "CKKS_EINVAL", -2: "CKKS_ERANGE", -3: "CKKS_ENOMEM", -4: "CKKS_EHIP",
          -5: "CKKS_EUNSUPPORTED"}


class CkksError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m rns_ckks_key_amd.build` (hipcc, gfx950)")

# torch brings its own HIP runtime under the same soname as the one the library
# links.  Loading torch first makes the library bind to that single runtime; the
# other order puts two HIP runtimes in the process and device calls then fail.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
U32 = ctypes.c_uint32
U64 = ctypes.c_uint64
PU32 = ctypes.POINTER(ctypes.c_uint32)
PU64 = ctypes.POINTER(ctypes.c_uint64)
PCTX = ctypes.c_void_p

class RotKey(ctypes.Structure):
    """ckks_rot_key of include/ckks_ks.h."""
    _fields_ = [("key_b", ctypes.c_void_p), ("key_a", ctypes.c_void_p), ("key_seed", ctypes.c_uint8 * 32),
                ("galois_elt", ctypes.c_uint32)]


class KsItem(ctypes.Structure):
    """ckks_ks_item of include/ckks_ks.h."""
    _fields_ = [("ct", ctypes.c_void_p), ("out", ctypes.c_void_p), ("key_b", ctypes.c_void_p),
                ("key_a", ctypes.c_void_p), ("key_seed", ctypes.c_uint8 * 32), ("level", ctypes.c_uint32),
                ("galois_elt", ctypes.c_uint32)]


_SIGS = {
    "ckks_build_id": (ctypes.c_char_p, []),
    "ckks_last_error": (ctypes.c_char_p, []),
    "ckks_chain_primes": (ctypes.c_int, [U32, U32, U32, PU32]),
    "ckks_ctx_create": (ctypes.c_int, [ctypes.POINTER(PCTX), U32, U32, U32, U32, PU32, U32]),
    "ckks_ctx_destroy": (None, [PCTX]),
    "ckks_ctx_info": (ctypes.c_int, [PCTX, PU32, PU32, PU32, PU32, PU32, PU32, PU64, PU32]),
    "ckks_ntt_fwd": (ctypes.c_int, [PCTX, P, U32, U32, U32, P]),
    "ckks_ntt_inv": (ctypes.c_int, [PCTX, P, U32, U32, U32, P]),
    "ckks_modup": (ctypes.c_int, [PCTX, P, U32, P, U32, P]),
    "ckks_moddown": (ctypes.c_int, [PCTX, P, U32, P, U32, P]),
    "ckks_keyswitch": (ctypes.c_int, [PCTX, P, U32, P, ctypes.c_char_p, P, U32, P, U32, P]),
    "ckks_keyswitch_noalloc": (ctypes.c_int, [PCTX, P, U32, P, ctypes.c_char_p, P, U32, P, U32, P]),
    "ckks_keyswitch_hoisted": (ctypes.c_int, [PCTX, P, U32, U32, ctypes.POINTER(P), ctypes.c_char_p,
                                              ctypes.POINTER(P), PU32, P, P]),
    "ckks_expand_a": (ctypes.c_int, [PCTX, ctypes.c_char_p, P, P]),
    "ckks_keyswitch_multi": (ctypes.c_int, [PCTX, U32, ctypes.POINTER(KsItem), P]),
    "ckks_rescale": (ctypes.c_int, [PCTX, P, U32, P, U32, P]),
    "ckks_linear_transform_bsgs": (ctypes.c_int, [PCTX, P, U32, U32, U32, ctypes.POINTER(RotKey),
                                                  ctypes.POINTER(RotKey), P, P, P]),
    "ckks_mul_relin_rescale": (ctypes.c_int, [PCTX, P, P, U32, P, ctypes.c_char_p, P, P, U32, P]),
    "ckks_ctx_set_regen_blocks": (ctypes.c_int, [PCTX, U32]),
    "ckks_ctx_set_conv_mfma": (ctypes.c_int, [PCTX, U32]),
    "ckks_ctx_set_fused": (ctypes.c_int, [PCTX, U32]),
    "ckks_profile_enable": (ctypes.c_int, [PCTX, ctypes.c_int]),
    "ckks_profile_read": (ctypes.c_int, [PCTX, ctypes.POINTER(ctypes.c_double), PU32, U32]),
}

KERNEL_CLASSES = ["row", "col", "modup_conv", "ip_special", "moddown_conv", "ip_final", "expand", "moddown_final",
                  "rescale_conv", "rescale_final", "baby", "diag", "digit_ntt", "ip_ext", "moddown_row"]

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check_build() -> None:
    """Refuse a library built from other sources than the ones beside it (a stale build)."""
    from rns_ckks_key_amd.build import source_digest

    built, now = lib.ckks_build_id().decode(), source_digest()
    if built != now:
        raise ImportError(f"{LIB_PATH} was built from other sources (digest {built}) than those in "
                          f"rns_ckks_key_amd/csrc and include/ ({now}); rebuild with "
                          f"`python -m rns_ckks_key_amd.build`")


_check_build()


def header_functions() -> list[str]:
    """Names of the functions include/ckks_ks.h declares."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(ckks_[a-z_0-9]+)\s*\(", text)))


def check(status: int) -> None:
    if status != 0:
        raise CkksError(status, lib.ckks_last_error().decode())
