"""ctypes view of libspd.so (declarations mirror include/spd.h).

The library is required: importing this module without a built libspd.so
raises ImportError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspd.so")

SPD_OK = 0
SPD_K_NAMES = ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv", "reconstruct", "pack_rows", "reconstruct_bwd",
               "pack_rows_bwd", "mask_to_varlen")
SPD_F32 = 0
SPD_BF16 = 1

_i32p = ctypes.POINTER(ctypes.c_int32)


class SpdPlan(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("P", ctypes.c_int64),
        ("group_of", ctypes.c_void_p), ("grp_off", ctypes.c_void_p), ("grp_idx", ctypes.c_void_p),
        ("rep", ctypes.c_void_p), ("prompt_off", ctypes.c_void_p), ("prompt_len", ctypes.c_void_p),
        ("resp_off", ctypes.c_void_p), ("resp_len", ctypes.c_void_p), ("src", ctypes.c_void_p),
        ("dst", ctypes.c_void_p), ("seg_start", ctypes.c_void_p), ("counts", ctypes.c_void_p),
        ("padded_with_mask", ctypes.c_int32),
    ]


class SpdAttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


# name -> (restype, argtypes)
_P = ctypes.c_void_p
_SIG = {
    "spd_group_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "spd_group": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(SpdPlan), _P,
                                 _P, ctypes.c_size_t, _P]),
    "spd_pack_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "spd_pack": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(SpdPlan), _P, _P, _P,
                                ctypes.c_size_t, _P]),
    "spd_pack_rows": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, _P, ctypes.c_int64, _P, _P]),
    "spd_reconstruct": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, _P, ctypes.c_int64, _P, _P]),
    "spd_reconstruct_bwd": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, _P, ctypes.c_int64,
                                           ctypes.c_int32, _P, _P]),
    "spd_pack_rows_bwd": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, _P, ctypes.c_int64, _P, _P]),
    "spd_share_prefix": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(SpdPlan),
                                        _P]),
    "spd_group_singletons": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(SpdPlan),
                                            _P]),
    "spd_repack_rows": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, ctypes.POINTER(SpdPlan),
                                       ctypes.c_int64, _P, ctypes.c_int64, _P, _P]),
    "spd_repack_rows_bwd": (ctypes.c_int, [ctypes.POINTER(SpdPlan), ctypes.c_int64, ctypes.POINTER(SpdPlan),
                                           ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
    "spd_mask_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64]),
    "spd_mask_to_varlen": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "spd_varlen_params": (ctypes.c_int, [ctypes.POINTER(SpdPlan), _P, _P, _P, _P, _P]),
    "spd_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SpdAttnDesc), ctypes.c_int64, ctypes.c_int64]),
    "spd_attn_fwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SpdAttnDesc), ctypes.c_int64,
                                                       ctypes.c_int64]),
    "spd_split_attn_fwd": (ctypes.c_int, [ctypes.POINTER(SpdAttnDesc), ctypes.POINTER(SpdPlan), ctypes.c_int64,
                                          _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "spd_split_attn_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(SpdAttnDesc), ctypes.POINTER(SpdPlan),
                                                  ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "spd_split_attn_bwd": (ctypes.c_int, [ctypes.POINTER(SpdAttnDesc), ctypes.POINTER(SpdPlan), ctypes.c_int64,
                                          _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "spd_profile_begin": (ctypes.c_int, []),
    "spd_profile_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
    "spd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "spd_last_hip_error": (ctypes.c_int, []),
    "spd_version": (ctypes.c_int, []),
}

EXPORTED = tuple(_SIG)


def _load():
    # One HIP runtime per process.  PyTorch ships its own libamdhip64 with the
    # same soname as the system one libspd.so is linked against; loading torch
    # first makes the dynamic linker bind libspd.so to torch's copy.  The other
    # order maps two runtimes, and torch's streams and allocations then reach a
    # runtime that does not own them.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m shared_prompt_dedup_amd.build` "
            "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIG.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class SpdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib.spd_status_string(status).decode()
        extra = f" (hip error {lib.spd_last_hip_error()})" if status == -5 else ""
        super().__init__(f"{fn}: {msg}{extra} [status {status}]")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != SPD_OK:
        raise SpdError(fn, status)
