"""ctypes loader for libsdv.so (the C ABI declared in include/sdv.h)."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdv.so")

SDV_OK, SDV_EINVAL, SDV_EWIDTH, SDV_ELAYOUT, SDV_ERANGE, SDV_EALIAS, SDV_EHIP = 0, -1, -2, -3, -4, -5, -6
MAX_ROWS, GROUP, MAX_EXPERTS, MAX_TOPK = 32, 64, 1024, 16
MODE_PLAIN, MODE_GATEUP_SWIGLU = 0, 1
ACT_BF16, ACT_F32 = 0, 1
ROUTE_SOFTMAX, ROUTE_SIGMOID = 0, 1
CONV_NONE, CONV_SILU = 0, 1
FMT_AFFINE_Q4, FMT_Q8_0, FMT_AFFINE_Q3 = 0, 1, 2
GATE_SIGMOID, GATE_SILU = 0, 1

EXPORTS = ("sdv_q4t_codes_bytes", "sdv_q4t_sb_bytes", "sdv_q4_repack", "sdv_q8_0t_codes_bytes", "sdv_q8_0_repack",
           "sdv_q3t_codes_bytes", "sdv_q3_repack",
           "sdv_qmv_k", "sdv_qmv_k_multi", "sdv_moe_route_k",
           "sdv_gather_qmv_k", "sdv_moe_experts_k", "sdv_moe_route_experts_k", "sdv_moe_experts_partial_bytes", "sdv_moe_combine_sliced_k",
           "sdv_moe_combine_k", "sdv_gdn_verify_k", "sdv_gdn_rollback",
           "sdv_gdn_rollback_copy", "sdv_gdn_prepare_k", "sdv_gdn_verify_prep_k", "sdv_gdn_verify_prep_norm_k",
           "sdv_gdn_layers_table", "sdv_gdn_verify_prep_k_layers", "sdv_gdn_gated_norm_k",
           "sdv_verify_accept_workspace_bytes", "sdv_verify_accept_k", "sdv_verify_accept_k_noalloc",
           "sdv_verify_accept_scratch_bytes",
           "sdv_status_string", "sdv_last_error", "sdv_build_info")


class SdvQ4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class SdvGdnLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("S_in", "qkv", "hist", "conv_w", "a", "b", "A_log", "dt_bias",
                                                 "window", "y")] + [("snaps", ctypes.c_void_p * MAX_ROWS)]


class SdvQ4T(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("sb", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("group", ctypes.c_int32),
                ("fused_gateup", ctypes.c_int32), ("format", ctypes.c_int32)]


class SdvQ3(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


class SdvQ8_0(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("d", ctypes.c_void_p), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32)]


class SdvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_LIB = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "sdv_q4t_codes_bytes": [_I, _I, _I, _I],
    "sdv_q4t_sb_bytes": [_I, _I, _I, _I],
    "sdv_q4_repack": [ctypes.POINTER(SdvQ4), _I, _P, _P, _P],
    "sdv_q8_0t_codes_bytes": [_I, _I, _I, _I],
    "sdv_q8_0_repack": [ctypes.POINTER(SdvQ8_0), _I, _P, _P, _P],
    "sdv_q3t_codes_bytes": [_I, _I, _I, _I],
    "sdv_q3_repack": [ctypes.POINTER(SdvQ3), _I, _P, _P, _P],
    "sdv_qmv_k": [ctypes.POINTER(SdvQ4T), _P, _I, _I, _I, _P, _P],
    "sdv_qmv_k_multi": [ctypes.POINTER(SdvQ4T), _I, _P, _I, _I, _I, ctypes.POINTER(_P), _P],
    "sdv_moe_route_k": [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P],
    "sdv_gather_qmv_k": [ctypes.POINTER(SdvQ4T), _I, _P, _I, _P, _P, _P, _P, _P, _I, _I, _P,
                         ctypes.POINTER(SdvQ4T), _P, _P, _P],
    "sdv_moe_experts_k": [ctypes.POINTER(SdvQ4T), ctypes.POINTER(SdvQ4T), _P, _P, _P, _P, _P, _P, _I, _I,
                          ctypes.POINTER(SdvQ4T), ctypes.POINTER(SdvQ4T), _P, _P],
    "sdv_moe_route_experts_k": [_P, _I, _I, ctypes.POINTER(SdvQ4T), ctypes.POINTER(SdvQ4T), _P, _I, _I,
                                ctypes.POINTER(SdvQ4T), ctypes.POINTER(SdvQ4T), _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "sdv_moe_experts_partial_bytes": [_I, _I, _I, _I],
    "sdv_moe_combine_sliced_k": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P],
    "sdv_moe_combine_k": [_P, _P, _P, _P, _I, _I, _I, _P, _P],
    "sdv_gdn_verify_k": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, ctypes.POINTER(_P), _P],
    "sdv_gdn_rollback": [_I, _I, ctypes.POINTER(_I)],
    "sdv_gdn_rollback_copy": [_P, _P, ctypes.POINTER(_P), _I, _I, ctypes.c_size_t, _P],
    "sdv_gdn_prepare_k": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                          _P, _P, _P, _P, _P, _P, _P],
    "sdv_gdn_verify_prep_k": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                              ctypes.POINTER(_P), _P],
    "sdv_gdn_verify_prep_norm_k": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                                   ctypes.POINTER(_P), _P, _P, _I, ctypes.c_float, _P, _P, _P],
    "sdv_gdn_layers_table": [ctypes.c_void_p, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t],
    "sdv_gdn_verify_prep_k_layers": [_P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P],
    "sdv_gdn_gated_norm_k": [_P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P],
    "sdv_verify_accept_workspace_bytes": [_I, _I],
    "sdv_verify_accept_k": [_P, _P, ctypes.c_float, _P, _I, _I, _I, _P, _P, _P, ctypes.c_size_t, _P],
    "sdv_verify_accept_k_noalloc": [_P, _P, ctypes.c_float, _P, _I, _I, _I, _P, _P, _P],
    "sdv_verify_accept_scratch_bytes": [],
    "sdv_status_string": [_I],
    "sdv_last_error": [],
    "sdv_build_info": [],
}


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build` "
                               "(hipcc, gfx950); there is no non-HIP implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            if name in ("sdv_status_string", "sdv_last_error", "sdv_build_info"):
                fn.restype = ctypes.c_char_p
            elif name in ("sdv_q4t_codes_bytes", "sdv_q4t_sb_bytes", "sdv_q8_0t_codes_bytes", "sdv_q3t_codes_bytes",
                          "sdv_moe_experts_partial_bytes", "sdv_verify_accept_workspace_bytes",
                          "sdv_verify_accept_scratch_bytes"):
                fn.restype = ctypes.c_size_t
            else:
                fn.restype = ctypes.c_int
        _LIB = L
    return _LIB


def check(status):
    if status != SDV_OK:
        L = lib()
        msg = L.sdv_last_error().decode() or L.sdv_status_string(status).decode()
        raise SdvError(status, msg)
    return status
