"""Device-side generation of the synthetic Q4 banks (same values as
``synth.counter``) and uploads of host-generated inputs."""

import ctypes
import os

import numpy as np
import torch

from .counter import BIAS_LO, BIAS_SPAN, SCALE_LO, SCALE_SPAN

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdvsynth.so")
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python __graft_entry__.py build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sdvsynth_fill_codes.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p]
        L.sdvsynth_fill_affine_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                                ctypes.c_uint64, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        _LIB = L
    return _LIB


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fill_codes(dst, key, first_word=0):
    rc = _lib().sdvsynth_fill_codes(ctypes.c_void_p(dst.data_ptr()), key, first_word, dst.numel(),
                                    _stream(dst.device))
    if rc:
        raise RuntimeError(f"sdvsynth_fill_codes failed ({rc})")


def fill_affine(dst, key, lo, span, first=0):
    rc = _lib().sdvsynth_fill_affine_bf16(ctypes.c_void_p(dst.data_ptr()), key, first, dst.numel(), lo, span,
                                          _stream(dst.device))
    if rc:
        raise RuntimeError(f"sdvsynth_fill_affine_bf16 failed ({rc})")


def q4_bank(keys, E, N, K, device):
    """A whole bank [E, N, K] generated in device memory: codes int32 [E, N, K/8],
    scales/biases int16 [E, N, K/64] (bit patterns)."""
    codes = torch.empty((E, N, K // 8), dtype=torch.int32, device=device)
    scales = torch.empty((E, N, K // 64), dtype=torch.int16, device=device)
    biases = torch.empty((E, N, K // 64), dtype=torch.int16, device=device)
    fill_codes(codes, keys.codes)
    fill_affine(scales, keys.scales, SCALE_LO, SCALE_SPAN)
    fill_affine(biases, keys.biases, BIAS_LO, BIAS_SPAN)
    return codes, scales, biases


def upload_q4(codes, scales, biases, device):
    """Host uint32/uint16 arrays to device int32/int16 tensors (bit patterns kept)."""
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).to(device)
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).to(device)
    b = torch.from_numpy(np.ascontiguousarray(biases).view(np.int16)).to(device)
    return c, s, b


def upload_bf16(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def upload_f32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
