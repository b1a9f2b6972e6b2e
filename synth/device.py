"""Fill device tensors with the seeded synthetic inputs (GPU twin of
:mod:`synth`), through ``synth/libsynth.so``.

The values are bit-identical to the NumPy generator's for the same flat
indices, so the CPU oracle can regenerate any slice it needs on its own.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import C_UNIT, C_W, RMS_EPS, TID_K, TID_LOGITS, TID_PROXY, TID_Q, TID_QIDX, TID_V, TID_W

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_long_context_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, U64, U32, F = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        L.synth_fill_bf16.argtypes = [P, U64, U64, U32, U64, F, P]
        L.synth_fill_f32.argtypes = [P, U64, U64, U32, U64, F, P]
        L.synth_fill_rms_rows_bf16.argtypes = [P, U64, ctypes.c_int32, U64, U32, U64, F, F, P]
        I32 = ctypes.c_int32
        L.synth_fill_corr.argtypes = [P, I32, U64, I32, I32, U64, U32, U64, F, F, P]
        for f in (L.synth_fill_bf16, L.synth_fill_f32, L.synth_fill_rms_rows_bf16, L.synth_fill_corr):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


def fill_bf16(t: torch.Tensor, seed: int, tid: int, idx0: int = 0) -> torch.Tensor:
    """Unit-variance bf16 values at flat indices idx0 .. idx0 + numel - 1."""
    assert t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous()
    _check(lib().synth_fill_bf16(t.data_ptr(), t.numel(), seed, tid, idx0, float(C_UNIT), _stream()),
           "synth_fill_bf16")
    return t


def fill_f32(t: torch.Tensor, seed: int, tid: int, idx0: int = 0, scale=C_UNIT) -> torch.Tensor:
    assert t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
    _check(lib().synth_fill_f32(t.data_ptr(), t.numel(), seed, tid, idx0, float(scale), _stream()),
           "synth_fill_f32")
    return t


def fill_rms_rows(t: torch.Tensor, seed: int, tid: int, row0: int = 0) -> torch.Tensor:
    """RMS-normalised bf16 rows over the last dim (rows row0 .. row0 + n - 1)."""
    assert t.dtype == torch.bfloat16 and t.is_cuda and t.is_contiguous()
    width = t.shape[-1]
    n_rows = t.numel() // width
    _check(lib().synth_fill_rms_rows_bf16(t.data_ptr(), n_rows, width, seed, tid, row0,
                                          float(C_UNIT), float(RMS_EPS), _stream()),
           "synth_fill_rms_rows_bf16")
    return t


__all__ = ["fill_bf16", "fill_f32", "fill_rms_rows", "lib", "TID_Q", "TID_K", "TID_V",
           "TID_QIDX", "TID_W", "TID_PROXY", "TID_LOGITS", "C_W"]


def fill_corr_rows(t: torch.Tensor, seed: int, tid: int, window: int, row0: int = 0,
                   scale=C_UNIT) -> torch.Tensor:
    """Correlated rows along dim 0 (a moving sum of `window` draws per value,
    see :mod:`synth`); bf16 or fp32 tensors, the row width is numel / size(0)."""
    import numpy as np
    assert t.dtype in (torch.bfloat16, torch.float32) and t.is_cuda and t.is_contiguous()
    n_rows = t.shape[0]
    width = t.numel() // max(n_rows, 1)
    c = float(np.float32(1.0 / np.sqrt(float(window))))
    _check(lib().synth_fill_corr(t.data_ptr(), 1 if t.dtype == torch.bfloat16 else 0, n_rows, width,
                                 int(window), seed, tid, row0, float(scale), c, _stream()),
           "synth_fill_corr")
    return t
