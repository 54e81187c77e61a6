"""Grouped tril mask softmax on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libgtms.so`` (built from ``csrc/`` by ``build.py``). The binding
only marshals arguments: every step of the operation runs in the library's HIP kernels,
on the caller's current torch stream. Torch provides device memory and streams.

    y = forward(x, seq_lens, scale)      # x: [B, M, S, S] f32/f16/bf16 on the GPU
    dx = backward(y, dy, seq_lens, scale)

There is no fallback: if the library is missing or cannot load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgtms.so")

# element-type, path and flag codes of include/gtms.h
F32, F16, BF16 = 0, 1, 2
PATH_AUTO, PATH_WAVE, PATH_BLOCK, PATH_STREAM = 0, 1, 2, 3
FLAG_PAIR_ROWS, FLAG_PLAIN_ORDER = 1, 2
PATHS = {"auto": PATH_AUTO, "wave": PATH_WAVE, "block": PATH_BLOCK, "stream": PATH_STREAM}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                           "python variable_length_causal_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32, u32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                             ctypes.c_uint)
    lib.gtms_forward.argtypes = [p, p, p, i64, i64, i64, f32, i32, p]
    lib.gtms_forward.restype = i32
    lib.gtms_forward_ex.argtypes = [p, p, p, i64, i64, i64, f32, i32, i32, u32, p]
    lib.gtms_forward_ex.restype = i32
    lib.gtms_backward.argtypes = [p, p, p, p, i64, i64, i64, f32, i32, p]
    lib.gtms_backward.restype = i32
    lib.gtms_backward_ex.argtypes = [p, p, p, p, i64, i64, i64, f32, i32, i32, u32, p]
    lib.gtms_backward_ex.restype = i32
    lib.gtms_status_string.argtypes = [i32]
    lib.gtms_status_string.restype = ctypes.c_char_p
    lib.gtms_version.argtypes = []
    lib.gtms_version.restype = i32
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def status_string(code: int) -> str:
    return _load().gtms_status_string(int(code)).decode()


def version() -> int:
    return _load().gtms_version()


_codes = None


def _dtype_code(t) -> int:
    global _codes
    if _codes is None:
        import torch
        _codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    code = _codes.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return code


def _check_scores(x, name="x"):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if x.dim() != 4 or x.shape[-1] != x.shape[-2]:
        raise ValueError(f"{name} must have shape [B, M, S, S], got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_lens(seq_lens, x):
    import torch
    if not seq_lens.is_cuda or seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be a 1-D int32 GPU tensor")
    if seq_lens.shape[0] != x.shape[0]:
        raise ValueError(f"seq_lens has {seq_lens.shape[0]} entries, batch is {x.shape[0]}")
    if seq_lens.device != x.device:
        raise ValueError("seq_lens and x must be on the same device")


def _raise(st: int, what: str):
    if st != 0:
        raise RuntimeError(f"{what}: {status_string(st)} (status {st})")


def _stream_of(t):
    """The current torch stream of t's device, as a hipStream_t."""
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


class _on_device:
    """Makes t's device current for the call (HIP launches go to the current device)."""

    def __init__(self, t):
        import torch
        self.torch, self.idx, self.prev = torch, t.device.index, None

    def __enter__(self):
        cur = self.torch.cuda.current_device()
        if cur != self.idx:
            self.prev = cur
            self.torch.cuda.set_device(self.idx)

    def __exit__(self, *exc):
        if self.prev is not None:
            self.torch.cuda.set_device(self.prev)


def forward(x, seq_lens, scale: float = 1.0, out=None, path: str = "auto", flags: int = 0):
    """Grouped tril mask softmax of x ([B, M, S, S]) with per-batch valid lengths.

    ``out`` may be x itself (in place). ``path``/``flags`` select a kernel explicitly
    (tests and tuning); the default is the library's own choice.
    """
    import torch
    _check_scores(x)
    _check_lens(seq_lens, x)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape, dtype and device")
    B, M, S, _ = x.shape
    L = _load()
    with _on_device(x):
        if path == "auto" and flags == 0:
            st = L.gtms_forward(x.data_ptr(), out.data_ptr(), seq_lens.data_ptr(), B, M, S,
                                float(scale), _dtype_code(x), _stream_of(x))
        else:
            st = L.gtms_forward_ex(x.data_ptr(), out.data_ptr(), seq_lens.data_ptr(), B, M, S,
                                   float(scale), _dtype_code(x), PATHS[path], int(flags),
                                   _stream_of(x))
    _raise(st, "gtms_forward")
    return out


def backward(y, dy, seq_lens, scale: float = 1.0, out=None, path: str = "auto", flags: int = 0):
    """Gradient with respect to the forward's input, given its output y and the upstream
    gradient dy (both [B, M, S, S]). ``out`` may be dy itself (in place), not y."""
    import torch
    _check_scores(y, "y")
    _check_scores(dy, "dy")
    _check_lens(seq_lens, y)
    if dy.shape != y.shape or dy.dtype != y.dtype or dy.device != y.device:
        raise ValueError("dy must match y in shape, dtype and device")
    if out is None:
        out = torch.empty_like(y)
    elif out.shape != y.shape or out.dtype != y.dtype or not out.is_contiguous() \
            or out.device != y.device:
        raise ValueError("out must be a contiguous tensor of y's shape, dtype and device")
    B, M, S, _ = y.shape
    L = _load()
    with _on_device(y):
        if path == "auto" and flags == 0:
            st = L.gtms_backward(y.data_ptr(), dy.data_ptr(), out.data_ptr(), seq_lens.data_ptr(),
                                 B, M, S, float(scale), _dtype_code(y), _stream_of(y))
        else:
            st = L.gtms_backward_ex(y.data_ptr(), dy.data_ptr(), out.data_ptr(),
                                    seq_lens.data_ptr(), B, M, S, float(scale), _dtype_code(y),
                                    PATHS[path], int(flags), _stream_of(y))
    _raise(st, "gtms_backward")
    return out
