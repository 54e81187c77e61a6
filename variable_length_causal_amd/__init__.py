"""Grouped tril mask softmax on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libgtms.so`` (built from ``csrc/`` by ``build.py``). The binding
only marshals arguments: every step of the operation runs in the library's HIP kernels,
on the caller's current torch stream. Torch provides device memory and streams.

    y = forward(x, seq_lens, scale)      # x: [B, M, S, S] f32/f16/bf16 on the GPU
    dx = backward(y, dy, seq_lens, scale)
    y = forward_band(x, seq_lens, lo, hi, scale)   # kept: lo <= c - r <= hi
    y = forward_masked(x, mask, seq_lens, scale)   # kept: mask != 0 ([B|1, M|1, S|1, S])
    dx = backward_band(...), backward_masked(...)  # their gradients
    o = attention(q, k, v, seq_lens, scale)        # fused: q, k, v [B, M, S, D] f16/bf16

There is no fallback: if the library is missing or cannot load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GTMS_LIBRARY names another build of the same library (the CPU sanitizer test loads one whose
# host code is built with AddressSanitizer); by default the in-tree build
LIB_PATH = os.environ.get("GTMS_LIBRARY") or os.path.join(HERE, "libgtms.so")

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
    lib.gtms_forward_band.argtypes = [p, p, p, i64, i64, i64, i64, i64, f32, i32, p]
    lib.gtms_forward_band.restype = i32
    lib.gtms_forward_band_ex.argtypes = [p, p, p, i64, i64, i64, i64, i64, f32, i32, i32, u32, p]
    lib.gtms_forward_band_ex.restype = i32
    lib.gtms_forward_masked.argtypes = [p, p, p, i64, i64, i64, p, i64, i64, i64, f32, i32, p]
    lib.gtms_forward_masked.restype = i32
    lib.gtms_forward_masked_ex.argtypes = [p, p, p, i64, i64, i64, p, i64, i64, i64, f32, i32,
                                           i32, u32, p]
    lib.gtms_forward_masked_ex.restype = i32
    lib.gtms_backward_band.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, f32, i32, i32, u32, p]
    lib.gtms_backward_band.restype = i32
    lib.gtms_backward_masked.argtypes = [p, p, p, p, i64, i64, i64, p, i64, i64, i64, f32, i32,
                                         i32, u32, p]
    lib.gtms_backward_masked.restype = i32
    lib.gtms_attention_forward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, f32, i32, p]
    lib.gtms_attention_forward.restype = i32
    lib.gtms_attention_forward_ex.argtypes = [p, p, p, p, p, i64, i64, i64, i64, f32, i32, i32, p]
    lib.gtms_attention_forward_ex.restype = i32
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


# ------------------------------------------------------------------------- mask variants

def _lens_ptr(seq_lens, x):
    if seq_lens is None:
        return None
    _check_lens(seq_lens, x)
    return seq_lens.data_ptr()


def _out_like(out, x):
    import torch
    if out is None:
        return torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of the input's shape, dtype and device")
    return out


def mask_strides(mask, x):
    """Byte strides (b, m, r) of a uint8/bool mask that broadcasts to x's [B, M, S, S]:
    each leading dimension is 1 (broadcast, stride 0) or x's size; columns contiguous."""
    import torch
    if not mask.is_cuda or mask.device != x.device:
        raise ValueError("mask must be on x's device")
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool (non-zero = kept)")
    if mask.dim() != 4 or mask.shape[3] != x.shape[3]:
        raise ValueError(f"mask must have shape [B|1, M|1, S|1, S], got {tuple(mask.shape)}")
    st = []
    for d in range(3):
        n = mask.shape[d]
        if n not in (1, x.shape[d]):
            raise ValueError(f"mask dimension {d} is {n}, expected 1 or {x.shape[d]}")
        st.append(0 if n == 1 else mask.stride(d))
    if mask.shape[3] > 1 and mask.stride(3) != 1:
        raise ValueError("mask columns must be contiguous")
    return st


def forward_band(x, seq_lens, lo: int, hi: int, scale: float = 1.0, out=None,
                 path: str = "auto", flags: int = 0):
    """Softmax over the band lo <= c - r <= hi of each row (and r, c below the valid
    length; seq_lens may be None: every length is S). Rows with nothing kept are zeros."""
    _check_scores(x)
    out = _out_like(out, x)
    B, M, S, _ = x.shape
    L = _load()
    with _on_device(x):
        if path == "auto" and flags == 0:
            st = L.gtms_forward_band(x.data_ptr(), out.data_ptr(), _lens_ptr(seq_lens, x), B, M,
                                     S, int(lo), int(hi), float(scale), _dtype_code(x),
                                     _stream_of(x))
        else:
            st = L.gtms_forward_band_ex(x.data_ptr(), out.data_ptr(), _lens_ptr(seq_lens, x), B,
                                        M, S, int(lo), int(hi), float(scale), _dtype_code(x),
                                        PATHS[path], int(flags), _stream_of(x))
    _raise(st, "gtms_forward_band")
    return out


def forward_masked(x, mask, seq_lens=None, scale: float = 1.0, out=None, path: str = "auto",
                   flags: int = 0):
    """Softmax over the elements where ``mask`` (uint8/bool, [B|1, M|1, S|1, S], size-1 or
    stride-0 dimensions broadcast) is non-zero, and r, c below the valid length."""
    _check_scores(x)
    sb, sm, sr = mask_strides(mask, x)
    out = _out_like(out, x)
    B, M, S, _ = x.shape
    L = _load()
    with _on_device(x):
        if path == "auto" and flags == 0:
            st = L.gtms_forward_masked(x.data_ptr(), out.data_ptr(), mask.data_ptr(), sb, sm, sr,
                                       _lens_ptr(seq_lens, x), B, M, S, float(scale),
                                       _dtype_code(x), _stream_of(x))
        else:
            st = L.gtms_forward_masked_ex(x.data_ptr(), out.data_ptr(), mask.data_ptr(), sb, sm,
                                          sr, _lens_ptr(seq_lens, x), B, M, S, float(scale),
                                          _dtype_code(x), PATHS[path], int(flags),
                                          _stream_of(x))
    _raise(st, "gtms_forward_masked")
    return out


def _check_grad_pair(y, dy):
    _check_scores(y, "y")
    _check_scores(dy, "dy")
    if dy.shape != y.shape or dy.dtype != y.dtype or dy.device != y.device:
        raise ValueError("dy must match y in shape, dtype and device")


def backward_band(y, dy, seq_lens, lo: int, hi: int, scale: float = 1.0, out=None,
                  path: str = "auto", flags: int = 0):
    """Gradient of forward_band with respect to its input (out may be dy, not y)."""
    _check_grad_pair(y, dy)
    out = _out_like(out, y)
    B, M, S, _ = y.shape
    L = _load()
    with _on_device(y):
        st = L.gtms_backward_band(y.data_ptr(), dy.data_ptr(), out.data_ptr(),
                                  _lens_ptr(seq_lens, y), B, M, S, int(lo), int(hi),
                                  float(scale), _dtype_code(y), PATHS[path], int(flags),
                                  _stream_of(y))
    _raise(st, "gtms_backward_band")
    return out


def backward_masked(y, dy, mask, seq_lens=None, scale: float = 1.0, out=None,
                    path: str = "auto", flags: int = 0):
    """Gradient of forward_masked with respect to its input (out may be dy, not y)."""
    _check_grad_pair(y, dy)
    sb, sm, sr = mask_strides(mask, y)
    out = _out_like(out, y)
    B, M, S, _ = y.shape
    L = _load()
    with _on_device(y):
        st = L.gtms_backward_masked(y.data_ptr(), dy.data_ptr(), out.data_ptr(), mask.data_ptr(),
                                    sb, sm, sr, _lens_ptr(seq_lens, y), B, M, S, float(scale),
                                    _dtype_code(y), PATHS[path], int(flags), _stream_of(y))
    _raise(st, "gtms_backward_masked")
    return out


ATTN_SPLITS = {"auto": 0, "off": 1, "on": 2}


def attention(q, k, v, seq_lens, scale: float | None = None, out=None, split: str = "auto"):
    """Fused attention with the grouped tril mask: for query row r < L_b,
    out[r] = sum_{c <= r} softmax_c(scale * q[r].k[c]) v[c]; rows r >= L_b are zero.
    q, k, v: [B, M, S, D] float16 or bfloat16 GPU tensors, D = 64 or 128. The default scale
    is 1 / sqrt(D). split: "auto", "off" or "on", the key split of each query tile over two
    groups of wavefronts (head size 64; see gtms_attention_forward_ex)."""
    import math
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, M, S, D] GPU tensor")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k and v must match in shape, dtype and device")
    _check_lens(seq_lens, q)
    B, M, S, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    L = _load()
    with _on_device(q):
        st = L.gtms_attention_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         out.data_ptr(), seq_lens.data_ptr(), B, M, S, D, sc,
                                         _dtype_code(q), ATTN_SPLITS[split], _stream_of(q))
    _raise(st, "gtms_attention_forward_ex")
    return out
