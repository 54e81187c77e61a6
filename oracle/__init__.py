"""Oracle for the grouped tril mask softmax: TEST INFRASTRUCTURE ONLY.

Python access to the plain fp64 C oracle in ``gtms_oracle.c``. Only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package. The GPU product package never imports it, and it imports nothing of the product.

Arrays cross this module as numpy arrays holding the raw element bits: ``float32`` for
binary32, ``uint16`` for binary16 and bfloat16 (``dtype`` code 0, 1, 2, the same codes the
C oracle uses).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gtms_oracle.c")
LIB = os.path.join(HERE, "liboracle_gtms.so")

F32, F16, BF16 = 0, 1, 2
STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

GCC_FLAGS = ["-O2", "-std=gnu99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    subprocess.run(["gcc", *GCC_FLAGS, f"-I{HERE}", src, "-o", out + ".tmp", "-lm"],
                   check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype not in STORAGE:
        raise ValueError(f"unknown element type code {dtype}")
    if x.dtype != STORAGE[dtype]:
        raise TypeError(f"dtype code {dtype} expects storage {STORAGE[dtype]}, got {x.dtype}")
    return np.ascontiguousarray(x)


def _lens(seq_lens, n: int) -> np.ndarray:
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if sl.shape != (n,):
        raise ValueError(f"expected {n} lengths, got shape {sl.shape}")
    return sl


def _nptr(a):
    return None if a is None else _ptr(a)


def mask_layout(mask: np.ndarray, B: int, M: int, S: int):
    """A contiguous uint8 copy of a [B|1, M|1, S|1, S] mask and its byte strides for b, m and
    r (zero where the dimension broadcasts)."""
    mk = np.ascontiguousarray(np.asarray(mask).astype(np.uint8))
    if mk.ndim != 4 or mk.shape[3] != S or any(d not in (1, n) for d, n in
                                               zip(mk.shape[:3], (B, M, S))):
        raise ValueError(f"mask shape {mk.shape} does not broadcast to [{B}, {M}, {S}, {S}]")
    st = [mk.strides[i] if mk.shape[i] > 1 else 0 for i in range(3)]
    return mk, st[0], st[1], st[2]


class Oracle:
    """One loaded copy of the C oracle (the default one, or a test build of it)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        for name in ("gtms_oracle_f64", "gtms_oracle"):
            fn = getattr(lib, name)
            fn.argtypes = [p, p, p, i64, i64, i64, f32, i32]
            fn.restype = i32
        lib.gtms_oracle_rows_f64.argtypes = [p, p, p, p, i64, i64, f32, i32]
        lib.gtms_oracle_rows_f64.restype = i32
        lib.gtms_oracle_backward_f64.argtypes = [p, p, p, p, i64, i64, i64, f32, i32]
        lib.gtms_oracle_backward_f64.restype = i32
        lib.gtms_oracle_backward_rows_f64.argtypes = [p, p, p, p, p, i64, i64, f32, i32]
        lib.gtms_oracle_backward_rows_f64.restype = i32
        lib.gtms_oracle_band_f64.argtypes = [p, p, p, i64, i64, i64, i64, i64, f32, i32]
        lib.gtms_oracle_band_f64.restype = i32
        lib.gtms_oracle_band_backward_f64.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, f32,
                                                      i32]
        lib.gtms_oracle_band_backward_f64.restype = i32
        lib.gtms_oracle_masked_f64.argtypes = [p, p, p, i64, i64, i64, p, i64, i64, i64, f32,
                                               i32]
        lib.gtms_oracle_masked_f64.restype = i32
        lib.gtms_oracle_masked_backward_f64.argtypes = [p, p, p, p, i64, i64, i64, p, i64, i64,
                                                        i64, f32, i32]
        lib.gtms_oracle_masked_backward_f64.restype = i32
        lib.gtms_oracle_attention_f64.argtypes = [p, p, p, p, p, i64, i64, i64, i64, f32, i32]
        lib.gtms_oracle_attention_f64.restype = i32
        lib.gtms_oracle_attention_row_f64.argtypes = [p, p, p, p, i64, ctypes.c_int32, i64, i64,
                                                      f32, i32]
        lib.gtms_oracle_attention_row_f64.restype = i32
        lib.gtms_oracle_decode.argtypes = [ctypes.c_uint32, i32]
        lib.gtms_oracle_decode.restype = ctypes.c_double
        lib.gtms_oracle_encode.argtypes = [ctypes.c_double, i32]
        lib.gtms_oracle_encode.restype = ctypes.c_uint32
        self.lib = lib
        self.path = path

    @staticmethod
    def _status(st: int, what: str):
        if st != 0:
            raise RuntimeError(f"{what}: oracle status {st}")

    def softmax_f64(self, x: np.ndarray, seq_lens, scale: float = 1.0,
                    dtype: int = F32) -> np.ndarray:
        """fp64 results for x of shape [B, M, S, S] (raw element storage)."""
        x = _check(x, dtype)
        B, M, S, S2 = x.shape
        assert S == S2
        sl = _lens(seq_lens, B)
        y = np.empty(x.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_f64(_ptr(x), _ptr(y), _ptr(sl), B, M, S, scale,
                                              dtype), "gtms_oracle_f64")
        return y

    def softmax(self, x: np.ndarray, seq_lens, scale: float = 1.0,
                dtype: int = F32) -> np.ndarray:
        """Results rounded to nearest-even into the element type (same storage as x)."""
        x = _check(x, dtype)
        B, M, S, S2 = x.shape
        assert S == S2
        sl = _lens(seq_lens, B)
        y = np.empty_like(x)
        self._status(self.lib.gtms_oracle(_ptr(x), _ptr(y), _ptr(sl), B, M, S, scale, dtype),
                     "gtms_oracle")
        return y

    def softmax_rows_f64(self, rows: np.ndarray, row_index, seq_len, scale: float = 1.0,
                         dtype: int = F32) -> np.ndarray:
        """fp64 results for independent rows: rows[i] (length S) is row row_index[i] of a
        plane whose batch has raw valid length seq_len[i]."""
        rows = _check(rows, dtype)
        n, S = rows.shape
        ri = np.ascontiguousarray(np.asarray(row_index, dtype=np.int64))
        sl = _lens(seq_len, n)
        assert ri.shape == (n,)
        y = np.empty((n, S), dtype=np.float64)
        self._status(self.lib.gtms_oracle_rows_f64(_ptr(rows), _ptr(y), _ptr(ri), _ptr(sl),
                                                   n, S, scale, dtype),
                     "gtms_oracle_rows_f64")
        return y

    def backward_f64(self, y: np.ndarray, dy: np.ndarray, seq_lens, scale: float = 1.0,
                     dtype: int = F32) -> np.ndarray:
        """fp64 gradient with respect to the input, given the output y and upstream dy."""
        y = _check(y, dtype)
        dy = _check(dy, dtype)
        B, M, S, S2 = y.shape
        assert S == S2 and dy.shape == y.shape
        sl = _lens(seq_lens, B)
        dx = np.empty(y.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_backward_f64(_ptr(y), _ptr(dy), _ptr(dx), _ptr(sl),
                                                       B, M, S, scale, dtype),
                     "gtms_oracle_backward_f64")
        return dx

    def backward_rows_f64(self, y_rows: np.ndarray, dy_rows: np.ndarray, row_index, seq_len,
                          scale: float = 1.0, dtype: int = F32) -> np.ndarray:
        """fp64 gradients for independent rows: y_rows[i] and dy_rows[i] (length S) are row
        row_index[i] of a plane whose batch has raw valid length seq_len[i]."""
        y_rows = _check(y_rows, dtype)
        dy_rows = _check(dy_rows, dtype)
        n, S = y_rows.shape
        assert dy_rows.shape == (n, S)
        ri = np.ascontiguousarray(np.asarray(row_index, dtype=np.int64))
        sl = _lens(seq_len, n)
        assert ri.shape == (n,)
        dx = np.empty((n, S), dtype=np.float64)
        self._status(self.lib.gtms_oracle_backward_rows_f64(_ptr(y_rows), _ptr(dy_rows),
                                                            _ptr(dx), _ptr(ri), _ptr(sl), n, S,
                                                            scale, dtype),
                     "gtms_oracle_backward_rows_f64")
        return dx

    # ---- mask variants: seq_lens may be None (every valid length is S)

    def softmax_band_f64(self, x: np.ndarray, seq_lens, lo: int, hi: int, scale: float = 1.0,
                         dtype: int = F32) -> np.ndarray:
        """fp64 results of the band variant: (r, c) kept when lo <= c - r <= hi (and r, c
        below the valid length)."""
        x = _check(x, dtype)
        B, M, S, S2 = x.shape
        assert S == S2
        sl = None if seq_lens is None else _lens(seq_lens, B)
        y = np.empty(x.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_band_f64(_ptr(x), _ptr(y), _nptr(sl), B, M, S,
                                                   int(lo), int(hi), scale, dtype),
                     "gtms_oracle_band_f64")
        return y

    def band_backward_f64(self, y: np.ndarray, dy: np.ndarray, seq_lens, lo: int, hi: int,
                          scale: float = 1.0, dtype: int = F32) -> np.ndarray:
        y = _check(y, dtype)
        dy = _check(dy, dtype)
        B, M, S, S2 = y.shape
        assert S == S2 and dy.shape == y.shape
        sl = None if seq_lens is None else _lens(seq_lens, B)
        dx = np.empty(y.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_band_backward_f64(_ptr(y), _ptr(dy), _ptr(dx),
                                                            _nptr(sl), B, M, S, int(lo),
                                                            int(hi), scale, dtype),
                     "gtms_oracle_band_backward_f64")
        return dx

    def softmax_masked_f64(self, x: np.ndarray, mask: np.ndarray, seq_lens,
                           scale: float = 1.0, dtype: int = F32) -> np.ndarray:
        """fp64 results of the explicit-mask variant: mask has shape [B|1, M|1, S|1, S]
        (a size-1 dimension broadcasts); an element is kept where the mask is non-zero."""
        x = _check(x, dtype)
        B, M, S, S2 = x.shape
        assert S == S2
        mk, sb, sm, sr = mask_layout(mask, B, M, S)
        sl = None if seq_lens is None else _lens(seq_lens, B)
        y = np.empty(x.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_masked_f64(_ptr(x), _ptr(y), _ptr(mk), sb, sm, sr,
                                                     _nptr(sl), B, M, S, scale, dtype),
                     "gtms_oracle_masked_f64")
        return y

    def masked_backward_f64(self, y: np.ndarray, dy: np.ndarray, mask: np.ndarray, seq_lens,
                            scale: float = 1.0, dtype: int = F32) -> np.ndarray:
        y = _check(y, dtype)
        dy = _check(dy, dtype)
        B, M, S, S2 = y.shape
        assert S == S2 and dy.shape == y.shape
        mk, sb, sm, sr = mask_layout(mask, B, M, S)
        sl = None if seq_lens is None else _lens(seq_lens, B)
        dx = np.empty(y.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_masked_backward_f64(_ptr(y), _ptr(dy), _ptr(dx),
                                                              _ptr(mk), sb, sm, sr, _nptr(sl),
                                                              B, M, S, scale, dtype),
                     "gtms_oracle_masked_backward_f64")
        return dx

    def attention_f64(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens,
                      scale: float, dtype: int = F32) -> np.ndarray:
        """fp64 attention output [B, M, S, D] with the grouped tril mask (raw storage in)."""
        q, k, v = _check(q, dtype), _check(k, dtype), _check(v, dtype)
        B, M, S, D = q.shape
        assert k.shape == q.shape and v.shape == q.shape
        sl = _lens(seq_lens, B)
        o = np.empty(q.shape, dtype=np.float64)
        self._status(self.lib.gtms_oracle_attention_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                                        _ptr(sl), B, M, S, D, scale, dtype),
                     "gtms_oracle_attention_f64")
        return o

    def attention_row_f64(self, q_head: np.ndarray, k_head: np.ndarray, v_head: np.ndarray,
                          r: int, seq_len: int, scale: float, dtype: int = F32) -> np.ndarray:
        """fp64 attention output of query row r of one head ([S, D] raw storage each)."""
        q, k, v = _check(q_head, dtype), _check(k_head, dtype), _check(v_head, dtype)
        S, D = q.shape
        o = np.empty(D, dtype=np.float64)
        self._status(self.lib.gtms_oracle_attention_row_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                                            int(r), int(seq_len), S, D, scale,
                                                            dtype),
                     "gtms_oracle_attention_row_f64")
        return o

    def decode(self, bits: int, dtype: int) -> float:
        return self.lib.gtms_oracle_decode(int(bits), dtype)

    def encode(self, v: float, dtype: int) -> int:
        return int(self.lib.gtms_oracle_encode(float(v), dtype))

    def decode_array(self, x: np.ndarray, dtype: int) -> np.ndarray:
        """Exact fp64 values of raw element storage, through the oracle's own codec."""
        x = _check(x, dtype)
        flat = x.view(np.uint32) if dtype == F32 else x
        out = np.array([self.lib.gtms_oracle_decode(int(b), dtype) for b in flat.reshape(-1)],
                       dtype=np.float64)
        return out.reshape(x.shape)


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``gtms_oracle.c`` (rebuilt when the source is newer), or the
    build named by the environment variable GTMS_ORACLE_LIB (the sanitizer test runs the pins
    against an AddressSanitizer / UndefinedBehaviorSanitizer build that way)."""
    global _default
    if _default is None:
        override = os.environ.get("GTMS_ORACLE_LIB")
        if override:
            _default = Oracle(override)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            _default = Oracle(LIB)
    return _default


def softmax_f64(*a, **k):
    return default().softmax_f64(*a, **k)


def softmax(*a, **k):
    return default().softmax(*a, **k)


def softmax_rows_f64(*a, **k):
    return default().softmax_rows_f64(*a, **k)


def backward_f64(*a, **k):
    return default().backward_f64(*a, **k)


def backward_rows_f64(*a, **k):
    return default().backward_rows_f64(*a, **k)


def decode(bits: int, dtype: int) -> float:
    return default().decode(bits, dtype)


def encode(v: float, dtype: int) -> int:
    return default().encode(v, dtype)


def softmax_band_f64(*a, **k):
    return default().softmax_band_f64(*a, **k)


def band_backward_f64(*a, **k):
    return default().band_backward_f64(*a, **k)


def softmax_masked_f64(*a, **k):
    return default().softmax_masked_f64(*a, **k)


def masked_backward_f64(*a, **k):
    return default().masked_backward_f64(*a, **k)


def attention_f64(*a, **k):
    return default().attention_f64(*a, **k)


def attention_row_f64(*a, **k):
    return default().attention_row_f64(*a, **k)
