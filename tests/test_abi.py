"""The C ABI without a GPU: the library loads, exports every declared symbol, and rejects
bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gtms_\w+)\s*\(", text, re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    import variable_length_causal_amd as g
    return g.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "gtms_forward" in names and "gtms_status_string" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings(lib):
    import variable_length_causal_amd as g
    for code in range(6):
        assert g.status_string(code)
    assert g.status_string(99) == "unknown status"
    assert g.version() >= 100


FAKE = 1 << 36  # a well-aligned pointer value that is never dereferenced


def fwd(lib, x=FAKE, y=FAKE * 4, sl=FAKE * 8, B=1, M=1, S=8, scale=1.0, dtype=0):
    return lib.gtms_forward(x, y, sl, B, M, S, scale, dtype, None)


def test_argument_checks(lib):
    assert fwd(lib, dtype=3) == 2                        # unknown element type
    assert fwd(lib, dtype=-1) == 2
    assert fwd(lib, B=-1) == 1                           # negative size
    assert fwd(lib, S=-4) == 1
    assert fwd(lib, x=0) == 1                            # null pointers
    assert fwd(lib, y=0) == 1
    assert fwd(lib, sl=0) == 1
    assert fwd(lib, B=0, x=0, y=0, sl=0) == 0            # empty: valid no-op
    assert fwd(lib, S=0, x=0, y=0, sl=0) == 0
    assert fwd(lib, B=1 << 40, M=1 << 20, S=1 << 10) == 1  # B*M*S*S overflows
    assert fwd(lib, S=(1 << 24) + 1) == 1                # beyond GTMS_MAX_S
    assert fwd(lib, x=FAKE + 2, dtype=0) == 3            # misaligned binary32
    assert fwd(lib, y=FAKE * 4 + 1, dtype=1) == 3        # misaligned binary16
    assert fwd(lib, sl=FAKE * 8 + 2) == 3                # misaligned lengths
    # partial overlap of in and out (identical pointers are allowed: in place)
    assert fwd(lib, x=FAKE, y=FAKE + 64, S=8) == 1


def test_path_checks(lib):
    def ex(path, S=8, dtype=0, flags=0):
        return lib.gtms_forward_ex(FAKE, FAKE * 4, FAKE * 8, 1, 1, S, 1.0, dtype, path, flags,
                                   None)
    assert ex(7) == 5 and ex(-1) == 5                    # unknown path
    assert ex(1, S=4100, dtype=0) == 5                   # row too long for the wave path
    assert ex(1, S=4088, dtype=0) == 5                   # ... once the line slack is added
    assert ex(1, S=8200, dtype=1) == 5
    assert ex(1, S=1025, dtype=0) == 5                   # unaligned rows: one element a slot
    assert ex(2, S=65540, dtype=0) == 5                  # ... and for the block path
    assert ex(2, S=16385, dtype=2) == 5


def test_backward_argument_checks(lib):
    Y, G, DX, SL = FAKE, FAKE * 4, FAKE * 16, FAKE * 64

    def bwd(y=Y, g=G, dx=DX, sl=SL, B=1, M=1, S=8, dtype=0):
        return lib.gtms_backward(y, g, dx, sl, B, M, S, 0.5, dtype, None)
    assert bwd(dtype=5) == 2
    assert bwd(g=0) == 1                                 # no upstream gradient
    assert bwd(dx=Y) == 1                                # dx may not replace y
    assert bwd(dx=Y + 64) == 1                           # ... nor overlap it
    assert bwd(dx=G + 64) == 1                           # partial overlap with dy
    assert bwd(g=G + 2) == 3                             # misaligned dy
    assert bwd(B=0, y=0, g=0, dx=0, sl=0) == 0
    assert lib.gtms_backward_ex(Y, G, DX, SL, 1, 1, 4100, 1.0, 0, 1, 0, None) == 5


def test_variant_argument_checks(lib):
    X, Y, SL, MK = FAKE, FAKE * 4, FAKE * 8, FAKE * 16

    def band(x=X, y=Y, sl=SL, S=8, lo=-8, hi=0, dtype=0, path=0):
        return lib.gtms_forward_band_ex(x, y, sl, 1, 1, S, lo, hi, 1.0, dtype, path, 0, None)

    def masked(x=X, y=Y, mk=MK, sb=0, sm=0, sr=8, sl=SL, B=1, S=8, dtype=0, path=0):
        return lib.gtms_forward_masked_ex(x, y, mk, sb, sm, sr, sl, B, 1, S, 1.0, dtype, path,
                                          0, None)
    assert band(dtype=4) == 2
    assert band(x=0) == 1
    assert band(x=X + 2) == 3
    assert band(x=X, y=X + 64) == 1                      # partial overlap
    # no lengths is valid for the variants: the call gets past the argument checks and is
    # only stopped by the unknown path
    assert band(sl=0, path=9) == 5
    assert masked(sl=0, path=9) == 5
    assert band(lo=5, hi=-5, path=9) == 5                # an empty band is a valid request
    assert masked(mk=0) == 1                             # no mask
    assert masked(sr=-8) == 1                            # negative stride
    assert masked(sb=-1, B=0, x=0, y=0, mk=0) == 1
    assert masked(B=0, x=0, y=0, mk=0, sl=0) == 0        # empty: no-op
    assert masked(dtype=2, x=X + 1) == 3
    assert lib.gtms_forward_band(0, 0, 0, 0, 4, 4, 0, 0, 1.0, 0, None) == 0
    assert lib.gtms_forward_masked(0, 0, 0, 0, 0, 4, 0, 0, 4, 4, 1.0, 0, None) == 0
    G, DX = FAKE * 32, FAKE * 64
    assert lib.gtms_backward_band(X, G, X, SL, 1, 1, 8, -8, 0, 1.0, 0, 0, 0, None) == 1
    assert lib.gtms_backward_band(X, 0, DX, SL, 1, 1, 8, -8, 0, 1.0, 0, 0, 0, None) == 1
    assert lib.gtms_backward_band(X, G, DX, 0, 1, 1, 8, -8, 0, 1.0, 0, 9, 0, None) == 5
    assert lib.gtms_backward_masked(X, G, DX, 0, 0, 0, 8, SL, 1, 1, 8, 1.0, 0, 0, 0, None) == 1
    assert lib.gtms_backward_masked(X, G, DX, MK, 0, -1, 8, SL, 1, 1, 8, 1.0, 0, 0, 0, None) == 1
    assert lib.gtms_backward_masked(X, G, DX, MK, 0, 0, 8, 0, 1, 1, 8, 1.0, 0, 9, 0, None) == 5


def test_attention_argument_checks(lib):
    """Every call here is rejected (or is a no-op) before anything reaches the GPU."""
    Q, K, V, O, SL = FAKE, FAKE * 2, FAKE * 4, FAKE * 8, FAKE * 16

    def attn(q=Q, k=K, v=V, o=O, sl=SL, B=1, M=1, S=8, D=64, dtype=2, split=0):
        return lib.gtms_attention_forward_ex(q, k, v, o, sl, B, M, S, D, 0.125, dtype, split,
                                             None)
    assert attn(dtype=0) == 2                            # binary32 is not an attention type
    assert attn(split=3) == 5 and attn(split=-1) == 5    # unknown work split
    assert attn(B=0, q=0, k=0, v=0, o=0, sl=0) == 0      # empty: no-op, nothing checked
    assert attn(D=96) == 5                               # head sizes 64 and 128 only
    assert attn(q=0) == 1 and attn(sl=0) == 1            # null pointers
    assert attn(v=V + 8) == 3                            # 16-byte alignment
    assert attn(o=Q + 64) == 1                           # out overlaps q
    assert attn(S=(1 << 24) - 64) == 1                   # one head's offsets past 2^31
    assert attn(B=-1) == 1
    assert lib.gtms_attention_forward(Q, K, V, O, SL, 1, 1, 8, 64, 0.125, 0, None) == 2
