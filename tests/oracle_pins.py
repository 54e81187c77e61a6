"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the oracle
breaks the fact. ``test_oracle_pins.py`` runs them on the oracle; ``test_oracle_mutations.py``
runs them on deliberately broken builds of it, to show that each plausible mistake is caught.

Sources of the facts:
  * page "Fused grouped tril mask softmax" (github aoxy/Attention-Mask-Optimization README):
    the masks and the output printed for its worked example (``golden/``), and the
    operator-behaviour listing (masked_fill with the most negative value, then softmax);
  * page "ops(8) self-attention CUDA (下)", section 2.1: the softmax derivative; sections 1-2:
    attention as scores, row softmax and weighted sum of values;
  * page "优化ScaledMaskSoftmax算子", sections 2.1, 4.1 and 6: the mask variants (minus
    infinity before the softmax, zero rows when every element is masked, masks built with
    tril, broadcast per-task masks, per-sample length masks);
  * mathematics: closed forms of the softmax, shift invariance, finite differences;
  * libraries: numpy's binary16 and binary32 conversions, torch's softmax in float64,
    torch's exact bfloat16 widening.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

F32, F16, BF16 = 0, 1, 2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- fixtures

def _read_blocks(name: str) -> np.ndarray:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([float(t) for t in line.split()])
    return np.asarray(rows)


def printed_masks() -> np.ndarray:
    """bool [3, 5, 5], True = masked, for lengths 3, 4, 5 (README worked example)."""
    return _read_blocks("page1_masks_S5.txt").reshape(3, 5, 5).astype(bool)


def printed_output() -> np.ndarray:
    """float [3, 2, 5, 5], the README's printed output (4 decimals)."""
    return _read_blocks("page1_output_S5.txt").reshape(3, 2, 5, 5)


def _bits_of(storage: np.ndarray, dtype: int) -> np.ndarray:
    return storage.view(np.uint32) if dtype == F32 else storage.view(np.uint16)


def _one_bits(dtype: int) -> int:
    return {F32: 0x3F800000, F16: 0x3C00, BF16: 0x3F80}[dtype]


def _storage(x64: np.ndarray, dtype: int) -> np.ndarray:
    """Element storage of values that are exactly representable in every element type."""
    if dtype == F32:
        return x64.astype(np.float32)
    if dtype == F16:
        h = x64.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), x64, equal_nan=True)
        return h.view(np.uint16)
    f = x64.astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64),
                          x64, equal_nan=True)
    return b


def _grid_values(rng, shape, lo=-4.0, hi=4.0, step=1 / 16):
    """Values on a coarse grid: exact in binary32, binary16 and bfloat16 alike."""
    n = int(round((hi - lo) / step))
    return lo + step * rng.integers(0, n + 1, size=shape).astype(np.float64)


def _kept(r, c, L):
    return r < L and c < L and c <= r


# ----------------------------------------------------------------------------- pins

def pin_printed_masks(orc):
    """The kept set equals the complement of the README's three printed masks."""
    masks = printed_masks()
    rng = np.random.default_rng(11)
    x = rng.uniform(-2.0, 2.0, size=(3, 2, 5, 5)).astype(np.float32)
    y = orc.softmax_f64(x, [3, 4, 5], 1.0, F32)
    for b in range(3):
        for m in range(2):
            assert np.array_equal(y[b, m] != 0.0, ~masks[b]), (b, m)


def pin_printed_output(orc):
    """Feeding ln(p) of the README's printed output gives back p / sum(p) on each kept row
    (the softmax of a log is the normalised argument) and so the printed values within
    their 4-decimal rounding; masked cells hold arbitrary values and do not matter."""
    P = printed_output()
    masks = printed_masks()
    rng = np.random.default_rng(12)
    x = rng.normal(0.0, 3.0, size=P.shape)
    for b in range(3):
        for m in range(2):
            kept = ~masks[b]
            x[b, m][kept] = np.log(P[b, m][kept])
    x32 = x.astype(np.float32)
    y = orc.softmax_f64(x32, [3, 4, 5], 1.0, F32)
    for b in range(3):
        for m in range(2):
            kept = ~masks[b]
            assert np.all(y[b, m][~kept] == 0.0)
            for r in range(5):
                ks = kept[r]
                if not ks.any():
                    continue
                p = np.exp(x32[b, m, r][ks].astype(np.float64))
                assert np.allclose(y[b, m, r][ks], p / p.sum(), rtol=1e-13, atol=0), (b, m, r)
                assert np.all(np.abs(y[b, m, r][ks] - P[b, m, r][ks]) <= 3e-4), (b, m, r)


def pin_row0(orc):
    """Row 0 of a batch with L >= 1 is [1, 0, ..., 0] exactly, in fp64 and every type."""
    rng = np.random.default_rng(13)
    x64 = _grid_values(rng, (3, 2, 9, 9))
    for dtype in (F32, F16, BF16):
        xs = _storage(x64, dtype)
        y = orc.softmax_f64(xs, [1, 5, 9], 0.75, dtype)
        yr = _bits_of(orc.softmax(xs, [1, 5, 9], 0.75, dtype), dtype)
        for b in range(3):
            for m in range(2):
                assert y[b, m, 0, 0] == 1.0 and np.all(y[b, m, 0, 1:] == 0.0)
                assert yr[b, m, 0, 0] == _one_bits(dtype) and np.all(yr[b, m, 0, 1:] == 0)


def pin_row_sums(orc):
    """Every kept row sums to 1 (within fp64 rounding); padded rows sum to 0."""
    rng = np.random.default_rng(14)
    x = rng.normal(0.0, 2.0, size=(2, 3, 37, 37)).astype(np.float32)
    lens = [37, 20]
    y = orc.softmax_f64(x, lens, 0.7, F32)
    sums = y.sum(axis=-1)
    for b, L in enumerate(lens):
        assert np.all(np.abs(sums[b, :, :L] - 1.0) <= 1e-12)
        assert np.all(sums[b, :, L:] == 0.0)


def pin_exact_zeros(orc):
    """Masked elements and padded rows are +0.0 exactly (bit pattern 0)."""
    rng = np.random.default_rng(15)
    x64 = _grid_values(rng, (3, 2, 11, 11))
    lens = [0, 6, 11]
    for dtype in (F32, F16, BF16):
        xs = _storage(x64, dtype)
        y = orc.softmax_f64(xs, lens, 1.0, dtype)
        yr = _bits_of(orc.softmax(xs, lens, 1.0, dtype), dtype)
        for b, L in enumerate(lens):
            for r in range(11):
                for c in range(11):
                    if not _kept(r, c, L):
                        assert y[b, :, r, c].view(np.uint64).tolist() == [0, 0]
                        assert yr[b, :, r, c].tolist() == [0, 0]


def _naive_row(z, r, L):
    """exp(z_c) / sum_k exp(z_k) over the kept columns, with no max subtraction."""
    S = len(z)
    out = [0.0] * S
    ks = [c for c in range(S) if _kept(r, c, L)]
    if ks:
        den = sum(math.exp(z[k]) for k in ks)
        for c in ks:
            out[c] = math.exp(z[c]) / den
    return out


def pin_brute_force(orc):
    """Tiny shapes, every length from -1 to S+1: matches (i) the naive formula without
    max subtraction in pure Python and (ii) torch.softmax in float64 over the row after
    masked_fill with -inf, as the README's listing does (with -inf for its fill value)."""
    import torch
    rng = np.random.default_rng(16)
    for S in range(1, 9):
        lens = list(range(-1, S + 2))
        B = len(lens)
        x = rng.uniform(-4.0, 4.0, size=(B, 2, S, S)).astype(np.float32)
        scale = 0.9
        y = orc.softmax_f64(x, lens, scale, F32)
        for b, L in enumerate(lens):
            for m in range(2):
                for r in range(S):
                    z = [float(np.float32(scale)) * float(v) for v in x[b, m, r]]
                    ref = _naive_row(z, r, L)
                    assert np.all(np.abs(y[b, m, r] - np.asarray(ref)) <= 1e-14), (S, L, m, r)
                if min(max(L, 0), S) > 0:
                    Lc = min(L, S)
                    zt = torch.from_numpy(x[b, m].astype(np.float64)) * float(np.float32(scale))
                    mask = torch.ones(S, S, dtype=torch.bool)
                    for r in range(S):
                        for c in range(S):
                            if _kept(r, c, Lc):
                                mask[r, c] = False
                    t = zt.masked_fill(mask, float("-inf"))[:Lc].softmax(-1).numpy()
                    assert np.allclose(y[b, m, :Lc], t, rtol=0, atol=1e-15), (S, L, m)
                    assert np.all(y[b, m, Lc:] == 0.0)


def pin_closed_forms(orc):
    """(i) scale 0 and (ii) constant rows give 1/(r+1); (iii) row 1 is the logistic
    function of the difference; (iv) a linear ramp z_c = c*t gives the normalised
    geometric sequence e^(ct) (e^t - 1) / (e^((r+1)t) - 1)."""
    rng = np.random.default_rng(17)
    S = 24
    x = rng.normal(0.0, 1.0, size=(2, 2, S, S)).astype(np.float32)
    y = orc.softmax_f64(x, [S, 13], 0.0, F32)
    const = np.full((2, 2, S, S), 1.75, dtype=np.float32)
    yc = orc.softmax_f64(const, [S, 13], 1.3, F32)
    for b, L in enumerate([S, 13]):
        for r in range(L):
            want = np.zeros(S)
            want[: r + 1] = 1.0 / (r + 1)
            for yy in (y, yc):
                assert np.all(np.abs(yy[b, :, r] - want) <= 1e-15), (b, r)
    # logistic on row 1
    z = orc.softmax_f64(x, [S, S], 1.0, F32)
    for b in range(2):
        for m in range(2):
            d = float(x[b, m, 1, 1]) - float(x[b, m, 1, 0])
            assert abs(z[b, m, 1, 0] - 1.0 / (1.0 + math.exp(d))) <= 1e-15
            assert abs(z[b, m, 1, 1] - 1.0 / (1.0 + math.exp(-d))) <= 1e-15
    # linear ramp
    ramp = np.broadcast_to(np.arange(S, dtype=np.float32), (1, 1, S, S)).copy()
    for t in (0.3, -0.45):
        yr = orc.softmax_f64(ramp, [S], t, F32)
        tt = float(np.float32(t))
        for r in range(S):
            c = np.arange(r + 1)
            want = np.exp(c * tt) * math.expm1(tt) / math.expm1((r + 1) * tt)
            assert np.allclose(yr[0, 0, r, : r + 1], want, rtol=1e-13, atol=0), (t, r)
            assert np.all(yr[0, 0, r, r + 1:] == 0.0)


def pin_shift_and_scale(orc):
    """Adding a constant to a row changes nothing (scale 1); softmax(2x) with scale 1
    equals softmax(x) with scale 2; scale -1 equals softmax of -x."""
    rng = np.random.default_rng(18)
    S = 19
    x64 = _grid_values(rng, (2, 2, S, S))
    shift = _grid_values(rng, (2, 2, S, 1), -8.0, 8.0)
    lens = [S, 7]
    y0 = orc.softmax_f64(x64.astype(np.float32), lens, 1.0, F32)
    y1 = orc.softmax_f64((x64 + shift).astype(np.float32), lens, 1.0, F32)
    assert np.all(np.abs(y0 - y1) <= 1e-14)
    y2 = orc.softmax_f64(x64.astype(np.float32), lens, 2.0, F32)
    y3 = orc.softmax_f64((2.0 * x64).astype(np.float32), lens, 1.0, F32)
    assert np.array_equal(y2, y3)
    y4 = orc.softmax_f64(x64.astype(np.float32), lens, -1.0, F32)
    y5 = orc.softmax_f64((-x64).astype(np.float32), lens, 1.0, F32)
    assert np.array_equal(y4, y5)


def pin_masked_poison(orc):
    """NaN and infinities in masked cells leave every output bit unchanged."""
    rng = np.random.default_rng(19)
    S = 13
    x64 = _grid_values(rng, (3, 2, S, S))
    lens = [S, 5, 0]
    for dtype in (F32, F16, BF16):
        clean = _storage(x64, dtype)
        ref = _bits_of(orc.softmax(clean, lens, 0.5, dtype), dtype)
        ref64 = orc.softmax_f64(clean, lens, 0.5, dtype)
        for poison in (np.nan, np.inf, -np.inf):
            p = x64.copy()
            for b, L in enumerate(lens):
                for r in range(S):
                    for c in range(S):
                        if not _kept(r, c, L):
                            p[b, :, r, c] = poison
            ps = _storage(p, dtype)
            assert np.array_equal(_bits_of(orc.softmax(ps, lens, 0.5, dtype), dtype), ref)
            assert np.array_equal(orc.softmax_f64(ps, lens, 0.5, dtype).view(np.uint64),
                                  ref64.view(np.uint64))


def pin_length_edges(orc):
    """L = 0 and L < 0: all zeros; L > S: identical to L = S; L = 1: only [0, 0] = 1."""
    rng = np.random.default_rng(20)
    S = 10
    x = rng.normal(size=(5, 2, S, S)).astype(np.float32)
    y = orc.softmax_f64(x, [0, -3, S + 4, S, 1], 1.0, F32)
    assert np.all(y[0].view(np.uint64) == 0) and np.all(y[1].view(np.uint64) == 0)
    assert np.array_equal(y[2], orc.softmax_f64(x[2:3], [S], 1.0, F32)[0])
    xs = x.copy()
    xs[2] = x[3]
    assert np.array_equal(orc.softmax_f64(xs, [0, -3, S + 4, S, 1], 1.0, F32)[2], y[3])
    one = np.zeros((2, S, S))
    one[:, 0, 0] = 1.0
    assert np.array_equal(y[4], one)


def _bf16_table():
    """All finite non-negative bfloat16 values (ascending) and their bits, by the exact
    widening bits << 16 done in numpy."""
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits


def _nearest_even(v: float, vals: np.ndarray, bits: np.ndarray, inf_bits: int) -> int:
    """Brute force round-to-nearest-even of v onto the sorted non-negative table, with
    exact rational comparisons; the step past the largest finite value is one spacing."""
    a = abs(v)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    i = int(np.searchsorted(vals, a))
    top_gap = Fraction(vals[-1]) - Fraction(vals[-2])
    candidates = []
    for j in (i - 1, i):
        if 0 <= j < len(vals):
            candidates.append((Fraction(vals[j]), int(bits[j])))
    candidates.append((Fraction(vals[-1]) + top_gap, inf_bits))
    fa = Fraction(a)
    best = min(abs(fa - c[0]) for c in candidates)
    ties = [c for c in candidates if abs(fa - c[0]) == best]
    if len(ties) > 1:
        ties = [c for c in ties if c[1] % 2 == 0]
    return sign | ties[0][1]


def pin_codec(orc):
    """Element codec: binary16 and binary32 against numpy; bfloat16 decoding against the
    exact widening and encoding against brute-force nearest-even over all values."""
    # binary16 decode: all patterns
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allh.view(np.float16).astype(np.float64)
    got = np.array([orc.decode(int(b), F16) for b in allh])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]),
                                                               np.signbit(ref[ok]))
    # bfloat16 decode: all patterns
    with np.errstate(invalid="ignore"):
        refb = (allh.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gotb = np.array([orc.decode(int(b), BF16) for b in allh])
    assert np.array_equal(np.isnan(gotb), np.isnan(refb))
    okb = ~np.isnan(refb)
    assert np.array_equal(gotb[okb], refb[okb])
    # encode: log-uniform magnitudes over every range, plus ties and near-ties
    rng = np.random.default_rng(21)
    mags = np.exp2(rng.uniform(-140.0, 130.0, size=3000))
    vals = np.concatenate([mags, -mags, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e300]])
    h = ref[ok & (ref > 0) & np.isfinite(ref)]
    h = np.unique(h)
    mids = (h[:-1] + h[1:]) / 2
    vals16 = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    with np.errstate(over="ignore"):
        want16 = vals16.astype(np.float16).view(np.uint16)
        want32 = vals.astype(np.float32).view(np.uint32)
    got16 = np.array([orc.encode(v, F16) for v in vals16], dtype=np.uint16)
    assert np.array_equal(got16, want16)
    got32 = np.array([orc.encode(v, F32) for v in vals], dtype=np.uint32)
    assert np.array_equal(got32, want32)
    tv, tb = _bf16_table()
    sel = vals[(np.abs(vals) < 3e38)][::3]
    bmid = (tv[1:2000] + tv[2:2001]) / 2
    bmid2 = (tv[16000:16600] + tv[16001:16601]) / 2
    for v in np.concatenate([sel, bmid, bmid2, np.nextafter(bmid2, 0), [3.4e38, 3.39e38]]):
        assert orc.encode(float(v), BF16) == _nearest_even(float(v), tv, tb, 0x7F80), v
    for dtype, nanmask in ((F32, 0x7F800000), (F16, 0x7C00), (BF16, 0x7F80)):
        nb = orc.encode(float("nan"), dtype)
        assert (nb & nanmask) == nanmask and (nb & ~nanmask & (nanmask - 1)) != 0


def pin_rounded_outputs(orc):
    """The rounded outputs are the fp64 results rounded to nearest-even: numpy's
    conversion for binary32 and binary16, brute force for bfloat16."""
    rng = np.random.default_rng(22)
    S = 33
    x = rng.normal(0.0, 2.0, size=(2, 2, S, S)).astype(np.float32)
    lens = [S, 17]
    y64 = orc.softmax_f64(x, lens, 0.6, F32)
    assert np.array_equal(orc.softmax(x, lens, 0.6, F32).view(np.uint32),
                          y64.astype(np.float32).view(np.uint32))
    xh = x.astype(np.float16).view(np.uint16)
    y64h = orc.softmax_f64(xh, lens, 0.6, F16)
    assert np.array_equal(orc.softmax(xh, lens, 0.6, F16),
                          y64h.astype(np.float16).view(np.uint16))
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y64b = orc.softmax_f64(xb, lens, 0.6, BF16)
    yb = orc.softmax(xb, lens, 0.6, BF16)
    tv, tb = _bf16_table()
    flat64, flatb = y64b.reshape(-1), yb.reshape(-1)
    for i in range(0, flat64.size, 7):
        assert int(flatb[i]) == _nearest_even(float(flat64[i]), tv, tb, 0x7F80)


def pin_rows_api(orc):
    """The row-sampling entry point gives the same bits as the full tensor."""
    rng = np.random.default_rng(23)
    S = 21
    x = rng.normal(size=(3, 2, S, S)).astype(np.float32)
    lens = np.array([S, 9, -1], dtype=np.int32)
    full = orc.softmax_f64(x, lens, 0.8, F32)
    idx = [(b, m, r) for b in range(3) for m in range(2) for r in range(S)]
    pick = [idx[i] for i in rng.choice(len(idx), size=40, replace=False)]
    rows = np.stack([x[b, m, r] for b, m, r in pick])
    got = orc.softmax_rows_f64(rows, [r for _, _, r in pick], [lens[b] for b, _, _ in pick],
                               0.8, F32)
    for i, (b, m, r) in enumerate(pick):
        assert np.array_equal(got[i], full[b, m, r])


def pin_backward(orc):
    """The backward equals (i) the softmax Jacobian-vector product written out from the
    derivative dy_i/dz_j = y_i (delta_ij - y_j), in pure Python, and (ii) central finite
    differences of the forward oracle; masked and padded positions get zero gradient."""
    rng = np.random.default_rng(24)
    S = 7
    lens = [S, 4, 0]
    scale = 0.8
    x64 = _grid_values(rng, (3, 2, S, S), -2.0, 2.0, 1 / 256)
    x = x64.astype(np.float32)
    y = orc.softmax(x, lens, scale, F32)              # forward output in binary32
    g = rng.normal(size=y.shape).astype(np.float32)   # upstream gradient
    dx = orc.backward_f64(y, g, lens, scale, F32)
    for b, L in enumerate(lens):
        for m in range(2):
            for r in range(S):
                ks = [c for c in range(S) if _kept(r, c, L)]
                for j in range(S):
                    if j not in ks:
                        assert dx[b, m, r, j] == 0.0
                        continue
                    jac = sum(float(g[b, m, r, i]) * float(y[b, m, r, i]) *
                              ((1.0 if i == j else 0.0) - float(y[b, m, r, j])) for i in ks)
                    assert abs(dx[b, m, r, j] - float(np.float32(scale)) * jac) <= 1e-14
    # finite differences of f(x) = sum(g * softmax(x)) in fp64, step exact in binary32
    h = 2.0 ** -10
    gd = g.astype(np.float64)
    for (b, m, r, j) in [(0, 0, 6, 2), (0, 1, 3, 3), (1, 0, 3, 0), (1, 1, 2, 1), (0, 0, 0, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[b, m, r, j] += np.float32(h)
        xm[b, m, r, j] -= np.float32(h)
        fp = float((gd * orc.softmax_f64(xp, lens, scale, F32)).sum())
        fm = float((gd * orc.softmax_f64(xm, lens, scale, F32)).sum())
        fd = (fp - fm) / (2 * h)
        assert abs(dx[b, m, r, j] - fd) <= 2e-5, (b, m, r, j, dx[b, m, r, j], fd)


def pin_backward_rows(orc):
    """The backward's row entry point gives the same bits as the full tensor; NaN and
    infinity outside a row's kept prefix change nothing; on rows of 3000 elements it agrees
    with central finite differences of the forward's row entry point."""
    rng = np.random.default_rng(25)
    S = 19
    lens = np.array([S, 8, -3], dtype=np.int32)
    y = rng.uniform(size=(3, 2, S, S)).astype(np.float32)
    g = rng.normal(size=(3, 2, S, S)).astype(np.float32)
    full = orc.backward_f64(y, g, lens, 0.7, F32)
    idx = [(b, m, r) for b in range(3) for m in range(2) for r in range(S)]
    pick = [idx[i] for i in rng.choice(len(idx), size=40, replace=False)]
    yr = np.stack([y[b, m, r] for b, m, r in pick])
    gr = np.stack([g[b, m, r] for b, m, r in pick])
    ri, li = [r for _, _, r in pick], [lens[b] for b, _, _ in pick]
    got = orc.backward_rows_f64(yr, gr, ri, li, 0.7, F32)
    for i, (b, m, r) in enumerate(pick):
        assert np.array_equal(got[i], full[b, m, r])
    for i, (b, m, r) in enumerate(pick):
        L = min(max(int(lens[b]), 0), S)
        off = np.array([not _kept(r, c, L) for c in range(S)])
        yr[i][off], gr[i][off] = np.float32("nan"), np.float32("inf")
    assert np.array_equal(orc.backward_rows_f64(yr, gr, ri, li, 0.7, F32), got)
    # long rows: f(x) = sum(g * softmax(x)), step exact in binary32
    S, L, scale, h = 3000, 2500, 0.8, 2.0 ** -10
    for r in (0, 1234, 2499):
        x = rng.normal(0.0, 2.0, size=(1, S)).astype(np.float32)
        g1 = rng.normal(size=(1, S)).astype(np.float32)
        y1 = orc.softmax_rows_f64(x, [r], [L], scale, F32).astype(np.float32)
        dx = orc.backward_rows_f64(y1, g1, [r], [L], scale, F32)[0]
        assert not dx[r + 1:].any()
        gd = g1.astype(np.float64)
        for j in sorted({0, r // 2, r}):
            xp, xm = x.copy(), x.copy()
            xp[0, j] += np.float32(h)
            xm[0, j] -= np.float32(h)
            fd = (float((gd * orc.softmax_rows_f64(xp, [r], [L], scale, F32)).sum()) -
                  float((gd * orc.softmax_rows_f64(xm, [r], [L], scale, F32)).sum())) / (2 * h)
            assert abs(dx[j] - fd) <= 1e-9 + 1e-5 * abs(fd), (r, j, dx[j], fd)


# ------------------------------------------------------------------------ mask variants
# The ScaledMaskSoftmax article ("优化ScaledMaskSoftmax算子") masks scores with minus infinity
# before the softmax (section 2.1), zeroes rows whose every element is masked (section
# 4.1), and in section 6 builds masks with tril for a local window, broadcasts per-task
# masks over the batch, and compares positions with per-sample lengths.

def _torch_masked_softmax(z, keep):
    """Reference in float64 with torch: masked_fill(-inf), softmax, rows without a kept
    element set to zero."""
    import torch
    t = torch.as_tensor(z, dtype=torch.float64).masked_fill(~keep, float("-inf"))
    y = t.softmax(-1)
    return torch.where(keep.any(-1, keepdim=True), y, torch.zeros_like(y)).numpy()


def _length_keep(S, L):
    import torch
    Lc = S if L is None else min(max(int(L), 0), S)
    i = torch.arange(S)
    return (i[:, None] < Lc) & (i[None, :] < Lc)


def _band_keep(S, lo, hi, L):
    """The band through torch's own triangle routines: tril(hi) keeps c - r <= hi and
    triu(lo) keeps c - r >= lo (tril(w) is the article's window mask)."""
    import torch
    ones = torch.ones(S, S)
    return (ones.tril(hi) * ones.triu(lo)).bool() & _length_keep(S, L)


def pin_band_brute_force(orc):
    """Band variant on tiny shapes, for many (lo, hi) and every length: matches torch's
    masked softmax over the band built by tril/triu, and the naive exp(z)/sum exp(z) in
    pure Python; masked elements are exactly +0."""
    rng = np.random.default_rng(31)
    for S in (1, 2, 3, 5, 8):
        lens = list(range(-1, S + 2))
        B = len(lens)
        x = rng.uniform(-4.0, 4.0, size=(B, 1, S, S)).astype(np.float32)
        scale = 0.7
        sc = float(np.float32(scale))
        for lo, hi in ((-S - 1, 0), (-2, 0), (0, 0), (-1, 1), (1, 3), (-S, S), (-3, -1),
                       (-(10 ** 12), 2), (2, 1)):
            y = orc.softmax_band_f64(x, lens, lo, hi, scale, F32)
            for b, L in enumerate(lens):
                keep = _band_keep(S, lo, hi, L)
                ref = _torch_masked_softmax(x[b, 0].astype(np.float64) * sc, keep)
                assert np.allclose(y[b, 0], ref, rtol=0, atol=1e-15), (S, lo, hi, L)
                assert np.all(y[b, 0][~keep.numpy()] == 0.0)
                assert not np.signbit(y[b, 0]).any()
                for r in range(S):
                    ks = [c for c in range(S) if keep[r, c]]
                    if ks:
                        den = sum(math.exp(sc * float(x[b, 0, r, c])) for c in ks)
                        for c in ks:
                            assert abs(y[b, 0, r, c] - math.exp(sc * float(x[b, 0, r, c])) / den) <= 1e-14
        y = orc.softmax_band_f64(x, None, -1, 0, scale, F32)   # no lengths: every L is S
        for b in range(B):
            ref = _torch_masked_softmax(x[b, 0].astype(np.float64) * sc, _band_keep(S, -1, 0, None))
            assert np.allclose(y[b, 0], ref, rtol=0, atol=1e-15)


def pin_band_closed_forms(orc):
    """(i) lo = hi = k: row r is one-hot at column r + k when that column is valid, else all
    zeros. (ii) scale 0: each kept element is 1 / (number kept in its row). (iii) the
    article's window tril(w) without lengths: row r keeps min(S, r + w + 1) columns.
    (iv) lo <= -S, hi >= S with lengths (the article's per-sample length mask, for rows and
    columns): each valid row is the plain softmax of its first L scores."""
    rng = np.random.default_rng(32)
    S = 9
    lens = [9, 5, 1, 0, 12]
    x = rng.normal(size=(5, 2, S, S)).astype(np.float32)
    for k in (-3, -1, 0, 2, 8, 9):
        y = orc.softmax_band_f64(x, lens, k, k, 1.3, F32)
        for b, L in enumerate(lens):
            Lc = min(L, S)
            for r in range(S):
                want = np.zeros(S)
                if r < Lc and 0 <= r + k < Lc:
                    want[r + k] = 1.0
                assert np.array_equal(y[b, :, r], np.broadcast_to(want, (2, S))), (k, L, r)
    for lo, hi in ((-2, 1), (-4, 0), (1, 5)):
        y = orc.softmax_band_f64(x, lens, lo, hi, 0.0, F32)
        for b, L in enumerate(lens):
            Lc = min(L, S)
            for r in range(S):
                c0, c1 = max(0, r + lo), min(Lc - 1, r + hi)
                n = c1 - c0 + 1 if r < Lc else 0
                for c in range(S):
                    want = 1.0 / n if n > 0 and c0 <= c <= c1 else 0.0
                    assert abs(y[b, 0, r, c] - want) <= 1e-15, (lo, hi, L, r, c)
    for w in (0, 1, 3):
        y = orc.softmax_band_f64(x, None, -(10 ** 9), w, 0.0, F32)
        for r in range(S):
            n = min(S, r + w + 1)
            assert np.allclose(y[:, :, r, :n], 1.0 / n, rtol=0, atol=1e-15)
            assert np.all(y[:, :, r, n:] == 0.0)
    # shift invariance far from zero: scores near 3000 at scale 0.5 (z near 1500, beyond
    # where exp overflows) give the same rows as the unshifted scores
    y0 = orc.softmax_band_f64(x, lens, -3, 1, 0.5, F32)
    y1 = orc.softmax_band_f64((x.astype(np.float64) + 3000.0).astype(np.float32), lens, -3, 1,
                              0.5, F32)
    assert np.allclose(y0, y1, rtol=0, atol=2e-4)   # 3000 + x rounds x to 2^-12 in binary32
    assert np.all((y0 == 0) == (y1 == 0))
    from scipy.special import softmax as sp_softmax
    y = orc.softmax_band_f64(x, lens, -S, S, 0.5, F32)
    for b, L in enumerate(lens):
        Lc = min(L, S)
        if Lc:
            ref = sp_softmax(0.5 * x[b, :, :Lc, :Lc].astype(np.float64), axis=-1)
            assert np.allclose(y[b, :, :Lc, :Lc], ref, rtol=0, atol=1e-15)
        assert np.all(y[b, :, Lc:] == 0.0) and np.all(y[b, :, :, Lc:] == 0.0)


def pin_masked_brute_force(orc):
    """Explicit-mask variant: random 0/1 masks of every broadcast layout (a shared [S, S]
    mask, per-batch masks, per-head masks, per-sample key masks [B, 1, 1, S]), with and
    without lengths, against torch's masked softmax on the expanded mask; a mask row of all
    zeros gives a zero row; the value of a masked score never matters."""
    import torch
    rng = np.random.default_rng(33)
    B, M, S = 3, 2, 7
    x = rng.uniform(-4.0, 4.0, size=(B, M, S, S)).astype(np.float32)
    for shape in ((1, 1, S, S), (B, 1, S, S), (1, M, S, S), (B, M, S, S), (B, 1, 1, S),
                  (1, 1, 1, S)):
        for density in (0.15, 0.5, 0.9):
            mask = (rng.uniform(size=shape) < density).astype(np.uint8)
            if shape[2] == S:
                mask[..., 3, :] = 0       # an all-masked row
            for lens in (None, [7, 4, 0]):
                y = orc.softmax_masked_f64(x, mask, lens, 1.1, F32)
                full = torch.as_tensor(np.broadcast_to(mask, (B, M, S, S)).copy()).bool()
                for b in range(B):
                    keep = full[b] & _length_keep(S, None if lens is None else lens[b])
                    ref = _torch_masked_softmax(x[b].astype(np.float64) * float(np.float32(1.1)), keep)
                    assert np.allclose(y[b], ref, rtol=0, atol=1e-15), (shape, density, lens, b)
                    assert np.all(y[b][~keep.numpy()] == 0.0)
                xp = x.copy()
                xp[~np.broadcast_to(mask, x.shape).astype(bool)] = np.nan
                yp = orc.softmax_masked_f64(xp, mask, lens, 1.1, F32)
                assert np.array_equal(yp, y)


def pin_variant_backward(orc):
    """Backward of both variants equals torch's autograd gradient of its float64 masked
    softmax (rows without a kept element contribute nothing)."""
    import torch
    rng = np.random.default_rng(34)
    B, M, S = 2, 2, 6
    x = rng.uniform(-2.0, 2.0, size=(B, M, S, S)).astype(np.float32)
    g = rng.normal(size=(B, M, S, S)).astype(np.float32)
    scale = 0.6
    lens = [6, 3]
    band = (-2, 1)
    mask = (rng.uniform(size=(B, 1, S, S)) < 0.6).astype(np.uint8)
    mask[0, 0, 2, :] = 0
    cases = []
    yb = orc.softmax_band_f64(x, lens, *band, scale, F32).astype(np.float32)
    cases.append((orc.band_backward_f64(yb, g, lens, *band, scale, F32), yb,
                  lambda b: _band_keep(S, band[0], band[1], lens[b]).expand(M, S, S)))
    ym = orc.softmax_masked_f64(x, mask, lens, scale, F32).astype(np.float32)
    cases.append((orc.masked_backward_f64(ym, g, mask, lens, scale, F32), ym,
                  lambda b: torch.as_tensor(mask[b]).bool().expand(M, S, S) & _length_keep(S, lens[b])))
    for dx, y, keep_of in cases:
        for b in range(B):
            keep = keep_of(b)
            # the gradient of sum(g * softmax(scale * x)) at the point whose softmax is y:
            # rebuild that point as log(y) on kept elements (softmax(log y) = y / sum y)
            yt = torch.as_tensor(y[b].astype(np.float64))
            z = torch.where(keep, torch.log(torch.where(keep, yt, torch.ones_like(yt))),
                            torch.zeros_like(yt)) / float(np.float32(scale))
            z.requires_grad_(True)
            s = (z * float(np.float32(scale))).masked_fill(~keep, float("-inf")).softmax(-1)
            s = torch.where(keep.any(-1, keepdim=True), s, torch.zeros_like(s))
            (gd,) = torch.autograd.grad((s * torch.as_tensor(g[b].astype(np.float64))).sum(), z)
            gd = torch.where(keep, gd, torch.zeros_like(gd)).numpy()
            # the oracle differentiates at the rounded y; the rebuilt point differs from it by
            # the normalisation of y, a relative change of order 2^-24
            assert np.allclose(dx[b], gd, rtol=0, atol=1e-6), float(np.abs(dx[b] - gd).max())
            assert np.all(dx[b][~keep.numpy()] == 0.0)
    # masked cells of y and dy are never read: poisoning them changes no bit
    for (dx, y, keep_of), fn in zip(cases, (
            lambda yy, gg: orc.band_backward_f64(yy, gg, lens, *band, scale, F32),
            lambda yy, gg: orc.masked_backward_f64(yy, gg, mask, lens, scale, F32))):
        full = np.stack([keep_of(b).numpy() for b in range(B)])
        yp, gp = y.copy(), g.copy()
        yp[~full] = np.nan
        gp[~full] = np.inf
        assert np.array_equal(fn(yp, gp), dx)


# ------------------------------------------------------------------------------ attention
# The self-attention article ("ops(8) self-attention CUDA") computes scores Q K^T, a softmax
# per score row and the weighted sum P V; with this operation's mask a query row r < L keeps
# the keys c <= r and a row r >= L is zero.

def pin_attention(orc):
    """(i) Equal to torch's float64 scaled_dot_product_attention with is_causal=True on the
    rows below each length, zero on the others, for several head sizes and lengths.
    (ii) Closed forms: row 0 is V[0]; keys all zero give the running mean of V; values all
    equal to one vector u give u. (iii) The values in padded query rows and in keys or values
    past the length never matter."""
    import torch
    rng = np.random.default_rng(41)
    for D in (1, 8, 64):
        S = 9
        lens = [9, 5, 1, 0, 12]
        B, M = len(lens), 2
        q, k, v = (rng.uniform(-2, 2, size=(B, M, S, D)).astype(np.float32) for _ in range(3))
        scale = 0.7
        o = orc.attention_f64(q, k, v, lens, scale, F32)
        t = [torch.as_tensor(a.astype(np.float64)) for a in (q, k, v)]
        ref = torch.nn.functional.scaled_dot_product_attention(
            *t, is_causal=True, scale=float(np.float32(scale))).numpy()
        for b, L in enumerate(lens):
            Lc = min(max(L, 0), S)
            assert np.allclose(o[b, :, :Lc], ref[b, :, :Lc], rtol=0, atol=1e-14), (D, L)
            assert np.all(o[b, :, Lc:] == 0.0)
            if Lc:
                assert np.allclose(o[b, :, 0], v[b, :, 0], rtol=0, atol=1e-15)
        # poison: queries of padded rows, keys and values past each length
        qp, kp, vp = q.copy(), k.copy(), v.copy()
        for b, L in enumerate(lens):
            Lc = min(max(L, 0), S)
            qp[b, :, Lc:] = np.nan
            kp[b, :, Lc:] = np.inf
            vp[b, :, Lc:] = np.nan
        assert np.array_equal(orc.attention_f64(qp, kp, vp, lens, scale, F32), o)
        # the one-row entry point gives the same bits as the full one
        for b, m, r in ((0, 1, 8), (1, 0, 3), (1, 0, 7), (2, 1, 0), (3, 0, 4)):
            row = orc.attention_row_f64(q[b, m], k[b, m], v[b, m], r, lens[b], scale, F32)
            assert np.array_equal(row, o[b, m, r])
    S, D = 7, 4
    v = rng.normal(size=(1, 1, S, D)).astype(np.float32)
    q = rng.normal(size=(1, 1, S, D)).astype(np.float32)
    o = orc.attention_f64(q, np.zeros_like(q), v, [S], 1.0, F32)
    for r in range(S):
        assert np.allclose(o[0, 0, r], v[0, 0, :r + 1].astype(np.float64).mean(0), rtol=0, atol=1e-15)
    u = rng.normal(size=(D,)).astype(np.float32)
    vv = np.broadcast_to(u, (1, 1, S, D)).copy()
    o = orc.attention_f64(q, rng.normal(size=q.shape).astype(np.float32), vv, [S], 1.3, F32)
    assert np.allclose(o[0, 0], np.broadcast_to(u.astype(np.float64), (S, D)), rtol=0, atol=1e-14)
    # 16-bit inputs are decoded exactly: the same values in binary32 give the same result
    q16 = rng.normal(size=(1, 2, S, 8)).astype(np.float16)
    k16 = rng.normal(size=(1, 2, S, 8)).astype(np.float16)
    v16 = rng.normal(size=(1, 2, S, 8)).astype(np.float16)
    a = orc.attention_f64(q16.view(np.uint16), k16.view(np.uint16), v16.view(np.uint16), [S],
                          0.5, F16)
    b = orc.attention_f64(q16.astype(np.float32), k16.astype(np.float32),
                          v16.astype(np.float32), [S], 0.5, F32)
    assert np.array_equal(a, b)


ALL_PINS = [
    pin_printed_masks, pin_printed_output, pin_row0, pin_row_sums, pin_exact_zeros,
    pin_brute_force, pin_closed_forms, pin_shift_and_scale, pin_masked_poison,
    pin_length_edges, pin_codec, pin_rounded_outputs, pin_rows_api, pin_backward,
    pin_backward_rows,
    pin_band_brute_force, pin_band_closed_forms, pin_masked_brute_force, pin_variant_backward,
    pin_attention,
]
