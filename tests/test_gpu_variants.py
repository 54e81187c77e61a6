"""GPU parity of the mask variants (band and explicit mask) against the CPU oracle.

The variants come from the ScaledMaskSoftmax article ("优化ScaledMaskSoftmax算子"): scores
outside the kept set count as minus infinity (section 2.1), rows with no kept element are
zeros (section 4.1), and section 6 builds window masks with tril, per-task masks
broadcast over the batch, and per-sample length masks. Every test calls the library
through its C ABI (the Python binding) and compares with the oracle's fp64 result:
elements outside the kept set must be +0.0 bit for bit, kept elements within the element
type's tolerance (binary32 2e-6, binary16 2e-3, bfloat16 8e-3). The kept set used for the
bit check is built here from the definition, not taken from either side.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gtms_check import (TOL, bits, check_planes_against_oracle, check_planes_backward_against_oracle,
                        check_rows_against_oracle, check_rows_backward_against_oracle, path_ok,
                        to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("GPU tests need a visible GPU", allow_module_level=True)

import variable_length_causal_amd as g  # noqa: E402

DTYPES = [workloads.F32, workloads.F16, workloads.BF16]
DNAME = {workloads.F32: "f32", workloads.F16: "f16", workloads.BF16: "bf16"}
PATHS = ("auto", "wave", "block", "stream")
U = {workloads.F32: 2.0 ** -21, workloads.F16: 2.0 ** -10, workloads.BF16: 2.0 ** -7}
TINY = {workloads.F32: 2.0 ** -150, workloads.F16: 2.0 ** -25, workloads.BF16: 2.0 ** -134}


def length_keep(S, L):
    Lc = S if L is None else min(max(int(L), 0), S)
    i = np.arange(S)
    return (i[:, None] < Lc) & (i[None, :] < Lc)


def band_keep(S, L, lo, hi):
    d = np.arange(S)[None, :] - np.arange(S)[:, None]
    return (d >= lo) & (d <= hi) & length_keep(S, L)


def expand_mask(mask, B, M, S):
    return np.broadcast_to(np.asarray(mask).astype(bool), (B, M, S, S))


def lens_dev(lens):
    return None if lens is None else torch.as_tensor(np.asarray(lens, np.int32)).cuda()


def check(out_dev, ref64, keep, dtype, tag):
    """keep: bool [B, M, S, S]."""
    st = workloads.to_storage(out_dev.cpu())
    ob = bits(st)
    assert not ob[~keep].any(), f"{tag}: nonzero bits outside the kept set"
    if keep.any():
        got = to_f64(st, dtype)
        err = np.abs(got[keep] - ref64[keep])
        assert np.all(np.isfinite(got[keep])), f"{tag}: non-finite kept output"
        assert float(err.max()) <= TOL[dtype], f"{tag}: max error {float(err.max()):.3g}"


def band_case(shape, dtype, lens, lo, hi, scale, paths, seed):
    B, M, S, _ = shape
    paths = [p for p in paths if path_ok(p, S, dtype)]
    x = workloads.scores_cpu(shape, dtype, 1.0, seed)
    ref = oracle.softmax_band_f64(workloads.to_storage(x), lens, lo, hi, scale, dtype)
    keep = np.stack([np.broadcast_to(band_keep(S, None if lens is None else lens[b], lo, hi),
                                     (M, S, S)) for b in range(B)])
    xd = x.cuda()
    for path in paths:
        print(f"band shape={shape} {DNAME[dtype]} lens={lens} lo={lo} hi={hi} path={path}",
              flush=True)
        y = g.forward_band(xd, lens_dev(lens), lo, hi, scale, path=path)
        torch.cuda.synchronize()
        check(y, ref, keep, dtype, f"band {shape} {lens} [{lo},{hi}] {path}")


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_band_sweep(dtype):
    for S in (1, 5, 64, 65, 200, 1000, 1025):
        bands = [(-S, 0), (-63, 0), (-1, 1), (0, 0), (-10 ** 12, 5), (3, 1), (-S, S),
                 (2, 40), (-(S // 2), -(S // 4))]
        for lens in ([S, max(1, S // 3), 0, S + 5], None):
            for lo, hi in bands:
                band_case((4, 1, S, S), dtype, lens, lo, hi, 0.8, PATHS, seed=S + lo % 97)


def test_band_equals_tril_bits():
    """lo <= -(S-1), hi = 0 is the grouped tril mask: the same bits as gtms_forward."""
    for dtype, S in ((workloads.F32, 1000), (workloads.F16, 4096), (workloads.BF16, 520)):
        lens = [S, S // 2, 7]
        x = workloads.scores_cpu((3, 2, S, S), dtype, 1.0, 11).cuda()
        sl = lens_dev(lens)
        a = g.forward(x, sl, 0.5)
        b = g.forward_band(x, sl, -S, 0, 0.5)
        c = g.forward_band(x, sl, -(10 ** 15), 0, 0.5)
        torch.cuda.synchronize()
        sa = bits(workloads.to_storage(a.cpu()))
        assert np.array_equal(sa, bits(workloads.to_storage(b.cpu())))
        assert np.array_equal(sa, bits(workloads.to_storage(c.cpu())))


def masked_case(shape, dtype, mask_np, lens, scale, paths, seed, as_bool=False, mask_dev=None):
    B, M, S, _ = shape
    paths = [p for p in paths if path_ok(p, S, dtype)]
    x = workloads.scores_cpu(shape, dtype, 1.0, seed)
    ref = oracle.softmax_masked_f64(workloads.to_storage(x), mask_np, lens, scale, dtype)
    if mask_dev is None:
        mask_dev = torch.as_tensor(mask_np.astype(bool) if as_bool else mask_np).cuda()
    keep = expand_mask(mask_np, B, M, S) & np.stack(
        [np.broadcast_to(length_keep(S, None if lens is None else lens[b]), (M, S, S))
         for b in range(B)])
    xd = x.cuda()
    for path in paths:
        print(f"masked shape={shape} {DNAME[dtype]} mask={tuple(mask_np.shape)} lens={lens} "
              f"path={path}", flush=True)
        y = g.forward_masked(xd, mask_dev, lens_dev(lens), scale, path=path)
        torch.cuda.synchronize()
        check(y, ref, keep, dtype, f"masked {shape} {tuple(mask_np.shape)} {lens} {path}")


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_masked_layouts(dtype):
    rng = np.random.default_rng(7)
    B, M = 3, 2
    for S in (7, 64, 300, 1000, 1030):
        layouts = [(1, 1, S, S), (B, 1, S, S), (1, M, S, S), (B, M, S, S), (B, 1, 1, S)]
        for li, shape in enumerate(layouts):
            mask = (rng.uniform(size=shape) < 0.6).astype(np.uint8)
            if shape[2] == S:
                mask[..., S // 2, :] = 0   # an all-masked row
            for lens in (None, [S, S // 3, 0]):
                masked_case((B, M, S, S), dtype, mask, lens, 1.2, PATHS, seed=S + li,
                            as_bool=(li % 2 == 1))


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_variants_in_place(dtype):
    """The variants follow gtms_forward's and gtms_backward's in-place rules: the band and the
    explicit-mask forwards with out = x, and their backwards with dx = dy, give the bits of
    the calls into separate outputs, on every path the rows fit."""
    B, M = 2, 2
    for S, lens in ((300, [300, 123]), (1030, [1030, 517])):
        sl = lens_dev(lens)
        rng = np.random.default_rng(S)
        mask = torch.as_tensor((rng.uniform(size=(1, M, S, S)) < 0.7).astype(np.uint8)).cuda()
        x = workloads.scores_cpu((B, M, S, S), dtype, 1.0, S + 11).cuda()
        dy = workloads.scores_cpu((B, M, S, S), dtype, 1.0, S + 12).cuda()
        ib = torch.int32 if dtype == workloads.F32 else torch.int16
        for path in [p for p in PATHS if path_ok(p, S, dtype)]:
            print(f"variants in place S={S} {DNAME[dtype]} path={path}", flush=True)
            for tag, fwd, bwd in (
                    ("band", lambda t, o: g.forward_band(t, sl, -40, 3, 0.7, out=o, path=path),
                     lambda y, d, o: g.backward_band(y, d, sl, -40, 3, 0.7, out=o, path=path)),
                    ("mask", lambda t, o: g.forward_masked(t, mask, sl, 0.7, out=o, path=path),
                     lambda y, d, o: g.backward_masked(y, d, mask, sl, 0.7, out=o, path=path))):
                y = fwd(x, None)
                xi = x.clone()
                fwd(xi, xi)
                dx = bwd(y, dy, None)
                dyi = dy.clone()
                bwd(y, dyi, dyi)
                torch.cuda.synchronize()
                assert torch.equal(xi.view(ib), y.view(ib)), f"{tag} forward in place, {path}"
                assert torch.equal(dyi.view(ib), dx.view(ib)), f"{tag} backward in place, {path}"


def test_masked_unaligned_mask_rows():
    """Mask rows at odd byte strides (a view into a wider buffer): the element-wise path."""
    for dtype, S in ((workloads.F32, 256), (workloads.BF16, 1000)):
        rng = np.random.default_rng(3)
        wide = (rng.uniform(size=(1, 1, S, S + 1)) < 0.5).astype(np.uint8)
        view_np = np.ascontiguousarray(wide[..., :S])
        mdev = torch.as_tensor(wide).cuda()[..., :S]
        assert mdev.stride(2) == S + 1
        masked_case((2, 2, S, S), dtype, view_np, [S, S - 9], 1.0, ("auto", "wave", "block"),
                    seed=5, mask_dev=mdev)


def test_masked_tril_matches_forward():
    """A tril mask of ones with lengths is the grouped tril mask. The kernels see a wider
    column interval ([0, L-1] instead of [0, r]), which changes which lane sums which
    elements, so results agree to rounding (same zeros, values within the tolerance)."""
    for dtype, S in ((workloads.F32, 1000), (workloads.F16, 4096)):
        lens = [S, S // 3]
        x = workloads.scores_cpu((2, 2, S, S), dtype, 1.0, 21).cuda()
        sl = lens_dev(lens)
        tril = torch.ones(S, S, dtype=torch.uint8, device="cuda").tril()[None, None]
        a = workloads.to_storage(g.forward(x, sl, 0.3).cpu())
        b = workloads.to_storage(g.forward_masked(x, tril, sl, 0.3).cpu())
        assert np.array_equal(bits(a) == 0, bits(b) == 0)
        assert float(np.max(np.abs(to_f64(a, dtype) - to_f64(b, dtype)))) <= TOL[dtype]


def test_variants_ignore_masked_scores():
    """NaN and infinity outside the kept set change no bit of either variant."""
    S, lens = 300, [300, 100]
    for dtype in DTYPES:
        x = workloads.scores_cpu((2, 2, S, S), dtype, 1.0, 31)
        keep_b = np.stack([np.broadcast_to(band_keep(S, L, -40, 3), (2, S, S)) for L in lens])
        rng = np.random.default_rng(9)
        mask = (rng.uniform(size=(2, 1, S, S)) < 0.5).astype(np.uint8)
        keep_m = expand_mask(mask, 2, 2, S) & np.stack(
            [np.broadcast_to(length_keep(S, L), (2, S, S)) for L in lens])
        mdev = torch.as_tensor(mask).cuda()
        sl = lens_dev(lens)
        for keep, run in ((keep_b, lambda t: g.forward_band(t, sl, -40, 3, 1.0)),
                          (keep_m, lambda t: g.forward_masked(t, mdev, sl, 1.0))):
            clean = run(x.cuda())
            xp = x.clone()
            kt = torch.as_tensor(keep)
            xp[~kt] = float("nan")
            xp[(~kt) & (torch.arange(S)[None, None, None, :] % 2 == 0)] = float("inf")
            dirty = run(xp.cuda())
            torch.cuda.synchronize()
            assert np.array_equal(bits(workloads.to_storage(clean.cpu())),
                                  bits(workloads.to_storage(dirty.cpu())))


def test_variant_long_rows():
    for dtype, S, lens in ((workloads.F16, 4096, [4096, 1500]), (workloads.BF16, 8192, [8000])):
        paths = ("auto", "block", "stream")
        band_case((len(lens), 1, S, S), dtype, lens, -511, 0, 0.125, paths, seed=41)
        band_case((len(lens), 1, S, S), dtype, None, -(10 ** 9), 300, 0.125, paths, seed=42)
        rng = np.random.default_rng(43)
        mask = (rng.uniform(size=(1, 1, S, S)) < 0.3).astype(np.uint8)
        masked_case((len(lens), 1, S, S), dtype, mask, lens, 0.125, ("auto", "stream"), seed=44)


def grad_check(dx_dev, ref, y_st, dy_st, keep, scale, dtype, tag):
    st = workloads.to_storage(dx_dev.cpu())
    assert not bits(st)[~keep].any(), f"{tag}: nonzero bits outside the kept set"
    got, yv, gv = to_f64(st, dtype), to_f64(y_st, dtype), to_f64(dy_st, dtype)
    gmax = np.max(np.where(keep, np.abs(gv), 0.0), axis=-1, keepdims=True)
    bound = U[dtype] * np.abs(ref) + 1e-5 * abs(scale) * yv * gmax + TINY[dtype]
    err = np.abs(got - ref)
    assert np.all(err[keep] <= bound[keep]), f"{tag}: {float(np.max((err - bound)[keep]))}"


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_variant_backward(dtype):
    rng = np.random.default_rng(51)
    for S in (5, 64, 300, 1000):
        B, M = 3, 2
        lens = [S, S // 3 + 1, 0]
        x = workloads.to_storage(workloads.scores_cpu((B, M, S, S), dtype, 1.0, S))
        dy = workloads.to_storage(workloads.scores_cpu((B, M, S, S), dtype, 1.0, S + 1))
        lo, hi = -(S // 4) - 1, 2
        mask = (rng.uniform(size=(B, 1, S, S)) < 0.5).astype(np.uint8)
        yb = workloads.to_storage(torch.as_tensor(
            oracle.softmax_band_f64(x, lens, lo, hi, 0.9, dtype)).to(workloads.torch_dtype(dtype)))
        ym = workloads.to_storage(torch.as_tensor(
            oracle.softmax_masked_f64(x, mask, lens, 0.9, dtype)).to(workloads.torch_dtype(dtype)))
        refb = oracle.band_backward_f64(yb, dy, lens, lo, hi, 0.9, dtype)
        refm = oracle.masked_backward_f64(ym, dy, mask, lens, 0.9, dtype)
        keep_b = np.stack([np.broadcast_to(band_keep(S, L, lo, hi), (M, S, S)) for L in lens])
        keep_m = expand_mask(mask, B, M, S) & np.stack(
            [np.broadcast_to(length_keep(S, L), (M, S, S)) for L in lens])
        sl = lens_dev(lens)
        mdev = torch.as_tensor(mask).cuda()
        dyd = workloads.from_storage(dy, dtype).cuda()
        for path in PATHS:
            if not path_ok(path, S, dtype):
                continue
            print(f"variant backward S={S} {DNAME[dtype]} path={path}", flush=True)
            dxb = g.backward_band(workloads.from_storage(yb, dtype).cuda(), dyd, sl, lo, hi, 0.9,
                                  path=path)
            dxm = g.backward_masked(workloads.from_storage(ym, dtype).cuda(), dyd, mdev, sl, 0.9,
                                    path=path)
            torch.cuda.synchronize()
            grad_check(dxb, refb, yb, dy, keep_b, 0.9, dtype, f"band bwd S={S} {path}")
            grad_check(dxm, refm, ym, dy, keep_m, 0.9, dtype, f"masked bwd S={S} {path}")


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_variants_widest_wave_rows(dtype):
    """Band and explicit mask, forward and backward, on rows of 4000 elements through the
    one-wavefront path: sixteen binary32 or eight 16-bit vectors per lane, the largest
    layouts of that path (random masks, one all-masked row, a shorter second sample)."""
    S, lens, scale = 4000, [4000, 1401], 0.9
    rng = np.random.default_rng(71)
    mask = (rng.uniform(size=(2, 1, S, S)) < 0.5).astype(np.uint8)
    mask[0, 0, 100, :] = 0
    band_case((2, 1, S, S), dtype, lens, -1500, 7, scale, ("wave",), seed=72)
    masked_case((2, 1, S, S), dtype, mask, lens, scale, ("wave",), seed=73)
    x = workloads.to_storage(workloads.scores_cpu((2, 1, S, S), dtype, 1.0, 74))
    dy = workloads.to_storage(workloads.scores_cpu((2, 1, S, S), dtype, 1.0, 75))
    tdt = workloads.torch_dtype(dtype)
    yb = workloads.to_storage(torch.as_tensor(
        oracle.softmax_band_f64(x, lens, -1500, 7, scale, dtype)).to(tdt))
    ym = workloads.to_storage(torch.as_tensor(
        oracle.softmax_masked_f64(x, mask, lens, scale, dtype)).to(tdt))
    keep_b = np.stack([band_keep(S, L, -1500, 7)[None] for L in lens])
    keep_m = expand_mask(mask, 2, 1, S) & np.stack([length_keep(S, L)[None] for L in lens])
    sl = lens_dev(lens)
    dyd = workloads.from_storage(dy, dtype).cuda()
    print(f"variant backward S={S} {DNAME[dtype]} path=wave", flush=True)
    dxb = g.backward_band(workloads.from_storage(yb, dtype).cuda(), dyd, sl, -1500, 7, scale,
                          path="wave")
    dxm = g.backward_masked(workloads.from_storage(ym, dtype).cuda(), dyd,
                            torch.as_tensor(mask).cuda(), sl, scale, path="wave")
    torch.cuda.synchronize()
    grad_check(dxb, oracle.band_backward_f64(yb, dy, lens, -1500, 7, scale, dtype), yb, dy,
               keep_b, scale, dtype, "band bwd wave")
    grad_check(dxm, oracle.masked_backward_f64(ym, dy, mask, lens, scale, dtype), ym, dy,
               keep_m, scale, dtype, "masked bwd wave")


def test_variants_block_rows_every_element():
    """Rows that fill the block path's registers (binary16 40000: eight 16-byte vectors per
    lane, the layout the 16-bit rows of 65536 use as well). A band [-S, 0] and a
    lower-triangular mask of ones, both with the valid length, keep exactly the grouped tril
    set, so every element compares with the oracle's tril row entry points, forward and
    backward, in blocks of rows."""
    for dtype, S in ((workloads.F16, 40000),):
        L = S - 17
        lens = np.asarray([L], np.int32)
        print(f"variant block rows S={S} {DNAME[dtype]}", flush=True)
        sl = lens_dev([L])
        tril = torch.ones((S, S), dtype=torch.uint8, device="cuda").tril_()[None, None]
        x = workloads.scores_device((1, 1, S, S), dtype, 1.0, S + 2)
        for tag, out in (("band", g.forward_band(x, sl, -S, 0, 0.5)),
                         ("masked", g.forward_masked(x, tril, sl, 0.5))):
            torch.cuda.synchronize()
            worst = check_rows_against_oracle(x, out, lens, 0.5, dtype)
            print(f"S={S} {tag}: every element checked, worst error {worst:.3g}", flush=True)
            del out
        del x
        torch.cuda.empty_cache()
        gen = torch.Generator(device="cuda")
        gen.manual_seed(S)
        # uniform in [0, 2/L): a row sums to about 1, as a forward output does
        y = torch.rand((1, 1, S, S), generator=gen, device="cuda").mul_(2.0 / L).to(
            workloads.torch_dtype(dtype))
        dy = workloads.scores_device((1, 1, S, S), dtype, 1.0, S + 3)
        for tag, run in (("band bwd", lambda: g.backward_band(y, dy, sl, -S, 0, 0.5)),
                         ("masked bwd", lambda: g.backward_masked(y, dy, tril, sl, 0.5))):
            dx = run()
            torch.cuda.synchronize()
            worst = check_rows_backward_against_oracle(y, dy, dx, lens, 0.5, dtype, U[dtype],
                                                       TINY[dtype])
            print(f"S={S} {tag}: every element checked, worst error {worst:.3g}", flush=True)
            del dx
        del y, dy, tril
        torch.cuda.empty_cache()


def test_shared_mask_long_rows_every_element():
    """A [1, 1, S, S] mask shared by 2 x 2 planes on binary16 rows of 33000 (66000 bytes: the
    rows are long enough for the unit order that takes blocks of 64 rows plane after plane,
    and 33000 = 515 * 64 + 40 leaves a shorter last block). The mask is the lower triangle
    of ones, which with the valid lengths keeps exactly the grouped tril set, so every
    element compares with the oracle's tril row entry points, forward and backward. The same
    mask materialised per plane (non-zero strides, so the plane-major order) gives the same
    bits, and so do paired rows (the order's blocks then run over pair indices) and the
    stream path with either mask."""
    dtype, S, B, M = workloads.F16, 33000, 2, 2
    lens = np.asarray([S - 17, S - 3001], np.int32)
    sl = lens_dev(lens)
    print(f"shared mask long rows S={S} B={B} M={M} lens={list(lens)}", flush=True)
    tril = torch.ones((S, S), dtype=torch.uint8, device="cuda").tril_()[None, None]
    x = workloads.scores_device((B, M, S, S), dtype, 1.0, S + 5)
    y = g.forward_masked(x, tril, sl, 0.5)
    torch.cuda.synchronize()
    worst = check_rows_against_oracle(x, y, lens, 0.5, dtype)
    print(f"shared mask forward: every element checked, worst error {worst:.3g}", flush=True)
    per_plane = tril.expand(B, M, S, S).contiguous()
    y2 = g.forward_masked(x, per_plane, sl, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), \
        "shared and per-plane masks differ (forward)"
    # rows paired (r, S-1-r): the blocks of the order then run over pair indices
    y2 = g.forward_masked(x, tril, sl, 0.5, flags=g.FLAG_PAIR_ROWS)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), \
        "paired rows differ (forward)"
    del x, y2
    torch.cuda.empty_cache()
    dy = workloads.scores_device((B, M, S, S), dtype, 1.0, S + 6)
    dx = g.backward_masked(y, dy, tril, sl, 0.5)
    torch.cuda.synchronize()
    worst = check_rows_backward_against_oracle(y, dy, dx, lens, 0.5, dtype, U[dtype], TINY[dtype])
    print(f"shared mask backward: every element checked, worst error {worst:.3g}", flush=True)
    dx2 = g.backward_masked(y, dy, per_plane, sl, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)), \
        "shared and per-plane masks differ (backward)"
    dx2 = g.backward_masked(y, dy, tril, sl, 0.5, flags=g.FLAG_PAIR_ROWS)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)), \
        "paired rows differ (backward)"
    del dx, dx2
    torch.cuda.empty_cache()
    # The stream path (forced) takes the same order with the shared mask: into outputs
    # filled with NaN, both orders must write the same bits everywhere (a unit skipped or
    # visited twice would leave NaN behind). Its arithmetic is checked against the oracle
    # in the path sweeps.
    x = workloads.scores_device((B, M, S, S), dtype, 1.0, S + 5)
    for tag, run in (
            ("forward", lambda m, o: g.forward_masked(x, m, sl, 0.5, out=o, path="stream")),
            ("backward", lambda m, o: g.backward_masked(y, dy, m, sl, 0.5, out=o, path="stream"))):
        a = torch.full_like(x, float("nan"))
        b = torch.full_like(x, float("nan"))
        run(tril, a)
        run(per_plane, b)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
            f"stream path: shared and per-plane masks differ ({tag})"
        assert not torch.isnan(a).any(), f"stream path: unwritten elements ({tag})"
        print(f"shared mask stream {tag}: same bits as the per-plane mask", flush=True)
        del a, b
        torch.cuda.empty_cache()
    del x, y, dy, per_plane, tril
    torch.cuda.empty_cache()


def test_full_size_window_and_key_masks():
    """Full workload shapes, every element of every plane against the oracle: a causal window
    of 512 columns on binary16 32 x 1 x 4096, and per-sample key masks [B, 1, 1, S] (the
    article's length mask) on binary32 3 x 64 x 1000."""
    w = workloads.WORKLOADS["scaled_f16_32x1x4096"]
    lens = workloads.seq_lens(w)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed, "cuda")
    y = g.forward_band(x, torch.as_tensor(lens).cuda(), -511, 0, w.scale)
    torch.cuda.synchronize()
    S = w.S

    def ref_band(x_plane, p):
        b = p // w.M
        ref = oracle.softmax_band_f64(x_plane, lens[b:b + 1], -511, 0, w.scale, w.dtype)[0, 0]
        return ref, band_keep(S, lens[b], -511, 0)
    worst = check_planes_against_oracle(x, y, lens, w.scale, w.dtype, plane_ref=ref_band)
    print(f"window tril(512) on {w.name}: every plane checked, worst error {worst:.3g}",
          flush=True)
    del x, y

    w = workloads.WORKLOADS["readme_f32_3x64x1000"]
    S = w.S
    key_lens = [700, 1000, 10]
    key = (np.arange(S)[None, :] < np.asarray(key_lens)[:, None]).astype(np.uint8)
    key = key.reshape(w.B, 1, 1, S)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed, "cuda")
    y = g.forward_masked(x, torch.as_tensor(key).cuda(), None, w.scale)
    torch.cuda.synchronize()

    def ref_key(x_plane, p):
        b = p // w.M
        ref = oracle.softmax_masked_f64(x_plane, key[b:b + 1], None, w.scale, w.dtype)[0, 0]
        return ref, np.broadcast_to(key[b, 0, 0].astype(bool), (S, S))
    worst = check_planes_against_oracle(x, y, None, w.scale, w.dtype, plane_ref=ref_key)
    print(f"key masks on {w.name}: every plane checked, worst error {worst:.3g}", flush=True)


def test_full_size_window_and_key_mask_backwards():
    """The backwards of the full-size variants, every element of every plane against the
    oracle's variant backwards: a causal window of 512 columns on binary16 32 x 1 x 4096, and
    per-sample key masks [B, 1, 1, S] on binary32 3 x 64 x 1000. y is drawn uniform in
    [0, 2/S) (the backward is defined for any y), dy normal."""
    w = workloads.WORKLOADS["scaled_f16_32x1x4096"]
    lens = workloads.seq_lens(w)
    S = w.S
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4301)
    y = torch.rand(w.shape, generator=gen, device="cuda",
                   dtype=workloads.torch_dtype(w.dtype)).mul_(2.0 / S)
    dy = workloads.scores_device(w.shape, w.dtype, 1.0, 4302)
    dx = g.backward_band(y, dy, torch.as_tensor(lens).cuda(), -511, 0, w.scale)
    torch.cuda.synchronize()

    def ref_band(y_plane, dy_plane, p):
        b = p // w.M
        ref = oracle.band_backward_f64(y_plane, dy_plane, lens[b:b + 1], -511, 0, w.scale,
                                       w.dtype)[0, 0]
        return ref, band_keep(S, lens[b], -511, 0)
    worst = check_planes_backward_against_oracle(y, dy, dx, lens, w.scale, w.dtype, U[w.dtype],
                                                 TINY[w.dtype], plane_ref=ref_band)
    print(f"window tril(512) backward on {w.name}: every plane checked, worst error {worst:.3g}",
          flush=True)
    del y, dy, dx

    w = workloads.WORKLOADS["readme_f32_3x64x1000"]
    S = w.S
    key = (np.arange(S)[None, :] < np.asarray([700, 1000, 10])[:, None]).astype(np.uint8)
    key = key.reshape(w.B, 1, 1, S)
    gen.manual_seed(4303)
    y = torch.rand(w.shape, generator=gen, device="cuda").mul_(2.0 / S)
    dy = workloads.scores_device(w.shape, w.dtype, 1.0, 4304)
    dx = g.backward_masked(y, dy, torch.as_tensor(key).cuda(), None, w.scale)
    torch.cuda.synchronize()

    def ref_key(y_plane, dy_plane, p):
        b = p // w.M
        ref = oracle.masked_backward_f64(y_plane, dy_plane, key[b:b + 1], None, w.scale,
                                         w.dtype)[0, 0]
        return ref, np.broadcast_to(key[b, 0, 0].astype(bool), (S, S))
    worst = check_planes_backward_against_oracle(y, dy, dx, None, w.scale, w.dtype, U[w.dtype],
                                                 TINY[w.dtype], plane_ref=ref_key)
    print(f"key mask backward on {w.name}: every plane checked, worst error {worst:.3g}",
          flush=True)


def test_band_forward_raw_long_rows():
    """A causal window of 70001 columns on bfloat16 rows of 100000 (forward): each row holds only
    its interval, up to 8766 vectors, which takes the block path at 16 raw vectors per lane.
    The scores below the window are set to -inf, so the grouped tril mask's softmax of the
    same input equals the window's (exp(-inf) = 0; the kernel never reads those cells), and
    every element compares with the oracle's tril rows, in blocks of rows."""
    S, L, lo = 100000, 100000 - 5, -70000
    dtype = workloads.BF16
    print(f"band forward S={S} L={L} lo={lo} {DNAME[dtype]}", flush=True)
    x = workloads.scores_device((1, 1, S, S), dtype, 1.0, 3301)
    cols = torch.arange(S, device="cuda")
    for r0 in range(0, S, 4096):
        r1 = min(S, r0 + 4096)
        rows = torch.arange(r0, r1, device="cuda")[:, None]
        x[0, 0, r0:r1].masked_fill_(cols[None, :] < rows + lo, float("-inf"))
    sl = lens_dev([L])
    y = g.forward_band(x, sl, lo, 0, 0.125)
    torch.cuda.synchronize()
    worst = check_rows_against_oracle(x, y, np.asarray([L], np.int32), 0.125, dtype)
    print(f"S={S} window {-lo + 1}: every element checked, worst error {worst:.3g}", flush=True)
    del x, y
    torch.cuda.empty_cache()
