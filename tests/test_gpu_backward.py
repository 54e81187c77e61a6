"""GPU parity of the backward kernels against the oracle's backward.

The forward output y and the upstream gradient dy are inputs of both sides: y comes from the
oracle's rounded forward (small shapes, the four benchmark workloads and the 65536- and
100000-wide rows at full size) or, for the block path's widest layouts and the LDS-stash rows,
a seeded uniform draw whose rows sum to about 1; never from the GPU path. Masked elements of dx must be +0 bit for bit. Kept elements must satisfy, per
element, the bound derived from the fp32 arithmetic:
    |dx_gpu - dx_ref| <= u * |dx_ref| + 1e-5 * scale * y_c * max_k |dy_k|
with u = 2^-21 (binary32), 2^-10 (binary16), 2^-7 (bfloat16): the output rounding plus a
few fp32 roundings, and the error of the fp32 dot product D (at most a few hundred terms
per thread and a 64-lane tree) relative to max |dy|; plus half the subnormal spacing of the
element type, the rounding floor near zero.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gtms_check import (bits, check_planes_backward_against_oracle,
                        check_rows_backward_against_oracle, kept_mask, kept_row,
                        oracle_forward_to_device, path_ok, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("GPU tests need a visible GPU", allow_module_level=True)

import variable_length_causal_amd as g  # noqa: E402

DTYPES = [workloads.F32, workloads.F16, workloads.BF16]
DNAME = {workloads.F32: "f32", workloads.F16: "f16", workloads.BF16: "bf16"}
U = {workloads.F32: 2.0 ** -21, workloads.F16: 2.0 ** -10, workloads.BF16: 2.0 ** -7}
# half the spacing of the element type's subnormals: the rounding error floor near zero
TINY = {workloads.F32: 2.0 ** -150, workloads.F16: 2.0 ** -25, workloads.BF16: 2.0 ** -134}


def check_rows(dx_st, ref, y_st, dy_st, lens_of_rows, rows_r, scale, dtype):
    """Rows given as 2-D arrays [n, S] with their row index and length."""
    got = to_f64(dx_st, dtype)
    gb = bits(dx_st)
    yv = to_f64(y_st, dtype)
    gv = to_f64(dy_st, dtype)
    S = dx_st.shape[-1]
    for i, (L, r) in enumerate(zip(lens_of_rows, rows_r)):
        keep = kept_row(S, L, r)
        assert not gb[i][~keep].any(), f"masked bits set in row {i} (r={r}, L={L})"
        if keep.any():
            gmax = float(np.max(np.abs(gv[i][keep])))
            bound = U[dtype] * np.abs(ref[i][keep]) + 1e-5 * abs(scale) * yv[i][keep] * gmax \
                + TINY[dtype]
            err = np.abs(got[i][keep] - ref[i][keep])
            assert np.all(err <= bound), (i, r, L, float(np.max(err - bound)))


def run_case(shape, dtype, lens, scale, path="auto", seed=0):
    B, M, S, _ = shape
    x = workloads.scores_cpu(shape, dtype, 1.0, seed)
    y_st = oracle.softmax(workloads.to_storage(x), lens, scale, dtype)   # the forward, oracle
    dy = workloads.scores_cpu(shape, dtype, 1.0, seed + 1)
    dy_st = workloads.to_storage(dy)
    ref = oracle.backward_f64(y_st, dy_st, lens, scale, dtype)
    y_dev = workloads.from_storage(y_st, dtype).cuda()
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    print(f"backward shape={shape} dtype={DNAME[dtype]} path={path} lens={list(lens)}",
          flush=True)
    dx = g.backward(y_dev, dy.cuda(), sl, scale, path=path)
    torch.cuda.synchronize()
    dx_st = workloads.to_storage(dx.cpu())
    n = B * M * S
    lens_rows = np.repeat(np.asarray(lens), M * S)
    rows_r = np.tile(np.arange(S), B * M)
    check_rows(dx_st.reshape(n, S), ref.reshape(n, S), y_st.reshape(n, S),
               dy_st.reshape(n, S), lens_rows, rows_r, scale, dtype)
    return dx_st, y_dev, dy, sl


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_backward_shape_sweep(dtype):
    for S in (1, 3, 5, 8, 17, 64, 65, 200, 513, 1000, 1025):
        lens = [S, max(1, S // 3), 0, S + 2]
        for path in ("auto", "wave", "block", "stream"):
            if path_ok(path, S, dtype):
                run_case((4, 2, S, S), dtype, lens, 0.7, path, seed=100 + S)


# Row lengths where the automatic choice changes kernel (see test_gpu_parity.SWITCH_CASES):
# the backward takes the same choice, by the same rule over its row slots.
SWITCH_CASES = [
    (workloads.F32, 1000, 0, "wave"), (workloads.F32, 1004, 0, "block"),
    (workloads.F32, 1008, 0, "wave"), (workloads.F32, 1012, 0, "block"),
    (workloads.F32, 1020, 0, "block"), (workloads.F32, 1024, 0, "wave"),
    (workloads.F32, 1028, 0, "block"), (workloads.F32, 1032, 0, "block"),
    (workloads.F32, 1024, 16, "block"),
] + [(dt, S, off, path) for dt in (workloads.F16, workloads.BF16) for S, off, path in (
    (2040, 0, "block"), (2047, 0, "block"), (2048, 0, "wave"), (2049, 0, "block"),
    (2056, 0, "block"), (2048, 16, "block"))]


def offset_copy(host, dtype, offset_bytes):
    """A device copy of a CPU tensor whose data starts offset_bytes past a 256-byte boundary."""
    es = 4 if dtype == workloads.F32 else 2
    n = host.numel()
    buf = torch.zeros(n + 256 // es, dtype=host.dtype, device="cuda")
    t = buf[offset_bytes // es:offset_bytes // es + n].view(host.shape)
    assert t.data_ptr() % 256 == offset_bytes
    t.copy_(host.cuda())
    return t


@pytest.mark.parametrize("case", SWITCH_CASES,
                         ids=lambda c: f"{DNAME[c[0]]}-{c[1]}-off{c[2]}-{c[3]}")
def test_backward_auto_path_switch_sizes(case):
    """The backward through the automatic choice at the row lengths where it changes kernel,
    lengths S, S - 1, S / 2 and 0, y from the oracle's forward: every element within the
    bound, and the same bits as the path the choice rule names."""
    dtype, S, off, expect = case
    lens = [S, S - 1, S // 2, 0]
    shape = (len(lens), 2, S, S)
    x = workloads.scores_cpu(shape, dtype, 1.0, 3600 + S + off)
    y_st = oracle.softmax(workloads.to_storage(x), lens, 0.8, dtype)
    dy = workloads.scores_cpu(shape, dtype, 1.0, 3601 + S + off)
    dy_st = workloads.to_storage(dy)
    ref = oracle.backward_f64(y_st, dy_st, lens, 0.8, dtype)
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    y_dev = offset_copy(workloads.from_storage(y_st, dtype), dtype, off)
    dy_dev = offset_copy(dy, dtype, off)
    got = {}
    for path in ("auto", expect):
        dx = offset_copy(torch.zeros_like(dy), dtype, off)
        print(f"backward switch S={S} dtype={DNAME[dtype]} offset={off} path={path}", flush=True)
        g.backward(y_dev, dy_dev, sl, 0.8, out=dx, path=path)
        torch.cuda.synchronize()
        got[path] = workloads.to_storage(dx.cpu())
    n = len(lens) * 2 * S
    check_rows(got["auto"].reshape(n, S), ref.reshape(n, S), y_st.reshape(n, S),
               dy_st.reshape(n, S), np.repeat(np.asarray(lens), 2 * S),
               np.tile(np.arange(S), len(lens) * 2), 0.8, dtype)
    assert np.array_equal(bits(got["auto"]), bits(got[expect]))


def test_backward_long_rows():
    for dtype, S, lens in ((workloads.F16, 4096, [4096, 1500]), (workloads.BF16, 8192, [8000])):
        for path in ("auto", "block", "stream"):
            run_case((len(lens), 1, S, S), dtype, lens, 0.125, path, seed=200 + S)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_backward_widest_wave_rows(dtype):
    """Rows of 4000 elements on the one-wavefront path: sixteen binary32 or eight 16-bit
    vectors per lane, the largest layouts of that path."""
    run_case((2, 1, 4000, 4000), dtype, [4000, 1401], 0.6, "wave", seed=400)


def test_backward_block_rows_every_element():
    """Rows that fill the block path's registers (binary16 40000 at eight 16-byte vectors per
    lane, binary32 65536 forced to sixteen; bfloat16 65536 at eight is the long workload's
    layout, checked by test_backward_full_long_rows), y uniform in [0, 2/L) (rows that sum to
    about 1, like the forward's outputs the error bound is derived for), dy normal; every
    element against the oracle's backward row entry point, in blocks of rows."""
    for dtype, S, path in ((workloads.F16, 40000, "auto"), (workloads.F32, 65536, "block")):
        L = S - 17
        print(f"backward block rows S={S} dtype={DNAME[dtype]} path={path}", flush=True)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(S)
        # uniform in [0, 2/L): a row sums to about 1, as a forward output does
        y = torch.rand((1, 1, S, S), generator=gen, device="cuda").mul_(2.0 / L).to(
            workloads.torch_dtype(dtype))
        dy = workloads.scores_device((1, 1, S, S), dtype, 1.0, S + 1)
        sl = torch.as_tensor(np.asarray([L], dtype=np.int32)).cuda()
        dx = g.backward(y, dy, sl, 0.3, path=path)
        torch.cuda.synchronize()
        worst = check_rows_backward_against_oracle(y, dy, dx, np.asarray([L], np.int32), 0.3,
                                                   dtype, U[dtype], TINY[dtype])
        print(f"S={S} {path}: every element of the backward checked, worst error {worst:.3g}",
              flush=True)
        del y, dy, dx
        torch.cuda.empty_cache()


def test_backward_in_place_and_poison():
    """dx written over dy gives the same bits; NaN in masked cells of y and dy changes
    nothing."""
    for dtype in DTYPES:
        S = 300
        lens = [S, 120, 0]
        dx_st, y_dev, dy, sl = run_case((3, 2, S, S), dtype, lens, 1.0, seed=300)
        dy_dev = dy.cuda()
        g.backward(y_dev, dy_dev, sl, 1.0, out=dy_dev)
        torch.cuda.synchronize()
        assert np.array_equal(bits(workloads.to_storage(dy_dev.cpu())), bits(dx_st))
        yp, gp = y_dev.clone(), dy.cuda()
        for b, L in enumerate(lens):
            masked = ~torch.as_tensor(kept_mask(S, L)).cuda()
            yp[b][:, masked] = float("nan")
            gp[b][:, masked] = float("inf")
        dxp = g.backward(yp, gp, sl, 1.0)
        torch.cuda.synchronize()
        assert np.array_equal(bits(workloads.to_storage(dxp.cpu())), bits(dx_st))


@pytest.mark.parametrize("name", ["readme_f32_3x64x1000", "readme_f32_12x64x1000",
                                  "scaled_f16_32x1x4096", "skewed_bf16_8x32x8192"])
def test_backward_full_workload(name):
    """A benchmark workload at full size through the default entry point, on real softmax
    rows: y is the oracle's rounded forward of the workload's own seeded scores (one-hot row
    0, peaked short rows, rows of every length up to S), dy normal; every element of every
    plane against the oracle's backward."""
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    print(f"backward full workload {name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    y = oracle_forward_to_device(x, lens, w.scale, w.dtype)
    del x
    torch.cuda.empty_cache()
    dy = workloads.scores_device(w.shape, w.dtype, 1.0, 4243)
    sl = torch.as_tensor(lens).cuda()
    dx = g.backward(y, dy, sl, w.scale)
    torch.cuda.synchronize()
    worst = check_planes_backward_against_oracle(y, dy, dx, lens, w.scale, w.dtype, U[w.dtype],
                                                 TINY[w.dtype])
    print(f"{name}: every plane of the backward checked, worst error {worst:.3g}", flush=True)
    del y, dy, dx
    torch.cuda.empty_cache()


def test_backward_full_long_rows():
    """The 65536-wide-row workload (bf16 2 x 2 x 65536, the block path at eight vectors per
    lane) at full size on real softmax rows: y is the oracle's rounded forward of the
    workload's own seeded scores (built in blocks of rows on host threads), dy normal; every
    element against the oracle's backward row entry point, in blocks of 512 rows."""
    w = workloads.WORKLOADS["long_bf16_2x2x65536"]
    lens = workloads.seq_lens(w)
    print(f"backward full workload {w.name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    y = oracle_forward_to_device(x, lens, w.scale, w.dtype)
    del x
    torch.cuda.empty_cache()
    dy = workloads.scores_device(w.shape, w.dtype, 1.0, 4245)
    dx = g.backward(y, dy, torch.as_tensor(lens).cuda(), w.scale)
    torch.cuda.synchronize()
    worst = check_rows_backward_against_oracle(y, dy, dx, lens, w.scale, w.dtype, U[w.dtype],
                                               TINY[w.dtype])
    print(f"{w.name}: every element of the backward checked, worst error {worst:.3g}", flush=True)
    del y, dy, dx
    torch.cuda.empty_cache()


def test_backward_full_long_bf16_2x1x100000():
    """The 100000-wide-row workload (bf16 2 x 1 x 100000, lengths 100000 and 70000) at full
    size on real softmax rows: y is the oracle's rounded forward of the workload's own seeded
    scores, dy normal. Rows whose kept prefix passes 65536 elements keep 8 vectors per lane in
    registers and the rest of y and dy in LDS; shorter rows of the same launch fit the
    registers, rows at or past the length are zeros. Every element against the oracle's
    backward row entry point; the forced block path (the same kernel) and the band [-S, 0]
    (the same kept set) give the same bits."""
    w = workloads.WORKLOADS["long_bf16_2x1x100000"]
    lens = workloads.seq_lens(w)
    print(f"backward full workload {w.name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    y = oracle_forward_to_device(x, lens, w.scale, w.dtype)
    del x
    torch.cuda.empty_cache()
    dy = workloads.scores_device(w.shape, w.dtype, 1.0, 4246)
    sl = torch.as_tensor(lens).cuda()
    dx = g.backward(y, dy, sl, w.scale)
    torch.cuda.synchronize()
    worst = check_rows_backward_against_oracle(y, dy, dx, lens, w.scale, w.dtype, U[w.dtype],
                                               TINY[w.dtype])
    print(f"{w.name}: every element of the backward checked, worst error {worst:.3g}", flush=True)
    for tag, run in (("block", lambda: g.backward(y, dy, sl, w.scale, path="block")),
                     ("band [-S, 0]", lambda: g.backward_band(y, dy, sl, -w.S, 0, w.scale))):
        other = run()
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), dx.view(torch.int16)), tag
        del other
    del y, dy, dx
    torch.cuda.empty_cache()


def test_backward_stash_rows():
    """Rows past 8 vectors per lane that the LDS stash takes: binary32 rows of 40000 (10000
    vectors, 8192 of them in registers), binary16 rows of 70000 (8750 vectors plus up to 6 of
    line slack), and a bfloat16 causal window of 70001 columns on rows
    of 100000, whose rows hold only their interval (up to 8766 vectors). y is uniform in
    [0, 2/n) over the kept set (n its width) and zero elsewhere, dy normal. With y zero
    outside the window, D and every kept dx of the window equal those of the grouped tril
    mask, so every element compares with the oracle's tril backward rows; the window's
    masked elements must also be +0 bit for bit. Paired rows and dx written over dy give the
    same bits."""
    cases = ((workloads.F32, 40000, 40000 - 3, None, 0.7),
             (workloads.F16, 70000, 70000 - 9, None, 0.45),
             (workloads.BF16, 100000, 100000 - 5, -70000, 0.3))
    for dtype, S, L, lo, scale in cases:
        print(f"backward stash rows S={S} dtype={DNAME[dtype]} L={L} lo={lo}", flush=True)
        n = L if lo is None else -lo + 1
        gen = torch.Generator(device="cuda")
        gen.manual_seed(S + 7)
        y = torch.rand((1, 1, S, S), generator=gen, device="cuda").mul_(2.0 / n).to(
            workloads.torch_dtype(dtype))
        if lo is not None:
            y.triu_(lo)
        dy = workloads.scores_device((1, 1, S, S), dtype, 1.0, S + 8)
        sl = torch.as_tensor(np.asarray([L], dtype=np.int32)).cuda()
        dx = (g.backward(y, dy, sl, scale) if lo is None
              else g.backward_band(y, dy, sl, lo, 0, scale))
        torch.cuda.synchronize()
        lens = np.asarray([L], np.int32)
        worst = check_rows_backward_against_oracle(y, dy, dx, lens, scale, dtype, U[dtype],
                                                   TINY[dtype])
        ib = torch.int32 if dtype == workloads.F32 else torch.int16
        if lo is not None:
            assert torch.equal(dx.triu(lo).view(ib), dx.view(ib)), "window: masked bits set"
        # the same bits with rows r and S-1-r paired in one unit (two rows through one stash
        # in turn), and with dx written over dy (both passes read dy before any dx store)
        paired = (g.backward(y, dy, sl, scale, flags=1) if lo is None
                  else g.backward_band(y, dy, sl, lo, 0, scale, flags=1))
        inplace = dy.clone()
        if lo is None:
            g.backward(y, inplace, sl, scale, out=inplace)
        else:
            g.backward_band(y, inplace, sl, lo, 0, scale, out=inplace)
        torch.cuda.synchronize()
        assert torch.equal(paired.view(ib), dx.view(ib)), "paired rows changed bits"
        assert torch.equal(inplace.view(ib), dx.view(ib)), "in place changed bits"
        del paired, inplace
        print(f"S={S}: every element checked, worst error {worst:.3g}", flush=True)
        del y, dy, dx
        torch.cuda.empty_cache()
