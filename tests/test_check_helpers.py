"""The every-plane parity checker of the GPU tests, run on host tensors: it accepts the
oracle's own rounded output and rejects a planted error in a kept element, a nonzero bit in
the masked region and a non-finite kept value."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gtms_check import (TOL, check_planes_against_oracle, check_planes_backward_against_oracle,
                        check_rows_against_oracle, check_rows_backward_against_oracle,
                        oracle_forward_to_device)

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.F16, workloads.BF16])
def test_every_plane_checker(dtype):
    lens = np.asarray([5, 0, 37, 41], dtype=np.int32)
    x = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=42)
    y = oracle.softmax(workloads.to_storage(x), lens, 0.7, dtype)
    y_t = workloads.from_storage(y, dtype)
    # a chunk of 5 planes: the 12 planes are checked in three chunks
    chunk = 5 * 2 * 40 * 40 * (4 if dtype == workloads.F32 else 2)
    assert check_planes_against_oracle(x, y_t, lens, 0.7, dtype, chunk_bytes=chunk) <= TOL[dtype]

    def planted(b, m, r, c, value):
        t = y_t.clone()
        t[b, m, r, c] = value
        return t

    kept_val = float(y_t[2, 1, 20, 3])
    with pytest.raises(AssertionError, match="max error"):
        check_planes_against_oracle(x, planted(2, 1, 20, 3, kept_val + 0.05), lens, 0.7, dtype,
                                    chunk_bytes=chunk)
    with pytest.raises(AssertionError, match="masked region"):
        check_planes_against_oracle(x, planted(0, 2, 4, 5, 1e-30 if dtype == workloads.F32
                                               else 1e-3), lens, 0.7, dtype, chunk_bytes=chunk)
    with pytest.raises(AssertionError, match="masked region"):
        check_planes_against_oracle(x, planted(1, 0, 0, 0, -0.0), lens, 0.7, dtype,
                                    chunk_bytes=chunk)
    with pytest.raises(AssertionError, match="non-finite"):
        check_planes_against_oracle(x, planted(3, 2, 39, 39, float("nan")), lens, 0.7, dtype,
                                    chunk_bytes=chunk)


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.F16, workloads.BF16])
def test_every_plane_backward_checker(dtype):
    u = {workloads.F32: 2.0 ** -21, workloads.F16: 2.0 ** -10, workloads.BF16: 2.0 ** -7}[dtype]
    tiny = {workloads.F32: 2.0 ** -150, workloads.F16: 2.0 ** -25, workloads.BF16: 2.0 ** -134}[dtype]
    lens = np.asarray([5, 0, 37, 41], dtype=np.int32)
    x = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=43)
    y_st = oracle.softmax(workloads.to_storage(x), lens, 0.7, dtype)
    dy = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=44)
    ref = oracle.backward_f64(y_st, workloads.to_storage(dy), lens, 0.7, dtype)
    y_t = workloads.from_storage(y_st, dtype)
    # the oracle's backward rounded to the element type passes
    dx = torch.as_tensor(ref).to(y_t.dtype)
    chunk = 5 * 3 * 40 * 40 * (4 if dtype == workloads.F32 else 2)
    check_planes_backward_against_oracle(y_t, dy, dx, lens, 0.7, dtype, u, tiny,
                                         chunk_bytes=chunk, row_block=16)

    def planted(b, m, r, c, value):
        t = dx.clone()
        t[b, m, r, c] = value
        return t

    with pytest.raises(AssertionError, match="beyond the bound"):
        check_planes_backward_against_oracle(
            y_t, dy, planted(2, 1, 20, 3, float(dx[2, 1, 20, 3]) + 0.05), lens, 0.7, dtype, u,
            tiny, chunk_bytes=chunk, row_block=16)
    with pytest.raises(AssertionError, match="masked region"):
        check_planes_backward_against_oracle(
            y_t, dy, planted(1, 0, 3, 2, -0.0), lens, 0.7, dtype, u, tiny, chunk_bytes=chunk,
            row_block=16)


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_row_block_checker(dtype):
    lens = np.asarray([5, 0, 37, 41], dtype=np.int32)
    x = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=45)
    y = workloads.from_storage(oracle.softmax(workloads.to_storage(x), lens, 0.7, dtype), dtype)
    assert check_rows_against_oracle(x, y, lens, 0.7, dtype, rows_per_call=16) <= TOL[dtype]
    bad = y.clone()
    bad[2, 1, 33, 30] += 0.05
    with pytest.raises(AssertionError, match="max error"):
        check_rows_against_oracle(x, bad, lens, 0.7, dtype, rows_per_call=16)
    bad = y.clone()
    bad[3, 0, 12, 13] = -0.0
    with pytest.raises(AssertionError, match="masked region"):
        check_rows_against_oracle(x, bad, lens, 0.7, dtype, rows_per_call=16)


def test_row_block_backward_checker():
    dtype = workloads.F16
    u, tiny = 2.0 ** -10, 2.0 ** -25
    lens = np.asarray([5, 0, 37, 41], dtype=np.int32)
    x = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=46)
    y_st = oracle.softmax(workloads.to_storage(x), lens, 0.7, dtype)
    dy = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=47)
    ref = oracle.backward_f64(y_st, workloads.to_storage(dy), lens, 0.7, dtype)
    y_t = workloads.from_storage(y_st, dtype)
    dx = torch.as_tensor(ref).to(y_t.dtype)
    check_rows_backward_against_oracle(y_t, dy, dx, lens, 0.7, dtype, u, tiny, rows_per_call=16)
    bad = dx.clone()
    bad[2, 1, 20, 3] += 0.05
    with pytest.raises(AssertionError, match="beyond the bound"):
        check_rows_backward_against_oracle(y_t, dy, bad, lens, 0.7, dtype, u, tiny,
                                           rows_per_call=16)
    bad = dx.clone()
    bad[0, 2, 4, 5] = 1e-3
    with pytest.raises(AssertionError, match="masked region"):
        check_rows_backward_against_oracle(y_t, dy, bad, lens, 0.7, dtype, u, tiny,
                                           rows_per_call=16)


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.F16, workloads.BF16])
def test_oracle_forward_to_device(dtype):
    """The chunked, per-plane, threaded forward that builds the full-size backward's y gives
    the bits of one oracle call over the whole tensor."""
    lens = np.asarray([5, 0, 37, 41], dtype=np.int32)
    x = workloads.scores_cpu((4, 3, 40, 40), dtype, 1.0, seed=48)
    whole = oracle.softmax(workloads.to_storage(x), lens, 0.7, dtype)
    chunk = 5 * 2 * 40 * 40 * (4 if dtype == workloads.F32 else 2)
    y = oracle_forward_to_device(x, lens, 0.7, dtype, chunk_bytes=chunk)
    assert y.dtype == x.dtype and tuple(y.shape) == tuple(x.shape)
    got = workloads.to_storage(y)
    assert np.array_equal(got.view(np.uint8), whole.view(np.uint8))
    # planes larger than a chunk: blocks of rows through the row entry point, rounded through
    # binary32 (the same values here except at rare ties of the 16-bit rounding)
    yr = oracle_forward_to_device(x, lens, 0.7, dtype, chunk_bytes=1000, rows_per_call=7)
    assert yr.dtype == x.dtype and tuple(yr.shape) == tuple(x.shape)
    got_r = workloads.to_storage(yr)
    ref = oracle.softmax_f64(workloads.to_storage(x), lens, 0.7, dtype)
    if dtype == workloads.F32:
        assert np.array_equal(got_r.view(np.uint8), whole.view(np.uint8))
    else:
        # within half an ulp of the 16-bit type plus the binary32 step, and masked cells +0
        from gtms_check import bits, to_f64
        assert not bits(got_r)[ref == 0].any()
        assert np.max(np.abs(to_f64(got_r, dtype) - ref)) <= 2.0 ** -8 * max(1.0, np.max(ref))


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.F16, workloads.BF16])
def test_window_by_minus_infinity(dtype):
    """The reduction behind the long-row band tests: with the scores below a causal window set
    to -inf, the oracle's grouped tril softmax (whole tensor and row entry point) equals its
    band softmax of the same input exactly, masked cells +0 included."""
    S, lo, L = 12, -4, 10
    x = workloads.scores_cpu((1, 1, S, S), dtype, 1.0, seed=61)
    for r in range(S):
        for c in range(S):
            if c < r + lo:
                x[0, 0, r, c] = float("-inf")
    xs = workloads.to_storage(x)
    band = oracle.softmax_band_f64(xs, [L], lo, 0, 0.3, dtype)
    tril = oracle.softmax_f64(xs, [L], 0.3, dtype)
    rows = oracle.softmax_rows_f64(xs[0, 0], np.arange(S), [L] * S, 0.3, dtype)
    assert np.array_equal(tril.view(np.uint64), band.view(np.uint64))
    assert np.array_equal(rows.view(np.uint64), band[0, 0].view(np.uint64))
