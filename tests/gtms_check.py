"""Helpers of the GPU parity tests: the kept set, comparisons against the oracle."""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import workloads

# tolerances: max |GPU - oracle fp64| on kept elements, per element type
TOL = {workloads.F32: 2e-6, workloads.F16: 2e-3, workloads.BF16: 8e-3}


def kept_mask(S: int, L: int) -> np.ndarray:
    """bool [S, S]: element (r, c) is kept when c <= r < L (L clamped to [0, S])."""
    L = min(max(int(L), 0), S)
    r = np.arange(S)[:, None]
    c = np.arange(S)[None, :]
    return (c <= r) & (r < L)


def kept_row(S: int, L: int, r: int) -> np.ndarray:
    """bool [S]: the kept columns of row r (c <= r < L, L clamped to [0, S])."""
    L = min(max(int(L), 0), S)
    return (np.arange(S) <= r) & (r < L)


def to_f64(storage: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp64 values of raw element storage (float32, or uint16 bits)."""
    if dtype == workloads.F32:
        return storage.astype(np.float64)
    if dtype == workloads.F16:
        return storage.view(np.float16).astype(np.float64)
    return (storage.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bits(storage: np.ndarray) -> np.ndarray:
    return storage.view(np.uint32) if storage.dtype == np.float32 else storage.view(np.uint16)


def check_against_oracle(out_storage: np.ndarray, ref64: np.ndarray, lens, dtype: int,
                         tol: float | None = None) -> float:
    """Masked elements must be +0 bit for bit; kept elements within the tolerance.
    Returns the max abs error on kept elements."""
    tol = TOL[dtype] if tol is None else tol
    B, M, S, _ = out_storage.shape
    got = to_f64(out_storage, dtype)
    ob = bits(out_storage)
    worst = 0.0
    for b in range(B):
        keep = kept_mask(S, lens[b])
        for m in range(M):
            masked_bits = ob[b, m][~keep]
            assert not masked_bits.any(), f"nonzero bits in masked region b={b} m={m}"
            if keep.any():
                err = np.abs(got[b, m][keep] - ref64[b, m][keep])
                e = float(np.nanmax(err)) if err.size else 0.0
                assert np.all(np.isfinite(got[b, m][keep])), f"non-finite output b={b} m={m}"
                assert e <= tol, f"b={b} m={m}: max error {e:.3g} > {tol:.3g}"
                worst = max(worst, e)
    return worst


def esize(dtype: int) -> int:
    return 4 if dtype == workloads.F32 else 2


def path_ok(path, S, dtype, aligned=True):
    """Whether a register-held path can take rows of S elements: a lane holds up to 16
    slots of 16 bytes (rows whose byte length is a multiple of 16, on an aligned tensor)
    or of one element otherwise; the block path has up to 16 wavefronts. A row of 16-byte
    slots of at least 128 bytes may also write up to (128 - gcd(bytes, 128)) / 16 slots of
    its predecessor's last line (torch allocations are 128-byte aligned)."""
    if path in ("auto", "stream"):
        return True
    row_bytes = S * esize(dtype)
    wide = aligned and row_bytes % 16 == 0
    vec = 16 // esize(dtype) if wide else 1
    slack = (128 - math.gcd(row_bytes, 128)) // 16 if wide and row_bytes >= 128 else 0
    return -(-S // vec) + slack <= 64 * 16 * (16 if path == "block" else 1)


def host_threads() -> int:
    """Host threads for oracle work: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def check_planes_against_oracle(x_dev, y_dev, lens, scale: float, dtype: int,
                                tol: float | None = None, chunk_bytes: int = 4 << 30,
                                plane_ref=None) -> float:
    """Every element of a [B, M, S, S] result on the device against the oracle's fp64 result:
    masked elements +0 bit for bit, kept elements finite and within the tolerance. Planes are
    copied to the host in chunks of at most chunk_bytes (input and output) and checked one
    oracle call per plane on host threads (ctypes releases the GIL during the call). Returns
    the max abs error on kept elements.

    plane_ref(x_plane, p) -> (ref [S, S] fp64, keep [S, S] bool) gives the reference and the
    kept set of flat plane p = b * M + m from its raw input [1, 1, S, S]; by default the
    grouped tril mask with the lengths `lens` (the mask variants pass their own)."""
    import oracle

    tol = TOL[dtype] if tol is None else tol
    B, M, S, _ = y_dev.shape
    es = esize(dtype)
    xf = x_dev.reshape(B * M, S, S)
    yf = y_dev.reshape(B * M, S, S)
    if plane_ref is None:
        keeps = {}
        for b in range(B):
            L = min(max(int(lens[b]), 0), S)
            if L not in keeps:
                keeps[L] = kept_mask(S, L)

        def plane_ref(x_plane, p):
            b = p // M
            ref = oracle.softmax_f64(x_plane, lens[b:b + 1], scale, dtype)[0, 0]
            return ref, keeps[min(max(int(lens[b]), 0), S)]

    per_chunk = max(1, chunk_bytes // (2 * S * S * es))
    worst = 0.0
    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        for p0 in range(0, B * M, per_chunk):
            p1 = min(B * M, p0 + per_chunk)
            xs = workloads.to_storage(xf[p0:p1].cpu())
            ys = workloads.to_storage(yf[p0:p1].cpu())

            def one(i, xs=xs, ys=ys, p0=p0):
                p = p0 + i
                ref, keep = plane_ref(xs[i:i + 1][None], p)
                assert not bits(ys[i])[~keep].any(), f"nonzero bits in masked region of plane {p}"
                got = to_f64(ys[i][keep], dtype)
                assert np.all(np.isfinite(got)), f"non-finite kept output in plane {p}"
                e = float(np.max(np.abs(got - ref[keep]))) if got.size else 0.0
                assert e <= tol, f"plane {p}: max error {e:.3g} > {tol:.3g}"
                return e

            worst = max([worst] + list(pool.map(one, range(p1 - p0))))
            del xs, ys
    return worst


def oracle_forward_to_device(x_dev, lens, scale: float, dtype: int,
                             chunk_bytes: int = 4 << 30, rows_per_call: int = 512):
    """The oracle's forward of a [B, M, S, S] device tensor, rounded into the element type and
    returned as a new device tensor. Planes that fit a host chunk (chunk_bytes for x and y
    together) go to the host a chunk at a time, one oracle call per plane on host threads, and
    come back rounded by the oracle. Larger planes go through the oracle's row entry point in
    blocks of rows_per_call rows on host threads; its fp64 rows are rounded to the element
    type through binary32 (for 16-bit types this differs from one rounding only at rare
    ties; the rows are inputs, and each test's reference takes them as they are). Lets a
    full-size backward run on real softmax rows that do not come from the GPU path. Prints
    its progress on large planes."""
    import oracle
    import torch

    B, M, S, _ = x_dev.shape
    y_dev = torch.empty_like(x_dev)
    per_chunk = chunk_bytes // (2 * S * S * esize(dtype))
    if per_chunk < 1:
        tasks = [(b, m, r0) for b in range(B) for m in range(M)
                 for r0 in range(0, S, rows_per_call)]
        done = [0]

        def rows(task):
            b, m, r0 = task
            r1 = min(S, r0 + rows_per_call)
            xs = workloads.to_storage(x_dev[b, m, r0:r1].cpu())
            ref = oracle.softmax_rows_f64(xs, np.arange(r0, r1), [lens[b]] * (r1 - r0), scale,
                                          dtype)
            y_dev[b, m, r0:r1].copy_(
                torch.from_numpy(ref).to(torch.float32).to(workloads.torch_dtype(dtype)))
            done[0] += 1
            if done[0] % max(1, len(tasks) // 10) == 0:
                print(f"oracle forward: {done[0]} of {len(tasks)} row blocks", flush=True)

        with ThreadPoolExecutor(max_workers=host_threads()) as pool:
            list(pool.map(rows, tasks))
        if y_dev.is_cuda:
            torch.cuda.synchronize()
        return y_dev
    xf = x_dev.reshape(B * M, S, S)
    yf = y_dev.reshape(B * M, S, S)
    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        for p0 in range(0, B * M, per_chunk):
            p1 = min(B * M, p0 + per_chunk)
            xs = workloads.to_storage(xf[p0:p1].cpu())
            ys = np.empty_like(xs)

            def one(i, xs=xs, ys=ys, p0=p0):
                b = (p0 + i) // M
                ys[i] = oracle.softmax(xs[i:i + 1][None], lens[b:b + 1], scale, dtype)[0, 0]

            list(pool.map(one, range(p1 - p0)))
            yf[p0:p1].copy_(workloads.from_storage(ys, dtype))
            del xs, ys
    return y_dev


def check_planes_backward_against_oracle(y_dev, dy_dev, dx_dev, lens, scale: float, dtype: int,
                                         u: float, tiny: float, chunk_bytes: int = 4 << 30,
                                         row_block: int = 1024, plane_ref=None) -> float:
    """Every element of a backward result dx [B, M, S, S] on the device against the oracle's
    fp64 backward of the same y and dy: masked elements +0 bit for bit; kept elements finite
    and within u * |dx_ref| + 1e-5 * |scale| * y_c * max_k |dy_k| + tiny (max over the row's
    kept columns). Planes go to the host in chunks of at most chunk_bytes (three tensors),
    one oracle call per plane on host threads; a plane is compared in blocks of row_block rows.
    Returns the max abs error on kept elements.

    plane_ref(y_plane, dy_plane, p) -> (ref [S, S] fp64, keep [S, S] bool) gives the reference
    and kept set of flat plane p from its raw inputs [1, 1, S, S]; by default the grouped tril
    mask with the lengths `lens` (the mask variants pass their own)."""
    import oracle

    B, M, S, _ = dx_dev.shape
    es = esize(dtype)
    flat = [t.reshape(B * M, S, S) for t in (y_dev, dy_dev, dx_dev)]
    if plane_ref is None:
        keeps = {}
        for b in range(B):
            L = min(max(int(lens[b]), 0), S)
            if L not in keeps:
                keeps[L] = kept_mask(S, L)

        def plane_ref(y_plane, dy_plane, p):
            b = p // M
            ref = oracle.backward_f64(y_plane, dy_plane, lens[b:b + 1], scale, dtype)[0, 0]
            return ref, keeps[min(max(int(lens[b]), 0), S)]

    per_chunk = max(1, chunk_bytes // (3 * S * S * es))
    worst = 0.0
    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        for p0 in range(0, B * M, per_chunk):
            p1 = min(B * M, p0 + per_chunk)
            ys, gs, ds = (workloads.to_storage(t[p0:p1].cpu()) for t in flat)

            def one(i, ys=ys, gs=gs, ds=ds, p0=p0):
                p = p0 + i
                ref, keep = plane_ref(ys[i:i + 1][None], gs[i:i + 1][None], p)
                assert not bits(ds[i])[~keep].any(), f"nonzero bits in masked region of plane {p}"
                e = 0.0
                for r0 in range(0, S, row_block):
                    r1 = min(S, r0 + row_block)
                    k = keep[r0:r1]
                    if not k.any():
                        continue
                    got = to_f64(ds[i, r0:r1], dtype)
                    yv = to_f64(ys[i, r0:r1], dtype)
                    gv = np.where(k, np.abs(to_f64(gs[i, r0:r1], dtype)), 0.0)
                    gmax = gv.max(axis=1, keepdims=True)
                    err = np.abs(got - ref[r0:r1])
                    bound = u * np.abs(ref[r0:r1]) + 1e-5 * abs(scale) * yv * gmax + tiny
                    assert np.all(np.isfinite(got[k])), f"non-finite kept output in plane {p}"
                    bad = k & ~(err <= bound)
                    assert not bad.any(), \
                        f"plane {p}: {int(bad.sum())} kept elements beyond the bound"
                    e = max(e, float(np.max(np.where(k, err, 0.0))))
                return e

            worst = max([worst] + list(pool.map(one, range(p1 - p0))))
            del ys, gs, ds
    return worst


def _run_blocks(one, tasks, what: str = "rows checked") -> float:
    """Runs one(task) on host threads and returns the max of the results, printing progress
    every tenth of the tasks (long checks must not run silently)."""
    done = [0]

    def step(task):
        e = one(task)
        done[0] += 1
        if len(tasks) >= 50 and done[0] % (len(tasks) // 10) == 0:
            print(f"{what}: {done[0]} of {len(tasks)} blocks", flush=True)
        return e

    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        return max([0.0] + list(pool.map(step, tasks)))


def check_rows_against_oracle(x_dev, y_dev, lens, scale: float, dtype: int,
                              tol: float | None = None, rows_per_call: int = 1024) -> float:
    """Every element of a [B, M, S, S] forward result on the device, for planes too large to
    hand to the oracle whole: blocks of rows_per_call rows go to the host and through the
    oracle's row entry point, one block per host thread. Masked elements +0 bit for bit, kept
    elements finite and within the tolerance. Returns the max abs error on kept elements."""
    import oracle

    tol = TOL[dtype] if tol is None else tol
    B, M, S, _ = y_dev.shape
    col = np.arange(S)[None, :]
    tasks = [(b, m, r0) for b in range(B) for m in range(M) for r0 in range(0, S, rows_per_call)]

    def one(task):
        b, m, r0 = task
        r1 = min(S, r0 + rows_per_call)
        L = min(max(int(lens[b]), 0), S)
        xs = workloads.to_storage(x_dev[b, m, r0:r1].cpu())
        ys = workloads.to_storage(y_dev[b, m, r0:r1].cpu())
        r = np.arange(r0, r1)[:, None]
        keep = (col <= r) & (r < L)
        assert not bits(ys)[~keep].any(), f"nonzero bits in masked region of b={b} m={m} rows {r0}.."
        if not keep.any():
            return 0.0
        ref = oracle.softmax_rows_f64(xs, np.arange(r0, r1), [lens[b]] * (r1 - r0), scale, dtype)
        got = to_f64(ys[keep], dtype)
        assert np.all(np.isfinite(got)), f"non-finite kept output in b={b} m={m} rows {r0}.."
        e = float(np.max(np.abs(got - ref[keep])))
        assert e <= tol, f"b={b} m={m} rows {r0}..{r1}: max error {e:.3g} > {tol:.3g}"
        return e

    return _run_blocks(one, tasks)


def check_rows_backward_against_oracle(y_dev, dy_dev, dx_dev, lens, scale: float, dtype: int,
                                       u: float, tiny: float, rows_per_call: int = 512) -> float:
    """The backward counterpart of check_rows_against_oracle: every element of dx against the
    oracle's backward row entry point, blocks of rows_per_call rows on host threads; masked
    elements +0 bit for bit, kept elements finite and within
    u * |dx_ref| + 1e-5 * |scale| * y_c * max_k |dy_k| + tiny. Returns the max abs error."""
    import oracle

    B, M, S, _ = dx_dev.shape
    col = np.arange(S)[None, :]
    tasks = [(b, m, r0) for b in range(B) for m in range(M) for r0 in range(0, S, rows_per_call)]

    def one(task):
        b, m, r0 = task
        r1 = min(S, r0 + rows_per_call)
        L = min(max(int(lens[b]), 0), S)
        ys, gs, ds = (workloads.to_storage(t[b, m, r0:r1].cpu()) for t in (y_dev, dy_dev, dx_dev))
        r = np.arange(r0, r1)[:, None]
        keep = (col <= r) & (r < L)
        assert not bits(ds)[~keep].any(), f"nonzero bits in masked region of b={b} m={m} rows {r0}.."
        if not keep.any():
            return 0.0
        ref = oracle.backward_rows_f64(ys, gs, np.arange(r0, r1), [lens[b]] * (r1 - r0), scale,
                                       dtype)
        got = to_f64(ds, dtype)
        yv = to_f64(ys, dtype)
        gmax = np.where(keep, np.abs(to_f64(gs, dtype)), 0.0).max(axis=1, keepdims=True)
        err = np.abs(got - ref)
        bound = u * np.abs(ref) + 1e-5 * abs(scale) * yv * gmax + tiny
        assert np.all(np.isfinite(got[keep])), f"non-finite kept output in b={b} m={m} rows {r0}.."
        bad = keep & ~(err <= bound)
        assert not bad.any(), f"b={b} m={m} rows {r0}..{r1}: {int(bad.sum())} kept elements beyond the bound"
        return float(np.max(np.where(keep, err, 0.0)))

    return _run_blocks(one, tasks)
