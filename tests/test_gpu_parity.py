"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Masked elements must be +0.0 bit for bit; kept elements must lie within the element type's
tolerance of the oracle's fp64 result (binary32 2e-6, binary16 2e-3, bfloat16 8e-3).
Small shapes and the benchmark workloads at full size, launched exactly as the benchmark
launches them, are compared element by element (the full sizes plane by plane on host
threads; rows of 40000 to 100000 elements, forced through each path, and the 65536-wide
workload in blocks of rows through the oracle's row entry point).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gtms_check import (bits, check_against_oracle, check_planes_against_oracle,
                        check_rows_against_oracle, kept_mask, oracle_forward_to_device, path_ok)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("GPU tests need a visible GPU", allow_module_level=True)

import variable_length_causal_amd as g  # noqa: E402

DTYPES = [workloads.F32, workloads.F16, workloads.BF16]
DNAME = {workloads.F32: "f32", workloads.F16: "f16", workloads.BF16: "bf16"}


def run_gpu(x_cpu, lens, scale, path="auto", flags=0, out=None):
    x = x_cpu.cuda()
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    y = g.forward(x, sl, scale, out=out, path=path, flags=flags)
    torch.cuda.synchronize()
    return y


def check_small(x_cpu, lens, scale, dtype, path="auto", flags=0):
    print(f"case shape={tuple(x_cpu.shape)} dtype={DNAME[dtype]} path={path} flags={flags} "
          f"lens={list(lens)} scale={scale}", flush=True)
    y = run_gpu(x_cpu, lens, scale, path, flags)
    out = workloads.to_storage(y.cpu())
    ref = oracle.softmax_f64(workloads.to_storage(x_cpu), lens, scale, dtype)
    return check_against_oracle(out, ref, lens, dtype)


# ------------------------------------------------------------------------ small shapes

def test_worked_example_shape():
    """The README's worked-example shape [3, 2, 5, 5] with lengths 3, 4, 5."""
    w = workloads.WORKLOADS["example_f32_3x2x5"]
    x = workloads.scores_cpu(w.shape, w.dtype, w.sigma, w.x_seed)
    lens = workloads.seq_lens(w)
    for path in ("auto", "wave", "block", "stream"):
        if path_ok(path, w.S, w.dtype):
            check_small(x, lens, w.scale, w.dtype, path)


S_SWEEP = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256,
           257, 511, 513, 1000, 1023, 1025]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_shape_sweep(dtype):
    """Every path over row lengths that cover one vector, several vectors, several 64-lane
    sweeps and ragged tails; lengths 0, 1, partial, S and beyond S, and negative."""
    for S in S_SWEEP:
        lens = [S, max(1, S // 2), 0, S + 3, -1, 1]
        x = workloads.scores_cpu((len(lens), 2, S, S), dtype, 1.5, seed=3000 + S)
        ref = oracle.softmax_f64(workloads.to_storage(x), lens, 0.7, dtype)
        for path in ("auto", "wave", "block", "stream"):
            if not path_ok(path, S, dtype):
                continue
            print(f"sweep S={S} dtype={DNAME[dtype]} path={path}", flush=True)
            y = run_gpu(x, lens, 0.7, path)
            check_against_oracle(workloads.to_storage(y.cpu()), ref, lens, dtype)


# Row lengths at which the automatic choice moves between the one-wavefront path and the
# block path. A wavefront holds 256 slots of 16 bytes; a row needs ceil(S / VEC) of them
# plus the slots it may write of its predecessor's last 128-byte line, (128 - gcd(row
# bytes, 128)) / 16 on a 128-byte aligned tensor and 7 on one that is not. Rows whose byte
# length is not a multiple of 16 take element accesses (one slot per element). Each case
# names the path the rule gives; the automatic call must match that forced path bit for bit.
SWITCH_CASES = [
    (workloads.F32, 1000, 0, "wave"), (workloads.F32, 1004, 0, "block"),
    (workloads.F32, 1008, 0, "wave"), (workloads.F32, 1012, 0, "block"),
    (workloads.F32, 1016, 0, "block"), (workloads.F32, 1020, 0, "block"),
    (workloads.F32, 1024, 0, "wave"), (workloads.F32, 1028, 0, "block"),
    (workloads.F32, 1032, 0, "block"), (workloads.F32, 1000, 16, "block"),
    (workloads.F32, 1024, 16, "block"),
] + [(dt, S, off, path) for dt in (workloads.F16, workloads.BF16) for S, off, path in (
    (2032, 0, "block"), (2040, 0, "block"), (2047, 0, "block"), (2048, 0, "wave"),
    (2049, 0, "block"), (2056, 0, "block"), (2048, 16, "block"))]


def offset_tensor(shape, dtype, offset_bytes):
    """A zeroed device tensor whose data starts offset_bytes past a 256-byte boundary."""
    tdt = workloads.torch_dtype(dtype)
    es = 4 if dtype == workloads.F32 else 2
    n = int(np.prod(shape))
    buf = torch.zeros(n + 256 // es, dtype=tdt, device="cuda")
    t = buf[offset_bytes // es:offset_bytes // es + n].view(shape)
    assert t.data_ptr() % 256 == offset_bytes
    return t


@pytest.mark.parametrize("case", SWITCH_CASES,
                         ids=lambda c: f"{DNAME[c[0]]}-{c[1]}-off{c[2]}-{c[3]}")
def test_auto_path_switch_sizes(case):
    """Forward through the automatic choice at the row lengths where it changes kernel,
    lengths S, S - 1, S / 2 and 0: every element against the oracle, and the same bits as
    the path the choice rule names."""
    dtype, S, off, expect = case
    lens = [S, S - 1, S // 2, 0]
    x_cpu = workloads.scores_cpu((len(lens), 2, S, S), dtype, 1.0, seed=3500 + S + off)
    ref = oracle.softmax_f64(workloads.to_storage(x_cpu), lens, 0.8, dtype)
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    got = {}
    for path in ("auto", expect):
        x = offset_tensor(x_cpu.shape, dtype, off)
        x.copy_(x_cpu.cuda())
        out = offset_tensor(x_cpu.shape, dtype, off)
        print(f"switch S={S} dtype={DNAME[dtype]} offset={off} path={path}", flush=True)
        g.forward(x, sl, 0.8, out=out, path=path)
        torch.cuda.synchronize()
        got[path] = workloads.to_storage(out.cpu())
    check_against_oracle(got["auto"], ref, lens, dtype)
    assert np.array_equal(bits(got["auto"]), bits(got[expect]))


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_unaligned_rows_take_the_scalar_path(dtype):
    """A tensor that starts off a 16-byte boundary, and rows whose byte length is not a
    multiple of 16, still give exact results (element-wide accesses)."""
    tdt = workloads.torch_dtype(dtype)
    for S in (12, 40, 100):
        lens = [S, S // 3, 0]
        x_cpu = workloads.scores_cpu((3, 2, S, S), dtype, 1.0, seed=4000 + S)
        n = x_cpu.numel()
        for path in ("auto", "wave", "block", "stream"):
            if not path_ok(path, S, dtype, aligned=False):
                continue
            buf_in = torch.zeros(n + 1, dtype=tdt, device="cuda")
            buf_out = torch.zeros(n + 1, dtype=tdt, device="cuda")
            x = buf_in[1:].view(x_cpu.shape)
            x.copy_(x_cpu.cuda())
            out = buf_out[1:].view(x_cpu.shape)
            assert x.data_ptr() % 16 != 0
            sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
            g.forward(x, sl, 1.0, out=out, path=path)
            torch.cuda.synchronize()
            ref = oracle.softmax_f64(workloads.to_storage(x_cpu), lens, 1.0, dtype)
            check_against_oracle(workloads.to_storage(out.cpu()), ref, lens, dtype)


@pytest.mark.parametrize("scale", [0.0, -1.25, 0.125, 3.0])
def test_scale_values(scale):
    for dtype in DTYPES:
        x = workloads.scores_cpu((2, 3, 70, 70), dtype, 1.0, seed=5000)
        check_small(x, [70, 33], scale, dtype)


def test_long_rows_every_path():
    """Rows of 4096 (binary16) and 8192 (bfloat16 and binary32) elements through each path
    that can hold them, compared on whole planes."""
    cases = [(workloads.F16, 4096, [4096, 2000], 0.125), (workloads.BF16, 8192, [8192], 0.125),
             (workloads.F32, 8192, [5000], 1.0)]
    for dtype, S, lens, scale in cases:
        x = workloads.scores_cpu((len(lens), 1, S, S), dtype, 2.0, seed=6000 + S)
        ref = oracle.softmax_f64(workloads.to_storage(x), lens, scale, dtype)
        for path in ("auto", "wave", "block", "stream"):
            if not path_ok(path, S, dtype):
                continue
            print(f"long rows S={S} dtype={DNAME[dtype]} path={path}", flush=True)
            y = run_gpu(x, lens, scale, path)
            check_against_oracle(workloads.to_storage(y.cpu()), ref, lens, dtype)


def test_very_long_rows_every_element():
    """Rows at the block path's widest layout, where each lane keeps sixteen raw 16-byte
    vectors (bfloat16 100000 and binary16 90000 through the automatic choice, 12.2 and 11
    vectors per lane with the last one partly used; binary32 65536 forced, exactly sixteen),
    beyond it (binary32 70000, the stream path) and at the automatic eight vectors per lane
    (binary16 40000): every element against the oracle, in blocks of 1024 rows through its
    row entry point."""
    for dtype, S, path in ((workloads.F32, 70000, "stream"), (workloads.F32, 65536, "block"),
                           (workloads.BF16, 100000, "auto"), (workloads.F16, 90000, "auto"),
                           (workloads.F16, 40000, "auto")):
        lens = [S - 17]
        print(f"very long rows S={S} dtype={DNAME[dtype]} path={path}", flush=True)
        x = workloads.scores_device((1, 1, S, S), dtype, 1.0, seed=7000 + S)
        sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
        y = g.forward(x, sl, 0.5, path=path)
        torch.cuda.synchronize()
        worst = check_rows_against_oracle(x, y, np.asarray(lens, np.int32), 0.5, dtype)
        print(f"S={S} {path}: every element checked, worst error {worst:.3g}", flush=True)
        del x, y
        torch.cuda.empty_cache()


# ------------------------------------------------------------------------ properties

def test_options_give_identical_bits():
    """Row pairing and the block order change the schedule, not the arithmetic."""
    for dtype in DTYPES:
        for S, path in ((300, "wave"), (1000, "block"), (700, "stream")):
            lens = [S, 123, 0, 1]
            x = workloads.scores_cpu((4, 2, S, S), dtype, 1.0, seed=8000 + S)
            base = bits(workloads.to_storage(run_gpu(x, lens, 0.9, path).cpu()))
            for flags in (g.FLAG_PAIR_ROWS, g.FLAG_PLAIN_ORDER, g.FLAG_PAIR_ROWS | g.FLAG_PLAIN_ORDER):
                other = bits(workloads.to_storage(run_gpu(x, lens, 0.9, path, flags).cpu()))
                assert np.array_equal(base, other), (DNAME[dtype], S, path, flags)


def test_empty_inputs_are_no_ops():
    """Zero batches, heads or rows: every entry point returns an empty result and launches
    nothing that touches memory."""
    for dtype in DTYPES:
        tdt = workloads.torch_dtype(dtype)
        for shape in ((0, 2, 5, 5), (2, 0, 5, 5), (2, 2, 0, 0)):
            B = shape[0]
            x = torch.zeros(shape, dtype=tdt, device="cuda")
            sl = torch.full((B,), 3, dtype=torch.int32, device="cuda")
            mask = torch.ones((1, 1, shape[2], shape[3]), dtype=torch.uint8, device="cuda")
            outs = [g.forward(x, sl, 1.0), g.backward(x, x.clone(), sl, 1.0),
                    g.forward_band(x, sl, -2, 0, 1.0), g.backward_band(x, x.clone(), sl, -2, 0),
                    g.forward_masked(x, mask, sl, 1.0), g.backward_masked(x, x.clone(), mask, sl)]
            torch.cuda.synchronize()
            for o in outs:
                assert tuple(o.shape) == shape and o.numel() == 0
    for dtype in (workloads.F16, workloads.BF16):
        tdt = workloads.torch_dtype(dtype)
        for shape in ((0, 2, 8, 64), (2, 0, 8, 64), (2, 2, 0, 64)):
            q = torch.zeros(shape, dtype=tdt, device="cuda")
            sl = torch.full((shape[0],), 3, dtype=torch.int32, device="cuda")
            o = g.attention(q, q.clone(), q.clone(), sl)
            torch.cuda.synchronize()
            assert tuple(o.shape) == shape and o.numel() == 0


def test_in_place_and_repeat_determinism():
    for dtype in DTYPES:
        S = 513
        lens = [S, 200, 0]
        x_cpu = workloads.scores_cpu((3, 2, S, S), dtype, 1.0, seed=9000)
        ref = bits(workloads.to_storage(run_gpu(x_cpu, lens, 1.0).cpu()))
        for _ in range(2):
            again = bits(workloads.to_storage(run_gpu(x_cpu, lens, 1.0).cpu()))
            assert np.array_equal(ref, again)
        x = x_cpu.cuda()
        sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
        g.forward(x, sl, 1.0, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(ref, bits(workloads.to_storage(x.cpu())))


def test_masked_poison_does_not_leak():
    """NaN and infinities in every masked cell leave the output bits unchanged."""
    for dtype in DTYPES:
        S = 200
        lens = [S, 77, 0]
        x = workloads.scores_cpu((3, 2, S, S), dtype, 1.0, seed=9100)
        ref = bits(workloads.to_storage(run_gpu(x, lens, 1.0).cpu()))
        for poison in (float("nan"), float("inf"), float("-inf")):
            p = x.clone()
            for b, L in enumerate(lens):
                keep = torch.as_tensor(kept_mask(S, L))
                p[b][:, ~keep] = poison
            for path in ("wave", "block", "stream"):
                got = bits(workloads.to_storage(run_gpu(p, lens, 1.0, path).cpu()))
                base = bits(workloads.to_storage(run_gpu(x, lens, 1.0, path).cpu()))
                assert np.array_equal(got, base), (DNAME[dtype], poison, path)
            assert np.array_equal(bits(workloads.to_storage(run_gpu(p, lens, 1.0).cpu())), ref)


def test_nan_in_kept_prefix_keeps_masked_zero():
    """A NaN among the kept scores makes that row's kept outputs NaN; its masked columns
    and every other row are unaffected."""
    S = 64
    x = workloads.scores_cpu((1, 1, S, S), workloads.F32, 1.0, seed=9200)
    x[0, 0, 40, 3] = float("nan")
    for path in ("wave", "block", "stream"):
        y = workloads.to_storage(run_gpu(x, [S], 1.0, path).cpu())
        assert np.all(np.isnan(y[0, 0, 40, :41]))
        assert not y[0, 0, 40, 41:].view(np.uint32).any()
        assert np.all(np.isfinite(y[0, 0, :40])) and np.all(np.isfinite(y[0, 0, 41:]))


# ------------------------------------------------------------------------ full workloads

def full_workload_check(name):
    """The workload at its real size, launched as the benchmark launches it (default entry
    point, fresh seeded input on the device): every element of every plane against the
    oracle (masked +0 bit for bit, kept within the tolerance), and kept rows summing to 1."""
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    print(f"full workload {name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    sl = torch.as_tensor(lens).cuda()
    y = g.forward(x, sl, w.scale)
    torch.cuda.synchronize()
    B, M, S, _ = w.shape
    worst = check_planes_against_oracle(x, y, lens, w.scale, w.dtype)
    sum_tol = {workloads.F32: 1e-5, workloads.F16: 4e-3, workloads.BF16: 1.6e-2}[w.dtype]
    for b in range(B):
        L = int(min(max(lens[b], 0), S))
        for m in range(M if L else 0):
            sums = y[b, m, :L].double().sum(dim=1)
            assert float((sums - 1).abs().max()) <= sum_tol, (name, b, m)
    print(f"{name}: every plane checked, worst error {worst:.3g}", flush=True)
    del x, y
    torch.cuda.empty_cache()


def test_full_readme_f32_3x64x1000():
    full_workload_check("readme_f32_3x64x1000")


def test_full_readme_f32_12x64x1000():
    full_workload_check("readme_f32_12x64x1000")


def test_full_scaled_f16_32x1x4096():
    full_workload_check("scaled_f16_32x1x4096")


def test_full_skewed_bf16_8x32x8192():
    full_workload_check("skewed_bf16_8x32x8192")


@pytest.mark.parametrize("case", ["readme_f32_3x64x1000", "scaled_f16_32x1x4096", "bf16_4x8x2048"])
def test_ulp_distance_to_rounded_oracle(case):
    """Diagnostic of pin P9: the distance in units in the last place between the GPU's output
    and the oracle's output rounded to the element type, over every kept element (outputs are
    non-negative, so bit patterns order like values). The tolerances above bound the absolute
    error; this reports how the results sit against correct rounding. Rounding into a 16-bit
    type from fp32 arithmetic (relative error near 1e-6, far below the type's half ulp) can
    land at most one step away from the correctly rounded value, which is asserted; binary32
    results carry the fp32 arithmetic's own error and are reported only."""
    if case in workloads.WORKLOADS:
        w = workloads.WORKLOADS[case]
        shape, dtype, sigma, scale, seed = w.shape, w.dtype, w.sigma, w.scale, w.x_seed
        lens = workloads.seq_lens(w)
    else:
        shape, dtype, sigma, scale, seed = (4, 8, 2048, 2048), workloads.BF16, 1.0, 0.125, 77
        lens = np.asarray([2048, 1500, 333, 1], np.int32)
    x = workloads.scores_device(shape, dtype, sigma, seed)
    y = g.forward(x, torch.as_tensor(lens).cuda(), scale)
    ref = oracle_forward_to_device(x, lens, scale, dtype)
    torch.cuda.synchronize()
    ib = torch.int32 if dtype == workloads.F32 else torch.int16
    S = shape[-1]
    keep = torch.ones((S, S), dtype=torch.bool, device="cuda").tril_()
    dmax, n, n0, n1 = 0, 0, 0, 0
    for b in range(shape[0]):
        L = int(min(max(int(lens[b]), 0), S))
        if L == 0:
            continue
        kb = keep[:L, :L]
        for m in range(shape[1]):
            d = (y[b, m, :L, :L].view(ib).to(torch.int64) -
                 ref[b, m, :L, :L].view(ib).to(torch.int64)).abs()[kb]
            dmax = max(dmax, int(d.max()))
            n += d.numel()
            n0 += int((d == 0).sum())
            n1 += int((d <= 1).sum())
    print(f"{case}: ulp distance to the rounded oracle over {n} kept elements: max {dmax}, "
          f"exact {n0 / n:.4f}, within 1 ulp {n1 / n:.6f}", flush=True)
    if dtype != workloads.F32:
        assert dmax <= 1, (case, dmax)
    del x, y, ref
    torch.cuda.empty_cache()


def test_side_stream_and_graph_replay():
    """The binding launches on the caller's current stream (a side stream here), and a
    captured HIP graph of forward + backward replays to the same bits as eager calls, with
    eager work and synchronisations between the replays."""
    S, lens = 520, [520, 300, 0]
    x = workloads.scores_cpu((3, 2, S, S), workloads.F32, 1.0, 77).cuda()
    dy = workloads.scores_cpu((3, 2, S, S), workloads.F32, 1.0, 78).cuda()
    sl = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
    ref_y = g.forward(x, sl, 0.5)
    ref_dx = g.backward(ref_y, dy, sl, 0.5)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.forward(x, sl, 0.5, out=y)
        g.backward(y, dy, sl, 0.5, out=dx)
    side.synchronize()
    assert torch.equal(y.view(torch.int32), ref_y.view(torch.int32))
    assert torch.equal(dx.view(torch.int32), ref_dx.view(torch.int32))
    graph = torch.cuda.CUDAGraph()
    y.fill_(float("nan"))
    dx.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.forward(x, sl, 0.5, out=y)
        g.backward(y, dy, sl, 0.5, out=dx)
    for i in range(3):
        y.fill_(float("nan"))
        dx.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref_y.view(torch.int32)), f"replay {i}"
        assert torch.equal(dx.view(torch.int32), ref_dx.view(torch.int32)), f"replay {i}"
        g.forward(x, sl, 0.25)   # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_variants_and_attention():
    """A captured HIP graph of the band and explicit-mask forwards, the band backward and the
    fused attention (whole tiles and the key split) replays to the eager calls' bits, three
    times, with eager work and synchronisations between the replays."""
    S, lens = 300, [300, 123, 0]
    x = workloads.scores_cpu((3, 2, S, S), workloads.BF16, 1.0, 91).cuda()
    dy = workloads.scores_cpu((3, 2, S, S), workloads.BF16, 1.0, 92).cuda()
    sl = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
    mask = torch.ones(S, S, dtype=torch.uint8, device="cuda").tril_(5)[None, None]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(93)
    Sa = 2048  # long enough for the key split
    q, k, v = (torch.randn((2, 2, Sa, 64), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    sla = torch.as_tensor(np.asarray([Sa, 1500], np.int32)).cuda()

    def run(outs):
        g.forward_band(x, sl, -40, 0, 0.5, out=outs[0])
        g.forward_masked(x, mask, sl, 0.5, out=outs[1])
        g.backward_band(outs[0], dy, sl, -40, 0, 0.5, out=outs[2])
        g.attention(q, k, v, sla, 0.125, out=outs[3], split="off")
        g.attention(q, k, v, sla, 0.125, out=outs[4], split="on")

    ref = [torch.empty_like(x) for _ in range(3)] + [torch.empty_like(q) for _ in range(2)]
    run(ref)
    torch.cuda.synchronize()
    outs = [torch.empty_like(t) for t in ref]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(outs)
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {i} output {j}"
        g.forward_band(x, sl, -7, 3, 0.25)  # eager work between replays
        torch.cuda.synchronize()


def test_full_long_bf16_2x1x100000():
    """Rows of 100000 bfloat16 elements (the block path at sixteen raw vectors per lane) at the
    benchmark's size, lengths 100000 and 70000: every element against the oracle, in blocks of
    1024 rows through the oracle's row entry point; the band [-S, 0] (the same kept set, row-
    relative slots) gives the same bits."""
    name = "long_bf16_2x1x100000"
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    print(f"full workload {name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    sl = torch.as_tensor(lens).cuda()
    y = g.forward(x, sl, w.scale)
    torch.cuda.synchronize()
    worst = check_rows_against_oracle(x, y, lens, w.scale, w.dtype)
    print(f"{name}: every element checked, worst error {worst:.3g}", flush=True)
    yb = g.forward_band(x, sl, -w.S, 0, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), y.view(torch.int16)), "band [-S, 0] changed bits"
    del x, y, yb
    torch.cuda.empty_cache()


def test_full_long_bf16_2x2x65536():
    """Rows of 65536 bfloat16 elements (the block path at eight 16-byte vectors per lane) at
    the benchmark's size: every element against the oracle, in blocks of 1024 rows through the
    oracle's row entry point (a plane of 4.3e9 elements is too large to hand over whole)."""
    name = "long_bf16_2x2x65536"
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    print(f"full workload {name} lens={list(lens)}", flush=True)
    x = workloads.scores_device(w.shape, w.dtype, w.sigma, w.x_seed)
    y = g.forward(x, torch.as_tensor(lens).cuda(), w.scale)
    torch.cuda.synchronize()
    worst = check_rows_against_oracle(x, y, lens, w.scale, w.dtype)
    print(f"{name}: every element checked, worst error {worst:.3g}", flush=True)
    del x, y
    torch.cuda.empty_cache()
