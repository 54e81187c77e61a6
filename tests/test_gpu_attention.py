"""GPU parity of the fused attention with the grouped tril mask against the CPU oracle.

The kernel computes, per query row r < L_b, sum_{c <= r} softmax(scale * q_r . k_c) v_c and
writes zeros for rows r >= L_b (the self-attention article's three steps with this
operation's softmax). Rows at or past the length must be +0.0 bit for bit. Kept rows must
satisfy, element by element, a bound derived from the arithmetic: the scores, exponentials
and sums are fp32 (relative errors of a few 2^-24), and two roundings into the element type
dominate, that of each probability before the product with v (relative u, so at most
u * sum_c p_c |v_c| <= u * max_c |v_c| in the row) and that of the output (u * |o|):
    |o_gpu - o_ref| <= u * (max_{c <= r} |v_c| + |o_ref|) + 1e-5 * max_{c <= r} |v_c|
with u = 2^-8 for bfloat16 and 2^-11 for binary16 (half an ulp of a 9- or 12-bit
significand).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads
from gtms_check import bits, host_threads, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("GPU tests need a visible GPU", allow_module_level=True)

import variable_length_causal_amd as g  # noqa: E402

DTYPES = [workloads.F16, workloads.BF16]
DNAME = {workloads.F16: "f16", workloads.BF16: "bf16"}
U = {workloads.F16: 2.0 ** -11, workloads.BF16: 2.0 ** -8}


def prefix_vmax(v_head_f64):
    """[S] running max over rows c <= r of max_d |v[c, d]| for one head [S, D]."""
    return np.maximum.accumulate(np.max(np.abs(v_head_f64), axis=1))


def check_rows(o_st, ref, vmax_rows, lens_rows, rows_r, S, dtype, tag):
    """o_st, ref: [n, D]; row i has index rows_r[i], length lens_rows[i] and
    vmax_rows[i] = max over its kept keys of |v|."""
    got = to_f64(o_st, dtype)
    ob = bits(o_st)
    for i, (L, r) in enumerate(zip(lens_rows, rows_r)):
        Lc = min(max(int(L), 0), S)
        if r >= Lc:
            assert not ob[i].any(), f"{tag}: row {r} >= L={L} is not zero"
            continue
        vmax = float(vmax_rows[i])
        bound = U[dtype] * (vmax + np.abs(ref[i])) + 1e-5 * vmax
        err = np.abs(got[i] - ref[i])
        assert np.all(err <= bound), f"{tag}: row {r} L={L} excess {float(np.max(err - bound)):.3g}"


def run_case(B, M, S, D, dtype, lens, scale, seed, split="auto"):
    shape = (B, M, S, D)
    q, k, v = (workloads.scores_cpu(shape, dtype, 1.0, seed + i) for i in range(3))
    qs, ks, vs = (workloads.to_storage(t) for t in (q, k, v))
    ref = oracle.attention_f64(qs, ks, vs, lens, scale, dtype)
    print(f"attention B={B} M={M} S={S} D={D} {DNAME[dtype]} lens={list(lens)} split={split}",
          flush=True)
    o = g.attention(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(np.asarray(lens, np.int32)).cuda(),
                    scale, split=split)
    torch.cuda.synchronize()
    o_st = workloads.to_storage(o.cpu())
    vf = to_f64(vs, dtype)
    for b in range(B):
        for m in range(M):
            check_rows(o_st[b, m], ref[b, m], prefix_vmax(vf[b, m]), [lens[b]] * S,
                       range(S), S, dtype, f"B={B} M={M} S={S} D={D} {DNAME[dtype]} b={b} m={m}")


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_shapes(dtype, D):
    for S in (1, 5, 31, 32, 33, 127, 128, 129, 300):
        lens = [S, max(1, S // 3), 0, S + 7]
        run_case(len(lens), 2, S, D, dtype, lens, 1.0 / np.sqrt(D), seed=10 * S + D)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_zero_and_negative_scales(dtype, D):
    """Any finite scale is accepted (the ScaledMaskSoftmax article multiplies the scores by
    it before the softmax): 0 and -0 give the running mean of v over the kept keys, and a
    negative scale takes the softmax of the negated scores. Lengths cover several query
    tiles, a partial tile, padded batches and a length past S."""
    S = 300
    lens = [S, 100, 0, S + 7]
    for scale in (0.0, -0.0, -0.125):
        run_case(len(lens), 2, S, D, dtype, lens, scale, seed=700 + D)


def test_attention_scales_and_long_rows():
    run_case(2, 2, 1000, 64, workloads.BF16, [1000, 611], 0.3, seed=5)
    run_case(1, 1, 700, 128, workloads.F16, [700], 0.05, seed=6)
    run_case(2, 1, 200, 64, workloads.F16, [200, 150], 2.0, seed=7)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_rising_scores(dtype, D):
    """Scores that rise along the keys, so that a row's maximum keeps moving up as the key
    blocks go by: by about 4 per 64 keys in the log2 domain (the kernel's running reference
    sometimes moves, probabilities reach 2^8) and by about 16 (it moves every block).
    Query dimension 0 is 1 and key dimension 0 carries the ramp; the other dimensions are
    small noise."""
    S, lens, scale = 640, [640, 300], 0.125
    for rise in (4.0, 16.0):
        shape = (2, 1, S, D)
        q, k, v = (workloads.scores_cpu(shape, workloads.F32, 1.0, 90 + i) for i in range(3))
        q.mul_(0.05)
        k.mul_(0.05)
        q[..., 0] = 1.0
        k[..., 0] = torch.arange(S, dtype=torch.float32) * (rise / 64.0 / (scale * np.log2(np.e)))
        q, k, v = (t.to(workloads.torch_dtype(dtype)) for t in (q, k, v))
        qs, ks, vs = (workloads.to_storage(t) for t in (q, k, v))
        ref = oracle.attention_f64(qs, ks, vs, lens, scale, dtype)
        print(f"attention rising scores D={D} {DNAME[dtype]} rise={rise}", flush=True)
        o = g.attention(q.cuda(), k.cuda(), v.cuda(),
                        torch.as_tensor(np.asarray(lens, np.int32)).cuda(), scale)
        torch.cuda.synchronize()
        o_st = workloads.to_storage(o.cpu())
        vf = to_f64(vs, dtype)
        for b in range(2):
            check_rows(o_st[b, 0], ref[b, 0], prefix_vmax(vf[b, 0]), [lens[b]] * S, range(S), S,
                       dtype, f"rising {rise} D={D} {DNAME[dtype]} b={b}")


def test_attention_ignores_padding():
    """Queries of padded rows and keys/values at or past the length change no bit."""
    B, M, S, D = 3, 2, 260, 64
    lens = [260, 100, 0]
    for dtype in DTYPES:
        q, k, v = (workloads.scores_cpu((B, M, S, D), dtype, 1.0, 50 + i).cuda() for i in range(3))
        sl = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
        clean = g.attention(q, k, v, sl)
        qp, kp, vp = q.clone(), k.clone(), v.clone()
        for b, L in enumerate(lens):
            qp[b, :, L:] = float("nan")
            kp[b, :, L:] = float("inf")
            vp[b, :, L:] = float("nan")
        dirty = g.attention(qp, kp, vp, sl)
        torch.cuda.synchronize()
        assert np.array_equal(bits(workloads.to_storage(clean.cpu())),
                              bits(workloads.to_storage(dirty.cpu())))


def test_attention_rejects_bad_arguments():
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16, device="cuda")
    sl = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):   # head size 32 is not served
        g.attention(torch.zeros(1, 1, 64, 32, dtype=torch.float16, device="cuda"),
                    torch.zeros(1, 1, 64, 32, dtype=torch.float16, device="cuda"),
                    torch.zeros(1, 1, 64, 32, dtype=torch.float16, device="cuda"), sl)
    with pytest.raises(RuntimeError, match="element type"):  # no binary32 path
        g.attention(q.float(), q.float(), q.float(), sl)
    with pytest.raises(RuntimeError):   # out over q
        g.attention(q, q.clone(), q.clone(), sl, out=q)


@pytest.mark.parametrize("name,split", [(n, "auto") for n in sorted(workloads.ATTN_WORKLOADS)]
                         + [("attn_f16_3x64x1000_d64", "on")])
def test_attention_full_workload(name, split):
    """The benchmark's shapes at full size through the default entry point (the automatic
    work split takes whole tiles on the two larger grids and the key split on bf16
    2 x 8 x 4096), and f16 3 x 64 x 1000 with the key split forced: every row of every head
    against the oracle (one oracle call per head on host threads), padded rows +0 bit for bit
    and kept rows within the bound."""
    w = workloads.ATTN_WORKLOADS[name]
    lens = workloads.seq_lens(w)
    print(f"attention full workload {name} lens={list(lens)} split={split}", flush=True)
    q, k, v = (workloads.scores_device(w.shape, w.dtype, 1.0, w.x_seed + i, "cuda")
               for i in range(3))
    o = g.attention(q, k, v, torch.as_tensor(lens).cuda(), w.scale, split=split)
    torch.cuda.synchronize()
    qs, ks, vs, os_ = (workloads.to_storage(t.cpu()) for t in (q, k, v, o))
    S, D = w.S, w.D

    def one(bm):
        b, m = bm
        L = min(max(int(lens[b]), 0), S)
        ob = bits(os_[b, m])
        assert not ob[L:].any(), f"{name} b={b} m={m}: padded rows are not zero"
        if L == 0:
            return 0.0
        ref = oracle.attention_f64(qs[b:b + 1, m:m + 1], ks[b:b + 1, m:m + 1],
                                   vs[b:b + 1, m:m + 1], lens[b:b + 1], w.scale, w.dtype)[0, 0, :L]
        got = to_f64(os_[b, m, :L], w.dtype)
        vmax = prefix_vmax(to_f64(vs[b, m], w.dtype))[:L, None]
        err = np.abs(got - ref)
        bound = U[w.dtype] * (vmax + np.abs(ref)) + 1e-5 * vmax
        assert np.all(np.isfinite(got)), f"{name} b={b} m={m}: non-finite output"
        assert np.all(err <= bound), \
            f"{name} b={b} m={m}: excess {float(np.max(err - bound)):.3g}"
        return float(err.max())

    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        worst = max(pool.map(one, [(b, m) for b in range(w.B) for m in range(w.M)]))
    print(f"{name}: every row of every head checked, worst error {worst:.3g}", flush=True)


def test_attention_plane_major_head_size_128():
    """bf16 [12, 8, 4096, 128]: the heads' K and V (201 MB) exceed what the tile-major block
    order is used for, so this runs the plane-major order at head size 128 (the choice depends
    on the shape, not on the lengths; lengths of 512 to 1200 keep the oracle's work small).
    Every row of every head against the oracle (one oracle call per head on host threads);
    padded rows +0 bit for bit."""
    B, M, S, D = 12, 8, 4096, 128
    lens = np.random.default_rng(3101).integers(512, 1201, B).astype(np.int32)
    q, k, v = (workloads.scores_device((B, M, S, D), workloads.BF16, 1.0, 3100 + i, "cuda")
               for i in range(3))
    o = g.attention(q, k, v, torch.as_tensor(lens).cuda(), 0.09)
    torch.cuda.synchronize()
    qs, ks, vs, os_ = (workloads.to_storage(t.cpu()) for t in (q, k, v, o))

    def one(bm):
        b, m = bm
        L = min(max(int(lens[b]), 0), S)
        assert not bits(os_[b, m])[L:].any(), f"b={b} m={m}: padded rows are not zero"
        ref = oracle.attention_f64(qs[b:b + 1, m:m + 1], ks[b:b + 1, m:m + 1],
                                   vs[b:b + 1, m:m + 1], lens[b:b + 1], 0.09,
                                   workloads.BF16)[0, 0, :L]
        got = to_f64(os_[b, m, :L], workloads.BF16)
        vmax = prefix_vmax(to_f64(vs[b, m], workloads.BF16))[:L, None]
        err = np.abs(got - ref)
        bound = U[workloads.BF16] * (vmax + np.abs(ref)) + 1e-5 * vmax
        assert np.all(np.isfinite(got)), f"b={b} m={m}: non-finite output"
        assert np.all(err <= bound), f"b={b} m={m}: excess {float(np.max(err - bound)):.3g}"
        return float(err.max())

    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        worst = max(pool.map(one, [(b, m) for b in range(B) for m in range(M)]))
    print(f"plane-major D=128: every row of every head checked, worst error {worst:.3g}",
          flush=True)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
@pytest.mark.parametrize("split", ["off", "on"])
def test_attention_key_split(dtype, split):
    """Head size 64 with each work split forced: whole tiles per workgroup, or each tile's key
    blocks split between two groups of wavefronts and merged (flash_decoding.py's split-KV
    reduction). Lengths give tiles of one key block (the first group then has none), two,
    and odd counts (the second group has one more), rows past the length, a length past S;
    the scales include 0 and a negative one; rising scores move the running max in one group
    and not the other. At head size 128 the choice is ignored: same bits."""
    for S in (1, 33, 64, 65, 127, 128, 129, 200, 300, 1000):
        lens = [S, max(1, S // 3), 0, S + 7]
        run_case(len(lens), 2, S, 64, dtype, lens, 0.125, seed=20 * S + 3, split=split)
    for scale in (0.0, -0.125, 2.0):
        run_case(2, 2, 300, 64, dtype, [300, 97], scale, seed=801, split=split)
    S, lens, scale = 640, [640, 300], 0.125
    shape = (2, 1, S, 64)
    q, k, v = (workloads.scores_cpu(shape, workloads.F32, 1.0, 95 + i) for i in range(3))
    q.mul_(0.05)
    k.mul_(0.05)
    q[..., 0] = 1.0
    k[..., 0] = torch.arange(S, dtype=torch.float32) * (16.0 / 64.0 / (scale * np.log2(np.e)))
    q, k, v = (t.to(workloads.torch_dtype(dtype)) for t in (q, k, v))
    qs, ks, vs = (workloads.to_storage(t) for t in (q, k, v))
    ref = oracle.attention_f64(qs, ks, vs, lens, scale, dtype)
    o = g.attention(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(np.asarray(lens, np.int32)).cuda(),
                    scale, split=split)
    torch.cuda.synchronize()
    o_st = workloads.to_storage(o.cpu())
    vf = to_f64(vs, dtype)
    for b in range(2):
        check_rows(o_st[b, 0], ref[b, 0], prefix_vmax(vf[b, 0]), [lens[b]] * S, range(S), S,
                   dtype, f"rising split={split} {DNAME[dtype]} b={b}")
    q, k, v = (workloads.scores_device((2, 2, 300, 128), dtype, 1.0, 900 + i, "cuda")
               for i in range(3))
    sl = torch.as_tensor(np.asarray([300, 111], np.int32)).cuda()
    a, b = g.attention(q, k, v, sl, split=split), g.attention(q, k, v, sl, split="auto")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_key_split_ignores_padding():
    """With the key split, queries of padded rows and keys/values at or past the length still
    change no bit."""
    B, M, S, D = 3, 2, 260, 64
    lens = [260, 97, 0]
    sl = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
    q, k, v = (workloads.scores_device((B, M, S, D), workloads.BF16, 1.0, 950 + i, "cuda")
               for i in range(3))
    clean = g.attention(q, k, v, sl, split="on")
    qp, kp, vp = q.clone(), k.clone(), v.clone()
    for b, L in enumerate(lens):
        for t in (qp, kp, vp):
            t[b, :, L:] = float("nan")
    dirty = g.attention(qp, kp, vp, sl, split="on")
    torch.cuda.synchronize()
    assert torch.equal(clean.view(torch.int16), dirty.view(torch.int16))


def test_attention_auto_split_small_grid():
    """bf16 [2, 8, 4096, 64]: 512 (head, tile) pairs, where the automatic choice takes the key
    split (same bits as forcing it). Every row of every head against the oracle (one oracle
    call per head on host threads)."""
    B, M, S, D = 2, 8, 4096, 64
    lens = np.asarray([4096, 3001], np.int32)
    q, k, v = (workloads.scores_device((B, M, S, D), workloads.BF16, 1.0, 3200 + i, "cuda")
               for i in range(3))
    sl = torch.as_tensor(lens).cuda()
    o = g.attention(q, k, v, sl, 0.125)
    forced = g.attention(q, k, v, sl, 0.125, split="on")
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), forced.view(torch.int16))
    qs, ks, vs, os_ = (workloads.to_storage(t.cpu()) for t in (q, k, v, o))

    def one(bm):
        b, m = bm
        L = int(lens[b])
        assert not bits(os_[b, m])[L:].any(), f"b={b} m={m}: padded rows are not zero"
        ref = oracle.attention_f64(qs[b:b + 1, m:m + 1], ks[b:b + 1, m:m + 1],
                                   vs[b:b + 1, m:m + 1], lens[b:b + 1], 0.125,
                                   workloads.BF16)[0, 0, :L]
        got = to_f64(os_[b, m, :L], workloads.BF16)
        vmax = prefix_vmax(to_f64(vs[b, m], workloads.BF16))[:L, None]
        err = np.abs(got - ref)
        bound = U[workloads.BF16] * (vmax + np.abs(ref)) + 1e-5 * vmax
        assert np.all(np.isfinite(got)), f"b={b} m={m}: non-finite output"
        assert np.all(err <= bound), f"b={b} m={m}: excess {float(np.max(err - bound)):.3g}"
        return float(err.max())

    with ThreadPoolExecutor(max_workers=host_threads()) as pool:
        worst = max(pool.map(one, [(b, m) for b in range(B) for m in range(M)]))
    print(f"bf16 [2, 8, 4096, 64] key split: every row checked, worst error {worst:.3g}",
          flush=True)
