"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: the quantised activations and scales and the prepared planes are
bit-exact; every output y satisfies |y_gpu - y_ref| <= 1e-5 * sum_g
|xs*ws*dot_g| + 1e-6 (the oracle returns that bound per output).  Outputs are
NaN-poisoned before every call, so an unwritten element fails.

Sizes: full element-by-element comparisons on shapes that span several
workgroup tiles with ragged row/column/group tails; at the full workload
sizes (the launch configuration the benchmark times) sampled outputs against
the oracle plus exact properties that hold at any size (negated activations
give exactly negated outputs, doubled weight scales exactly doubled ones,
one column does not depend on the others).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


@functools.lru_cache(maxsize=None)
def _pq2():
    import gemm_int8_act_amd as pq2
    return pq2


# ------------------------------------------------------------------ helpers
def gpu_planes(raw_np, n, k):
    pq2 = _pq2()
    raw = torch.from_numpy(np.ascontiguousarray(raw_np)).to(DEV)
    planes = torch.empty(n * (k // 128) * 34, dtype=torch.uint8, device=DEV)
    pq2.pq2_prepare_planes(raw, n, k, planes)
    return planes


def gpu_quantize(x, k=None):
    pq2 = _pq2()
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    q = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xs = torch.full((m, k // 128), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_quantize_act_i8(x, q, xs)
    return q, xs


def gpu_matmul(fn, q, xs, planes, n, **kw):
    m = q.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    fn(q, xs, planes, y, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y_gpu, y_ref, bound, what):
    y_gpu = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output (unwritten element?)"
    excess = np.abs(y_gpu - y_ref) - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, (f"{what}: |diff| {abs(y_gpu[worst] - y_ref[worst]):.3e} > bound "
                                f"{bound[worst]:.3e} at {worst}")


def quantise_both(x_cpu, k=None):
    """Quantise on the GPU and in the oracle; require bit equality; return
    the (device) q, xs and the oracle's numpy copies."""
    qo, xso = oracle.quantize_act_i8(workloads.bf16_bits(x_cpu) if x_cpu.dtype == torch.bfloat16
                                     else x_cpu.numpy(), "bf16" if x_cpu.dtype == torch.bfloat16 else "f32", k=k)
    q, xs = gpu_quantize(x_cpu.to(DEV), k)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), qo), "q differs from the oracle"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xso.view(np.uint32)), "xs differs from the oracle"
    return q, xs, qo, xso


@functools.lru_cache(maxsize=None)
def workload_case(name):
    w = workloads.WORKLOADS[name]
    raw, x = workloads.workload_inputs(name)
    return w, raw, x


# ------------------------------------------------------------------ quantiser
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_quantize_bit_exact_workloads(name):
    w, _, x = workload_case(name)
    announce(f"quantize {name} m={x.shape[0]} k={w.k}")
    quantise_both(x)


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("m,k,stride_pad", [(1, 128, 0), (3, 640, 5), (7, 5120, 8), (33, 1024, 3)])
def test_quantize_dtypes_and_strides(dtype, m, k, stride_pad):
    announce(f"quantize dtype={dtype} m={m} k={k} pad={stride_pad}")
    x = workloads.make_activations(m, k + stride_pad, 70 + m, "laplace").float() * 3.0
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    xt = x.to(tdt)
    if dtype == "f32":
        bits = xt.numpy()
    else:
        bits = xt.view(torch.int16).numpy().view(np.uint16)
    qo, xso = oracle.quantize_act_i8(bits, dtype, k=k)
    # Row stride k + pad (elements): unaligned rows take the kernel's scalar path.
    q, xs = gpu_quantize(xt.to(DEV), k)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xso.view(np.uint32))


def test_quantize_special_groups():
    """Zero group, subnormal scale, exact ties, +-amax."""
    announce("quantize special groups")
    g = np.zeros((1, 128 * 4), dtype=np.float32)
    g[0, 128:132] = [2.0 ** -130, -3 * 2.0 ** -131, 2.0 ** -126, 5 * 2.0 ** -133]
    g[0, 256] = 127.0
    g[0, 257:263] = [0.5, 1.5, 2.5, -2.5, 126.5, -0.5]
    g[0, 384:512] = np.arange(-64, 64) * 0.37
    x = torch.tensor(g).to(torch.bfloat16)
    q, xs, qo, xso = quantise_both(x)
    assert xso[0, 0] == 0.0 and xso[0, 2] == 1.0


# ------------------------------------------------------------------ prepare
@pytest.mark.parametrize("n,k,pad", [(1, 128, 0), (37, 640, 3), (256, 5120, 0), (19, 17408, 6)])
def test_prepare_byte_exact(n, k, pad):
    announce(f"prepare n={n} k={k} pad={pad}")
    raw = workloads.make_raw_weights(n, k, seed=80 + n, codes="ternary+3", row_pad=pad)
    planes = gpu_planes(raw, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(planes.cpu().numpy(), oracle.prepare_planes(raw, n, k))


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_prepare_byte_exact_workloads(name):
    w, raw, _ = workload_case(name)
    announce(f"prepare workload {name}")
    planes = gpu_planes(raw, w.n, w.k)
    torch.cuda.synchronize()
    assert np.array_equal(planes.cpu().numpy(), oracle.prepare_planes(raw, w.n, w.k))


# ------------------------------------------------------------------ small m: full comparisons
SMALL_SHAPES = [
    # (m, n, k): several row tiles, ragged row tail, partial last segment of groups
    (1, 1024, 512), (1, 1, 128), (2, 333, 640), (3, 97, 1152), (4, 1000, 5120),
    (5, 77, 2176), (8, 130, 384), (9, 61, 1024), (16, 40, 17408), (12, 300, 3072),
    (6, 513, 9216), (4, 64, 34816), (2, 24, 65536), (1, 4096, 16384), (11, 70, 9216),
]


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_small_m_full(m, n, k):
    announce(f"small_m full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    y = gpu_matmul(_pq2().pq2_matmul_small_m, q, xs, planes, n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"small_m m={m} n={n} k={k}")


def test_small_m_tiny_workload():
    w, raw, x = workload_case("tiny")
    announce("small_m tiny workload")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, w.n, w.k)
    y = gpu_matmul(_pq2().pq2_matmul_small_m, q, xs, planes, w.n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, w.n, w.k)
    assert_within(y, y_ref, bound, "tiny")


def test_small_m_zero_activations():
    announce("small_m zero activations")
    n, k = 100, 1024
    raw = workloads.make_raw_weights(n, k, seed=5)
    x = torch.zeros((3, k), dtype=torch.bfloat16)
    q, xs, _, _ = quantise_both(x)
    y = gpu_matmul(_pq2().pq2_matmul_small_m, q, xs, gpu_planes(raw, n, k), n)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_small_m_matrix_core_engine_full(m, n, k):
    """The matrix-core engines against the oracle, and bit-identical to the
    packed-dot engine, on every full-comparison shape, both input orders and
    every row-block count of the row-streaming engine."""
    pq2 = _pq2()
    announce(f"small_m matrix-core engine m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    y = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, engine=2)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"engine 2 m={m} n={n} k={k}")
    y1 = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, engine=1)
    assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), "engines differ"
    qp, xsp, qsum = gpu_quantize_planes(x.to(DEV))
    yp = gpu_matmul_planes(pq2.pq2_matmul_small_m_planes_tuned, qp, xsp, qsum, planes, n, engine=2)
    assert np.array_equal(yp.view(np.uint32), y1.view(np.uint32)), "plane-order matrix-core path differs"
    for engine in (3, 4):
        for rows in (0, 1):  # the library's row blocks per workgroup, and one
            y3 = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, rows=rows, engine=engine)
            assert np.array_equal(y3.view(np.uint32), y1.view(np.uint32)), \
                f"workgroup-staged engine {engine} rows={rows} differs"
            y3p = gpu_matmul_planes(pq2.pq2_matmul_small_m_planes_tuned, qp, xsp, qsum, planes, n, rows=rows,
                                    engine=engine)
            assert np.array_equal(y3p.view(np.uint32), y1.view(np.uint32)), \
                f"plane-order engine {engine} rows={rows} differs"


@pytest.mark.parametrize("m", [1, 4, 11])
def test_small_m_tuning_variants(m):
    """Every rows / k-split / engine setting is within the bound; neither
    rows nor the engine (packed dots, matrix cores, workgroup-staged matrix
    cores) changes the summation order, so they keep the bits."""
    pq2 = _pq2()
    n, k = 200, 5248
    announce(f"small_m variants m={m}")
    raw = workloads.make_raw_weights(n, k, seed=7, codes="ternary+3")
    x = workloads.make_activations(m, k, 8, "laplace")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    y0 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, n)
    assert_within(y0, y_ref, bound, "default")
    for waves in (1, 2, 3, 5, 8):
        ys = []
        for rows, engine in ((1, 1), (2, 1), (1, 2), (1, 3), (2, 3), (1, 4), (2, 4)):
            y = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, rows=rows, max_waves=waves,
                           engine=engine)
            assert_within(y, y_ref, bound, f"rows={rows} waves={waves} engine={engine}")
            ys.append(y)
        for y in ys[1:]:
            assert np.array_equal(ys[0].view(np.uint32), y.view(np.uint32)), \
                f"waves={waves}: rows per lane or engine changed the bits"


# ------------------------------------------------------------------ small m: full workload sizes
def _sample_indices(m, n, count, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([[0, 1, n // 2, n - 2, n - 1], rng.integers(0, n, count)])
    mi = np.repeat(np.arange(m), len(rows))
    ni = np.tile(rows, m)
    return mi, ni


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_small_m_workloads_sampled(name):
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    planes = gpu_planes(raw, w.n, w.k)
    ys = {}
    for m in w.ms:
        announce(f"small_m workload {name} m={m}")
        q, xs, qo, xso = quantise_both(x[:m].contiguous())
        y = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)
        mi, ni = _sample_indices(m, w.n, 400, seed=m)
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi, ni)
        assert_within(y[mi, ni], y_ref, bound, f"{name} m={m}")
        assert np.all(np.isfinite(y))
        ys[m] = y
    # Batch invariance: column c is bit-identical whatever the number of columns.
    mmax = max(w.ms)
    for m, y in ys.items():
        assert np.array_equal(y.view(np.uint32), ys[mmax][:m].view(np.uint32)), f"batch variance at m={m}"


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_small_m_workloads_exact_properties(name):
    """At full size: determinism, exact negation, exact scale doubling."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    m = 4
    announce(f"small_m properties {name}")
    planes = gpu_planes(raw, w.n, w.k)
    q, xs = gpu_quantize(x[:m].contiguous().to(DEV))
    y1 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)
    y2 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not deterministic"
    yneg = gpu_matmul(pq2.pq2_matmul_small_m, -q, xs, planes, w.n)
    assert np.array_equal(yneg, -y1), "negated activations must negate outputs exactly"
    planes2 = planes.clone()
    sc = planes2[w.n * w.k // 4:].view(torch.float16)
    sc.mul_(2.0)
    y2x = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes2, w.n)
    assert np.array_equal(y2x, 2.0 * y1), "doubled weight scales must double outputs exactly"


# ------------------------------------------------------------------ small m: tile layout
def gpu_tiles(raw_np, n, k):
    pq2 = _pq2()
    raw = torch.from_numpy(np.ascontiguousarray(raw_np)).to(DEV)
    tiles = torch.full((pq2.pq2_tiles_bytes(n, k),), 0xA5, dtype=torch.uint8, device=DEV)  # poisoned
    pq2.pq2_prepare_tiles(raw, n, k, tiles)
    return tiles


@pytest.mark.parametrize("n,k,pad", [(1, 128, 0), (37, 384, 3), (33, 640, 0), (256, 5120, 0), (19, 17408, 6)])
def test_prepare_tiles_byte_exact(n, k, pad):
    announce(f"prepare tiles n={n} k={k} pad={pad}")
    raw = workloads.make_raw_weights(n, k, seed=82 + n, codes="ternary+3", row_pad=pad)
    tiles = gpu_tiles(raw, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(tiles.cpu().numpy(), oracle.prepare_tiles(raw, n, k))


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_small_m_tiles_full(m, n, k):
    """The tile-layout engine against the oracle, and bit-identical to
    pq2_matmul_small_m on the row-major planes at the same k split (the
    default one for k <= 8192, where both give each wave one segment; up to
    8 waves through the tuning hook for longer k)."""
    pq2 = _pq2()
    announce(f"small_m tiles m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    tiles = gpu_tiles(raw, n, k)
    y = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"tiles m={m} n={n} k={k}")
    y1 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, gpu_planes(raw, n, k), n)
    y8 = gpu_matmul(pq2.pq2_matmul_small_m_tiles_tuned, q, xs, tiles, n, max_waves=8)
    assert np.array_equal(y8.view(np.uint32), y1.view(np.uint32)), "tile layout and planes differ (8 waves)"
    if k <= 8192:
        assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), "tile layout and planes differ"


@pytest.mark.parametrize("m", [1, 3, 4, 6, 13])
def test_small_m_tiles_waves(m):
    """Every k split gives the bits of the planes path at the same split."""
    pq2 = _pq2()
    n, k = 200, 5248
    announce(f"small_m tiles waves m={m}")
    raw = workloads.make_raw_weights(n, k, seed=7, codes="ternary+3")
    x = workloads.make_activations(m, k, 8, "laplace")
    q, xs, qo, xso = quantise_both(x)
    tiles, planes = gpu_tiles(raw, n, k), gpu_planes(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    for waves in (1, 2, 3, 5, 8):
        y1 = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, max_waves=waves)
        nseg = -(-(k // 128) // 8)
        slices = -(-nseg // -(-nseg // waves))
        for split in (1, 2, 4):
            if slices * split > 16:  # more than 16 waves per workgroup: not offered
                continue
            y = gpu_matmul(pq2.pq2_matmul_small_m_tiles_tuned, q, xs, tiles, n, max_waves=waves, split=split)
            assert_within(y, y_ref, bound, f"tiles waves={waves} split={split}")
            assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), \
                f"waves={waves} split={split}: tiles differ from planes"


def test_small_m_tiles_zero_activations_and_tiny():
    pq2 = _pq2()
    announce("small_m tiles zero activations / tiny workload")
    n, k = 100, 1024
    raw = workloads.make_raw_weights(n, k, seed=5)
    q, xs, _, _ = quantise_both(torch.zeros((3, k), dtype=torch.bfloat16))
    y = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, gpu_tiles(raw, n, k), n)
    assert np.all(y == 0.0)
    w, raw, x = workload_case("tiny")
    q, xs, qo, xso = quantise_both(x)
    y = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, gpu_tiles(raw, w.n, w.k), w.n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, w.n, w.k)
    assert_within(y, y_ref, bound, "tiles tiny")


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_small_m_tiles_workloads(name):
    """Full workload sizes: sampled outputs against the oracle, every output
    bit-identical to the planes path at the same k split, and each column's
    bits independent of the column count."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles, planes = gpu_tiles(raw, w.n, w.k), gpu_planes(raw, w.n, w.k)
    ys = {}
    for m in w.ms:
        announce(f"small_m tiles workload {name} m={m}")
        q, xs, qo, xso = quantise_both(x[:m].contiguous())
        y = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, w.n)
        mi, ni = _sample_indices(m, w.n, 400, seed=m)
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi, ni)
        assert_within(y[mi, ni], y_ref, bound, f"tiles {name} m={m}")
        y1 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)
        y8 = y if w.k <= 8192 else gpu_matmul(pq2.pq2_matmul_small_m_tiles_tuned, q, xs, tiles, w.n, max_waves=8)
        assert np.array_equal(y8.view(np.uint32), y1.view(np.uint32)), f"{name} m={m}: tiles differ from planes"
        ys[m] = y
    mmax = max(w.ms)
    for m, y in ys.items():
        assert np.array_equal(y.view(np.uint32), ys[mmax][:m].view(np.uint32)), f"batch variance at m={m}"


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_small_m_repeatable(name):
    """48 back-to-back launches of each decode path, every one with its own
    output buffer, give the same bits as the first (an intermittent hazard
    or race would show up as a differing launch)."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles, planes = gpu_tiles(raw, w.n, w.k), gpu_planes(raw, w.n, w.k)
    reps = 48
    for m in w.ms:
        announce(f"repeatable {name} m={m}")
        q, xs, _, _ = quantise_both(x[:m].contiguous())
        xd = x[:m].contiguous().to(DEV)
        calls = {
            "tiles": lambda out: pq2.pq2_matmul_small_m_tiles(q, xs, tiles, out),
            "tiles fused": lambda out: pq2.pq2_matmul_small_m_tiles_fused(xd, tiles, out),
            "planes": lambda out: pq2.pq2_matmul_small_m(q, xs, planes, out),
        }
        for what, call in calls.items():
            ys = torch.full((reps, m, w.n), float("nan"), dtype=torch.float32, device=DEV)
            for i in range(reps):
                call(ys[i])
            torch.cuda.synchronize()
            bits = ys.view(torch.int32)
            same = (bits == bits[0:1]).all(dim=(1, 2)).cpu().numpy()
            assert same.all(), f"{name} m={m} {what}: launches {np.nonzero(~same)[0].tolist()} differ from the first"
            assert torch.isfinite(ys[0]).all(), f"{name} m={m} {what}: unwritten outputs"


# ------------------------------------------------------------------ prefill
PREFILL_SHAPES = [(1, 64, 128), (5, 200, 640), (128, 128, 1024), (130, 257, 384), (300, 96, 5120),
                  (257, 513, 2048), (70, 80, 9088)]


@pytest.mark.parametrize("m,n,k", PREFILL_SHAPES)
def test_prefill_full(m, n, k):
    announce(f"prefill full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=110 + n, codes="ternary+3", row_pad=1)
    x = workloads.make_activations(m, k, 111 + m, "normal")
    q, xs, qo, xso = quantise_both(x)
    y = gpu_matmul(_pq2().pq2_matmul_prefill, q, xs, gpu_planes(raw, n, k), n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"prefill m={m} n={n} k={k}")
    yt = gpu_matmul(_pq2().pq2_matmul_prefill_tiles, q, xs, gpu_tiles(raw, n, k), n)
    assert np.array_equal(yt.view(np.uint32), y.view(np.uint32)), "prefill from the tile layout differs"


@pytest.mark.parametrize("name", ["prefill_gate", "prefill_up"])
def test_prefill_workloads_sampled(name):
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    planes = gpu_planes(raw, w.n, w.k)
    tiles = gpu_tiles(raw, w.n, w.k)
    for m in w.ms:
        announce(f"prefill workload {name} m={m}")
        q, xs, qo, xso = quantise_both(x[:m].contiguous())
        y = gpu_matmul(pq2.pq2_matmul_prefill, q, xs, planes, w.n)
        assert np.all(np.isfinite(y))
        qp, xsp, _ = gpu_quantize_planes(x[:m].contiguous().to(DEV))
        yp = gpu_matmul(pq2.pq2_matmul_prefill_planes, qp, xsp, planes, w.n)
        assert np.array_equal(yp.view(np.uint32), y.view(np.uint32)), "plane-order prefill differs"
        yt = gpu_matmul(pq2.pq2_matmul_prefill_tiles, q, xs, tiles, w.n)
        assert np.array_equal(yt.view(np.uint32), y.view(np.uint32)), "prefill from the tile layout differs"
        rng = np.random.default_rng(m)
        mi = np.concatenate([[0, m - 1, 0, m - 1], rng.integers(0, m, 1500)])
        ni = np.concatenate([[0, 0, w.n - 1, w.n - 1], rng.integers(0, w.n, 1500)])
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi, ni)
        assert_within(y[mi, ni], y_ref, bound, f"{name} m={m}")
        # Exact property at full size: a column does not depend on the others.
        if m == w.ms[0]:
            y_first = gpu_matmul(pq2.pq2_matmul_prefill, q[:1].contiguous(), xs[:1].contiguous(), planes, w.n)
            assert np.all(np.isfinite(y_first))
            mi1 = np.zeros(64, dtype=np.int64)
            ni1 = np.arange(0, w.n, w.n // 64)[:64]
            y1_ref, b1 = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi1, ni1)
            assert_within(y_first[0, ni1], y1_ref, b1, f"{name} m=1")


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5])
def test_prefill_tiles(tile):
    """Every workgroup tile, from natural- and plane-order activations, gives
    outputs within the bound, with ragged row, column and group tails, and
    the same bits as the default tile."""
    pq2 = _pq2()
    m, n, k = 200, 333, 1408
    announce(f"prefill tile={tile}")
    raw = workloads.make_raw_weights(n, k, seed=120 + tile, codes="ternary+3", row_pad=3)
    x = workloads.make_activations(m, k, 121, "laplace")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    y = gpu_matmul(pq2.pq2_matmul_prefill_tuned, q, xs, planes, n, tile=tile)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"prefill tile={tile}")
    y0 = gpu_matmul(pq2.pq2_matmul_prefill, q, xs, planes, n)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32)), "tile changed the bits"
    qp, xsp, _ = gpu_quantize_planes(x.to(DEV))
    yp = gpu_matmul(pq2.pq2_matmul_prefill_planes_tuned, qp, xsp, planes, n, tile=tile)
    assert np.array_equal(yp.view(np.uint32), y0.view(np.uint32)), "plane-order prefill changed the bits"
    yt = gpu_matmul(pq2.pq2_matmul_prefill_tiles_tuned, q, xs, gpu_tiles(raw, n, k), n, tile=tile)
    assert np.array_equal(yt.view(np.uint32), y0.view(np.uint32)), "prefill from the tile layout changed the bits"


@pytest.mark.parametrize("m,n,k", [(1, 200, 128), (127, 130, 1152), (129, 384, 1152), (256, 128, 5120),
                                   (300, 272, 2176)])
def test_prefill_tiles_lds_direct_edges(m, n, k):
    """The 128x128 tile on eight waves from the tile layout, whose
    activations go straight into LDS one group ahead: rows past m inside a
    workgroup tile, a single group, group counts that are not a multiple of
    8, several row tiles.  Within the bound, and the bits of the 64x128 tile
    (same summation order)."""
    pq2 = _pq2()
    announce(f"prefill lds-direct m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=130 + m, codes="ternary+3", row_pad=1)
    x = workloads.make_activations(m, k, 131 + n, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    tiles = gpu_tiles(raw, n, k)
    y5 = gpu_matmul(pq2.pq2_matmul_prefill_tiles_tuned, q, xs, tiles, n, tile=5)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y5, y_ref, bound, f"prefill lds-direct m={m} n={n} k={k}")
    y2 = gpu_matmul(pq2.pq2_matmul_prefill_tiles_tuned, q, xs, tiles, n, tile=2)
    assert np.array_equal(y5.view(np.uint32), y2.view(np.uint32)), "128x128 tile changed the bits"
    y5b = gpu_matmul(pq2.pq2_matmul_prefill_tiles_tuned, q, xs, tiles, n, tile=5)
    assert np.array_equal(y5b.view(np.uint32), y5.view(np.uint32)), "repeat call differs"


def test_prefill_matches_small_m():
    """Both paths compute the same definition: agree within twice the bound."""
    pq2 = _pq2()
    m, n, k = 16, 300, 5120
    announce("prefill vs small_m")
    raw = workloads.make_raw_weights(n, k, seed=3)
    x = workloads.make_activations(m, k, 4, "normal")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    ya = gpu_matmul(pq2.pq2_matmul_prefill, q, xs, planes, n)
    yb = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, n)
    _, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert np.all(np.abs(ya.astype(np.float64) - yb) <= 2 * bound)


# ------------------------------------------------------------------ plane-order path
def to_plane_order(q):
    """The layout pq2_quantize_act_i8_planes documents: inside each 16-byte
    block of a row, qp[16t + 4s + j] = q[16t + 4j + s] (a 4x4 byte transpose)."""
    m, k = q.shape
    return np.ascontiguousarray(q.reshape(m, k // 16, 4, 4).transpose(0, 1, 3, 2).reshape(m, k))


def gpu_quantize_planes(x, k=None):
    pq2 = _pq2()
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    qp = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xs = torch.full((m, k // 128), float("nan"), dtype=torch.float32, device=DEV)
    qsum = torch.full((m, k // 128), -(1 << 30), dtype=torch.int32, device=DEV)
    pq2.pq2_quantize_act_i8_planes(x, qp, xs, qsum)
    return qp, xs, qsum


def quantise_planes_both(x_cpu, dtype="bf16", k=None):
    """Plane-order quantiser vs the oracle: the same q values (moved by the
    documented transpose), bit-equal xs, and qsum = the oracle q's group sums."""
    bits = workloads.bf16_bits(x_cpu) if dtype == "bf16" else (
        x_cpu.numpy() if dtype == "f32" else x_cpu.view(torch.int16).numpy().view(np.uint16))
    qo, xso = oracle.quantize_act_i8(bits, dtype, k=k)
    qp, xs, qsum = gpu_quantize_planes(x_cpu.to(DEV), k)
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), to_plane_order(qo)), "qp is not the plane-ordered oracle q"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xso.view(np.uint32)), "xs differs from the oracle"
    m, kk = qo.shape
    sums = qo.astype(np.int64).reshape(m, kk // 128, 128).sum(axis=2)
    assert np.array_equal(qsum.cpu().numpy().astype(np.int64), sums), "qsum is not the group sum of q"
    return qp, xs, qsum, qo, xso


def test_plane_order_helper_is_a_transpose():
    q = np.arange(2 * 128, dtype=np.int64).reshape(2, 128) % 251 - 125
    p = to_plane_order(q.astype(np.int8))
    assert p[0, 4 * 1 + 2] == q[0, 4 * 2 + 1] and p[1, 16 * 3 + 4 * 3 + 0] == q[1, 16 * 3 + 0 + 3]
    assert np.array_equal(to_plane_order(p), q.astype(np.int8))  # an involution


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_quantize_planes_workloads(name):
    w, _, x = workload_case(name)
    announce(f"quantize planes {name} m={x.shape[0]} k={w.k}")
    quantise_planes_both(x)


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("m,k,stride_pad", [(1, 128, 0), (3, 640, 5), (7, 5120, 8), (33, 1024, 3)])
def test_quantize_planes_dtypes_and_strides(dtype, m, k, stride_pad):
    announce(f"quantize planes dtype={dtype} m={m} k={k} pad={stride_pad}")
    x = workloads.make_activations(m, k + stride_pad, 170 + m, "laplace").float() * 3.0
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    quantise_planes_both(x.to(tdt), dtype, k=k)


def test_quantize_planes_special_groups():
    announce("quantize planes special groups")
    g = np.zeros((1, 128 * 4), dtype=np.float32)
    g[0, 128:132] = [2.0 ** -130, -3 * 2.0 ** -131, 2.0 ** -126, 5 * 2.0 ** -133]
    g[0, 256] = 127.0
    g[0, 257:263] = [0.5, 1.5, 2.5, -2.5, 126.5, -0.5]
    g[0, 384:512] = -127.0  # a group at the clamp: qsum = -16256
    quantise_planes_both(torch.tensor(g).to(torch.bfloat16))


def gpu_matmul_planes(fn, qp, xs, qsum, planes, n, **kw):
    m = qp.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    fn(qp, xs, qsum, planes, y, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_small_m_planes_full(m, n, k):
    """Within the bound of the oracle, and the same bits as the natural-order
    path (same exact integer dots, same summation order)."""
    pq2 = _pq2()
    announce(f"small_m planes full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    qp, xs, qsum, qo, xso = quantise_planes_both(x)
    planes = gpu_planes(raw, n, k)
    y = gpu_matmul_planes(pq2.pq2_matmul_small_m_planes, qp, xs, qsum, planes, n)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    assert_within(y, y_ref, bound, f"small_m planes m={m} n={n} k={k}")
    q, xs2 = gpu_quantize(x.to(DEV))
    y_nat = gpu_matmul(pq2.pq2_matmul_small_m, q, xs2, planes, n)
    assert np.array_equal(y.view(np.uint32), y_nat.view(np.uint32)), "plane-order and natural paths differ"


@pytest.mark.parametrize("rows,waves,engine", [(1, 1, 1), (1, 5, 1), (2, 3, 1), (2, 8, 1), (2, 3, 3), (1, 8, 3), (2, 3, 4), (0, 8, 4)])
def test_small_m_planes_tuning_variants(rows, waves, engine):
    pq2 = _pq2()
    m, n, k = 4, 200, 5248
    announce(f"small_m planes variants rows={rows} waves={waves} engine={engine}")
    raw = workloads.make_raw_weights(n, k, seed=7, codes="ternary+3")
    x = workloads.make_activations(m, k, 8, "laplace")
    qp, xs, qsum, qo, xso = quantise_planes_both(x)
    planes = gpu_planes(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    y = gpu_matmul_planes(pq2.pq2_matmul_small_m_planes_tuned, qp, xs, qsum, planes, n, rows=rows,
                          max_waves=waves, engine=engine)
    assert_within(y, y_ref, bound, f"planes rows={rows} waves={waves} engine={engine}")
    q, xs2 = gpu_quantize(x.to(DEV))
    y_nat = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs2, planes, n, rows=rows, max_waves=waves, engine=engine)
    assert np.array_equal(y.view(np.uint32), y_nat.view(np.uint32)), "same settings, same bits"


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_small_m_planes_workloads_sampled(name):
    """Full workload sizes in the benchmark's launch configuration: sampled
    outputs against the oracle, bitwise batch invariance, and the same bits as
    the natural-order path everywhere."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    planes = gpu_planes(raw, w.n, w.k)
    ys = {}
    for m in w.ms:
        announce(f"small_m planes workload {name} m={m}")
        qp, xs, qsum, qo, xso = quantise_planes_both(x[:m].contiguous())
        y = gpu_matmul_planes(pq2.pq2_matmul_small_m_planes, qp, xs, qsum, planes, w.n)
        mi, ni = _sample_indices(m, w.n, 400, seed=m)
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi, ni)
        assert_within(y[mi, ni], y_ref, bound, f"{name} m={m}")
        q, xs2 = gpu_quantize(x[:m].contiguous().to(DEV))
        y_nat = gpu_matmul(pq2.pq2_matmul_small_m, q, xs2, planes, w.n)
        assert np.array_equal(y.view(np.uint32), y_nat.view(np.uint32)), f"paths differ at m={m}"
        ys[m] = y
    mmax = max(w.ms)
    for m, y in ys.items():
        assert np.array_equal(y.view(np.uint32), ys[mmax][:m].view(np.uint32)), f"batch variance at m={m}"


# ------------------------------------------------------------------ fused quantise + matmul
def gpu_fused(x_dev, planes, n, **kw):
    pq2 = _pq2()
    y = torch.full((x_dev.shape[0], n), float("nan"), dtype=torch.float32, device=DEV)
    if kw:
        pq2.pq2_matmul_small_m_fused_tuned(x_dev, planes, y, **kw)
    else:
        pq2.pq2_matmul_small_m_fused(x_dev, planes, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(np.asarray(a, dtype=np.float32).view(np.uint32), np.asarray(b, dtype=np.float32).view(np.uint32))


FUSED_SHAPES = [(1, 1024, 512), (1, 1, 128), (2, 333, 640), (3, 97, 1152), (4, 1000, 5120), (5, 77, 2176),
                (8, 130, 384), (16, 40, 17408), (12, 300, 3072), (2, 24, 65536)]


@pytest.mark.parametrize("m,n,k", FUSED_SHAPES)
def test_fused_full(m, n, k):
    """Quantise + matmul in one launch: within the bound of the oracle (which
    quantises with the definition), and bit-identical to the two-launch path
    for every engine and rows-per-lane setting."""
    pq2 = _pq2()
    announce(f"fused full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    planes = gpu_planes(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    xd = x.to(DEV)
    for rows, engine in ((1, 1), (2, 1), (1, 2), (0, 3), (1, 3), (0, 4), (1, 4)):
        yf = gpu_fused(xd, planes, n, rows=rows, engine=engine)
        assert_within(yf, y_ref, bound, f"fused rows={rows} engine={engine}")
        yu = gpu_matmul(pq2.pq2_matmul_small_m_tuned, q, xs, planes, n, rows=rows, engine=engine)
        assert same_bits(yf, yu), f"fused rows={rows} engine={engine} differs from quantise + matmul"
    y0 = gpu_fused(xd, planes, n)
    assert same_bits(y0, gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, n)), "default fused path differs"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k,pad", [(1, 200, 1024, 0), (3, 150, 640, 8), (4, 64, 5120, 16), (7, 90, 2048, 24)])
def test_fused_dtypes_and_strides(dtype, m, n, k, pad):
    pq2 = _pq2()
    announce(f"fused dtype={dtype} m={m} n={n} k={k} pad={pad}")
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    xt = (workloads.make_activations(m, k + pad, 170 + m, "laplace").float() * 3.0).to(tdt)
    bits = xt.numpy() if dtype == "f32" else xt.view(torch.int16).numpy().view(np.uint16)
    qo, xso = oracle.quantize_act_i8(bits, dtype, k=k)
    raw = workloads.make_raw_weights(n, k, seed=171 + n, codes="ternary+3")
    planes = gpu_planes(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    xd = xt.to(DEV)
    yf = gpu_fused(xd[:, :k], planes, n)  # row stride k + pad elements
    assert_within(yf, y_ref, bound, f"fused {dtype}")
    q, xs = gpu_quantize(xd, k)
    assert same_bits(yf, gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, n))


def probe_weights(k):
    """Raw rows that read one activation each: row r has weight +1 (code 2)
    at position r, weight 0 (code 1) elsewhere, and every scale is fp16 1.0,
    so y[m][r] = float(q[m][r]) * xs[m][r // 128] exactly."""
    groups = k // 128
    raw = np.zeros((k, groups, 34), dtype=np.uint8)
    raw[:, :, 0], raw[:, :, 1] = 0x00, 0x3C  # 1.0 = 0x3C00, little-endian
    raw[:, :, 2:] = 0x55
    r = np.arange(k)
    i = r % 128
    shift = 2 * (i % 4)
    raw[r, r // 128, 2 + i // 4] = (0x55 & ~(3 << shift)) | (2 << shift)
    return raw.reshape(k, groups * 34)


def probe_activations(dtype, k):
    """16 columns: random groups of several distributions and magnitudes, and
    groups built for the edge cases of the quantiser's quotient: exact
    rounding ties (power-of-two scales), a zero group, subnormal scales (with
    f32 input also a scale that makes the clamp bind), repeated +-amax, and
    huge values."""
    m = 16
    cols = [workloads.make_activations(1, k, 300 + c, "normal+outliers" if c % 2 else "laplace").float()[0]
            * (10.0 ** (c % 5 - 2)) for c in range(m)]
    x = torch.stack(cols)
    g = x[5].view(k // 128, 128)
    g[0] = 0.0
    g[1] = torch.tensor([(j - 63.5) * 0.125 for j in range(128)])          # d = 2^-3: every element a tie
    g[1, 0] = 127 * 0.125
    g[2] = torch.tensor([((j % 9) - 4) * 2.0 ** -131 for j in range(128)])  # subnormal scale
    g[3] = torch.tensor([(-1.0) ** j * 3.0e30 for j in range(128)])        # all at +-amax
    g[4] = torch.tensor([(j - 64) * 0.5 + 0.25 for j in range(128)])       # d = 0.5: ties
    g[4, 0] = 63.5
    if dtype == "f32":
        g[5] = torch.tensor([(j % 7 - 3) * 2.0 ** -149 for j in range(128)], dtype=torch.float64).float()
        g[5, 0] = 190 * 2.0 ** -149                                         # scale rounds to 2^-149: clamp
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return x.to(tdt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_quantiser_codes_exact(dtype):
    """Every code and scale of the fused quantiser, read back through
    single-weight rows: y[m][r] must equal the oracle's q * xs bit for bit
    (exact ties and near-ties of the quotient, subnormal scales and the
    clamp)."""
    k = 2048
    announce(f"fused quantiser probe dtype={dtype} k={k}")
    x = probe_activations(dtype, k)
    bits = x.numpy() if dtype == "f32" else workloads.bf16_bits(x)
    qo, xso = oracle.quantize_act_i8(bits, dtype)
    assert np.any(np.abs(qo) == 127)
    raw = probe_weights(k)
    planes = gpu_planes(raw, k, k)
    expect = qo.astype(np.float32) * np.repeat(xso, 128, axis=1)
    for rows, engine in ((1, 1), (1, 2), (1, 3), (2, 3), (1, 4), (3, 4)):
        y = gpu_fused(x.to(DEV), planes, k, rows=rows, engine=engine)
        bad = np.argwhere(y.view(np.uint32) != expect.view(np.uint32))
        assert bad.size == 0, f"engine={engine}: {len(bad)} codes differ, first at {tuple(bad[0])}: " \
                              f"{y[tuple(bad[0])]!r} vs {expect[tuple(bad[0])]!r}"


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_fused_workloads(name):
    """Full workload sizes: bit-identical to quantise + matmul at every M,
    and sampled outputs within the oracle's bound."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    planes = gpu_planes(raw, w.n, w.k)
    for m in w.ms:
        announce(f"fused workload {name} m={m}")
        xd = x[:m].contiguous().to(DEV)
        yf = gpu_fused(xd, planes, w.n)
        q, xs, qo, xso = quantise_both(x[:m].contiguous())
        assert same_bits(yf, gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)), f"{name} m={m}"
        mi, ni = _sample_indices(m, w.n, 200, seed=50 + m)
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw, w.n, w.k, mi, ni)
        assert_within(yf[mi, ni], y_ref, bound, f"fused {name} m={m}")


# ------------------------------------------------------------------ fused quantise + tile-layout matmul
def gpu_tiles_fused(x_dev, tiles, n, **kw):
    pq2 = _pq2()
    y = torch.full((x_dev.shape[0], n), float("nan"), dtype=torch.float32, device=DEV)
    if kw:
        pq2.pq2_matmul_small_m_tiles_fused_tuned(x_dev, tiles, y, **kw)
    else:
        pq2.pq2_matmul_small_m_tiles_fused(x_dev, tiles, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _tiles_splits(k, waves=16):
    """The (max_waves, split) settings offered for this k (at most 16 waves)."""
    nseg = -(-(k // 128) // 8)
    slices = -(-nseg // -(-nseg // waves))
    return [s for s in (1, 2, 4) if slices * s <= 16]


@pytest.mark.parametrize("m,n,k", FUSED_SHAPES)
def test_tiles_fused_full(m, n, k):
    """Quantise + tile matmul in one launch: within the oracle's bound and
    bit-identical to pq2_quantize_act_i8 + pq2_matmul_small_m_tiles for
    every split."""
    pq2 = _pq2()
    announce(f"tiles fused full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=90 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 91 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    tiles = gpu_tiles(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    xd = x.to(DEV)
    for split in _tiles_splits(k):
        yf = gpu_tiles_fused(xd, tiles, n, split=split)
        assert_within(yf, y_ref, bound, f"tiles fused split={split}")
        yu = gpu_matmul(pq2.pq2_matmul_small_m_tiles_tuned, q, xs, tiles, n, split=split)
        assert same_bits(yf, yu), f"tiles fused split={split} differs from quantise + matmul"
    if k <= 8192:  # the same k split as the planes engine
        assert same_bits(gpu_tiles_fused(xd, tiles, n),
                         gpu_matmul(pq2.pq2_matmul_small_m, q, xs, gpu_planes(raw, n, k), n))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k,pad", [(1, 200, 1024, 0), (3, 150, 640, 8), (4, 64, 5120, 16), (7, 90, 2048, 24)])
def test_tiles_fused_dtypes_and_strides(dtype, m, n, k, pad):
    pq2 = _pq2()
    announce(f"tiles fused dtype={dtype} m={m} n={n} k={k} pad={pad}")
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    xt = (workloads.make_activations(m, k + pad, 170 + m, "laplace").float() * 3.0).to(tdt)
    bits = xt.numpy() if dtype == "f32" else xt.view(torch.int16).numpy().view(np.uint16)
    qo, xso = oracle.quantize_act_i8(bits, dtype, k=k)
    raw = workloads.make_raw_weights(n, k, seed=171 + n, codes="ternary+3")
    tiles = gpu_tiles(raw, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    xd = xt.to(DEV)
    yf = gpu_tiles_fused(xd[:, :k], tiles, n)  # row stride k + pad elements
    assert_within(yf, y_ref, bound, f"tiles fused {dtype}")
    q, xs = gpu_quantize(xd, k)
    assert same_bits(yf, gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, n))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiles_fused_quantiser_codes_exact(dtype):
    """Every code and scale of the tile engine's in-kernel quantiser, read
    back through single-weight rows, equals the oracle's q * xs bit for bit."""
    k = 2048
    announce(f"tiles fused quantiser probe dtype={dtype} k={k}")
    x = probe_activations(dtype, k)
    bits = x.numpy() if dtype == "f32" else workloads.bf16_bits(x)
    qo, xso = oracle.quantize_act_i8(bits, dtype)
    tiles = gpu_tiles(probe_weights(k), k, k)
    expect = qo.astype(np.float32) * np.repeat(xso, 128, axis=1)
    for split in _tiles_splits(k):
        y = gpu_tiles_fused(x.to(DEV), tiles, k, split=split)
        bad = np.argwhere(y.view(np.uint32) != expect.view(np.uint32))
        assert bad.size == 0, f"split={split}: {len(bad)} codes differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_tiles_fused_workloads(name):
    """Full workload sizes: bit-identical to quantise + tile matmul at every M."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles = gpu_tiles(raw, w.n, w.k)
    for m in w.ms:
        announce(f"tiles fused workload {name} m={m}")
        xd = x[:m].contiguous().to(DEV)
        q, xs = gpu_quantize(xd)
        assert same_bits(gpu_tiles_fused(xd, tiles, w.n), gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, w.n)), \
            f"{name} m={m}"


@pytest.mark.parametrize("name", ["qkv", "up", "down"])
def test_gemv_tiles_same_bits(name):
    """pq2_gemv_tiles (fused at one or two columns and k <= 8192, two
    launches otherwise or when the rows are not 16-byte aligned) gives the
    bits of quantise + tile matmul at every M."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles = gpu_tiles(raw, w.n, w.k)
    for m in w.ms:
        announce(f"gemv tiles {name} m={m}")
        q, xs, _, _ = quantise_both(x[:m].contiguous())
        y0 = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, w.n)
        xd = x[:m].contiguous().to(DEV)
        y = torch.full((m, w.n), float("nan"), dtype=torch.float32, device=DEV)
        qw = torch.empty((m, w.k), dtype=torch.int8, device=DEV)
        xw = torch.empty((m, w.k // 128), dtype=torch.float32, device=DEV)
        pq2.pq2_gemv_tiles(xd, tiles, y, qw, xw)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32)), f"{name} m={m}"
        fused = m <= 2 and w.k <= 8192 and m * -(-w.n // 16) <= 1600
        if fused:  # the fused path needs no scratch
            y.fill_(float("nan"))
            pq2.pq2_gemv_tiles(xd, tiles, y)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32)), f"{name} m={m} no scratch"
        if m == 2 and w.k <= 8192:
            # Rows 8 bf16 elements + 2 apart: the fused kernel cannot read them
            # (16-byte rows), so the call takes the two-launch path.
            xp = torch.zeros((m, w.k + 10), dtype=x.dtype, device=DEV)
            xp[:, 2:2 + w.k] = xd
            xv = xp[:, 2:2 + w.k]
            y.fill_(float("nan"))
            pq2.pq2_gemv_tiles(xv, tiles, y, qw, xw)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32)), f"{name} m=2 unaligned rows"


# ------------------------------------------------------------------ smaller activation groups
# Page "Kernel experiments: recorded evidence", section C (Tests 8 and 9).
def quantise_g_both(x_cpu, agroup, dtype="bf16", k=None):
    """Activation-group quantiser on the GPU and in the oracle, bit-equal."""
    pq2 = _pq2()
    bits = workloads.bf16_bits(x_cpu) if dtype == "bf16" else (
        x_cpu.numpy() if dtype == "f32" else x_cpu.view(torch.int16).numpy().view(np.uint16))
    qo, xso = oracle.quantize_act_i8_g(bits, agroup, dtype, k=k)
    m = x_cpu.shape[0]
    k = x_cpu.shape[1] if k is None else k
    q = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xs = torch.full((m, k // agroup), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_quantize_act_i8_g(x_cpu.to(DEV), q, xs, agroup)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), qo), f"agroup {agroup}: q differs from the oracle"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), xso.view(np.uint32)), f"agroup {agroup}: xs differs"
    return q, xs, qo, xso


@pytest.mark.parametrize("agroup", [64, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_quantize_g_bit_exact(agroup, dtype):
    announce(f"quantize agroup={agroup} {dtype}")
    x = workloads.make_activations(5, 1152, 60 + agroup, "normal+outliers")
    x[1, :64] = 0                                    # zero groups
    x[2, 128:256] = torch.linspace(-3, 3, 128)       # exact ties at power-of-two scales
    x[3, 256:288] = 1e-38                            # tiny group (subnormal scale)
    xc = {"bf16": x, "f16": x.float().to(torch.float16), "f32": x.float()}[dtype]
    quantise_g_both(xc, agroup, dtype)
    if agroup == 64:  # a padded row stride takes the unaligned path
        wide = torch.zeros((5, 1160), dtype=xc.dtype)
        wide[:, :1152] = xc
        quantise_g_both(wide, agroup, dtype, k=1152)


G_SHAPES = [(1, 1024, 512), (2, 333, 640), (3, 97, 1152), (4, 1000, 5120), (5, 77, 2176), (9, 61, 1024),
            (16, 40, 17408)]


@pytest.mark.parametrize("agroup", [64, 32])
@pytest.mark.parametrize("m,n,k", G_SHAPES)
def test_small_m_tiles_g_full(agroup, m, n, k):
    pq2 = _pq2()
    announce(f"tiles agroup={agroup} m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=70 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 71 + k, "normal+outliers")
    q, xs, qo, xso = quantise_g_both(x, agroup)
    tiles = gpu_tiles(raw, n, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_g(q, xs, tiles, y, agroup)
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_raw_g(qo, xso, raw, n, k, agroup)
    assert_within(y.cpu().numpy(), y_ref, bound, f"tiles agroup={agroup} m={m} n={n} k={k}")


def test_small_m_tiles_g_128_is_the_tile_matmul():
    pq2 = _pq2()
    m, n, k = 4, 300, 3072
    raw = workloads.make_raw_weights(n, k, seed=73, codes="ternary+3")
    x = workloads.make_activations(m, k, 74, "laplace")
    q, xs, _, _ = quantise_g_both(x, 128)
    tiles = gpu_tiles(raw, n, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_g(q, xs, tiles, y, 128)
    y0 = gpu_matmul(pq2.pq2_matmul_small_m_tiles, q, xs, tiles, n)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32))


FUSED_G_SHAPES = [(1, 1024, 512), (2, 333, 640), (3, 97, 1152), (4, 1000, 5120), (5, 77, 2176), (16, 40, 17408)]


@pytest.mark.parametrize("agroup", [64, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", FUSED_G_SHAPES)
def test_tiles_fused_g_same_bits(agroup, dtype, m, n, k):
    """Quantise + tile matmul in one launch with activation groups of 64 or
    32: the bits of pq2_quantize_act_i8_g followed by
    pq2_matmul_small_m_tiles_g (the quantiser is checked against the oracle
    here, the matmul against the oracle's bound in test_small_m_tiles_g_full),
    with a zero group, ragged rows and column passes past four."""
    pq2 = _pq2()
    announce(f"tiles fused agroup={agroup} {dtype} m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=80 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 81 + k, "normal+outliers")
    x[0, :agroup] = 0
    xc = {"bf16": x, "f16": x.float().to(torch.float16), "f32": x.float()}[dtype]
    q, xs, _, _ = quantise_g_both(xc, agroup, dtype)
    tiles = gpu_tiles(raw, n, k)
    y0 = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_g(q, xs, tiles, y0, agroup)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_fused_g(xc.to(DEV), tiles, y, agroup)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.cpu().numpy().view(np.uint32)), \
        f"fused agroup={agroup} {dtype} m={m} n={n} k={k}"


def test_tiles_fused_g_128_is_the_fused_matmul():
    pq2 = _pq2()
    m, n, k = 3, 300, 3072
    raw = workloads.make_raw_weights(n, k, seed=83, codes="ternary+3")
    xd = workloads.make_activations(m, k, 84, "laplace").to(DEV)
    tiles = gpu_tiles(raw, n, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_fused_g(xd, tiles, y, 128)
    y0 = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_tiles_fused(xd, tiles, y0)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y0.view(torch.int32))


@pytest.mark.parametrize("name", ["qkv", "up"])
def test_tiles_fused_g_workloads(name):
    """Full workload sizes, every M: the fused call with activation groups of
    64 and 32 has the bits of the two calls."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles = gpu_tiles(raw, w.n, w.k)
    for agroup in (64, 32):
        for m in w.ms:
            announce(f"tiles fused agroup={agroup} workload {name} m={m}")
            xm = x[:m].contiguous()
            q, xs, _, _ = quantise_g_both(xm, agroup)
            y0 = torch.full((m, w.n), float("nan"), dtype=torch.float32, device=DEV)
            pq2.pq2_matmul_small_m_tiles_g(q, xs, tiles, y0, agroup)
            y = torch.full((m, w.n), float("nan"), dtype=torch.float32, device=DEV)
            pq2.pq2_matmul_small_m_tiles_fused_g(xm.to(DEV), tiles, y, agroup)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), y0.view(torch.int32)), f"{name} m={m} agroup={agroup}"


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_small_m_tiles_g_workloads(name):
    """Full workload sizes, sampled outputs against the oracle, and 16
    repeated launches with identical bits."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles = gpu_tiles(raw, w.n, w.k)
    for agroup in (64, 32):
        for m in w.ms:
            announce(f"tiles agroup={agroup} workload {name} m={m}")
            q, xs, qo, xso = quantise_g_both(x[:m].contiguous(), agroup)
            ys = torch.full((16, m, w.n), float("nan"), dtype=torch.float32, device=DEV)
            for i in range(16):
                pq2.pq2_matmul_small_m_tiles_g(q, xs, tiles, ys[i], agroup)
            torch.cuda.synchronize()
            bits = ys.view(torch.int32)
            assert bool((bits == bits[0:1]).all()), f"{name} m={m} agroup={agroup}: launches differ"
            y = ys[0].cpu().numpy()
            mi, ni = _sample_indices(m, w.n, 300, seed=m + agroup)
            y_ref, bound = oracle.matmul_raw_sample_g(qo, xso, raw, w.n, w.k, agroup, mi, ni)
            assert_within(y[mi, ni], y_ref, bound, f"tiles agroup={agroup} {name} m={m}")


@pytest.mark.parametrize("agroup", [64, 32])
@pytest.mark.parametrize("m,n,k", PREFILL_SHAPES)
def test_prefill_tiles_g_full(agroup, m, n, k):
    """Tile-layout prefill with smaller activation groups against the oracle,
    element by element, with ragged row, column and group tails."""
    pq2 = _pq2()
    announce(f"prefill agroup={agroup} m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=130 + n, codes="ternary+3", row_pad=1)
    x = workloads.make_activations(m, k, 131 + m, "normal+outliers")
    q, xs, qo, xso = quantise_g_both(x, agroup)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_prefill_tiles_g(q, xs, gpu_tiles(raw, n, k), y, agroup)
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_raw_g(qo, xso, raw, n, k, agroup)
    assert_within(y.cpu().numpy(), y_ref, bound, f"prefill agroup={agroup} m={m} n={n} k={k}")


def test_prefill_tiles_g_128_is_the_tile_prefill():
    pq2 = _pq2()
    m, n, k = 200, 333, 1408
    raw = workloads.make_raw_weights(n, k, seed=132, codes="ternary+3")
    x = workloads.make_activations(m, k, 133, "laplace")
    q, xs, _, _ = quantise_g_both(x, 128)
    tiles = gpu_tiles(raw, n, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_prefill_tiles_g(q, xs, tiles, y, 128)
    y0 = gpu_matmul(pq2.pq2_matmul_prefill_tiles, q, xs, tiles, n)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("name", ["prefill_gate", "prefill_up"])
def test_prefill_tiles_g_workloads(name):
    """Full prefill sizes: sampled outputs against the oracle, and two
    launches with identical bits."""
    pq2 = _pq2()
    w, raw, x = workload_case(name)
    tiles = gpu_tiles(raw, w.n, w.k)
    for agroup in (64, 32):
        for m in w.ms:
            announce(f"prefill agroup={agroup} workload {name} m={m}")
            q, xs, qo, xso = quantise_g_both(x[:m].contiguous(), agroup)
            ys = torch.full((2, m, w.n), float("nan"), dtype=torch.float32, device=DEV)
            for i in range(2):
                pq2.pq2_matmul_prefill_tiles_g(q, xs, tiles, ys[i], agroup)
            torch.cuda.synchronize()
            assert torch.equal(ys[0].view(torch.int32), ys[1].view(torch.int32)), f"{name} m={m}: launches differ"
            y = ys[0].cpu().numpy()
            rng = np.random.default_rng(m + agroup)
            mi = np.concatenate([[0, m - 1, 0, m - 1], rng.integers(0, m, 1000)])
            ni = np.concatenate([[0, 0, w.n - 1, w.n - 1], rng.integers(0, w.n, 1000)])
            y_ref, bound = oracle.matmul_raw_sample_g(qo, xso, raw, w.n, w.k, agroup, mi, ni)
            assert_within(y[mi, ni], y_ref, bound, f"prefill agroup={agroup} {name} m={m}")


def gpu_raw(raw_np, shift=0):
    """The raw rows on the device as [n][stride] bytes, starting `shift`
    bytes past a 256-byte boundary."""
    n, stride = raw_np.shape
    buf = torch.full((n * stride + shift,), 0xEE, dtype=torch.uint8, device=DEV)
    raw = buf[shift:].view(n, stride)
    raw.copy_(torch.from_numpy(np.ascontiguousarray(raw_np)))
    return raw


# (m, n, k, row padding, pointer shift): strides of 0 and 2 mod 4, padded
# rows (pad bytes 0xEE, never read), a raw pointer 2 bytes off a 4-byte
# boundary, one and two rows per lane, several column passes.
RAW_SHAPES = [(1, 1024, 512, 0, 0), (2, 333, 640, 0, 0), (3, 97, 1152, 6, 0), (4, 1000, 5120, 0, 2),
              (5, 77, 2176, 2, 0), (9, 61, 1024, 0, 2), (16, 40, 17408, 4, 2), (1, 1, 128, 0, 0),
              (12, 300, 3072, 10, 0), (2, 24, 65536, 0, 2)]


@pytest.mark.parametrize("m,n,k,pad,shift", RAW_SHAPES)
def test_small_m_raw_full(m, n, k, pad, shift):
    """The raw-layout reader against the oracle, element by element, and
    bit-identical to pq2_matmul_small_m on the prepared planes."""
    pq2 = _pq2()
    announce(f"small_m raw m={m} n={n} k={k} pad={pad} shift={shift}")
    raw_np = workloads.make_raw_weights(n, k, seed=140 + m + n, codes="ternary+3", row_pad=pad)
    x = workloads.make_activations(m, k, 141 + k, "normal+outliers")
    q, xs, qo, xso = quantise_both(x)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    pq2.pq2_matmul_small_m_raw(q, xs, gpu_raw(raw_np, shift), y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, bound = oracle.matmul_raw(qo, xso, raw_np, n, k)
    assert_within(y, y_ref, bound, f"raw m={m} n={n} k={k}")
    y1 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, gpu_planes(raw_np, n, k), n)
    assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), "raw reader and planes differ"


@pytest.mark.parametrize("name", ["qkv", "down"])
def test_small_m_raw_workloads(name):
    """Full workload sizes: bit-identical to the planes path, sampled outputs
    against the oracle."""
    pq2 = _pq2()
    w, raw_np, x = workload_case(name)
    raw = gpu_raw(raw_np)
    planes = gpu_planes(raw_np, w.n, w.k)
    for m in w.ms:
        announce(f"raw workload {name} m={m}")
        q, xs, qo, xso = quantise_both(x[:m].contiguous())
        y = torch.full((m, w.n), float("nan"), dtype=torch.float32, device=DEV)
        pq2.pq2_matmul_small_m_raw(q, xs, raw, y)
        y1 = gpu_matmul(pq2.pq2_matmul_small_m, q, xs, planes, w.n)
        y = y.cpu().numpy()
        assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), f"{name} m={m}: raw reader and planes differ"
        mi, ni = _sample_indices(m, w.n, 300, seed=m + 7)
        y_ref, bound = oracle.matmul_raw_sample(qo, xso, raw_np, w.n, w.k, mi, ni)
        assert_within(y[mi, ni], y_ref, bound, f"raw {name} m={m}")


def _xor_dwords(buf_u8):
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(buf_u8).view(np.uint32)))


@pytest.mark.parametrize("n,k", [(1, 128), (33, 640), (1000, 5120), (37, 17408), (300, 1152)])
def test_read_probe_reads_every_byte_once(n, k):
    """The read probe's XOR folds equal the XOR of every dword of the layout
    (planes: code dwords and zero-extended scales), computed on the host
    from the oracle's own preparation of the same weights."""
    pq2 = _pq2()
    announce(f"read probe n={n} k={k}")
    raw_np = workloads.make_raw_weights(n, k, seed=150 + n, codes="ternary+3", row_pad=2)
    planes_ref = oracle.prepare_planes(raw_np, n, k)
    tiles_ref = oracle.prepare_tiles(raw_np, n, k)
    codes_bytes = n * (k // 4)
    want = {
        pq2.LAYOUT_PLANES: _xor_dwords(planes_ref[:codes_bytes])
        ^ int(np.bitwise_xor.reduce(planes_ref[codes_bytes:].view(np.uint16).astype(np.uint32))),
        pq2.LAYOUT_TILES: _xor_dwords(tiles_ref),
    }
    for layout, weights in ((pq2.LAYOUT_PLANES, gpu_planes(raw_np, n, k)), (pq2.LAYOUT_TILES, gpu_tiles(raw_np, n, k))):
        words = pq2.pq2_read_probe_words(layout, n, k)
        out = torch.full((words,), -1, dtype=torch.int32, device=DEV)
        pq2.pq2_read_probe(weights, layout, n, k, out)
        torch.cuda.synchronize()
        got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
        assert got == want[layout], f"layout {layout}: probe fold {got:#x}, layout xor {want[layout]:#x}"
