"""The split-k tile matmul and the measurement probes on the GPU, through
the C ABI.

Split k (page "Kernel experiments: recorded evidence", Test 30; page
"KERNEL_REPORT: PTQ1_0 small-batch decoding", "Facts"): one 1024-element
segment per slice, the slices of a tile spread over workgroups, the last
workgroup at the tile's counter adding them in index order.  Checked: within
the oracle's bound element by element (ragged rows, partial last segment,
long k), the bits of pq2_matmul_small_m_tiles wherever both cut k the same
way (k <= 8192) for every workgroup width, batch invariance over m,
repeated calls giving the same bits with the counters back at zero, and the
long-k workload at full size (sampled).

Probes: the stream probe reads every byte of the buffer exactly once (the
XOR of its words is the XOR of the buffer's dwords, for ragged sizes and
several grids); the empty probe launches and returns.
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


def quantise(x_cpu):
    qo, xso = oracle.quantize_act_i8(workloads.bf16_bits(x_cpu), "bf16")
    pq2 = _pq2()
    m, k = x_cpu.shape
    q = torch.empty((m, k), dtype=torch.int8, device=DEV)
    xs = torch.empty((m, k // 128), dtype=torch.float32, device=DEV)
    pq2.pq2_quantize_act_i8(x_cpu.to(DEV), q, xs)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(xs.cpu().numpy().view(np.uint32), xso.view(np.uint32))
    return q, xs, qo, xso


def tiles_of(raw, n, k):
    pq2 = _pq2()
    t = torch.full((pq2.pq2_tiles_bytes(n, k),), 0xA5, dtype=torch.uint8, device=DEV)
    pq2.pq2_prepare_tiles(torch.from_numpy(np.ascontiguousarray(raw)).to(DEV), n, k, t)
    return t


class SplitK:
    """Caller-owned scratch for one shape: partials (poisoned) and counters (zero)."""

    def __init__(self, m, n, k):
        pq2 = _pq2()
        self.partials = torch.full((pq2.pq2_tiles_splitk_partial_floats(m, n, k),), float("nan"),
                                   dtype=torch.float32, device=DEV)
        self.counters = torch.zeros(pq2.pq2_tiles_splitk_counter_words(n), dtype=torch.int32, device=DEV)

    def run(self, q, xs, tiles, n, waves=0):
        y = torch.full((q.shape[0], n), float("nan"), dtype=torch.float32, device=DEV)
        _pq2().pq2_matmul_small_m_tiles_splitk_tuned(q, xs, tiles, y, self.partials, self.counters, waves)
        torch.cuda.synchronize()
        return y.cpu().numpy()


def plain(q, xs, tiles, n):
    y = torch.full((q.shape[0], n), float("nan"), dtype=torch.float32, device=DEV)
    _pq2().pq2_matmul_small_m_tiles(q, xs, tiles, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y_gpu, y_ref, bound, what):
    y_gpu = y_gpu.astype(np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output (unwritten element?)"
    excess = np.abs(y_gpu - y_ref) - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, f"{what}: |diff| {abs(y_gpu[worst] - y_ref[worst]):.3e} > {bound[worst]:.3e}"


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


SPLITK_SHAPES = [
    # (m, n, k): ragged row tiles, a partial last segment, long k, 8-column passes
    (1, 1024, 512), (1, 1, 128), (2, 333, 640), (3, 97, 1152), (4, 1000, 5120), (5, 77, 2176),
    (8, 130, 384), (16, 40, 17408), (6, 513, 9216), (4, 64, 34816), (2, 24, 65536), (1, 700, 16384),
    (11, 70, 9216), (4, 250, 17408),
]


@pytest.mark.parametrize("m,n,k", SPLITK_SHAPES)
def test_splitk_full(m, n, k):
    pq2 = _pq2()
    announce(f"splitk full m={m} n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=300 + m + n, codes="ternary+3", row_pad=2)
    x = workloads.make_activations(m, k, 301 + k, "normal+outliers")
    q, xs, qo, xso = quantise(x)
    tiles = tiles_of(raw, n, k)
    sk = SplitK(m, n, k)
    y_ref, bound = oracle.matmul_raw(qo, xso, raw, n, k)
    y6 = sk.run(q, xs, tiles, n)
    assert_within(y6, y_ref, bound, f"splitk m={m} n={n} k={k}")
    # Every workgroup width cuts k into the same slices: same bits.
    for waves in (1, 2, 3, 16):
        assert same_bits(sk.run(q, xs, tiles, n, waves), y6), f"waves={waves}"
    if (k // 128 + 7) // 8 <= 8:
        # One segment per wave in the single-workgroup kernel too.
        assert same_bits(plain(q, xs, tiles, n), y6), "differs from pq2_matmul_small_m_tiles"
    assert not sk.counters.any().item(), "counters not back at zero"


def test_splitk_repeat_and_batch_invariance():
    pq2 = _pq2()
    n, k, mmax = 520, 17408, 16
    announce(f"splitk repeat n={n} k={k}")
    raw = workloads.make_raw_weights(n, k, seed=311, codes="ternary+3", row_pad=0)
    x = workloads.make_activations(mmax, k, 312, "laplace")
    tiles = tiles_of(raw, n, k)
    q, xs, qo, xso = quantise(x)
    sk = SplitK(mmax, n, k)
    ys = {}
    for m in (1, 2, 3, 4, 5, 8, 16):
        ys[m] = sk.run(q[:m].contiguous(), xs[:m].contiguous(), tiles, n)
    for m, y in ys.items():
        assert same_bits(y, ys[mmax][:m]), f"batch variance at m={m}"
    first = ys[4]
    for _ in range(24):  # back-to-back calls on one stream, counters reused
        y = torch.full((4, n), float("nan"), dtype=torch.float32, device=DEV)
        pq2.pq2_matmul_small_m_tiles_splitk(q[:4].contiguous(), xs[:4].contiguous(), tiles, y, sk.partials, sk.counters)
    torch.cuda.synchronize()
    assert same_bits(y.cpu().numpy(), first)
    assert not sk.counters.any().item()
    y_ref, bound = oracle.matmul_raw(qo[:4], xso[:4], raw, n, k)
    assert_within(first, y_ref, bound, "laplace long k")


def test_splitk_down_workload_sampled():
    w = workloads.WORKLOADS["down"]
    raw, x = workloads.workload_inputs("down")
    tiles = tiles_of(raw, w.n, w.k)
    q, xs, qo, xso = quantise(x[: max(w.ms)].contiguous())
    sk = SplitK(max(w.ms), w.n, w.k)
    ys = {}
    for m in w.ms:
        announce(f"splitk down m={m}")
        ys[m] = sk.run(q[:m].contiguous(), xs[:m].contiguous(), tiles, w.n)
        rng = np.random.default_rng(m)
        rows = np.concatenate([[0, 1, w.n // 2, w.n - 1], rng.integers(0, w.n, 300)])
        mi, ni = np.repeat(np.arange(m), len(rows)), np.tile(rows, m)
        y_ref, bound = oracle.matmul_raw_sample(qo[:m], xso[:m], raw, w.n, w.k, mi, ni)
        assert_within(ys[m][mi, ni], y_ref, bound, f"down m={m}")
    for m, y in ys.items():
        assert same_bits(y, ys[max(w.ms)][:m]), f"batch variance at m={m}"


@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (1024, 1), (4096 + 48, 3), (1 << 20, 7),
                                                (13926400, 2048), (23674880, 2048), (5 << 20, 1)])
def test_stream_probe_reads_every_byte_once(nbytes, workgroups):
    pq2 = _pq2()
    announce(f"stream probe bytes={nbytes} workgroups={workgroups}")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((pq2.pq2_stream_probe_words(workgroups),), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    pq2.pq2_stream_probe(buf, nbytes, workgroups, out, store_all=True)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host), "stream probe did not read each byte exactly once"
    # Timed mode: no word is written unless a fold equals the sentinel.
    out.fill_(7)
    pq2.pq2_stream_probe(buf, nbytes, workgroups, out, store_all=False, sentinel=0x7FFFFFFF)
    pq2.pq2_empty_probe(workgroups, 4)
    torch.cuda.synchronize()
    words = out.cpu().numpy().view(np.uint32)
    assert np.all((words == 7) | (words == 0x7FFFFFFF))


# Configurable stream probe: every load instruction and cache policy, loads
# in flight per lane 1..16, 1..16 waves, ragged tails (a last iteration that
# covers part of the grid; a partial 1 KB block for the buffer loads).
STREAM_CFG_CASES = [(1024, 1, 1, 1), (5120, 3, 2, 4), ((1 << 20) + 3072, 7, 3, 16), (23674880, 1024, 4, 4),
                    (13926400, 256, 16, 4), (5 << 20, 1, 1, 8), (3 << 20, 2048, 8, 2), (9216, 1, 4, 16)]


@pytest.mark.parametrize("policy", [0, 1, 2, 3])
@pytest.mark.parametrize("nbytes,workgroups,waves,loads", STREAM_CFG_CASES)
def test_stream_probe_cfg_reads_every_byte_once(policy, nbytes, workgroups, waves, loads):
    pq2 = _pq2()
    if policy < 2 and nbytes % 1024 == 0:
        nbytes -= 48  # buffer loads take any multiple of 16: a partial last block
    announce(f"stream probe cfg policy={policy} bytes={nbytes} workgroups={workgroups} waves={waves} loads={loads}")
    rng = np.random.default_rng(nbytes + policy)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((workgroups * waves,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    pq2.pq2_stream_probe_cfg(buf, nbytes, workgroups, waves, loads, policy, out, store_all=True)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host), "stream probe did not read each byte exactly once"
    out.fill_(7)
    pq2.pq2_stream_probe_cfg(buf, nbytes, workgroups, waves, loads, policy, out, store_all=False,
                             sentinel=0x7FFFFFFF)
    torch.cuda.synchronize()
    words = out.cpu().numpy().view(np.uint32)
    assert np.all((words == 7) | (words == 0x7FFFFFFF))
