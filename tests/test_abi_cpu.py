"""The C ABI without a GPU: the library loads, exports every symbol that
include/*.h declares (pq2.h, pq2_measure.h, pq2_tuning.h), and rejects bad
arguments on the host before any HIP call (every case below fails validation
or, without a GPU, the device check, so nothing is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pq2.h", "pq2_measure.h", "pq2_tuning.h")]

import gemm_int8_act_amd as pq2  # noqa: E402

OK, EINVAL, ESHAPE, EALIGN, EDEVICE = pq2.PQ2_OK, pq2.PQ2_EINVAL, pq2.PQ2_ESHAPE, pq2.PQ2_EALIGN, pq2.PQ2_EDEVICE

# Fake device addresses: never dereferenced, because validation fails first.
A = 0x7F0000000000          # 4 KiB aligned
B = 0x7F0100000000
C = 0x7F0200000000
D = 0x7F0300000000
E = 0x7F0400000000


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0  # counts devices without initialising the runtime


def _declared_symbols():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(pq2_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_symbols_exported():
    names = _declared_symbols()
    assert len(names) == 41
    lib = ctypes.CDLL(pq2.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(pq2.EXPORTED)


def test_layout_version_and_status_strings():
    assert pq2.pq2_layout_version() == 1
    for s in range(6):
        assert pq2.pq2_status_str(s)
    assert pq2.pq2_status_str(99) == "unknown status"
    assert pq2.pq2_last_hip_error() == "hipSuccess"


def test_prepare_validation():
    f = pq2.lib.pq2_prepare_planes
    assert f(None, 34, 4, 128, B, None) == EINVAL
    assert f(A, 34, 4, 128, None, None) == EINVAL
    assert f(A, 34, 0, 128, B, None) == ESHAPE
    assert f(A, 34, 4, 100, B, None) == ESHAPE
    assert f(A, 34, 4, 0, B, None) == ESHAPE
    assert f(A, 33, 4, 128, B, None) == ESHAPE          # row stride below 34 bytes per block
    assert f(A, 34 * 2, 4, 384, B, None) == ESHAPE
    assert f(A, 34, 4, 128, B + 8, None) == EALIGN     # planes not 16-byte aligned
    assert f(A, 34, 4, 128, A + 64, None) == EINVAL    # planes overlap raw


def test_quantize_validation():
    f = pq2.lib.pq2_quantize_act_i8
    assert f(None, 0, 128, 1, 128, B, C, None) == EINVAL
    assert f(A, 3, 128, 1, 128, B, C, None) == EINVAL    # unknown dtype
    assert f(A, 0, 128, 0, 128, B, C, None) == ESHAPE
    assert f(A, 0, 128, 1, 96, B, C, None) == ESHAPE
    assert f(A, 0, 100, 1, 128, B, C, None) == ESHAPE     # stride < k
    assert f(A, 0, 1 << 17, 1, 1 << 17, B, C, None) == ESHAPE  # k beyond the limit
    assert f(A + 1, 0, 128, 1, 128, B, C, None) == EALIGN  # bf16 not 2-byte aligned
    assert f(A + 2, 2, 128, 1, 128, B, C, None) == EALIGN  # f32 not 4-byte aligned
    assert f(A, 0, 128, 1, 128, B + 4, C, None) == EALIGN  # q not 8-byte aligned
    assert f(A, 0, 128, 1, 128, B, C + 2, None) == EALIGN
    assert f(A, 0, 128, 2, 128, A + 16, C, None) == EINVAL  # q overlaps x


@pytest.mark.parametrize("name", ["pq2_matmul_small_m", "pq2_matmul_prefill", "pq2_matmul_prefill_planes",
                                  "pq2_matmul_small_m_tiles", "pq2_matmul_prefill_tiles"])
def test_matmul_validation(name):
    f = getattr(pq2.lib, name)
    assert f(None, B, C, 1, 8, 128, D, None) == EINVAL
    assert f(A, None, C, 1, 8, 128, D, None) == EINVAL
    assert f(A, B, None, 1, 8, 128, D, None) == EINVAL
    assert f(A, B, C, 1, 8, 128, None, None) == EINVAL
    assert f(A, B, C, 0, 8, 128, D, None) == ESHAPE
    assert f(A, B, C, 1, 0, 128, D, None) == ESHAPE
    assert f(A, B, C, 1, 8, 200, D, None) == ESHAPE
    assert f(A, B, C, 1, 8, 1 << 17, D, None) == ESHAPE
    assert f(A + 8, B, C, 1, 8, 128, D, None) == EALIGN   # q 16-byte alignment
    assert f(A, B + 2, C, 1, 8, 128, D, None) == EALIGN
    assert f(A, B, C + 8, 1, 8, 128, D, None) == EALIGN   # planes 16-byte alignment
    assert f(A, B, C, 1, 8, 128, D + 2, None) == EALIGN
    assert f(A, B, C, 1, 8, 128, C + 16, None) == EINVAL  # y overlaps planes


def test_small_m_column_limit_and_tuning_validation():
    f = pq2.lib.pq2_matmul_small_m
    assert f(A, B, C, 17, 8, 128, D, None) == ESHAPE
    t = pq2.lib.pq2_matmul_small_m_tuned
    assert t(A, B, C, 1, 8, 128, D, 3, 0, 1, None) == EINVAL   # rows per lane of the packed-dot engine
    assert t(A, B, C, 1, 8, 128, D, 4, 0, 1, None) == EINVAL
    assert t(A, B, C, 1, 8, 128, D, 2, 0, 2, None) == EINVAL   # one row block per matrix-core workgroup
    assert t(A, B, C, 1, 8, 128, D, 100, 0, 3, None) == EINVAL  # more row blocks than a workgroup's waves run
    assert t(A, B, C, 4, 8, 65536, D, 2, 0, 3, None) == EINVAL  # more items per wave than it holds
    assert t(A, B, C, 1, 8, 128, D, 0, 9, 0, None) == EINVAL   # waves
    assert t(A, B, C, 1, 8, 128, D, 0, 0, 5, None) == EINVAL   # engine
    assert t(A, B, C, 17, 8, 128, D, 1, 1, 1, None) == ESHAPE


@pytest.mark.skipif(_gpu_visible(), reason="the device check passes on a GPU")
def test_small_m_valid_settings_reach_the_device_check():
    """Every supported (rows, engine) setting passes validation: without a
    GPU the call gets as far as the device check."""
    t = pq2.lib.pq2_matmul_small_m_tuned
    for rows, engine in ((0, 0), (1, 1), (2, 1), (1, 2), (1, 3), (2, 3), (0, 3), (1, 4), (0, 4)):
        assert t(A, B, C, 4, 8, 128, D, rows, 0, engine, None) == EDEVICE, (rows, engine)


def test_tiles_bytes():
    """T*S8*4352 with T = ceil(n/16), S8 = ceil(G/8)."""
    f = pq2.pq2_tiles_bytes
    assert f(10240, 5120) == 10240 * 40 * 34           # no padding: equal to the prepared planes
    assert f(5120, 17408) == 5120 * 136 * 34
    assert f(1, 128) == 4352                           # one tile, one (padded) segment unit
    assert f(17, 1152) == 2 * 2 * 4352
    for n, k in ((0, 128), (1, 100), (1, 0), (1, 1 << 17), ((1 << 30) + 1, 128)):
        assert pq2.lib.pq2_tiles_bytes(n, k) == -1, (n, k)


def test_prepare_tiles_validation():
    f = pq2.lib.pq2_prepare_tiles
    assert f(None, 34, 4, 128, B, None) == EINVAL
    assert f(A, 34, 4, 128, None, None) == EINVAL
    assert f(A, 34, 0, 128, B, None) == ESHAPE
    assert f(A, 34, 4, 100, B, None) == ESHAPE
    assert f(A, 33, 4, 128, B, None) == ESHAPE          # row stride below 34 bytes per block
    assert f(A, 34, 4, 128, B + 8, None) == EALIGN     # tiles not 16-byte aligned
    assert f(A, 34, 4, 128, A + 64, None) == EINVAL    # tiles overlap raw
    assert f(A, 34, 4, 128, A - 4096, None) == EINVAL  # the 4352-byte tiles end inside raw's 136 bytes
    if not _gpu_visible():
        assert f(A, 34, 4, 128, A + 144, None) == EDEVICE  # adjacent, no overlap: valid


def test_small_m_tiles_validation():
    f = pq2.lib.pq2_matmul_small_m_tiles
    assert f(A, B, C, 17, 8, 128, D, None) == ESHAPE
    assert f(A, B, C, 1, 8, 128, C + 4096, None) == EINVAL  # y overlaps the tiles (4352 bytes)
    t = pq2.lib.pq2_matmul_small_m_tiles_tuned
    assert t(A, B, C, 1, 8, 128, D, 17, 0, None) == EINVAL    # waves (at most 16)
    assert t(A, B, C, 1, 8, 128, D, -1, 0, None) == EINVAL
    assert t(A, B, C, 1, 8, 128, D, 0, 3, None) == EINVAL     # split
    assert t(A, B, C, 1, 8, 65536, D, 8, 4, None) == EINVAL   # 8 slices x 4 waves > 16
    if not _gpu_visible():
        for waves, split in ((0, 0), (1, 1), (8, 2), (1, 4), (5, 0)):
            assert t(A, B, C, 4, 8, 5120, D, waves, split, None) == EDEVICE, (waves, split)


def test_small_m_tiles_fused_validation():
    f = pq2.lib.pq2_matmul_small_m_tiles_fused
    assert f(None, 0, 128, C, 1, 8, 128, D, None) == EINVAL
    assert f(A, 3, 128, C, 1, 8, 128, D, None) == EINVAL        # dtype
    assert f(A, 0, 128, C, 17, 8, 128, D, None) == ESHAPE       # columns
    assert f(A, 0, 100, C, 1, 8, 128, D, None) == ESHAPE        # stride < k
    assert f(A + 2, 0, 128, C, 1, 8, 128, D, None) == EALIGN    # x not 16-byte aligned
    assert f(A, 0, 129, C, 2, 8, 128, D, None) == EALIGN        # row stride not 16-byte aligned
    assert f(A, 0, 128, C, 1, 8, 128, C + 64, None) == EINVAL   # y overlaps the tiles
    t = pq2.lib.pq2_matmul_small_m_tiles_fused_tuned
    assert t(A, 0, 128, C, 1, 8, 128, D, 17, 0, None) == EINVAL
    assert t(A, 0, 128, C, 1, 8, 128, D, 0, 3, None) == EINVAL
    if not _gpu_visible():
        assert t(A, 2, 5120, C, 4, 8, 5120, D, 0, 0, None) == EDEVICE


def test_gemv_tiles_validation():
    f = pq2.lib.pq2_gemv_tiles
    # m <= 2, k <= 8192: the fused path's checks; no scratch needed.
    assert f(None, 0, 128, C, 1, 8, 128, D, None, None, None) == EINVAL
    assert f(A, 3, 128, C, 1, 8, 128, D, None, None, None) == EINVAL         # dtype
    assert f(A + 2, 0, 128, C, 1, 8, 128, D, None, None, None) == EALIGN     # x not 16-byte aligned
    # Otherwise the two-launch path: scratch required, everything checked first.
    assert f(A, 0, 128, C, 3, 8, 128, D, None, E, None) == EINVAL            # no q scratch
    assert f(A, 0, 128, C, 3, 8, 128, D, B, None, None) == EINVAL            # no xs scratch
    assert f(A, 0, 128, C, 17, 8, 128, D, B, E, None) == ESHAPE              # columns
    assert f(A, 0, 100, C, 3, 8, 128, D, B, E, None) == ESHAPE               # stride < k
    assert f(A, 0, 128, C, 3, 8, 128, D, B + 8, E, None) == EALIGN           # q scratch not 16-byte aligned
    assert f(A + 1, 0, 128, C, 3, 8, 128, D, B, E, None) == EALIGN           # bf16 x not 2-byte aligned
    assert f(A, 0, 128, C, 3, 8, 128, D, A + 64, E, None) == EINVAL          # q scratch overlaps x
    assert f(A, 0, 128, C, 3, 8, 128, A + 128, B, E, None) == EINVAL         # y overlaps x
    assert f(A, 0, 128, C, 3, 8, 128, D, B, C + 64, None) == EINVAL          # xs scratch overlaps the tiles
    assert f(A, 0, 16384, C, 1, 8, 16384, D, None, None, None) == EINVAL     # long k takes the two-launch path
    if not _gpu_visible():
        assert f(A, 0, 5120, C, 1, 8, 5120, D, None, None, None) == EDEVICE
        assert f(A, 0, 5120, C, 4, 8, 5120, D, B, E, None) == EDEVICE


def test_activation_group_validation():
    f = pq2.lib.pq2_quantize_act_i8_g
    for bad in (0, 16, 96, 256):
        assert f(A, 0, 128, 1, 128, bad, B, C, None) == EINVAL, bad
    assert f(None, 0, 128, 1, 128, 64, B, C, None) == EINVAL
    assert f(A, 3, 128, 1, 128, 64, B, C, None) == EINVAL        # dtype
    assert f(A, 0, 128, 1, 96, 32, B, C, None) == ESHAPE         # k % 128
    assert f(A, 0, 100, 1, 128, 64, B, C, None) == ESHAPE        # stride < k
    assert f(A, 0, 128, 1, 128, 32, B + 4, C, None) == EALIGN    # q not 8-byte aligned
    assert f(A, 0, 256, 1, 256, 32, B, B + 128, None) == EINVAL  # xs (8 floats) overlaps q
    g = pq2.lib.pq2_matmul_small_m_tiles_g
    for bad in (0, 16, 96, 256):
        assert g(A, B, C, 1, 8, 128, bad, D, None) == EINVAL, bad
    assert g(A, B, C, 17, 8, 128, 64, D, None) == ESHAPE         # columns
    assert g(A + 8, B, C, 1, 8, 128, 64, D, None) == EALIGN      # q not 16-byte aligned
    assert g(A, B, C, 1, 8, 256, 32, B + 16, None) == EINVAL     # y overlaps xs (8 floats)
    h = pq2.lib.pq2_matmul_prefill_tiles_g
    for bad in (0, 16, 96, 256):
        assert h(A, B, C, 64, 8, 128, bad, D, None) == EINVAL, bad
    assert h(A, B, C, 0, 8, 128, 64, D, None) == ESHAPE          # no rows
    assert h(A, B, C, 64, 8, 96, 64, D, None) == ESHAPE          # k % 128
    assert h(A + 8, B, C, 64, 8, 128, 64, D, None) == EALIGN     # q not 16-byte aligned
    assert h(A, B, C, 1, 8, 256, 32, B + 16, None) == EINVAL     # y overlaps xs (8 floats)
    u = pq2.lib.pq2_matmul_small_m_tiles_fused_g  # (x, dtype, stride, tiles, m, n, k, agroup, y)
    for bad in (0, 16, 96, 256):
        assert u(A, 0, 128, C, 1, 8, 128, bad, D, None) == EINVAL, bad
    assert u(None, 0, 128, C, 1, 8, 128, 64, D, None) == EINVAL
    assert u(A, 3, 128, C, 1, 8, 128, 64, D, None) == EINVAL        # dtype
    assert u(A, 0, 128, C, 17, 8, 128, 64, D, None) == ESHAPE       # columns
    assert u(A, 0, 128, C, 1, 8, 96, 32, D, None) == ESHAPE         # k % 128
    assert u(A, 0, 100, C, 1, 8, 128, 64, D, None) == ESHAPE        # stride < k
    assert u(A + 8, 0, 128, C, 1, 8, 128, 64, D, None) == EALIGN    # x not 16-byte aligned
    assert u(A, 0, 132, C, 2, 8, 128, 64, D, None) == EALIGN        # rows 264 bytes apart
    assert u(A, 0, 128, C, 1, 8, 128, 32, A + 16, None) == EINVAL   # y overlaps x
    if not _gpu_visible():
        for agroup in (128, 64, 32):
            assert f(A, 0, 5120, 4, 5120, agroup, B, C, None) == EDEVICE
            assert g(A, B, C, 4, 8, 5120, agroup, D, None) == EDEVICE
            assert h(A, B, C, 256, 8, 5120, agroup, D, None) == EDEVICE
            assert u(A, 0, 5120, C, 4, 8, 5120, agroup, D, None) == EDEVICE


def test_prefill_tile_validation():
    t = pq2.lib.pq2_matmul_prefill_tuned
    assert t(A, B, C, 1, 8, 128, D, 6, None) == EINVAL
    assert pq2.lib.pq2_matmul_prefill_planes_tuned(A, B, C, 1, 8, 128, D, 6, None) == EINVAL
    assert pq2.lib.pq2_matmul_prefill_tiles_tuned(A, B, C, 1, 8, 128, D, 6, None) == EINVAL
    assert pq2.lib.pq2_matmul_prefill_planes(A + 8, B, C, 1, 8, 128, D, None) == EALIGN
    assert t(A, B, C, 1, 8, 128, D, -1, None) == EINVAL
    assert t(A, B, C, 0, 8, 128, D, 1, None) == ESHAPE


def test_quantize_planes_validation():
    f = pq2.lib.pq2_quantize_act_i8_planes
    assert f(None, 0, 128, 1, 128, B, C, D, None) == EINVAL
    assert f(A, 0, 128, 1, 128, B, C, None, None) == EINVAL   # no qsum
    assert f(A, 3, 128, 1, 128, B, C, D, None) == EINVAL      # unknown dtype
    assert f(A, 0, 128, 0, 128, B, C, D, None) == ESHAPE
    assert f(A, 0, 128, 1, 96, B, C, D, None) == ESHAPE
    assert f(A, 0, 100, 1, 128, B, C, D, None) == ESHAPE      # stride < k
    assert f(A, 0, 128, 1, 128, B + 8, C, D, None) == EALIGN  # qp not 16-byte aligned
    assert f(A, 0, 128, 1, 128, B, C + 2, D, None) == EALIGN
    assert f(A, 0, 128, 1, 128, B, C, D + 2, None) == EALIGN  # qsum not 4-byte aligned
    assert f(A, 0, 128, 2, 128, B, C, C, None) == EINVAL      # qsum overlaps xs
    assert f(A, 0, 128, 2, 128, A + 16, C, D, None) == EINVAL  # qp overlaps x


def test_small_m_planes_validation():
    f = pq2.lib.pq2_matmul_small_m_planes
    assert f(None, B, E, C, 1, 8, 128, D, None) == EINVAL
    assert f(A, B, None, C, 1, 8, 128, D, None) == EINVAL     # no qsum
    assert f(A, B, E, C, 17, 8, 128, D, None) == ESHAPE
    assert f(A, B, E, C, 1, 8, 200, D, None) == ESHAPE
    assert f(A + 8, B, E, C, 1, 8, 128, D, None) == EALIGN    # qp 16-byte alignment
    assert f(A, B, E + 2, C, 1, 8, 128, D, None) == EALIGN    # qsum 4-byte alignment
    assert f(A, B, E, C, 1, 8, 128, E, None) == EINVAL        # y overlaps qsum
    t = pq2.lib.pq2_matmul_small_m_planes_tuned
    assert t(A, B, E, C, 1, 8, 128, D, 4, 0, 1, None) == EINVAL  # rows per lane
    assert t(A, B, E, C, 1, 8, 128, D, 100, 0, 3, None) == EINVAL  # row blocks
    assert t(A, B, E, C, 1, 8, 128, D, 0, 9, 0, None) == EINVAL  # waves
    assert t(A, B, E, C, 1, 8, 128, D, 0, 0, 7, None) == EINVAL  # engine


def test_small_m_fused_validation():
    f = pq2.lib.pq2_matmul_small_m_fused
    assert f(None, 0, 128, C, 1, 8, 128, D, None) == EINVAL
    assert f(A, 0, 128, None, 1, 8, 128, D, None) == EINVAL
    assert f(A, 0, 128, C, 1, 8, 128, None, None) == EINVAL
    assert f(A, 3, 128, C, 1, 8, 128, D, None) == EINVAL        # unknown dtype
    assert f(A, 0, 128, C, 0, 8, 128, D, None) == ESHAPE
    assert f(A, 0, 128, C, 17, 8, 128, D, None) == ESHAPE       # column limit
    assert f(A, 0, 128, C, 1, 0, 128, D, None) == ESHAPE
    assert f(A, 0, 200, C, 1, 8, 200, D, None) == ESHAPE        # k % 128
    assert f(A, 0, 100, C, 1, 8, 128, D, None) == ESHAPE        # stride < k
    assert f(A, 2, 1 << 26, C, 16, 8, 128, D, None) == ESHAPE   # x span beyond 2^31 bytes
    assert f(A + 2, 0, 128, C, 1, 8, 128, D, None) == EALIGN    # x 16-byte alignment
    assert f(A, 0, 132, C, 2, 8, 128, D, None) == EALIGN        # row stride 264 bytes
    assert f(A, 0, 128, C + 8, 1, 8, 128, D, None) == EALIGN    # planes 16-byte alignment
    assert f(A, 0, 128, C, 1, 8, 128, D + 2, None) == EALIGN
    assert f(A, 0, 128, C, 1, 8, 128, A + 64, None) == EINVAL   # y overlaps x
    assert f(A, 0, 128, C, 1, 8, 128, C + 16, None) == EINVAL   # y overlaps planes
    t = pq2.lib.pq2_matmul_small_m_fused_tuned
    assert t(A, 0, 128, C, 1, 8, 128, D, 3, 0, 1, None) == EINVAL  # rows per lane
    assert t(A, 0, 128, C, 1, 8, 128, D, 100, 0, 3, None) == EINVAL  # row blocks
    assert t(A, 0, 128, C, 1, 8, 128, D, 0, 9, 0, None) == EINVAL  # waves
    assert t(A, 0, 128, C, 1, 8, 128, D, 0, 0, 5, None) == EINVAL  # engine


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros((1, 128), dtype=torch.int8)
    xs = torch.zeros((1, 1), dtype=torch.float32)
    planes = torch.zeros(34, dtype=torch.uint8)
    y = torch.zeros((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        pq2.pq2_matmul_small_m(q, xs, planes, y)


@pytest.mark.parametrize("order", ["package_first", "torch_first"])
def test_single_hip_runtime_whatever_the_import_order(order):
    """Regression: importing the package before torch used to map a second
    HIP runtime (the system one) next to torch's, and kernels launched through
    it on torch's memory crashed the process."""
    import subprocess
    import sys
    first, second = ("gemm_int8_act_amd", "torch") if order == "package_first" else ("torch", "gemm_int8_act_amd")
    code = (f"import {first}; import {second}; "
            "maps = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_raw_reader_validation():
    r = pq2.lib.pq2_matmul_small_m_raw
    assert r(None, B, C, 34, 1, 8, 128, D, None) == EINVAL
    assert r(A, B, C, 33, 1, 8, 128, D, None) == ESHAPE           # stride below one block
    assert r(A, B, C, 35, 1, 8, 128, D, None) == ESHAPE           # odd stride
    assert r(A, B, C, 1 << 27, 1, 8, 128, D, None) == ESHAPE      # stride too large
    assert r(A, B, C, 34, 17, 8, 128, D, None) == ESHAPE          # columns
    assert r(A, B, C, 34, 1, 8, 96, D, None) == ESHAPE            # k % 128
    assert r(A, B, C + 1, 34, 1, 8, 128, D, None) == EALIGN       # raw not 2-byte aligned
    assert r(A + 8, B, C, 34, 1, 8, 128, D, None) == EALIGN       # q not 16-byte aligned
    assert r(A, B, C, 34, 1, 8, 128, C + 16, None) == EINVAL      # y overlaps raw
    if not _gpu_visible():
        assert r(A, B, C + 2, 170, 4, 8, 640, D, None) == EDEVICE


def test_read_probe_validation_and_grid():
    w = pq2.pq2_read_probe_words
    # One word per wave: the decode engines' grids and k split (segments of
    # 8 groups over at most 8 waves).
    assert w(pq2.LAYOUT_TILES, 10240, 5120) == 640 * 5
    assert w(pq2.LAYOUT_PLANES, 10240, 5120) == 1280 * 5
    assert w(pq2.LAYOUT_TILES, 5120, 17408) == 320 * 9       # 17 segments: 9 waves of 2 (up to 16 waves)
    assert w(pq2.LAYOUT_PLANES, 5120, 17408) == 640 * 6      # 17 segments: 6 waves of 3 (up to 8 waves)
    assert w(pq2.LAYOUT_PLANES, 33, 640) == 5                # ragged rows, one partial segment
    assert w(pq2.LAYOUT_TILES, 17, 8192) == 2 * 8
    assert w(2, 8, 128) == 0 and w(0, 0, 128) == 0 and w(0, 8, 96) == 0
    r = pq2.lib.pq2_read_probe
    assert r(None, 0, 8, 128, D, None) == EINVAL
    assert r(A, 2, 8, 128, D, None) == EINVAL                # layout
    assert r(A, 0, 0, 128, D, None) == ESHAPE
    assert r(A, 1, 8, 96, D, None) == ESHAPE
    assert r(A + 4, 0, 8, 128, D, None) == EALIGN            # weights not 16-byte aligned
    assert r(A, 0, 8, 128, D + 2, None) == EALIGN            # out not 4-byte aligned
    assert r(A, 0, 8, 128, A + 16, None) == EINVAL           # out overlaps the weights
    if not _gpu_visible():
        assert r(A, 1, 10240, 5120, D, None) == EDEVICE


def test_splitk_validation_and_sizes():
    pf, cw = pq2.pq2_tiles_splitk_partial_floats, pq2.pq2_tiles_splitk_counter_words
    assert pf(1, 5120, 17408) == 17 * 5120          # one slice per 1024-element segment
    assert pf(4, 10240, 5120) == 5 * 4 * 10240
    assert pf(3, 33, 640) == 1 * 3 * 33               # one partial segment
    assert cw(5120) == 4 * 320 and cw(33) == 4 * 3
    assert pq2.lib.pq2_tiles_splitk_partial_floats(0, 8, 128) == -1
    assert pq2.lib.pq2_tiles_splitk_partial_floats(17, 8, 128) == -1
    assert pq2.lib.pq2_tiles_splitk_counter_words(0) == -1
    f = pq2.lib.pq2_matmul_small_m_tiles_splitk
    # q, xs, tiles, m, n, k, y, partials, counters, stream
    assert f(A, B, C, 1, 8, 128, D, None, E, None) == EINVAL            # no partials
    assert f(A, B, C, 1, 8, 128, D, E, None, None) == EINVAL            # no counters
    assert f(A, B, C, 17, 8, 128, D, E, E + 4096, None) == ESHAPE       # columns
    assert f(A, B, C, 1, 8, 96, D, E, E + 4096, None) == ESHAPE         # k % 128
    assert f(A, B, C, 1, 8, 128, D, E + 2, E + 4096, None) == EALIGN    # partials not 4-byte aligned
    assert f(A, B, C, 1, 8, 128, D, E, E + 4098, None) == EALIGN        # counters not 4-byte aligned
    assert f(A, B, C, 1, 8, 128, D, E, E + 16, None) == EINVAL          # counters overlap partials
    assert f(A, B, C, 1, 8, 128, D, D + 16, E, None) == EINVAL          # partials overlap y
    assert f(A, B, C, 1, 8, 128, D, C + 64, E, None) == EINVAL          # partials overlap the tiles
    t = pq2.lib.pq2_matmul_small_m_tiles_splitk_tuned
    assert t(A, B, C, 1, 8, 128, D, E, E + 4096, 17, None) == EINVAL    # more than 16 waves
    assert t(A, B, C, 1, 8, 128, D, E, E + 4096, -1, None) == EINVAL
    if not _gpu_visible():
        assert f(A, B, C, 4, 5120, 17408, D, E, E + (1 << 24), None) == EDEVICE
        assert t(A, B, C, 4, 5120, 17408, D, E, E + (1 << 24), 3, None) == EDEVICE


def test_stream_and_empty_probe_validation():
    w = pq2.pq2_stream_probe_words
    assert w(2048) == 8192 and w(1) == 4 and w(0) == 0 and w(65537) == 0
    s = pq2.lib.pq2_stream_probe
    # buf, bytes, workgroups, store_all, sentinel, out, stream
    assert s(None, 1024, 8, 1, 0, D, None) == EINVAL
    assert s(A, 1024, 8, 1, 0, None, None) == EINVAL
    assert s(A, 1000, 8, 1, 0, D, None) == ESHAPE            # not a multiple of 16
    assert s(A, 0, 8, 1, 0, D, None) == ESHAPE
    assert s(A, 1 << 31, 8, 1, 0, D, None) == ESHAPE          # 32-bit offsets
    assert s(A, 1024, 0, 1, 0, D, None) == ESHAPE
    assert s(A, 1024, 65537, 1, 0, D, None) == ESHAPE
    assert s(A + 8, 1024, 8, 1, 0, D, None) == EALIGN
    assert s(A, 1024, 8, 1, 0, D + 2, None) == EALIGN
    assert s(A, 1024, 8, 1, 0, A + 512, None) == EINVAL       # out overlaps buf
    c = pq2.lib.pq2_stream_probe_cfg
    # buf, bytes, workgroups, waves, loads per lane, policy, store_all, sentinel, out, stream
    assert c(None, 4096, 8, 4, 2, 1, 1, 0, D, None) == EINVAL
    assert c(A, 4096, 8, 4, 2, 1, 1, 0, None, None) == EINVAL
    assert c(A, 4096, 8, 4, 2, -1, 1, 0, D, None) == EINVAL       # policy
    assert c(A, 4096, 8, 4, 2, 4, 1, 0, D, None) == EINVAL
    assert c(A, 4096, 8, 0, 2, 1, 1, 0, D, None) == ESHAPE        # waves
    assert c(A, 4096, 8, 17, 2, 1, 1, 0, D, None) == ESHAPE
    for u in (0, 3, 5, 32):                                        # loads per lane: 1, 2, 4, 8 or 16
        assert c(A, 4096, 8, 1, u, 1, 1, 0, D, None) == ESHAPE
    assert c(A, 4096, 8, 8, 16, 1, 1, 0, D, None) == ESHAPE       # more than 64 KB per workgroup and chunk
    assert c(A, 4096, 65536, 16, 2, 1, 1, 0, D, None) == ESHAPE   # an iteration spans more than 1 GiB
    assert c(A, 1040, 8, 4, 2, 2, 1, 0, D, None) == ESHAPE        # LDS loads: whole 1 KB blocks
    assert c(A, 1040, 8, 4, 2, 3, 1, 0, D, None) == ESHAPE
    assert c(A, 1000, 8, 4, 2, 0, 1, 0, D, None) == ESHAPE
    assert c(A + 8, 4096, 8, 4, 2, 1, 1, 0, D, None) == EALIGN
    assert c(A, 4096, 8, 4, 2, 1, 1, 0, A + 1024, None) == EINVAL  # out overlaps buf
    e = pq2.lib.pq2_empty_probe
    assert e(0, 1, None) == ESHAPE and e(1, 0, None) == ESHAPE and e(1, 17, None) == ESHAPE
    assert e((1 << 20) + 1, 1, None) == ESHAPE
    if not _gpu_visible():
        assert s(A, 1024, 8, 1, 0, D, None) == EDEVICE
        assert e(256, 4, None) == EDEVICE
        assert c(A, 4096, 8, 4, 2, 3, 1, 0, D, None) == EDEVICE
        assert c(A, 1040, 8, 4, 2, 1, 1, 0, D, None) == EDEVICE   # buffer loads: any multiple of 16
    text = open(os.path.join(ROOT, "include", "pq2_measure.h")).read()
    for name, value in (("BUFFER", pq2.STREAM_BUFFER), ("BUFFER_NT", pq2.STREAM_BUFFER_NT),
                        ("LDS", pq2.STREAM_LDS), ("LDS_NT", pq2.STREAM_LDS_NT)):
        assert re.search(rf"PQ2_STREAM_{name} = {value}\b", text), name


def test_gemv_static_validation():
    f = pq2.lib.pq2_gemv_tiles_static
    # x, dtype, stride, tiles, m, n, k, y, stream
    assert f(A, 0, 128, C, 0, 8, 128, D, None) == ESHAPE
    assert f(A, 0, 128, C, 17, 8, 128, D, None) == ESHAPE      # beyond the static scratch (16 columns)
    assert f(A, 0, 1 << 17, C, 1, 8, 1 << 17, D, None) == ESHAPE  # k beyond 65536
    assert f(A, 0, 96, C, 1, 8, 96, D, None) == ESHAPE
    assert f(A, 0, 128, C, 1, 0, 128, D, None) == ESHAPE
    if not _gpu_visible():
        assert f(A, 0, 5120, C, 4, 8, 5120, D, None) == EDEVICE
