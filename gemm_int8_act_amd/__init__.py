"""gemm_int8_act_amd -- packed-ternary (PQ2) x INT8-activation matmul on MI355X.

A thin ctypes binding over ``libpq2.so`` (hand-written HIP for gfx950, C ABI
in ``include/pq2.h``).  Every function here has the name of the C entry point
it calls and only marshals arguments: torch tensors give device pointers and
shapes, the current torch stream gives the HIP stream.  All arithmetic runs
in the HIP kernels; there is no CPU or PyTorch fallback.  If the library is
missing, importing the package raises ImportError; build it with
``python gemm_int8_act_amd/build.py``.

Status codes map to exceptions: EINVAL, ESHAPE and EALIGN raise ValueError;
ELAUNCH and EDEVICE raise RuntimeError.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpq2.so")

PQ2_OK, PQ2_EINVAL, PQ2_ESHAPE, PQ2_EALIGN, PQ2_ELAUNCH, PQ2_EDEVICE = range(6)
PQ2_BF16, PQ2_F16, PQ2_F32 = 0, 1, 2
PQ2_MAX_SMALL_M = 16
PQ2_MAX_K = 65536

EXPORTED = (
    "pq2_layout_version",
    "pq2_status_str",
    "pq2_last_hip_error",
    "pq2_prepare_planes",
    "pq2_quantize_act_i8",
    "pq2_matmul_small_m",
    "pq2_matmul_prefill",
    "pq2_matmul_small_m_tuned",
    "pq2_quantize_act_i8_planes",
    "pq2_matmul_small_m_planes",
    "pq2_matmul_small_m_planes_tuned",
    "pq2_matmul_prefill_tuned",
    "pq2_tiles_bytes",
    "pq2_prepare_tiles",
    "pq2_matmul_small_m_tiles",
    "pq2_matmul_small_m_tiles_tuned",
    "pq2_matmul_small_m_tiles_fused",
    "pq2_matmul_small_m_tiles_fused_tuned",
    "pq2_matmul_small_m_tiles_fused_g",
    "pq2_matmul_prefill_tiles",
    "pq2_matmul_prefill_tiles_tuned",
    "pq2_matmul_prefill_planes",
    "pq2_matmul_prefill_planes_tuned",
    "pq2_matmul_small_m_fused",
    "pq2_matmul_small_m_fused_tuned",
    "pq2_quantize_act_i8_g",
    "pq2_matmul_small_m_tiles_g",
    "pq2_gemv_tiles",
    "pq2_matmul_prefill_tiles_g",
    "pq2_matmul_small_m_raw",
    "pq2_read_probe",
    "pq2_read_probe_words",
    "pq2_matmul_small_m_tiles_splitk",
    "pq2_matmul_small_m_tiles_splitk_tuned",
    "pq2_tiles_splitk_partial_floats",
    "pq2_tiles_splitk_counter_words",
    "pq2_stream_probe",
    "pq2_stream_probe_words",
    "pq2_stream_probe_cfg",
    "pq2_empty_probe",
    "pq2_gemv_tiles_static",
)


def _hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as fh:
            return sorted({line.split()[-1] for line in fh if "libamdhip64" in line})
    except OSError:
        return []


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: the HIP library must be built "
            "(python gemm_int8_act_amd/build.py); there is no fallback path")
    # torch brings its own HIP runtime.  It must be loaded BEFORE libpq2.so so
    # that the dynamic loader binds libpq2's libamdhip64 dependency to that
    # same copy; loading libpq2 first maps the system runtime, torch then maps
    # its own, and kernels launched through one runtime on memory and streams
    # of the other crash the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process ({runtimes}); "
                          "libpq2 must share torch's runtime")
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.pq2_layout_version.argtypes = []
    lib.pq2_layout_version.restype = i32
    lib.pq2_status_str.argtypes = [i32]
    lib.pq2_status_str.restype = ctypes.c_char_p
    lib.pq2_last_hip_error.argtypes = []
    lib.pq2_last_hip_error.restype = ctypes.c_char_p
    lib.pq2_prepare_planes.argtypes = [p, i64, i64, i64, p, p]
    lib.pq2_prepare_planes.restype = i32
    lib.pq2_quantize_act_i8.argtypes = [p, i32, i64, i64, i64, p, p, p]
    lib.pq2_quantize_act_i8.restype = i32
    lib.pq2_matmul_small_m.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m.restype = i32
    lib.pq2_matmul_prefill.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_prefill.restype = i32
    lib.pq2_matmul_small_m_tuned.argtypes = [p, p, p, i64, i64, i64, p, i32, i32, i32, p]
    lib.pq2_matmul_small_m_tuned.restype = i32
    lib.pq2_quantize_act_i8_planes.argtypes = [p, i32, i64, i64, i64, p, p, p, p]
    lib.pq2_quantize_act_i8_planes.restype = i32
    lib.pq2_matmul_small_m_planes.argtypes = [p, p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_planes.restype = i32
    lib.pq2_matmul_small_m_planes_tuned.argtypes = [p, p, p, p, i64, i64, i64, p, i32, i32, i32, p]
    lib.pq2_matmul_small_m_planes_tuned.restype = i32
    lib.pq2_matmul_prefill_tuned.argtypes = [p, p, p, i64, i64, i64, p, i32, p]
    lib.pq2_matmul_prefill_tuned.restype = i32
    lib.pq2_matmul_prefill_planes.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_prefill_planes.restype = i32
    lib.pq2_matmul_prefill_planes_tuned.argtypes = [p, p, p, i64, i64, i64, p, i32, p]
    lib.pq2_matmul_prefill_planes_tuned.restype = i32
    lib.pq2_matmul_small_m_fused.argtypes = [p, i32, i64, p, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_fused.restype = i32
    lib.pq2_matmul_small_m_fused_tuned.argtypes = [p, i32, i64, p, i64, i64, i64, p, i32, i32, i32, p]
    lib.pq2_matmul_small_m_fused_tuned.restype = i32
    lib.pq2_tiles_bytes.argtypes = [i64, i64]
    lib.pq2_tiles_bytes.restype = i64
    lib.pq2_prepare_tiles.argtypes = [p, i64, i64, i64, p, p]
    lib.pq2_prepare_tiles.restype = i32
    lib.pq2_matmul_small_m_tiles.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_tiles.restype = i32
    lib.pq2_gemv_tiles.argtypes = [p, i32, i64, p, i64, i64, i64, p, p, p, p]
    lib.pq2_gemv_tiles.restype = i32
    lib.pq2_quantize_act_i8_g.argtypes = [p, i32, i64, i64, i64, i64, p, p, p]
    lib.pq2_quantize_act_i8_g.restype = i32
    lib.pq2_matmul_small_m_tiles_g.argtypes = [p, p, p, i64, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_tiles_g.restype = i32
    lib.pq2_matmul_prefill_tiles_g.argtypes = [p, p, p, i64, i64, i64, i64, p, p]
    lib.pq2_matmul_prefill_tiles_g.restype = i32
    lib.pq2_matmul_small_m_raw.argtypes = [p, p, p, i64, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_raw.restype = i32
    lib.pq2_read_probe.argtypes = [p, i32, i64, i64, p, p]
    lib.pq2_read_probe.restype = i32
    lib.pq2_read_probe_words.argtypes = [i32, i64, i64]
    lib.pq2_read_probe_words.restype = i64
    lib.pq2_matmul_small_m_tiles_tuned.argtypes = [p, p, p, i64, i64, i64, p, i32, i32, p]
    lib.pq2_matmul_small_m_tiles_tuned.restype = i32
    lib.pq2_matmul_prefill_tiles.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.pq2_matmul_prefill_tiles.restype = i32
    lib.pq2_matmul_prefill_tiles_tuned.argtypes = [p, p, p, i64, i64, i64, p, i32, p]
    lib.pq2_matmul_prefill_tiles_tuned.restype = i32
    lib.pq2_matmul_small_m_tiles_fused.argtypes = [p, i32, i64, p, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_tiles_fused.restype = i32
    lib.pq2_matmul_small_m_tiles_fused_tuned.argtypes = [p, i32, i64, p, i64, i64, i64, p, i32, i32, p]
    lib.pq2_matmul_small_m_tiles_fused_tuned.restype = i32
    lib.pq2_matmul_small_m_tiles_fused_g.argtypes = [p, i32, i64, p, i64, i64, i64, i64, p, p]
    lib.pq2_matmul_small_m_tiles_fused_g.restype = i32
    lib.pq2_matmul_small_m_tiles_splitk.argtypes = [p, p, p, i64, i64, i64, p, p, p, p]
    lib.pq2_matmul_small_m_tiles_splitk.restype = i32
    lib.pq2_matmul_small_m_tiles_splitk_tuned.argtypes = [p, p, p, i64, i64, i64, p, p, p, i32, p]
    lib.pq2_matmul_small_m_tiles_splitk_tuned.restype = i32
    lib.pq2_tiles_splitk_partial_floats.argtypes = [i64, i64, i64]
    lib.pq2_tiles_splitk_partial_floats.restype = i64
    lib.pq2_tiles_splitk_counter_words.argtypes = [i64]
    lib.pq2_tiles_splitk_counter_words.restype = i64
    lib.pq2_stream_probe.argtypes = [p, i64, i64, i32, ctypes.c_uint32, p, p]
    lib.pq2_stream_probe.restype = i32
    lib.pq2_stream_probe_words.argtypes = [i64]
    lib.pq2_stream_probe_cfg.argtypes = [p, i64, i64, i32, i32, i32, i32, ctypes.c_uint32, p, p]
    lib.pq2_stream_probe_cfg.restype = i32
    lib.pq2_stream_probe_words.restype = i64
    lib.pq2_empty_probe.argtypes = [i64, i32, p]
    lib.pq2_empty_probe.restype = i32
    lib.pq2_gemv_tiles_static.argtypes = [p, i32, i64, p, i64, i64, i64, p, p]
    lib.pq2_gemv_tiles_static.restype = i32
    return lib


lib = _load_library()


class Pq2Error(Exception):
    pass


def pq2_status_str(status: int) -> str:
    return lib.pq2_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status == PQ2_OK:
        return
    msg = f"{what}: {pq2_status_str(status)} (status {status})"
    if status in (PQ2_EINVAL, PQ2_ESHAPE, PQ2_EALIGN):
        raise ValueError(msg)
    if status == PQ2_ELAUNCH:
        msg += f" [{pq2_last_hip_error()}]"
    raise RuntimeError(msg)


def pq2_last_hip_error() -> str:
    return lib.pq2_last_hip_error().decode()


def pq2_layout_version() -> int:
    return lib.pq2_layout_version()


def _dev_ptr(t, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def pq2_prepare_planes(raw, n: int, k: int, planes, stream=None) -> None:
    """raw: uint8 device tensor [n][row_stride] (row stride = raw.stride(0));
    planes: uint8 device tensor of n*(k/128)*34 bytes."""
    import torch
    if raw.dtype != torch.uint8 or planes.dtype != torch.uint8 or raw.dim() != 2 or raw.stride(1) != 1:
        raise ValueError("raw must be a 2-D uint8 tensor with unit column stride; planes uint8")
    if planes.numel() < n * (k // 128) * 34 or not planes.is_contiguous():
        raise ValueError("planes must be a contiguous uint8 tensor of n*(k/128)*34 bytes")
    _check(lib.pq2_prepare_planes(_dev_ptr(raw, "raw"), raw.stride(0), n, k, _dev_ptr(planes, "planes"),
                                  _stream(stream)), "pq2_prepare_planes")


_DTYPES = None


def _dtype_code(x) -> int:
    global _DTYPES
    import torch
    if _DTYPES is None:
        _DTYPES = {torch.bfloat16: PQ2_BF16, torch.float16: PQ2_F16, torch.float32: PQ2_F32}
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    return _DTYPES[x.dtype]


def pq2_quantize_act_i8(x, q, xs, stream=None) -> None:
    """x: [m][>=k] bf16/f16/f32 device tensor (unit column stride); q: int8
    [m][k]; xs: float32 [m][k/128] (both contiguous)."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or not q.is_contiguous() or not xs.is_contiguous():
        raise ValueError("q must be contiguous int8 and xs contiguous float32")
    m, k = q.shape
    if x.shape[0] != m or x.shape[1] < k or xs.numel() != m * (k // 128):
        raise ValueError("shape mismatch between x, q and xs")
    _check(lib.pq2_quantize_act_i8(_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), m, k, _dev_ptr(q, "q"),
                                   _dev_ptr(xs, "xs"), _stream(stream)), "pq2_quantize_act_i8")


def _matmul_args(q, xs, planes, y):
    import torch
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or planes.dtype != torch.uint8 or y.dtype != torch.float32:
        raise ValueError("q int8, xs float32, planes uint8, y float32 expected")
    for name, t in (("q", q), ("xs", xs), ("planes", planes), ("y", y)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    m, k = q.shape
    n = y.shape[1]
    if y.shape[0] != m or xs.numel() != m * (k // 128) or planes.numel() < n * (k // 128) * 34:
        raise ValueError("shape mismatch between q, xs, planes and y")
    return (_dev_ptr(q, "q"), _dev_ptr(xs, "xs"), _dev_ptr(planes, "planes"), m, n, k, _dev_ptr(y, "y"))


def pq2_matmul_small_m(q, xs, planes, y, stream=None) -> None:
    """y[m][n] = PQ2 planes x INT8 activations, 1 <= m <= 16."""
    _check(lib.pq2_matmul_small_m(*_matmul_args(q, xs, planes, y), _stream(stream)), "pq2_matmul_small_m")


def pq2_matmul_small_m_tuned(q, xs, planes, y, rows=0, max_waves=0, engine=0, stream=None) -> None:
    _check(lib.pq2_matmul_small_m_tuned(*_matmul_args(q, xs, planes, y), rows, max_waves, engine,
                                        _stream(stream)), "pq2_matmul_small_m_tuned")


def pq2_tiles_bytes(n: int, k: int) -> int:
    """Bytes of the tile layout of an n x k weight matrix (ValueError on a bad shape)."""
    size = lib.pq2_tiles_bytes(n, k)
    if size < 0:
        raise ValueError(f"pq2_tiles_bytes: unsupported shape n={n} k={k}")
    return size


def pq2_prepare_tiles(raw, n: int, k: int, tiles, stream=None) -> None:
    """raw: uint8 device tensor [n][row_stride]; tiles: contiguous uint8
    device tensor of pq2_tiles_bytes(n, k) bytes."""
    import torch
    if raw.dtype != torch.uint8 or tiles.dtype != torch.uint8 or raw.dim() != 2 or raw.stride(1) != 1:
        raise ValueError("raw must be a 2-D uint8 tensor with unit column stride; tiles uint8")
    if tiles.numel() < pq2_tiles_bytes(n, k) or not tiles.is_contiguous():
        raise ValueError("tiles must be a contiguous uint8 tensor of pq2_tiles_bytes(n, k) bytes")
    _check(lib.pq2_prepare_tiles(_dev_ptr(raw, "raw"), raw.stride(0), n, k, _dev_ptr(tiles, "tiles"),
                                 _stream(stream)), "pq2_prepare_tiles")


def _tiles_args(q, xs, tiles, y):
    import torch
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or tiles.dtype != torch.uint8 or y.dtype != torch.float32:
        raise ValueError("q int8, xs float32, tiles uint8, y float32 expected")
    for name, t in (("q", q), ("xs", xs), ("tiles", tiles), ("y", y)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    m, k = q.shape
    n = y.shape[1]
    if y.shape[0] != m or xs.numel() != m * (k // 128) or tiles.numel() < pq2_tiles_bytes(n, k):
        raise ValueError("shape mismatch between q, xs, tiles and y")
    return (_dev_ptr(q, "q"), _dev_ptr(xs, "xs"), _dev_ptr(tiles, "tiles"), m, n, k, _dev_ptr(y, "y"))


def pq2_matmul_small_m_tiles(q, xs, tiles, y, stream=None) -> None:
    """pq2_matmul_small_m from the tile layout (same bits)."""
    _check(lib.pq2_matmul_small_m_tiles(*_tiles_args(q, xs, tiles, y), _stream(stream)),
           "pq2_matmul_small_m_tiles")


def pq2_matmul_small_m_tiles_tuned(q, xs, tiles, y, max_waves=0, split=0, stream=None) -> None:
    _check(lib.pq2_matmul_small_m_tiles_tuned(*_tiles_args(q, xs, tiles, y), max_waves, split, _stream(stream)),
           "pq2_matmul_small_m_tiles_tuned")


def pq2_gemv_tiles(x, tiles, y, q_work=None, xs_work=None, stream=None) -> None:
    """y = W x from activations: one fused launch at m <= 2 (k <= 8192), else
    the quantiser into q_work (int8 [m][k]) / xs_work (float32 [m][k/128])
    and the tile matmul; the same bits either way."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if tiles.dtype != torch.uint8 or y.dtype != torch.float32 or not tiles.is_contiguous() or not y.is_contiguous():
        raise ValueError("tiles contiguous uint8 and y contiguous float32 expected")
    m, n = y.shape
    k = x.shape[1] if q_work is None else q_work.shape[1]
    if x.shape[0] != m or x.shape[1] < k or tiles.numel() < pq2_tiles_bytes(n, k):
        raise ValueError("shape mismatch between x, tiles and y")
    qp = xp = None
    if q_work is not None or xs_work is not None:
        if q_work is None or xs_work is None or q_work.dtype != torch.int8 or xs_work.dtype != torch.float32 or \
                not q_work.is_contiguous() or not xs_work.is_contiguous() or q_work.shape != (m, k) or \
                xs_work.numel() != m * (k // 128):
            raise ValueError("q_work int8 [m][k] and xs_work float32 [m][k/128], contiguous, expected")
        qp, xp = _dev_ptr(q_work, "q_work"), _dev_ptr(xs_work, "xs_work")
    _check(lib.pq2_gemv_tiles(_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), _dev_ptr(tiles, "tiles"), m, n, k,
                              _dev_ptr(y, "y"), qp, xp, _stream(stream)), "pq2_gemv_tiles")


def pq2_tiles_splitk_partial_floats(m: int, n: int, k: int) -> int:
    """Floats of partial sums pq2_matmul_small_m_tiles_splitk needs."""
    v = int(lib.pq2_tiles_splitk_partial_floats(m, n, k))
    if v < 0:
        raise ValueError(f"invalid shape m={m} n={n} k={k}")
    return v


def pq2_tiles_splitk_counter_words(n: int) -> int:
    """Counter words pq2_matmul_small_m_tiles_splitk needs (zero before the
    first call; every call leaves them zero)."""
    v = int(lib.pq2_tiles_splitk_counter_words(n))
    if v < 0:
        raise ValueError(f"invalid n={n}")
    return v


def _splitk_args(q, xs, tiles, y, partials, counters):
    import torch
    args = _tiles_args(q, xs, tiles, y)
    m, n, k = args[3], args[4], args[5]
    if partials.dtype != torch.float32 or not partials.is_contiguous() or \
            partials.numel() < pq2_tiles_splitk_partial_floats(m, n, k):
        raise ValueError("partials: contiguous float32 of pq2_tiles_splitk_partial_floats(m, n, k) expected")
    if counters.dtype != torch.int32 or not counters.is_contiguous() or \
            counters.numel() < pq2_tiles_splitk_counter_words(n):
        raise ValueError("counters: contiguous int32 of pq2_tiles_splitk_counter_words(n) (all zero) expected")
    return args + (_dev_ptr(partials, "partials"), _dev_ptr(counters, "counters"))


def pq2_matmul_small_m_tiles_splitk(q, xs, tiles, y, partials, counters, stream=None) -> None:
    """Split-k tile matmul: partials float32 scratch, counters int32 words
    that are zero before the first call (each call leaves them zero)."""
    _check(lib.pq2_matmul_small_m_tiles_splitk(*_splitk_args(q, xs, tiles, y, partials, counters), _stream(stream)),
           "pq2_matmul_small_m_tiles_splitk")


def pq2_matmul_small_m_tiles_splitk_tuned(q, xs, tiles, y, partials, counters, waves=0, stream=None) -> None:
    _check(lib.pq2_matmul_small_m_tiles_splitk_tuned(*_splitk_args(q, xs, tiles, y, partials, counters), waves,
                                                     _stream(stream)), "pq2_matmul_small_m_tiles_splitk_tuned")


def pq2_stream_probe_words(workgroups: int) -> int:
    """Words pq2_stream_probe writes (4 per workgroup)."""
    return int(lib.pq2_stream_probe_words(workgroups))


def pq2_stream_probe(buf, nbytes: int, workgroups: int, out, store_all: bool = False, sentinel: int = 0,
                     stream=None) -> None:
    """Linear streaming read of the first nbytes of buf (any contiguous
    device tensor); out int32 [pq2_stream_probe_words(workgroups)]."""
    import torch
    if not buf.is_contiguous() or not out.is_contiguous() or out.dtype != torch.int32:
        raise ValueError("buf contiguous and out contiguous int32 expected")
    if buf.numel() * buf.element_size() < nbytes or out.numel() < pq2_stream_probe_words(workgroups):
        raise ValueError("buf or out too small")
    _check(lib.pq2_stream_probe(_dev_ptr(buf, "buf"), nbytes, workgroups, 1 if store_all else 0,
                                sentinel & 0xFFFFFFFF, _dev_ptr(out, "out"), _stream(stream)), "pq2_stream_probe")


def pq2_stream_probe_cfg(buf, nbytes: int, workgroups: int, waves: int, loads_per_lane: int, policy: int, out,
                         store_all: bool = False, sentinel: int = 0, stream=None) -> None:
    """The stream read with its grid, loads in flight per lane and load
    instruction (STREAM_*) as parameters; out int32 [workgroups * waves]."""
    import torch
    if not buf.is_contiguous() or not out.is_contiguous() or out.dtype != torch.int32:
        raise ValueError("buf contiguous and out contiguous int32 expected")
    if buf.numel() * buf.element_size() < nbytes or out.numel() < workgroups * waves:
        raise ValueError("buf or out too small")
    _check(lib.pq2_stream_probe_cfg(_dev_ptr(buf, "buf"), nbytes, workgroups, waves, loads_per_lane, policy,
                                    1 if store_all else 0, sentinel & 0xFFFFFFFF, _dev_ptr(out, "out"),
                                    _stream(stream)), "pq2_stream_probe_cfg")


def pq2_empty_probe(workgroups: int = 1, waves: int = 1, stream=None) -> None:
    """An empty kernel (the launch floor of back-to-back launches)."""
    _check(lib.pq2_empty_probe(workgroups, waves, _stream(stream)), "pq2_empty_probe")


def pq2_gemv_tiles_static(x, tiles, y, k=None, stream=None) -> None:
    """pq2_gemv_tiles with the library's own static scratch (no allocation);
    k defaults to x.shape[1]."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if tiles.dtype != torch.uint8 or y.dtype != torch.float32 or not tiles.is_contiguous() or not y.is_contiguous():
        raise ValueError("tiles contiguous uint8 and y contiguous float32 expected")
    m, n = y.shape
    k = x.shape[1] if k is None else k
    if x.shape[0] != m or x.shape[1] < k or tiles.numel() < pq2_tiles_bytes(n, k):
        raise ValueError("shape mismatch between x, tiles and y")
    _check(lib.pq2_gemv_tiles_static(_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), _dev_ptr(tiles, "tiles"), m, n,
                                     k, _dev_ptr(y, "y"), _stream(stream)), "pq2_gemv_tiles_static")


def pq2_quantize_act_i8_g(x, q, xs, agroup: int, stream=None) -> None:
    """Quantisation in activation groups of agroup = 128, 64 or 32 elements:
    x [m][>=k] bf16/f16/f32 (unit column stride), q int8 [m][k], xs float32
    [m][k/agroup] (both contiguous)."""
    import torch
    if agroup not in (128, 64, 32):
        raise ValueError("agroup must be 128, 64 or 32")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or not q.is_contiguous() or not xs.is_contiguous():
        raise ValueError("q must be contiguous int8 and xs contiguous float32")
    m, k = q.shape
    if x.shape[0] != m or x.shape[1] < k or xs.numel() != m * (k // agroup):
        raise ValueError("shape mismatch between x, q and xs")
    _check(lib.pq2_quantize_act_i8_g(_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), m, k, agroup, _dev_ptr(q, "q"),
                                     _dev_ptr(xs, "xs"), _stream(stream)), "pq2_quantize_act_i8_g")


def _tiles_g_args(q, xs, tiles, y, agroup):
    import torch
    if agroup not in (128, 64, 32):
        raise ValueError("agroup must be 128, 64 or 32")
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or tiles.dtype != torch.uint8 or y.dtype != torch.float32:
        raise ValueError("q int8, xs float32, tiles uint8, y float32 expected")
    for name, t in (("q", q), ("xs", xs), ("tiles", tiles), ("y", y)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    m, k = q.shape
    n = y.shape[1]
    if y.shape[0] != m or xs.numel() != m * (k // agroup) or tiles.numel() < pq2_tiles_bytes(n, k):
        raise ValueError("shape mismatch between q, xs, tiles and y")
    return (_dev_ptr(q, "q"), _dev_ptr(xs, "xs"), _dev_ptr(tiles, "tiles"), m, n, k, agroup, _dev_ptr(y, "y"))


def pq2_matmul_small_m_tiles_g(q, xs, tiles, y, agroup: int, stream=None) -> None:
    """Tile-layout decode matmul with activation groups of agroup elements
    (q, xs from pq2_quantize_act_i8_g with the same agroup)."""
    _check(lib.pq2_matmul_small_m_tiles_g(*_tiles_g_args(q, xs, tiles, y, agroup), _stream(stream)),
           "pq2_matmul_small_m_tiles_g")


def pq2_matmul_small_m_raw(q, xs, raw, y, stream=None) -> None:
    """pq2_matmul_small_m reading the raw block layout in place: raw uint8
    [n][stride] (stride >= k/128*34 bytes, even; row padding is not read),
    same bits as pq2_matmul_small_m on the prepared planes."""
    import torch
    if q.dtype != torch.int8 or xs.dtype != torch.float32 or raw.dtype != torch.uint8 or y.dtype != torch.float32:
        raise ValueError("q int8, xs float32, raw uint8, y float32 expected")
    for name, t in (("q", q), ("xs", xs), ("y", y)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if raw.dim() != 2 or raw.stride(1) != 1:
        raise ValueError("raw must be [n][stride] bytes with unit column stride")
    m, k = q.shape
    n = y.shape[1]
    if y.shape[0] != m or xs.numel() != m * (k // 128) or raw.shape[0] != n or raw.shape[1] < k // 128 * 34:
        raise ValueError("shape mismatch between q, xs, raw and y")
    _check(lib.pq2_matmul_small_m_raw(_dev_ptr(q, "q"), _dev_ptr(xs, "xs"), _dev_ptr(raw, "raw"), raw.stride(0), m, n,
                                      k, _dev_ptr(y, "y"), _stream(stream)), "pq2_matmul_small_m_raw")


LAYOUT_PLANES = 0
LAYOUT_TILES = 1
STREAM_BUFFER, STREAM_BUFFER_NT, STREAM_LDS, STREAM_LDS_NT = 0, 1, 2, 3


def pq2_read_probe_words(layout: int, n: int, k: int) -> int:
    """Words pq2_read_probe writes (one per wave of its grid)."""
    return int(lib.pq2_read_probe_words(layout, n, k))


def pq2_read_probe(weights, layout: int, n: int, k: int, out, stream=None) -> None:
    """Read-only probe: the decode engine's weight loads for this layout with
    no arithmetic; out uint32-sized int32 [pq2_read_probe_words(...)] gets
    each wave's XOR fold."""
    import torch
    if weights.dtype != torch.uint8 or out.dtype != torch.int32:
        raise ValueError("weights uint8 and out int32 expected")
    if not weights.is_contiguous() or not out.is_contiguous():
        raise ValueError("weights and out must be contiguous")
    words = pq2_read_probe_words(layout, n, k)
    if words == 0:
        raise ValueError("bad layout or shape")
    need = pq2_tiles_bytes(n, k) if layout == LAYOUT_TILES else n * (k // 128) * 34
    if weights.numel() < need or out.numel() < words:
        raise ValueError("weights or out too small")
    _check(lib.pq2_read_probe(_dev_ptr(weights, "weights"), layout, n, k, _dev_ptr(out, "out"), _stream(stream)),
           "pq2_read_probe")


def pq2_matmul_prefill_tiles_g(q, xs, tiles, y, agroup: int, stream=None) -> None:
    """Tile-layout prefill matmul with activation groups of agroup elements
    (q, xs from pq2_quantize_act_i8_g with the same agroup)."""
    _check(lib.pq2_matmul_prefill_tiles_g(*_tiles_g_args(q, xs, tiles, y, agroup), _stream(stream)),
           "pq2_matmul_prefill_tiles_g")


def pq2_matmul_prefill_tiles(q, xs, tiles, y, stream=None) -> None:
    """pq2_matmul_prefill from the tile layout (same bits)."""
    _check(lib.pq2_matmul_prefill_tiles(*_tiles_args(q, xs, tiles, y), _stream(stream)), "pq2_matmul_prefill_tiles")


def pq2_matmul_prefill_tiles_tuned(q, xs, tiles, y, tile=0, stream=None) -> None:
    _check(lib.pq2_matmul_prefill_tiles_tuned(*_tiles_args(q, xs, tiles, y), tile, _stream(stream)),
           "pq2_matmul_prefill_tiles_tuned")


def _tiles_fused_args(x, tiles, y):
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if tiles.dtype != torch.uint8 or y.dtype != torch.float32 or not tiles.is_contiguous() or not y.is_contiguous():
        raise ValueError("tiles uint8 and y float32, both contiguous, expected")
    m, n = y.shape
    k = x.shape[1]
    if x.shape[0] != m or tiles.numel() < pq2_tiles_bytes(n, k):
        raise ValueError("shape mismatch between x, tiles and y")
    return (_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), _dev_ptr(tiles, "tiles"), m, n, k, _dev_ptr(y, "y"))


def pq2_matmul_small_m_tiles_fused(x, tiles, y, stream=None) -> None:
    """Quantise x (bf16/f16/f32 [m][k]) and multiply by the tile layout in one launch."""
    _check(lib.pq2_matmul_small_m_tiles_fused(*_tiles_fused_args(x, tiles, y), _stream(stream)),
           "pq2_matmul_small_m_tiles_fused")


def pq2_matmul_small_m_tiles_fused_g(x, tiles, y, agroup: int, stream=None) -> None:
    """pq2_matmul_small_m_tiles_fused with activation groups of agroup = 128,
    64 or 32 elements (the bits of pq2_quantize_act_i8_g followed by
    pq2_matmul_small_m_tiles_g)."""
    xp, dt, stride, tp, m, n, k, yp = _tiles_fused_args(x, tiles, y)
    _check(lib.pq2_matmul_small_m_tiles_fused_g(xp, dt, stride, tp, m, n, k, agroup, yp, _stream(stream)),
           "pq2_matmul_small_m_tiles_fused_g")


def pq2_matmul_small_m_tiles_fused_tuned(x, tiles, y, max_waves=0, split=0, stream=None) -> None:
    _check(lib.pq2_matmul_small_m_tiles_fused_tuned(*_tiles_fused_args(x, tiles, y), max_waves, split,
                                                    _stream(stream)), "pq2_matmul_small_m_tiles_fused_tuned")


def _fused_args(x, planes, y):
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if planes.dtype != torch.uint8 or y.dtype != torch.float32 or not planes.is_contiguous() or not y.is_contiguous():
        raise ValueError("planes contiguous uint8 and y contiguous float32 expected")
    m, k = x.shape
    n = y.shape[1]
    if y.shape[0] != m or planes.numel() < n * (k // 128) * 34:
        raise ValueError("shape mismatch between x, planes and y")
    return (_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), _dev_ptr(planes, "planes"), m, n, k, _dev_ptr(y, "y"))


def pq2_matmul_small_m_fused(x, planes, y, stream=None) -> None:
    """Quantise x ([m][k] bf16/f16/f32, unit column stride, any row stride)
    and multiply in one launch: the y of pq2_quantize_act_i8 followed by
    pq2_matmul_small_m, bit for bit, 1 <= m <= 16."""
    _check(lib.pq2_matmul_small_m_fused(*_fused_args(x, planes, y), _stream(stream)), "pq2_matmul_small_m_fused")


def pq2_matmul_small_m_fused_tuned(x, planes, y, rows=0, max_waves=0, engine=0, stream=None) -> None:
    _check(lib.pq2_matmul_small_m_fused_tuned(*_fused_args(x, planes, y), rows, max_waves, engine,
                                              _stream(stream)), "pq2_matmul_small_m_fused_tuned")


def pq2_matmul_prefill(q, xs, planes, y, stream=None) -> None:
    """y[m][n] on the INT8 matrix cores (any m >= 1)."""
    _check(lib.pq2_matmul_prefill(*_matmul_args(q, xs, planes, y), _stream(stream)), "pq2_matmul_prefill")


def pq2_matmul_prefill_tuned(q, xs, planes, y, tile=0, stream=None) -> None:
    _check(lib.pq2_matmul_prefill_tuned(*_matmul_args(q, xs, planes, y), tile, _stream(stream)),
           "pq2_matmul_prefill_tuned")


def pq2_quantize_act_i8_planes(x, qp, xs, qsum, stream=None) -> None:
    """As pq2_quantize_act_i8, writing q in code-plane order (qp, int8
    [m][k]) plus the int32 group sums qsum [m][k/128]."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if (qp.dtype != torch.int8 or xs.dtype != torch.float32 or qsum.dtype != torch.int32
            or not qp.is_contiguous() or not xs.is_contiguous() or not qsum.is_contiguous()):
        raise ValueError("qp contiguous int8, xs contiguous float32, qsum contiguous int32 expected")
    m, k = qp.shape
    if x.shape[0] != m or x.shape[1] < k or xs.numel() != m * (k // 128) or qsum.numel() != m * (k // 128):
        raise ValueError("shape mismatch between x, qp, xs and qsum")
    _check(lib.pq2_quantize_act_i8_planes(_dev_ptr(x, "x"), _dtype_code(x), x.stride(0), m, k,
                                          _dev_ptr(qp, "qp"), _dev_ptr(xs, "xs"), _dev_ptr(qsum, "qsum"),
                                          _stream(stream)), "pq2_quantize_act_i8_planes")


def _planes_args(qp, xs, qsum, planes, y):
    import torch
    if qsum.dtype != torch.int32 or not qsum.is_contiguous():
        raise ValueError("qsum must be contiguous int32")
    qa, xa, pa, m, n, k, ya = _matmul_args(qp, xs, planes, y)
    if qsum.numel() != m * (k // 128):
        raise ValueError("qsum must hold m*k/128 group sums")
    return (qa, xa, _dev_ptr(qsum, "qsum"), pa, m, n, k, ya)


def pq2_matmul_small_m_planes(qp, xs, qsum, planes, y, stream=None) -> None:
    """pq2_matmul_small_m from the plane-order quantiser's outputs."""
    _check(lib.pq2_matmul_small_m_planes(*_planes_args(qp, xs, qsum, planes, y), _stream(stream)),
           "pq2_matmul_small_m_planes")


def pq2_matmul_small_m_planes_tuned(qp, xs, qsum, planes, y, rows=0, max_waves=0, engine=0,
                                    stream=None) -> None:
    _check(lib.pq2_matmul_small_m_planes_tuned(*_planes_args(qp, xs, qsum, planes, y), rows,
                                               max_waves, engine, _stream(stream)), "pq2_matmul_small_m_planes_tuned")


def pq2_matmul_prefill_planes(qp, xs, planes, y, stream=None) -> None:
    """pq2_matmul_prefill from plane-order activations (pq2_quantize_act_i8_planes)."""
    _check(lib.pq2_matmul_prefill_planes(*_matmul_args(qp, xs, planes, y), _stream(stream)),
           "pq2_matmul_prefill_planes")


def pq2_matmul_prefill_planes_tuned(qp, xs, planes, y, tile=0, stream=None) -> None:
    _check(lib.pq2_matmul_prefill_planes_tuned(*_matmul_args(qp, xs, planes, y), tile, _stream(stream)),
           "pq2_matmul_prefill_planes_tuned")
