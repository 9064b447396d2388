"""Plain CPU oracle for the packed-ternary x INT8-activation matmul.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``gemm_int8_act_amd``) never imports it and shares no code with it.

The arithmetic lives in ``pq2_oracle.c`` (plain C, FP32 quantiser steps as
single IEEE operations, FP64 scaling and summation); this module compiles it
with gcc and wraps it with numpy.  Every function follows the definition on
the pages "Kernel experiments: recorded evidence" and "Baseline and the
integer breakthrough" (see the C file's header for the passages).  Each
function is pinned by tests in ``tests/test_oracle_pins.py`` against values
the pages print, closed forms, exact rational arithmetic and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pq2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GROUP = 128
BLOCK_BYTES = 34
DTYPE_CODES = {"bf16": 0, "f16": 1, "f32": 2}

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_decode_weight.argtypes = [p, i32]
    lib.oracle_decode_weight.restype = i32
    lib.oracle_decode_byte.argtypes = [ctypes.c_uint8, p]
    lib.oracle_decode_byte.restype = None
    lib.oracle_prepare_planes.argtypes = [p, i64, i64, i64, p]
    lib.oracle_prepare_planes.restype = i32
    lib.oracle_tiles_bytes.argtypes = [i64, i64]
    lib.oracle_tiles_bytes.restype = i64
    lib.oracle_prepare_tiles.argtypes = [p, i64, i64, i64, p]
    lib.oracle_prepare_tiles.restype = i32
    lib.oracle_quantize_act_i8.argtypes = [p, i32, i64, i64, i64, p, p]
    lib.oracle_quantize_act_i8.restype = i32
    lib.oracle_matmul_raw.argtypes = [p, p, p, i64, i64, i64, i64, p, p]
    lib.oracle_matmul_raw.restype = i32
    lib.oracle_matmul_raw_sample.argtypes = [p, p, p, i64, i64, i64, i64, p, p, i64, p, p]
    lib.oracle_matmul_raw_sample.restype = i32
    lib.oracle_quantize_act_i8_g.argtypes = [p, i32, i64, i64, i64, i64, p, p]
    lib.oracle_quantize_act_i8_g.restype = i32
    lib.oracle_matmul_raw_g.argtypes = [p, p, p, i64, i64, i64, i64, i64, p, p]
    lib.oracle_matmul_raw_g.restype = i32
    lib.oracle_matmul_raw_sample_g.argtypes = [p, p, p, i64, i64, i64, i64, i64, p, p, i64, p, p]
    lib.oracle_matmul_raw_sample_g.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def decode_byte(byte: int) -> np.ndarray:
    """Four weight values of one code byte: element s is weight 4b+s."""
    out = np.zeros(4, dtype=np.int8)
    _load().oracle_decode_byte(ctypes.c_uint8(byte), _ptr(out))
    return out


def decode_block_codes(codes32: np.ndarray) -> np.ndarray:
    """128 weight values (int) of one block's 32 code bytes, in weight order."""
    codes32 = np.ascontiguousarray(codes32, dtype=np.uint8)
    assert codes32.shape == (32,)
    lib = _load()
    return np.array([lib.oracle_decode_weight(_ptr(codes32), i) for i in range(GROUP)], dtype=np.int64)


def prepare_planes(raw: np.ndarray, n: int, k: int) -> np.ndarray:
    """Raw [n][row_stride] uint8 blocks -> prepared planes (n*k/128*34 bytes)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    assert raw.ndim == 2 and raw.shape[0] == n
    planes = np.empty(n * (k // GROUP) * BLOCK_BYTES, dtype=np.uint8)
    rc = _load().oracle_prepare_planes(_ptr(raw), raw.shape[1], n, k, _ptr(planes))
    if rc:
        raise ValueError("oracle_prepare_planes: bad shape")
    return planes


def tiles_bytes(n: int, k: int) -> int:
    return int(_load().oracle_tiles_bytes(n, k))


def prepare_tiles(raw: np.ndarray, n: int, k: int) -> np.ndarray:
    """Raw [n][row_stride] uint8 blocks -> the tile layout of the decode GEMV."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    assert raw.ndim == 2 and raw.shape[0] == n
    out = np.empty(tiles_bytes(n, k), dtype=np.uint8)
    rc = _load().oracle_prepare_tiles(_ptr(raw), raw.shape[1], n, k, _ptr(out))
    if rc:
        raise ValueError("oracle_prepare_tiles: bad shape")
    return out


def quantize_act_i8(x_bits: np.ndarray, dtype: str = "bf16", k: int | None = None):
    """Group-128 quantisation of the first k columns of each row of x_bits.

    x_bits is [m][width]: uint16 bit patterns for bf16/f16, float32 values for
    f32; the row stride is ``width`` (k defaults to width).  Returns
    (q int8 [m][k], xs float32 [m][k/128])."""
    code = DTYPE_CODES[dtype]
    x_bits = np.ascontiguousarray(x_bits, dtype=np.float32 if code == 2 else np.uint16)
    m, width = x_bits.shape
    return _quantize(x_bits, code, width, m, width if k is None else k)


def _quantize(x_bits, code, row_stride, m, k):
    q = np.empty((m, k), dtype=np.int8)
    xs = np.empty((m, k // GROUP), dtype=np.float32)
    rc = _load().oracle_quantize_act_i8(_ptr(x_bits), code, row_stride, m, k, _ptr(q), _ptr(xs))
    if rc:
        raise ValueError("oracle_quantize_act_i8: bad shape")
    return q, xs


def matmul_raw(q: np.ndarray, xs: np.ndarray, raw: np.ndarray, n: int, k: int):
    """y[m][n] (float64) and the acceptance bound[m][n] from raw blocks."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    m = q.shape[0]
    assert q.shape == (m, k) and xs.shape == (m, k // GROUP) and raw.shape[0] == n
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = _load().oracle_matmul_raw(_ptr(q), _ptr(xs), _ptr(raw), raw.shape[1], m, n, k, _ptr(y), _ptr(bound))
    if rc:
        raise ValueError("oracle_matmul_raw: bad shape")
    return y, bound


def matmul_raw_sample(q, xs, raw, n: int, k: int, mi, ni):
    """Selected outputs y[mi[c]][ni[c]] and bounds (float64 vectors)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    m = q.shape[0]
    count = mi.shape[0]
    y = np.empty(count, dtype=np.float64)
    bound = np.empty(count, dtype=np.float64)
    rc = _load().oracle_matmul_raw_sample(_ptr(q), _ptr(xs), _ptr(raw), raw.shape[1], m, n, k,
                                          _ptr(mi), _ptr(ni), count, _ptr(y), _ptr(bound))
    if rc:
        raise ValueError("oracle_matmul_raw_sample: bad shape or index")
    return y, bound


# ---------------------------------------------------------------- smaller activation groups
# Page "Kernel experiments: recorded evidence", section C (Diagram 3, Tests 8
# and 9): weight blocks stay 128 weights with one fp16 scale; activations get
# one scale per `agroup` = 128, 64 or 32 elements.
AGROUPS = (128, 64, 32)


def quantize_act_i8_g(x_bits: np.ndarray, agroup: int, dtype: str = "bf16", k: int | None = None):
    """Quantisation in activation groups of ``agroup`` elements.  Returns
    (q int8 [m][k], xs float32 [m][k/agroup])."""
    code = DTYPE_CODES[dtype]
    x_bits = np.ascontiguousarray(x_bits, dtype=np.float32 if code == 2 else np.uint16)
    m, width = x_bits.shape
    k = width if k is None else k
    q = np.empty((m, k), dtype=np.int8)
    xs = np.empty((m, k // agroup if agroup else 0), dtype=np.float32)
    rc = _load().oracle_quantize_act_i8_g(_ptr(x_bits), code, width, m, k, agroup, _ptr(q), _ptr(xs))
    if rc:
        raise ValueError("oracle_quantize_act_i8_g: bad shape or group")
    return q, xs


def matmul_raw_g(q: np.ndarray, xs: np.ndarray, raw: np.ndarray, n: int, k: int, agroup: int):
    """y[m][n] (float64) and bound[m][n] with activation groups of ``agroup``."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    m = q.shape[0]
    assert q.shape == (m, k) and xs.shape == (m, k // agroup) and raw.shape[0] == n
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = _load().oracle_matmul_raw_g(_ptr(q), _ptr(xs), _ptr(raw), raw.shape[1], m, n, k, agroup, _ptr(y),
                                     _ptr(bound))
    if rc:
        raise ValueError("oracle_matmul_raw_g: bad shape or group")
    return y, bound


def matmul_raw_sample_g(q, xs, raw, n: int, k: int, agroup: int, mi, ni):
    """Selected outputs y[mi[c]][ni[c]] and bounds with activation groups of ``agroup``."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    m = q.shape[0]
    count = mi.shape[0]
    y = np.empty(count, dtype=np.float64)
    bound = np.empty(count, dtype=np.float64)
    rc = _load().oracle_matmul_raw_sample_g(_ptr(q), _ptr(xs), _ptr(raw), raw.shape[1], m, n, k, agroup,
                                            _ptr(mi), _ptr(ni), count, _ptr(y), _ptr(bound))
    if rc:
        raise ValueError("oracle_matmul_raw_sample_g: bad shape, group or index")
    return y, bound
