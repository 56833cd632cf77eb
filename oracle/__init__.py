"""Plain CPU oracle for the VBQ packed GEMV / small-batch GEMM.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path. It wraps
``vbq_oracle.c`` (scalar loops, double-precision accumulation) through ctypes
and shares no code with the HIP library. What it computes, and the packed
layout it reads, are stated in the header of ``vbq_oracle.c`` and follow the
VBQ paper (arXiv 2607.02893): §3.1 Eq. (1) for w_hat = s * q and its grid, §6
for the per-group fused decode over packed {1, 2, 4, 8}-bit groups.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .build import LIB_PATH, build

OK, ERR_NULL, ERR_SHAPE, ERR_WIDTH, ERR_CODE, ERR_SCALE, ERR_CAPACITY, ERR_OFFSETS = range(8)

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f64p = ctypes.POINTER(ctypes.c_double)
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64

_lib = None


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} failed with status {status}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the compiled oracle (compiling it first only if it is absent)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_pack_sizes.argtypes = [_u32, _u32, _u8p, _u64p]
    lib.oracle_pack.argtypes = [_u32, _u32, _u8p, _i8p, _u16p, _u8p, _u16p, _u32p, _u8p, _u64]
    lib.oracle_check_offsets.argtypes = [_u32, _u32, _u8p, _u32p, _u64]
    lib.oracle_unpack.argtypes = [_u32, _u32, _u8p, _u32p, _u8p, _u64, _i8p]
    lib.oracle_gemm.argtypes = [_u32, _u32, _u8p, _u16p, _u32p, _u8p, _u64, _u16p, _u32, _f64p, _u32, _u32]
    lib.oracle_gemv.argtypes = [_u32, _u32, _u8p, _u16p, _u32p, _u8p, _u64, _u16p, _f64p, _u32, _u32]
    for f in (lib.oracle_pack_sizes, lib.oracle_pack, lib.oracle_check_offsets, lib.oracle_unpack,
              lib.oracle_gemm, lib.oracle_gemv):
        f.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _p(a, t):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


@dataclass
class Packed:
    """Host copy of one packed matrix (the four arrays of the layout)."""
    n: int
    k: int
    widths: np.ndarray       # uint8
    scales: np.ndarray       # uint16 (binary16 bits)
    tile_offsets: np.ndarray  # uint32 [tiles+1]
    payload: np.ndarray      # uint8

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.size)

    @property
    def total_bytes(self) -> int:
        return int(self.widths.size + 2 * self.scales.size + 4 * self.tile_offsets.size + self.payload.size)


def half_to_double(h: int, lib=None) -> float:
    return (lib or load()).oracle_half_to_double(int(h))


def pack_sizes(n: int, k: int, bits: np.ndarray, lib=None) -> dict:
    lib = lib or load()
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.zeros(5, dtype=np.uint64)
    st = lib.oracle_pack_sizes(n, k, _p(bits, _u8p), _p(out, _u64p))
    if st:
        raise OracleError(st, "pack_sizes")
    return dict(zip(("widths", "scales", "tile_offsets", "payload", "total"), (int(v) for v in out)))


def pack(n: int, k: int, bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, lib=None) -> Packed:
    lib = lib or load()
    bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
    codes = np.ascontiguousarray(codes, dtype=np.int8).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
    sz = pack_sizes(n, k, bits, lib)
    widths = np.zeros(sz["widths"], dtype=np.uint8)
    sc = np.zeros(sz["scales"] // 2, dtype=np.uint16)
    offs = np.zeros(sz["tile_offsets"] // 4, dtype=np.uint32)
    payload = np.zeros(sz["payload"], dtype=np.uint8)
    st = lib.oracle_pack(n, k, _p(bits, _u8p), _p(codes, _i8p), _p(scales, _u16p), _p(widths, _u8p),
                         _p(sc, _u16p), _p(offs, _u32p), _p(payload, _u8p), sz["payload"])
    if st:
        raise OracleError(st, "pack")
    return Packed(n, k, widths, sc, offs, payload)


def check_offsets(p: Packed, lib=None) -> int:
    lib = lib or load()
    return lib.oracle_check_offsets(p.n, p.k, _p(p.widths, _u8p), _p(p.tile_offsets, _u32p), p.payload_bytes)


def unpack(p: Packed, lib=None) -> np.ndarray:
    lib = lib or load()
    out = np.zeros((p.n, p.k), dtype=np.int8)
    st = lib.oracle_unpack(p.n, p.k, _p(p.widths, _u8p), _p(p.tile_offsets, _u32p), _p(p.payload, _u8p),
                           p.payload_bytes, _p(out, _i8p))
    if st:
        raise OracleError(st, "unpack")
    return out


def gemm(p: Packed, x: np.ndarray, rows=None, lib=None) -> np.ndarray:
    """Y[m][n] in float64; x is binary16 bits [m, k]. rows=(begin, end) limits the rows computed
    (other entries are NaN)."""
    lib = lib or load()
    x = np.asarray(x, dtype=np.uint16)
    x = np.ascontiguousarray(x.reshape(1, -1) if x.ndim == 1 else x)
    if x.shape[1] != p.k:
        raise ValueError(f"x has {x.shape[1]} columns, the matrix has k = {p.k}")
    m = x.shape[0]
    b, e = rows if rows is not None else (0, p.n)
    y = np.full((m, p.n), np.nan, dtype=np.float64)
    st = lib.oracle_gemm(p.n, p.k, _p(p.widths, _u8p), _p(p.scales, _u16p), _p(p.tile_offsets, _u32p),
                         _p(p.payload, _u8p), p.payload_bytes, _p(x, _u16p), m, _p(y, _f64p), b, e)
    if st:
        raise OracleError(st, "gemm")
    return y


def gemv(p: Packed, x: np.ndarray, rows=None, lib=None) -> np.ndarray:
    return gemm(p, np.asarray(x, dtype=np.uint16).reshape(1, -1), rows, lib)[0]


def gemv_threaded(p: Packed, x: np.ndarray, row_begin: int, row_end: int, threads: int, lib=None) -> np.ndarray:
    """Rows [row_begin, row_end) split over `threads` host threads (ctypes drops the GIL while the C
    loop runs). Returns y for those rows."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
    y = np.full(p.n, np.nan, dtype=np.float64)
    bounds = np.linspace(row_begin, row_end, threads + 1).astype(np.int64)

    def run(i):
        b, e = int(bounds[i]), int(bounds[i + 1])
        if e > b:
            st = lib.oracle_gemv(p.n, p.k, _p(p.widths, _u8p), _p(p.scales, _u16p), _p(p.tile_offsets, _u32p),
                                 _p(p.payload, _u8p), p.payload_bytes, _p(x, _u16p), _p(y, _f64p), b, e)
            if st:
                raise OracleError(st, "gemv")

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, range(threads)))
    return y[row_begin:row_end]


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Gated-MLP intermediate silu(g) * u = g * u / (1 + e^-g), fp64 (VBQ §6, "Granularity is
    deployment-friendly", where the padded channels are inert because silu(0) * u = 0)."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * np.asarray(u, np.float64)
