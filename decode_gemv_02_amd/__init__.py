"""VBQ packed mixed-bit decode on AMD MI355X: Python binding of ``libvbq.so``.

Thin ctypes layer with the C ABI's names (``include/vbq.h``): it only
marshals pointers, sizes and the HIP stream. Every step of the packed GEMV /
GEMM runs in the library's HIP kernels; PyTorch supplies device memory and
streams. There is no fallback: if the compiled library is missing, importing
the binding raises.

Method: VBQ paper (arXiv 2607.02893), §3.1 Eq. (1) (groups of 64 weights with
their own width b in {1,2,4,8} and scale s, w_hat = s*q) and §6 (fused
dequantise-and-multiply decode over packed groups).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # import before the library so it binds to the HIP runtime torch has mapped

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvbq.so")
ABI_VERSION = 3
GROUP = 64
MAX_K = 65536
MAX_BATCH = 64
MAX_MULTI = 32
TILE_ROWS = 64
TILE_GROUPS = 4

OK, ERR_NULL, ERR_SHAPE, ERR_WIDTH, ERR_CODE, ERR_SCALE, ERR_CAPACITY, ERR_OFFSETS, ERR_ALIGN, \
    ERR_TOO_LARGE, ERR_HIP, ERR_ABI, ERR_PADDING, ERR_FORMAT, ERR_NOMEM, ERR_INTERNAL = range(16)
NOALLOC_SCRATCH_BYTES = 4 << 20
NOALLOC_COUNTER_BYTES = 64 << 10
CONTAINER_HEADER = 128


class VbqSizes(ctypes.Structure):
    _fields_ = [("widths_bytes", ctypes.c_uint64), ("scales_bytes", ctypes.c_uint64),
                ("offsets_bytes", ctypes.c_uint64), ("payload_bytes", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64)]


class VbqMatrix(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("n", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("payload_bytes", ctypes.c_uint32), ("widths", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tile_offsets", ctypes.c_void_p), ("payload", ctypes.c_void_p), ("uniform_bits", ctypes.c_uint32),
                ("stream_index", ctypes.c_void_p)]


class VbqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    U32 = ctypes.c_uint32
    lib.vbq_abi_version.restype = U32
    lib.vbq_abi_version.argtypes = []
    lib.vbq_status_string.restype = ctypes.c_char_p
    lib.vbq_status_string.argtypes = [ctypes.c_int]
    lib.vbq_last_error.restype = ctypes.c_char_p
    lib.vbq_last_error.argtypes = []
    lib.vbq_pack_sizes.argtypes = [U32, U32, P, ctypes.POINTER(VbqSizes)]
    lib.vbq_pack.argtypes = [U32, U32, P, P, P, P, P, P, P, ctypes.c_uint64]
    lib.vbq_validate_host.argtypes = [ctypes.POINTER(VbqMatrix)]
    lib.vbq_tile_count.restype = ctypes.c_uint64
    lib.vbq_tile_count.argtypes = [U32, U32]
    lib.vbq_gemv_multi.argtypes = [ctypes.POINTER(ctypes.POINTER(VbqMatrix)), ctypes.POINTER(P), ctypes.POINTER(P),
                                   U32, P]
    lib.vbq_gemv_multi_noalloc.argtypes = [ctypes.POINTER(ctypes.POINTER(VbqMatrix)), ctypes.POINTER(P),
                                           ctypes.POINTER(P), U32, P]
    lib.vbq_gemm_smallbatch_multi.argtypes = [ctypes.POINTER(ctypes.POINTER(VbqMatrix)), P, U32, ctypes.POINTER(P),
                                              U32, P]
    lib.vbq_gemv.argtypes = [ctypes.POINTER(VbqMatrix), P, P, P]
    lib.vbq_gemv_multi_f16.argtypes = [ctypes.POINTER(ctypes.POINTER(VbqMatrix)), ctypes.POINTER(P),
                                       ctypes.POINTER(P), U32, P]
    lib.vbq_gemv_swiglu.argtypes = [ctypes.POINTER(VbqMatrix), ctypes.POINTER(VbqMatrix), P, P, P]
    lib.vbq_uniform_width.argtypes = [ctypes.POINTER(VbqMatrix), ctypes.POINTER(U32)]
    lib.vbq_gemm_smallbatch.argtypes = [ctypes.POINTER(VbqMatrix), P, U32, P, P]
    lib.vbq_unpack_codes.argtypes = [ctypes.POINTER(VbqMatrix), P, P]
    lib.vbq_stream_index_bytes.argtypes = [U32, U32, ctypes.POINTER(ctypes.c_uint64)]
    lib.vbq_build_stream_index.argtypes = [ctypes.POINTER(VbqMatrix), P, P]
    lib.vbq_quantize.argtypes = [U32, U32, P, P, P, P, P]
    lib.vbq_soft_quantize.argtypes = [U32, U32, P, P, P, ctypes.c_float, P, P, P, P, P]
    lib.vbq_recipe_head_bits.argtypes = [U32, P, P]
    lib.vbq_recipe_head_order.argtypes = [U32, P, P]
    lib.vbq_recipe_head_tiers.argtypes = [U32, P, P, P]
    lib.vbq_gemv_head_grouped.argtypes = [ctypes.POINTER(ctypes.POINTER(VbqMatrix)), U32, P, P, P, U32, P]
    lib.vbq_probe_stream_read.argtypes = [P, ctypes.c_uint64, P, U32, P]
    lib.vbq_probe_dense_gemv.argtypes = [P, P, P, U32, U32, P]
    lib.vbq_check_padding.argtypes = [ctypes.POINTER(VbqMatrix), U32, U32, U32]
    lib.vbq_container_size.argtypes = [ctypes.POINTER(VbqMatrix), ctypes.POINTER(ctypes.c_uint64)]
    lib.vbq_container_write.argtypes = [ctypes.POINTER(VbqMatrix), P, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
    lib.vbq_container_open.argtypes = [P, ctypes.c_uint64, ctypes.POINTER(VbqMatrix)]
    for f in (lib.vbq_pack_sizes, lib.vbq_pack, lib.vbq_validate_host, lib.vbq_gemv, lib.vbq_gemv_multi,
              lib.vbq_gemm_smallbatch, lib.vbq_unpack_codes, lib.vbq_quantize, lib.vbq_recipe_head_bits,
              lib.vbq_check_padding, lib.vbq_container_size, lib.vbq_container_write, lib.vbq_container_open,
              lib.vbq_gemv_swiglu, lib.vbq_uniform_width, lib.vbq_recipe_head_order, lib.vbq_gemv_multi_f16,
              lib.vbq_soft_quantize, lib.vbq_gemv_multi_noalloc, lib.vbq_recipe_head_tiers,
              lib.vbq_probe_stream_read, lib.vbq_probe_dense_gemv, lib.vbq_gemm_smallbatch_multi,
              lib.vbq_stream_index_bytes, lib.vbq_build_stream_index, lib.vbq_gemv_head_grouped):
        f.restype = ctypes.c_int
    if lib.vbq_abi_version() != ABI_VERSION:
        raise ImportError(f"libvbq.so ABI {lib.vbq_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def _check(status: int):
    if status != OK:
        raise VbqError(status, lib.vbq_last_error().decode())


def _np_ptr(a):
    return None if a is None or a.size == 0 else a.ctypes.data


def _stream_handle(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


# ------------------------------------------------------------------ host side

@dataclass
class HostMatrix:
    """The four packed arrays in host memory."""
    n: int
    k: int
    widths: np.ndarray       # uint8
    scales: np.ndarray       # uint16 binary16 bits
    tile_offsets: np.ndarray  # uint32 [tiles+1]
    payload: np.ndarray      # uint8

    @property
    def payload_bytes(self) -> int:
        return int(self.payload.size)

    @property
    def total_bytes(self) -> int:
        return int(self.widths.size + 2 * self.scales.size + 4 * self.tile_offsets.size + self.payload.size)

    def view(self) -> VbqMatrix:
        return VbqMatrix(ABI_VERSION, self.n, self.k, self.payload_bytes, _np_ptr(self.widths),
                         _np_ptr(self.scales), _np_ptr(self.tile_offsets), _np_ptr(self.payload))


def vbq_pack_sizes(n: int, k: int, bits: np.ndarray) -> dict:
    bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
    out = VbqSizes()
    _check(lib.vbq_pack_sizes(n, k, _np_ptr(bits), ctypes.byref(out)))
    return {f: int(getattr(out, f)) for f, _ in VbqSizes._fields_}


def vbq_pack(n: int, k: int, bits: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> HostMatrix:
    """Pack int8 codes [n,k], per-group widths [n,k/64] and binary16 scales [n,k/64]."""
    bits = np.ascontiguousarray(bits, dtype=np.uint8).reshape(-1)
    codes = np.ascontiguousarray(codes, dtype=np.int8).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
    sz = vbq_pack_sizes(n, k, bits)
    widths = np.zeros(sz["widths_bytes"], np.uint8)
    sc = np.zeros(sz["scales_bytes"] // 2, np.uint16)
    offs = np.zeros(sz["offsets_bytes"] // 4, np.uint32)
    payload = np.zeros(sz["payload_bytes"], np.uint8)
    _check(lib.vbq_pack(n, k, _np_ptr(bits), _np_ptr(codes), _np_ptr(scales), _np_ptr(widths), _np_ptr(sc),
                        offs.ctypes.data, _np_ptr(payload), payload.size))
    return HostMatrix(n, k, widths, sc, offs, payload)


def vbq_uniform_width(m: HostMatrix) -> int:
    """b when every group of m has width b, else 0."""
    v = m.view()
    out = ctypes.c_uint32()
    _check(lib.vbq_uniform_width(ctypes.byref(v), ctypes.byref(out)))
    return int(out.value)


def vbq_validate_host(m: HostMatrix) -> None:
    v = m.view()
    _check(lib.vbq_validate_host(ctypes.byref(v)))


# ------------------------------------------------------------------ device side

class DeviceMatrix:
    """Packed matrix resident in device memory (torch tensors own the bytes)."""

    def __init__(self, host: HostMatrix, device="cuda", uniform: bool = True, stream_index: bool = True):
        """uniform: declare the matrix's single width (when it has one) so launches take the
        uniform-width kernels; False keeps it on the mixed-width kernel. stream_index: build the
        matrix's stream index on the device (vbq_build_stream_index, 264 bytes per tile), which the
        mixed-width kernel then reads instead of deriving each tile's counts and list."""
        self.n, self.k = host.n, host.k
        self.uniform_bits = vbq_uniform_width(host) if uniform else 0
        self.payload_bytes = host.payload_bytes
        self.total_bytes = host.total_bytes
        dev = torch.device(device)
        self.device = dev

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self._widths = up(host.widths)
        self._scales = up(host.scales.view(np.int16))
        self._offsets = up(host.tile_offsets.view(np.int32))
        self._payload = up(host.payload)
        self.struct = VbqMatrix(ABI_VERSION, self.n, self.k, self.payload_bytes, self._widths.data_ptr(),
                                self._scales.data_ptr(), self._offsets.data_ptr(), self._payload.data_ptr(),
                                self.uniform_bits, None)
        self._index = None
        if stream_index and self.n and self.k:
            self._index = torch.empty(vbq_stream_index_bytes(self.n, self.k), dtype=torch.uint8, device=dev)
            s = torch.cuda.current_stream(dev)
            _check(lib.vbq_build_stream_index(ctypes.byref(self.struct), self._index.data_ptr(), int(s.cuda_stream)))
            s.synchronize()   # built once; later calls may run on any stream
            self.struct.stream_index = self._index.data_ptr()
        self.index_bytes = 0 if self._index is None else self._index.numel()


def vbq_gemv(w: DeviceMatrix, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[n] (fp32) = W x (x fp16 [k]); enqueued on `stream` (default: torch's current stream)."""
    assert x.dtype == torch.float16 and y.dtype == torch.float32
    assert x.is_contiguous() and y.is_contiguous() and x.numel() == w.k and y.numel() >= w.n
    _check(lib.vbq_gemv(ctypes.byref(w.struct), x.data_ptr(), y.data_ptr(), _stream_handle(stream, w.device)))
    return y


def vbq_gemv_swiglu(gate: DeviceMatrix, up: DeviceMatrix, x: torch.Tensor, h: torch.Tensor,
                    stream=None) -> torch.Tensor:
    """h[n] (fp16) = silu(gate x) * (up x), x fp16 [k]; one launch."""
    assert x.dtype == torch.float16 and h.dtype == torch.float16 and x.is_contiguous() and h.is_contiguous()
    assert x.numel() == gate.k and h.numel() >= gate.n
    _check(lib.vbq_gemv_swiglu(ctypes.byref(gate.struct), ctypes.byref(up.struct), x.data_ptr(), h.data_ptr(),
                               _stream_handle(stream, gate.device)))
    return h


def vbq_tile_count(n: int, k: int) -> int:
    return int(lib.vbq_tile_count(n, k))


def vbq_stream_index_bytes(n: int, k: int) -> int:
    out = ctypes.c_uint64()
    _check(lib.vbq_stream_index_bytes(n, k, ctypes.byref(out)))
    return int(out.value)


def vbq_build_stream_index(w: DeviceMatrix, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Write w's stream index to the uint8 device tensor out (vbq_stream_index_bytes(n, k) bytes)."""
    assert out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= vbq_stream_index_bytes(w.n, w.k)
    _check(lib.vbq_build_stream_index(ctypes.byref(w.struct), out.data_ptr(), _stream_handle(stream, w.device)))
    return out


def _multi_args(ws, xs, ys, ydtype):
    count = len(ws)
    assert len(xs) == count and len(ys) == count
    for w, x, y in zip(ws, xs, ys):
        assert x.dtype == torch.float16 and y.dtype == ydtype and x.is_contiguous() and y.is_contiguous()
        assert x.numel() == w.k and y.numel() >= w.n
    wa = (ctypes.POINTER(VbqMatrix) * max(count, 1))(*[ctypes.pointer(w.struct) for w in ws])
    xa = (ctypes.c_void_p * max(count, 1))(*[x.data_ptr() for x in xs])
    ya = (ctypes.c_void_p * max(count, 1))(*[y.data_ptr() for y in ys])
    dev = ws[0].device if count else torch.device("cuda")
    return wa, xa, ya, count, dev


def vbq_gemv_multi(ws, xs, ys, stream=None):
    """Several independent GEMVs (ys[i] = W_i xs[i]) in one launch; up to MAX_MULTI."""
    wa, xa, ya, count, dev = _multi_args(ws, xs, ys, torch.float32)
    _check(lib.vbq_gemv_multi(wa, xa, ya, count, _stream_handle(stream, dev)))
    return ys


def vbq_gemv_multi_noalloc(ws, xs, ys, stream=None):
    """vbq_gemv_multi that never allocates: its scratch is the library's fixed per-GPU array (calls that
    overlap on one GPU race)."""
    wa, xa, ya, count, dev = _multi_args(ws, xs, ys, torch.float32)
    _check(lib.vbq_gemv_multi_noalloc(wa, xa, ya, count, _stream_handle(stream, dev)))
    return ys


def vbq_gemv_multi_f16(ws, xs, ys, stream=None):
    """vbq_gemv_multi with fp16 outputs (ys: float16 tensors)."""
    wa, xa, ya, count, dev = _multi_args(ws, xs, ys, torch.float16)
    _check(lib.vbq_gemv_multi_f16(wa, xa, ya, count, _stream_handle(stream, dev)))
    return ys


def vbq_gemm_smallbatch(w: DeviceMatrix, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[m][n] (fp32) = x[m][k] (fp16) W^T, m <= 64."""
    assert x.dtype == torch.float16 and y.dtype == torch.float32 and x.dim() == 2 and x.shape[1] == w.k
    assert x.is_contiguous() and y.is_contiguous() and y.numel() >= x.shape[0] * w.n
    _check(lib.vbq_gemm_smallbatch(ctypes.byref(w.struct), x.data_ptr(), x.shape[0], y.data_ptr(),
                                   _stream_handle(stream, w.device)))
    return y


def vbq_gemm_smallbatch_multi(ws, x: torch.Tensor, ys, stream=None):
    """ys[i][m][n_i] (fp32) = x[m][k] (fp16) W_i^T for matrices sharing x (q/k/v, gate/up), few launches."""
    count = len(ws)
    assert count == len(ys) and x.dtype == torch.float16 and x.dim() == 2 and x.is_contiguous()
    for w, y in zip(ws, ys):
        assert w.k == x.shape[1] and y.dtype == torch.float32 and y.is_contiguous() and y.numel() >= x.shape[0] * w.n
    wa = (ctypes.POINTER(VbqMatrix) * max(count, 1))(*[ctypes.pointer(w.struct) for w in ws])
    ya = (ctypes.c_void_p * max(count, 1))(*[y.data_ptr() for y in ys])
    _check(lib.vbq_gemm_smallbatch_multi(wa, x.data_ptr(), x.shape[0], ya, count, _stream_handle(stream, x.device)))
    return ys


def vbq_unpack_codes(w: DeviceMatrix, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Decoded int8 codes [n][k] (device)."""
    assert out.dtype == torch.int8 and out.is_contiguous() and out.numel() >= w.n * w.k
    _check(lib.vbq_unpack_codes(ctypes.byref(w.struct), out.data_ptr(), _stream_handle(stream, w.device)))
    return out


def vbq_quantize(w: torch.Tensor, bits: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 stream=None):
    """Eq. (1) per group on the device: w fp32 [n][k], bits uint8 [n][k/64] -> codes int8 [n][k]
    and scales (int16 tensor holding binary16 bit patterns) [n][k/64]."""
    assert w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()
    n, k = w.shape
    assert bits.dtype == torch.uint8 and bits.is_contiguous() and bits.numel() == n * (k // GROUP)
    assert codes.dtype == torch.int8 and codes.is_contiguous() and codes.numel() >= n * k
    assert scales.dtype == torch.int16 and scales.is_contiguous() and scales.numel() >= n * (k // GROUP)
    _check(lib.vbq_quantize(n, k, w.data_ptr(), bits.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                            _stream_handle(stream, w.device)))
    return codes, scales


def vbq_recipe_head_bits(freq: np.ndarray) -> np.ndarray:
    """Per-row widths of the frequency-tiered head (host, uint8 [rows])."""
    freq = np.ascontiguousarray(freq, dtype=np.uint64).reshape(-1)
    out = np.zeros(freq.size, np.uint8)
    _check(lib.vbq_recipe_head_bits(freq.size, _np_ptr(freq), _np_ptr(out)))
    return out


def vbq_check_padding(m: HostMatrix, n_real: int, k_real: int, k_multiple: int = 512) -> None:
    """Raises VbqError unless every padded row/column of m dequantizes to zero and k % k_multiple == 0."""
    v = m.view()
    _check(lib.vbq_check_padding(ctypes.byref(v), n_real, k_real, k_multiple))


def vbq_container_bytes(m: HostMatrix) -> np.ndarray:
    """The container image of m (uint8 array)."""
    v = m.view()
    size = ctypes.c_uint64()
    _check(lib.vbq_container_size(ctypes.byref(v), ctypes.byref(size)))
    out = np.zeros(size.value, np.uint8)
    written = ctypes.c_uint64()
    _check(lib.vbq_container_write(ctypes.byref(v), out.ctypes.data, out.size, ctypes.byref(written)))
    return out


def vbq_container_open(image: np.ndarray) -> HostMatrix:
    """HostMatrix whose arrays are views into image (checked by the library first)."""
    image = np.ascontiguousarray(image, dtype=np.uint8).reshape(-1)
    v = VbqMatrix()
    _check(lib.vbq_container_open(image.ctypes.data, image.size, ctypes.byref(v)))
    base = image.ctypes.data
    groups = v.n * (v.k // GROUP)

    def part(ptr, count, dtype):
        if not ptr or count == 0:
            return np.zeros(0, dtype)
        start = ptr - base
        return image[start:start + count * np.dtype(dtype).itemsize].view(dtype)

    tiles = vbq_tile_count(v.n, v.k)
    return HostMatrix(v.n, v.k, part(v.widths, (groups + 3) // 4, np.uint8), part(v.scales, groups, np.uint16),
                      part(v.tile_offsets, tiles + 1, np.uint32), part(v.payload, v.payload_bytes, np.uint8))


def vbq_save(path: str, m: HostMatrix) -> None:
    vbq_container_bytes(m).tofile(path)


def vbq_load(path: str) -> HostMatrix:
    return vbq_container_open(np.fromfile(path, dtype=np.uint8))


def vbq_recipe_head_order(freq: np.ndarray) -> np.ndarray:
    """Vocabulary rows in rank order (descending frequency, ties to the lower row), uint32."""
    freq = np.ascontiguousarray(freq, dtype=np.uint64).reshape(-1)
    out = np.zeros(freq.size, np.uint32)
    _check(lib.vbq_recipe_head_order(freq.size, _np_ptr(freq), _np_ptr(out)))
    return out


def vbq_probe_stream_read(buf: torch.Tensor, nbytes: int, sink: torch.Tensor, blocks: int, stream=None):
    """Read nbytes of buf (device) once: the HBM read ceiling of a launch that size (measurement only)."""
    assert buf.is_contiguous() and nbytes <= buf.numel() * buf.element_size()
    assert sink.dtype == torch.int32 and sink.numel() >= blocks * 256
    _check(lib.vbq_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                     _stream_handle(stream, buf.device)))


def vbq_probe_dense_gemv(w: torch.Tensor, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[n] (fp32) = W x for dense fp16 W [n][k]: the dense baseline (measurement only)."""
    assert w.dtype == torch.float16 and x.dtype == torch.float16 and y.dtype == torch.float32
    assert w.dim() == 2 and w.is_contiguous() and x.is_contiguous() and y.is_contiguous()
    n, k = w.shape
    assert x.numel() == k and y.numel() >= n
    _check(lib.vbq_probe_dense_gemv(w.data_ptr(), x.data_ptr(), y.data_ptr(), n, k, _stream_handle(stream, w.device)))
    return y


def vbq_gemv_head_grouped(tiers, x: torch.Tensor, row_map: torch.Tensor, y: torch.Tensor, stream=None):
    """y[row_map[rank]] = the grouped head's logit of that rank; tiers are DeviceMatrix row blocks in rank
    order (same k), row_map a device uint32 tensor (torch.int32 storage) with one entry per rank."""
    count = len(tiers)
    assert count <= MAX_MULTI and x.dtype == torch.float16 and y.dtype == torch.float32
    assert row_map.dtype in (torch.int32, torch.uint32) and row_map.is_contiguous() and y.is_contiguous()
    assert row_map.numel() == sum(t.n for t in tiers) and all(t.k == x.numel() for t in tiers)
    arr = (ctypes.POINTER(VbqMatrix) * max(count, 1))(*[ctypes.pointer(t.struct) for t in tiers])
    dev = tiers[0].device if count else y.device
    _check(lib.vbq_gemv_head_grouped(arr, count, x.data_ptr(), row_map.data_ptr(), y.data_ptr(), y.numel(),
                                     _stream_handle(stream, dev)))
    return y


def vbq_recipe_head_tiers(freq: np.ndarray):
    """(order, tier_rows): rows in rank order and the rank counts of the 8-, 4-, 2- and 1-bit tiers."""
    freq = np.ascontiguousarray(freq, dtype=np.uint64).reshape(-1)
    order = np.zeros(freq.size, np.uint32)
    tiers = np.zeros(4, np.uint32)
    _check(lib.vbq_recipe_head_tiers(freq.size, _np_ptr(freq), _np_ptr(order), tiers.ctypes.data))
    return order, tiers


def vbq_pack_grouped_head(freq: np.ndarray, codes: np.ndarray, scales: np.ndarray):
    """The recipe head as one-width row blocks: returns (order, [HostMatrix per tier present]).

    codes int8 [rows][k] and scales uint16 [rows][k/64] are in vocabulary order and must follow the
    widths vbq_recipe_head_bits(freq) gives each row. The library ranks the rows and cuts the tiers
    (vbq_recipe_head_tiers); each block holds one tier's rows in rank order (8, 4, 2, 1 bits), and the
    blocks' outputs, concatenated, are the logits of rows `order`."""
    order, tiers = vbq_recipe_head_tiers(freq)
    rows, k = codes.shape
    blocks = []
    start = 0
    for b, cnt in zip((8, 4, 2, 1), tiers):
        if cnt == 0:
            continue
        sel = order[start:start + cnt]
        blocks.append(vbq_pack(int(cnt), k, np.full((int(cnt), k // GROUP), b, np.uint8),
                               np.ascontiguousarray(codes[sel]), np.ascontiguousarray(scales[sel])))
        start += int(cnt)
    return order, blocks


def vbq_soft_quantize(w: torch.Tensor, logits: torch.Tensor, gumbel: torch.Tensor, tau: float, w_soft: torch.Tensor,
                      pi: torch.Tensor, group_bits: torch.Tensor, mean_bits: torch.Tensor, stream=None):
    """§3.2 soft quantizer on the device: w fp32 [n][k]; logits, gumbel, pi fp32 [n*k/64][4];
    w_soft fp32 [n][k]; group_bits fp32 [n*k/64]; mean_bits float64 [1]."""
    assert w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()
    n, k = w.shape
    groups = n * (k // GROUP)
    for t, dt, cnt in ((logits, torch.float32, 4 * groups), (gumbel, torch.float32, 4 * groups),
                       (pi, torch.float32, 4 * groups), (w_soft, torch.float32, n * k),
                       (group_bits, torch.float32, groups), (mean_bits, torch.float64, 1)):
        assert t.dtype == dt and t.is_contiguous() and t.numel() >= cnt
    _check(lib.vbq_soft_quantize(n, k, w.data_ptr(), logits.data_ptr(), gumbel.data_ptr(), float(tau),
                                 w_soft.data_ptr(), pi.data_ptr(), group_bits.data_ptr(), mean_bits.data_ptr(),
                                 _stream_handle(stream, w.device)))
    return w_soft, pi, group_bits, mean_bits
