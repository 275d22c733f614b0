"""Python binding of the gfx950 RHT + lattice + bit-strip + Rice codec (``libhq.so``).

Argument marshalling only: every step of the method runs in the HIP kernels behind the C ABI
declared in ``include/hq.h``.  PyTorch provides device memory and the stream.  There is no CPU
fallback: if the library is missing the calls raise.

Entry points mirror the C ABI: ``hq_encode``, ``hq_decode``, ``hq_rate``, ``hq_codes``,
``hq_status``, ``hq_fallbacks``, ``hq_workspace_size``, ``hq_stream_fixed_bytes``, ``hq_encode_bound``,
``hq_version``, ``hq_strerror``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhq.so")

HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_NONFINITE = 0, -1, -2, -3
HQ_ERR_CAPACITY, HQ_ERR_CORRUPT, HQ_ERR_RATE, HQ_ERR_HIP, HQ_ERR_TIMEOUT, HQ_ERR_SCRATCH = -4, -5, -6, -7, -8, -9
HQ_Z, HQ_D4, HQ_E8, HQ_A2 = 0, 1, 2, 3
HQ_F32, HQ_BF16 = 0, 1
LATTICES = {"z": HQ_Z, "d4": HQ_D4, "e8": HQ_E8, "a2": HQ_A2}

EXPORTS = ("hq_version", "hq_strerror", "hq_workspace_size", "hq_stream_fixed_bytes", "hq_encode_bound", "hq_rate",
           "hq_encode", "hq_encode_noalloc", "hq_decode", "hq_status", "hq_fallbacks", "hq_codes",
           "hq_gemv_workspace_size", "hq_gemv",
           "hq_haar_matrix", "hq_rotate", "hq_srft_encode", "hq_srft_decode")


class HqParams(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_uint32), ("lattice", ctypes.c_int32), ("target_bps", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("dither", ctypes.c_uint32), ("step", ctypes.c_float),
                ("rice_k", ctypes.c_int32)]


class HqInfo(ctypes.Structure):
    _fields_ = [("step", ctypes.c_float), ("rice_k", ctypes.c_int32), ("bytes", ctypes.c_uint64),
                ("payload_bits", ctypes.c_uint64), ("payload_bps", ctypes.c_double),
                ("side_bps", ctypes.c_double), ("total_bps", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class HqError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def lib():
    """Load ``libhq.so`` (built in-tree by ``kv_quantization_tile_amd/build.py``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with kv_quantization_tile_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, u64, i32, sz = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_size_t
        L.hq_version.restype = ctypes.c_uint32
        L.hq_strerror.argtypes = [ctypes.c_int]
        L.hq_strerror.restype = ctypes.c_char_p
        L.hq_workspace_size.argtypes = [u64, P, ctypes.POINTER(sz)]
        L.hq_stream_fixed_bytes.argtypes = [u64, i32, i32, ctypes.c_uint32, ctypes.POINTER(u64)]
        L.hq_encode_bound.argtypes = [u64, P, ctypes.POINTER(u64)]
        L.hq_rate.argtypes = [P, i32, u64, P, P, P, sz, P]
        L.hq_encode.argtypes = [P, i32, u64, P, P, u64, P, P, P, sz, P]
        L.hq_encode_noalloc.argtypes = [P, i32, u64, P, P, u64, P, P, P]
        L.hq_decode.argtypes = [P, u64, P, i32, u64, P, sz, P]
        L.hq_status.argtypes = [P, P]
        L.hq_fallbacks.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32)]
        L.hq_codes.argtypes = [P, i32, u64, P, P, P, P, sz, P]
        L.hq_gemv_workspace_size.argtypes = [u64, u64, ctypes.POINTER(sz)]
        L.hq_gemv.argtypes = [P, u64, u64, u64, P, i32, P, P, sz, P]
        L.hq_haar_matrix.argtypes = [u64, P]
        L.hq_rotate.argtypes = [P, u64, P, i32, P, P]
        L.hq_srft_encode.argtypes = [P, i32, u64, u64, P, i32, P, P, P]
        L.hq_srft_decode.argtypes = [P, P, u64, u64, P, i32, P, i32, P]
        for name in EXPORTS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().hq_strerror(code).decode()


def hq_version() -> int:
    return int(lib().hq_version())


def _check(rc: int, what: str):
    if rc != HQ_OK:
        raise HqError(rc, what)


# Dither flags: bit 0 on; bit 1 the dither's Philox calls take 7 rounds instead of 10; bit 2 a
# 24-bit draw instead of 16.  True / False mean 1 / 0.
HQ_DITHER, HQ_DITHER_PHILOX7, HQ_DITHER_24BIT = 1, 2, 4


def dither_flags(dither) -> int:
    return (1 if dither else 0) if isinstance(dither, bool) else int(dither)


def make_params(lattice="e8", target_bps=4.0, seed=0, dither=False, step=0.0, rice_k=-1, tile=128) -> HqParams:
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    return HqParams(tile=tile, lattice=lat, target_bps=float(target_bps), seed=int(seed),
                    dither=dither_flags(dither), step=float(step), rice_k=int(rice_k))


def hq_workspace_size(n: int, params: HqParams | None = None) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().hq_workspace_size(n, ctypes.byref(params) if params else None, ctypes.byref(out)),
           "hq_workspace_size")
    return out.value


def hq_stream_fixed_bytes(n: int, lattice, rice_k: int, tile: int = 128) -> int:
    out = ctypes.c_uint64(0)
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    _check(lib().hq_stream_fixed_bytes(n, lat, rice_k, tile, ctypes.byref(out)), "hq_stream_fixed_bytes")
    return out.value


def hq_encode_bound(n: int, lattice="e8", step=0.0, rice_k=-1, dither=False, tile=128) -> int:
    """Worst-case stream bytes of an encode of n values (host only; see include/hq.h)."""
    out = ctypes.c_uint64(0)
    p = make_params(lattice, 4.0, 0, dither, step, rice_k, tile)
    _check(lib().hq_encode_bound(n, ctypes.byref(p), ctypes.byref(out)), "hq_encode_bound")
    return out.value


# ---- torch-side helpers (device memory and streams only) ------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return HQ_F32
    if t.dtype == torch.bfloat16:
        return HQ_BF16
    raise TypeError("input must be float32 or bfloat16")


def _stream_handle(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace(n: int, device="cuda"):
    torch = _torch()
    return torch.empty(hq_workspace_size(n), dtype=torch.uint8, device=device)


def capacity_estimate(n: int, lattice, target_bps: float, rice_k: int = -1, step: float = 0.0,
                      tile: int = 128) -> int:
    """A starting output size: the fixed plane at a generous Rice k plus 4 unary bits per value."""
    if rice_k >= 0:
        k = rice_k
    elif step > 0:
        k = 15
    else:
        k = min(15, int(target_bps) + 3)
    return hq_stream_fixed_bytes(n, lattice, k, tile) + n // 2 + 4096


def hq_encode(x, lattice="e8", target_bps=4.0, seed=0, dither=False, step=0.0, rice_k=-1, out=None,
              ws=None, stream=None, blocking=True, tile=128):
    """Encode a contiguous CUDA tensor (fp32 or bf16, numel a multiple of the tile length 64, 128
    or 256).

    Returns (stream bytes as a uint8 CUDA tensor, info dict).  With blocking=False the call only
    enqueues work and returns (out, None); the size is then in the stream header.  Without `out`,
    the asynchronous call sizes the buffer with hq_encode_bound: at the given step (step > 0), or,
    with rate control (step == 0), at the operating point of a blocking hq_rate on the workspace,
    which the asynchronous encode then uses (step == -1)."""
    torch = _torch()
    assert x.is_cuda and x.is_contiguous()
    n = x.numel()
    p = make_params(lattice, target_bps, seed, dither, step, rice_k, tile)
    if ws is None:
        ws = workspace(n, x.device)
    sh = _stream_handle(stream)
    if out is None and not blocking:
        if step > 0:
            cap = hq_encode_bound(n, p.lattice, step, rice_k, p.dither, tile)
        elif step == 0:
            point = hq_rate(x, lattice, target_bps, seed, dither, 0.0, rice_k, ws=ws, stream=stream, tile=tile)
            cap = hq_encode_bound(n, p.lattice, point["step"], point["rice_k"], p.dither, tile)
            p = make_params(lattice, target_bps, seed, dither, -1.0, rice_k, tile)
        else:
            raise ValueError("an asynchronous encode at the workspace's operating point (step=-1) needs `out`")
        out = torch.empty(cap, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty(capacity_estimate(n, p.lattice, target_bps, rice_k, step, tile), dtype=torch.uint8,
                          device=x.device)
    assert out.is_cuda and out.is_contiguous() and out.dtype == torch.uint8
    if not blocking:
        _check(lib().hq_encode(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ctypes.byref(p),
                               ctypes.c_void_p(out.data_ptr()), out.numel(), None, None,
                               ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh), "hq_encode")
        return out, None
    info = HqInfo()
    nbytes = ctypes.c_uint64(0)
    while True:
        rc = lib().hq_encode(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ctypes.byref(p),
                             ctypes.c_void_p(out.data_ptr()), out.numel(), ctypes.byref(nbytes),
                             ctypes.byref(info), ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh)
        if rc == HQ_ERR_CAPACITY and nbytes.value > out.numel():
            out = torch.empty(nbytes.value, dtype=torch.uint8, device=x.device)
            continue
        _check(rc, "hq_encode")
        break
    return out[: nbytes.value], info.as_dict()


def hq_decode(stream_bytes, n: int, out_dtype=None, out=None, ws=None, stream=None, check=True):
    """Decode a uint8 CUDA tensor holding a stream into n values (bf16 by default)."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    assert stream_bytes.is_cuda and stream_bytes.is_contiguous() and stream_bytes.dtype == torch.uint8
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=stream_bytes.device)
    # the kernels write n values of out's type: a shorter or strided tensor would be written past
    assert out.is_cuda and out.is_contiguous() and out.numel() >= n, "out must be a contiguous CUDA tensor of n values"
    assert out.dtype in (torch.float32, torch.bfloat16), "out must be float32 or bfloat16"
    if ws is None:
        ws = workspace(0, stream_bytes.device)
    sh = _stream_handle(stream)
    _check(lib().hq_decode(ctypes.c_void_p(stream_bytes.data_ptr()), stream_bytes.numel(),
                           ctypes.c_void_p(out.data_ptr()), _dtype_code(out), n,
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh), "hq_decode")
    if check:
        _check(lib().hq_status(ctypes.c_void_p(ws.data_ptr()), sh), "hq_decode")
    return out


def hq_gemv_workspace_size(rows: int, cols: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().hq_gemv_workspace_size(rows, cols, ctypes.byref(out)), "hq_gemv_workspace_size")
    return out.value


def hq_gemv(stream_bytes, rows: int, cols: int, x, y=None, ws=None, stream=None, check=True):
    """y = W_hat x for a stream of a [rows][cols] matrix: fused decode + matrix-vector product
    (float32 output)."""
    torch = _torch()
    assert x.is_cuda and x.is_contiguous() and x.numel() == cols
    assert stream_bytes.is_cuda and stream_bytes.is_contiguous() and stream_bytes.dtype == torch.uint8
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=x.device)
    # the kernels write `rows` binary32 values
    assert y.is_cuda and y.is_contiguous() and y.dtype == torch.float32 and y.numel() >= rows, \
        "y must be a contiguous float32 CUDA tensor of `rows` values"
    if ws is None:
        ws = torch.empty(hq_gemv_workspace_size(rows, cols), dtype=torch.uint8, device=x.device)
    sh = _stream_handle(stream)
    _check(lib().hq_gemv(ctypes.c_void_p(stream_bytes.data_ptr()), stream_bytes.numel(), rows, cols,
                         ctypes.c_void_p(x.data_ptr()), _dtype_code(x), ctypes.c_void_p(y.data_ptr()),
                         ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh), "hq_gemv")
    if check:
        _check(lib().hq_status(ctypes.c_void_p(ws.data_ptr()), sh), "hq_gemv")
    return y


def hq_haar_matrix(seed: int):
    """The per-layer Haar-uniform rotation Q of a seed, as a float32 numpy array [128, 128]."""
    import numpy as np
    q = np.zeros(128 * 128, dtype=np.float32)
    _check(lib().hq_haar_matrix(seed, ctypes.c_void_p(q.ctypes.data)), "hq_haar_matrix")
    return q.reshape(128, 128)


def hq_rotate(x, q, transpose: bool = False, out=None, stream=None):
    """y_v = Q x_v (or Q^T x_v) for the 128-value bf16 vectors of x; q a float32 CUDA tensor [128, 128]."""
    torch = _torch()
    assert x.is_cuda and x.is_contiguous() and x.dtype == torch.bfloat16
    assert q.is_cuda and q.is_contiguous() and q.dtype == torch.float32 and q.numel() == 128 * 128
    if out is None:
        out = torch.empty_like(x)
    assert out.is_cuda and out.is_contiguous() and out.dtype == torch.bfloat16 and out.numel() >= x.numel()
    _check(lib().hq_rotate(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_void_p(q.data_ptr()),
                           1 if transpose else 0, ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)),
           "hq_rotate")
    return out


def _host_lambda(lam):
    import numpy as np
    if lam is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(lam, dtype=np.float32).reshape(-1))
    if a.size != 128:
        raise ValueError("lambda holds one scale per coordinate: 128 values")
    return a, ctypes.c_void_p(a.ctypes.data)


def hq_srft_encode(x, seed: int = 0, bits: int = 4, lam=None, codes=None, scales=None, stream=None):
    """SRFT fixed-rate codes of x (bf16 or float32 CUDA tensor, numel % 128 == 0): returns (codes
    uint8 [vectors][64 | 128], scales int16 view of binary16 [vectors][16]).  lam: 128 host floats."""
    torch = _torch()
    assert x.is_cuda and x.is_contiguous()
    n = x.numel()
    nv = n // 128
    if codes is None:
        codes = torch.empty((nv, 64 if bits == 4 else 128), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((nv, 16), dtype=torch.int16, device=x.device)
    assert codes.is_cuda and codes.is_contiguous() and codes.numel() * codes.element_size() >= nv * (64 if bits == 4 else 128)
    assert scales.is_cuda and scales.is_contiguous() and scales.numel() * scales.element_size() >= nv * 32
    keep, lp = _host_lambda(lam)
    _check(lib().hq_srft_encode(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, int(seed), lp, int(bits),
                                ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                _stream_handle(stream)), "hq_srft_encode")
    return codes, scales


def hq_srft_decode(codes, scales, n: int, seed: int = 0, bits: int = 4, lam=None, out=None,
                   out_dtype=None, stream=None):
    """Decode n values from SRFT codes and scales (CUDA tensors) into bf16 (default) or float32."""
    torch = _torch()
    assert codes.is_cuda and scales.is_cuda and codes.is_contiguous() and scales.is_contiguous()
    if out is None:
        out = torch.empty(n, dtype=out_dtype or torch.bfloat16, device=codes.device)
    assert out.is_cuda and out.is_contiguous() and out.numel() >= n and out.dtype in (torch.float32, torch.bfloat16)
    keep, lp = _host_lambda(lam)
    _check(lib().hq_srft_decode(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), n,
                                int(seed), lp, int(bits), ctypes.c_void_p(out.data_ptr()), _dtype_code(out),
                                _stream_handle(stream)), "hq_srft_decode")
    return out


def hq_rate(x, lattice="e8", target_bps=4.0, seed=0, dither=False, step=0.0, rice_k=-1, ws=None, stream=None,
            blocking=True, tile=128):
    """Rate control alone.  blocking=False only enqueues it; a following hq_encode(..., step=-1,
    ws=<same workspace>) then encodes at the chosen operating point."""
    assert x.is_cuda and x.is_contiguous()
    n = x.numel()
    p = make_params(lattice, target_bps, seed, dither, step, rice_k, tile)
    if ws is None:
        ws = workspace(n, x.device)
    info = HqInfo()
    _check(lib().hq_rate(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ctypes.byref(p),
                         ctypes.byref(info) if blocking else None, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                         _stream_handle(stream)), "hq_rate")
    return info.as_dict() if blocking else None


def hq_codes(x, step: float, lattice="e8", seed=0, dither=False, ws=None, stream=None, tile=128):
    """Integer lattice codes (int32, per value) and bf16 tile-scale bits (int16 view, per tile)."""
    torch = _torch()
    assert x.is_cuda and x.is_contiguous()
    n = x.numel()
    p = make_params(lattice, 4.0, seed, dither, step, -1, tile)
    if ws is None:
        ws = workspace(0, x.device)
    codes = torch.empty(n, dtype=torch.int32, device=x.device)
    scales = torch.empty(max(n // tile, 1), dtype=torch.int16, device=x.device)
    sh = _stream_handle(stream)
    _check(lib().hq_codes(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), n, ctypes.byref(p),
                          ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh), "hq_codes")
    _check(lib().hq_status(ctypes.c_void_p(ws.data_ptr()), sh), "hq_codes")
    return codes, scales[: n // tile]


def hq_status(ws, stream=None) -> int:
    return int(lib().hq_status(ctypes.c_void_p(ws.data_ptr()), _stream_handle(stream)))


# bits of hq_fallbacks
FALLBACK_LOOKBACK, FALLBACK_CENTRE, FALLBACK_PRIVATE = 1, 2, 4


def hq_fallbacks(ws, stream=None) -> int:
    """Which bounded waits of the workspace's last call took their (slower, same-result) fallback:
    bit 0 a look-back aggregate, bit 1 pass A's centre, bit 2 a pass's private evaluation."""
    f = ctypes.c_uint32(0)
    _check(lib().hq_fallbacks(ctypes.c_void_p(ws.data_ptr()), _stream_handle(stream), ctypes.byref(f)),
           "hq_fallbacks")
    return int(f.value)


def header_fields(stream_bytes_host) -> dict:
    """Parse the 128-byte stream header (host bytes) into a dict."""
    import struct
    b = bytes(stream_bytes_host[:128])
    magic, ver, lat, flags, tile, k, clog, step_bits = struct.unpack_from("<IHBBHBBI", b, 0)
    seed, n, T = struct.unpack_from("<QQQ", b, 16)
    chunks, F = struct.unpack_from("<II", b, 40)
    fixed_off, unary_off, words, ubits, payload, total = struct.unpack_from("<QQQQQQ", b, 48)
    return dict(magic=magic, version=ver, lattice=lat, dither=flags, tile=tile, k=k, chunk_log2=clog,
                step_bits=step_bits, seed=seed, n=n, tiles=T, chunks=chunks, F=F, fixed_off=fixed_off,
                unary_off=unary_off, unary_words=words, unary_bits=ubits, payload_bits=payload,
                total_bytes=total)
