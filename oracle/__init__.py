"""CPU oracle for the RHT + lattice + bit-strip + Rice codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (``kv_quantization_tile_amd``) never imports it, and it never imports
the product.  The C source ``hq_oracle.c`` is compiled with gcc, ``-O2 -ffp-contract=off``, no
fast-math, so that every binary32 operation is rounded exactly once in the order written.

The method follows the HyperQuant technical summaries (gist.science/ko/paper/2606.23406 and
gist.science/ja/paper/2606.23406), "Methodology: the HyperQuant pipeline", components 1-4.

Parity: the tests pin each function to something outside this package (a dense Hadamard matrix,
brute-force nearest-point search, closed forms, the rocRAND Philox source, statistical invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "hq_oracle.c"), os.path.join(_HERE, "srft_oracle.c")]
_LIB = os.path.join(_HERE, "libhq_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same sources (host code only).  lib()
# loads it when HQO_SANITIZE is set; the process must then have libasan preloaded (the Python
# interpreter itself is not instrumented), e.g.
#   LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 HQO_SANITIZE=1 \
#     python -m pytest tests -m "not gpu"
_LIB_SAN = os.path.join(_HERE, "libhq_oracle_san.so")

LAT_Z, LAT_D4, LAT_E8, LAT_A2 = 0, 1, 2, 3
LATTICES = {"z": LAT_Z, "d4": LAT_D4, "e8": LAT_E8, "a2": LAT_A2}
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NONFINITE, ERR_CAPACITY, ERR_CORRUPT, ERR_RATE = (
    0, -1, -2, -3, -4, -5, -6)


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle into ``oracle/libhq_oracle.so`` with gcc (``libhq_oracle_san.so`` with
    AddressSanitizer and UndefinedBehaviorSanitizer when ``sanitize``; any report aborts)."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out):
        san = (["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
               if sanitize else [])
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-Wextra", *san, "-o", out + ".tmp", *_SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        sanitize = bool(os.environ.get("HQO_SANITIZE"))
        path = _LIB_SAN if sanitize else _LIB
        if not os.path.exists(path):
            build(sanitize=sanitize)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        u64, u32, i32, f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float
        L.hqo_philox4x32_10.argtypes = [P, P, P]
        L.hqo_philox4x32_r.argtypes = [P, P, i32, P]
        L.hqo_philox4x32_span.argtypes = [P, P, i32, i32, P]
        L.hqo_signs.argtypes = [u64, P]
        L.hqo_signs_n.argtypes = [u64, i32, P]
        L.hqo_fwht128.argtypes = [P]
        L.hqo_fwht_n.argtypes = [P, i32]
        L.hqo_sumsq128.argtypes = [P]
        L.hqo_sumsq128.restype = f32
        L.hqo_sumsq_n.argtypes = [P, i32]
        L.hqo_sumsq_n.restype = f32
        L.hqo_scale_bits.argtypes = [f32]
        L.hqo_scale_bits.restype = ctypes.c_uint16
        L.hqo_scale_bits_n.argtypes = [f32, i32]
        L.hqo_scale_bits_n.restype = ctypes.c_uint16
        L.hqo_nearest_octet.argtypes = [i32, P, P]
        L.hqo_nearest_batch.argtypes = [i32, P, u64, P]
        L.hqo_dither_octet.argtypes = [u64, u64, i32, i32, P]
        L.hqo_dither_octet_flags.argtypes = [u64, u64, i32, i32, i32, P]
        L.hqo_strip_octet.argtypes = [i32, P, P, P]
        L.hqo_unstrip_octet.argtypes = [i32, P, i32, P]
        L.hqo_tile_fixed_bits.argtypes = [i32, i32]
        L.hqo_tile_fixed_bits.restype = u32
        L.hqo_tile_fixed_bits_n.argtypes = [i32, i32, i32]
        L.hqo_tile_fixed_bits_n.restype = u32
        L.hqo_quantize.argtypes = [P, i32, u64, i32, i32, u64, f32, P, P, i32]
        L.hqo_dequantize.argtypes = [P, P, u64, i32, i32, u64, f32, P, i32]
        L.hqo_lattice_inputs.argtypes = [P, i32, u64, i32, i32, u64, f32, P, i32]
        L.hqo_sample_tile.argtypes = [u64, u64, u64]
        L.hqo_sample_tile.restype = u64
        L.hqo_rate.argtypes = [P, i32, u64, i32, i32, u64, f32, f32, i32, P, P, i32]
        L.hqo_rice_roundtrip.argtypes = [P, u64, i32, P, P, P, u64, P]
        L.hqo_encode_layout.argtypes = [u64, i32, i32, P, P, P, i32]
        L.hqo_encode.argtypes = [P, i32, u64, i32, i32, u64, f32, f32, i32, P, u64, P, P, i32]
        L.hqo_decode.argtypes = [P, u64, u64, P, i32]
        L.hqo_decode_coords.argtypes = [P, u64, u64, P]
        L.hqo_haar_matrix.argtypes = [u64, P]
        L.hqo_haar_gaussians.argtypes = [u64, P]
        L.hqo_srft_twiddle.argtypes = [u32, u32, P]
        L.hqo_srft_forward.argtypes = [P, u64, P, P]
        L.hqo_srft_inverse.argtypes = [P, u64, P]
        L.hqo_srft_encode.argtypes = [P, i32, u64, u64, P, i32, P, P]
        L.hqo_srft_decode.argtypes = [P, P, u64, u64, P, i32, P, i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:  # bfloat16 bit patterns
        return 1
    raise TypeError("oracle input must be float32 or uint16 (bfloat16 bits)")


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(rc, what)


# ---- primitives ---------------------------------------------------------------------------------

def philox4x32_10(counter, key) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().hqo_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def philox4x32_span(counter, key, r0: int, r1: int) -> np.ndarray:
    """Rounds r0 .. r1-1 of Philox4x32 (the key first bumped r0 times); (0, R) is Philox4x32-R."""
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().hqo_philox4x32_span(_p(c), _p(k), r0, r1, _p(out))
    return out


TILES = (64, 128, 256)


def signs(seed: int, tile: int = 128) -> np.ndarray:
    d = np.zeros(tile, dtype=np.float32)
    if tile == 128:
        lib().hqo_signs(seed, _p(d))
    else:
        lib().hqo_signs_n(seed, tile, _p(d))
    return d


def fwht128(x) -> np.ndarray:
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    assert y.shape == (128,)
    lib().hqo_fwht128(_p(y))
    return y


def fwht(x) -> np.ndarray:
    """The unnormalised transform of one tile of 64, 128 or 256 values."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    assert y.shape in ((64,), (128,), (256,))
    lib().hqo_fwht_n(_p(y), y.size)
    return y


def sumsq128(y) -> float:
    y = np.ascontiguousarray(y, dtype=np.float32)
    return float(lib().hqo_sumsq128(_p(y)))


def sumsq(y) -> float:
    y = np.ascontiguousarray(y, dtype=np.float32)
    return float(lib().hqo_sumsq_n(_p(y), y.size))


def scale_bits(S: float, tile: int = 128) -> int:
    if tile == 128:
        return int(lib().hqo_scale_bits(ctypes.c_float(S)))
    return int(lib().hqo_scale_bits_n(ctypes.c_float(S), tile))


def nearest(lattice: int, v) -> np.ndarray:
    """Nearest-point integer codes for an array of octets, shape (..., 8)."""
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1, 8)
    out = np.zeros(v.shape, dtype=np.int32)
    _check(lib().hqo_nearest_batch(lattice, _p(v), v.shape[0], _p(out)), "nearest")
    return out


def dither_octet(seed: int, tile: int, octet: int, lattice: int, flags: int = 1) -> np.ndarray:
    """U of octet `octet` of tile `tile`; flags as in dither_flags (1: 16-bit draw, 10 rounds)."""
    u = np.zeros(8, dtype=np.float32)
    if flags == 1:
        lib().hqo_dither_octet(seed, tile, octet, lattice, _p(u))
    else:
        lib().hqo_dither_octet_flags(seed, tile, octet, lattice, flags, _p(u))
    return u


# Dither flags: bit 0 on; bit 1 the dither's Philox calls take 7 rounds instead of 10; bit 2 a
# 24-bit draw instead of 16.  True / False mean 1 / 0.
DITHER_PHILOX7, DITHER_24BIT = 2, 4


def dither_flags(dither) -> int:
    return int(dither) if not isinstance(dither, bool) else (1 if dither else 0)


def strip_octet(lattice: int, code):
    c = np.ascontiguousarray(code, dtype=np.int32)
    sym = np.zeros(8, dtype=np.uint32)
    cos = ctypes.c_int(0)
    _check(lib().hqo_strip_octet(lattice, _p(c), _p(sym), ctypes.byref(cos)), "strip")
    return sym, cos.value


def unstrip_octet(lattice: int, sym, coset: int) -> np.ndarray:
    s = np.ascontiguousarray(sym, dtype=np.uint32)
    out = np.zeros(8, dtype=np.int32)
    _check(lib().hqo_unstrip_octet(lattice, _p(s), coset, _p(out)), "unstrip")
    return out


def tile_fixed_bits(lattice: int, k: int, tile: int = 128) -> int:
    if tile == 128:
        return int(lib().hqo_tile_fixed_bits(lattice, k))
    return int(lib().hqo_tile_fixed_bits_n(lattice, k, tile))


def sample_tile(i: int, T: int, N: int) -> int:
    return int(lib().hqo_sample_tile(i, T, N))


def rice_roundtrip(vals, k: int):
    v = np.ascontiguousarray(vals, dtype=np.uint32)
    n = v.size
    out = np.zeros(n, dtype=np.uint32)
    fixed = np.zeros((k * n + 7) // 8 + 8, dtype=np.uint8)
    ubits = int(sum(int(a) >> k for a in v) + n)
    unary = np.zeros((ubits + 7) // 8 + 8, dtype=np.uint8)
    ulen = ctypes.c_uint64(0)
    _check(lib().hqo_rice_roundtrip(_p(v), n, k, _p(out), _p(fixed), _p(unary), ubits + 64,
                                    ctypes.byref(ulen)), "rice")
    return out, ulen.value


# ---- the codec ----------------------------------------------------------------------------------

def quantize(x: np.ndarray, lattice: int, step: float, seed: int = 0, dither: bool = False, tile: int = 128):
    """Per-value integer codes (int32) and per-tile bf16 scale bits (uint16) at a fixed step."""
    x = np.ascontiguousarray(x).reshape(-1)
    n = x.size
    codes = np.zeros(n, dtype=np.int32)
    scales = np.zeros(max(n // tile, 1), dtype=np.uint16)
    _check(lib().hqo_quantize(_p(x), _dtype_code(x), n, lattice, dither_flags(dither), seed,
                              ctypes.c_float(step), _p(codes), _p(scales), tile), "quantize")
    return codes, scales[: n // tile]


def lattice_inputs(x, lattice: int, step: float, seed: int = 0, dither: bool = False,
                   tile: int = 128) -> np.ndarray:
    """The binary32 values fed to the nearest-point step (y * m, plus U with dither)."""
    x = np.ascontiguousarray(x).reshape(-1)
    v = np.zeros(x.size, dtype=np.float32)
    _check(lib().hqo_lattice_inputs(_p(x), _dtype_code(x), x.size, lattice, dither_flags(dither), seed,
                                    ctypes.c_float(step), _p(v), tile), "lattice_inputs")
    return v


def dequantize(codes, scales, lattice: int, step: float, seed: int = 0, dither: bool = False, tile: int = 128):
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.zeros(codes.size, dtype=np.float32)
    _check(lib().hqo_dequantize(_p(codes), _p(scales), codes.size, lattice, dither_flags(dither), seed,
                                ctypes.c_float(step), _p(out), tile), "dequantize")
    return out


def rate(x, lattice: int, target_bps: float, seed: int = 0, dither: bool = False, step: float = 0.0,
         rice_k: int = -1, tile: int = 128):
    """Rate control only: returns (step as float32, step bit pattern, k)."""
    x = np.ascontiguousarray(x).reshape(-1)
    sb = ctypes.c_uint32(0)
    k = ctypes.c_int(0)
    _check(lib().hqo_rate(_p(x), _dtype_code(x), x.size, lattice, dither_flags(dither), seed,
                          ctypes.c_float(target_bps), ctypes.c_float(step), rice_k,
                          ctypes.byref(sb), ctypes.byref(k), tile), "rate")
    step_f = np.array([sb.value], dtype=np.uint32).view(np.float32)[0]
    return float(step_f), sb.value, k.value


def layout(n: int, lattice: int, k: int, tile: int = 128):
    fo, uo, F = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint32(0)
    _check(lib().hqo_encode_layout(n, lattice, k, ctypes.byref(fo), ctypes.byref(uo), ctypes.byref(F), tile),
           "layout")
    return fo.value, uo.value, F.value


def encode(x, lattice: int, target_bps: float = 4.0, seed: int = 0, dither: bool = False,
           step: float = 0.0, rice_k: int = -1, capacity: int | None = None, tile: int = 128):
    """Full encoder.  Returns (stream bytes as uint8 array, info dict)."""
    x = np.ascontiguousarray(x).reshape(-1)
    n = x.size
    if capacity is None:
        capacity = 4096 + n * 4
    info = np.zeros(4, dtype=np.uint64)
    nbytes = ctypes.c_uint64(0)
    while True:
        out = np.zeros(capacity, dtype=np.uint8)
        rc = lib().hqo_encode(_p(x), _dtype_code(x), n, lattice, dither_flags(dither), seed,
                              ctypes.c_float(target_bps), ctypes.c_float(step), rice_k, _p(out),
                              capacity, ctypes.byref(nbytes), _p(info), tile)
        if rc == ERR_CAPACITY and nbytes.value > capacity:
            capacity = int(nbytes.value)
            continue
        _check(rc, "encode")
        break
    step_f = np.array([info[0]], dtype=np.uint64).astype(np.uint32).view(np.float32)[0]
    d = {"step": float(step_f), "step_bits": int(info[0]), "k": int(info[1]),
         "payload_bits": int(info[2]), "unary_bits": int(info[3]), "bytes": int(nbytes.value),
         "payload_bps": float(info[2]) / n if n else 0.0,
         "total_bps": 8.0 * float(nbytes.value) / n if n else 0.0}
    return out[: nbytes.value].copy(), d


def decode(stream, n: int, out_dtype: str = "f32"):
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    if out_dtype == "f32":
        out = np.zeros(n, dtype=np.float32)
        code = 0
    else:
        out = np.zeros(n, dtype=np.uint16)
        code = 1
    _check(lib().hqo_decode(_p(s), s.size, n, _p(out), code), "decode")
    return out


def decode_coords(stream, n: int) -> np.ndarray:
    """yhat = (c - U) * (s * step) per value, binary64: the exact reconstruction of tile t is
    D H yhat_t / tile."""
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(n, dtype=np.float64)
    _check(lib().hqo_decode_coords(_p(s), s.size, n, _p(out)), "decode_coords")
    return out


def hadamard(n: int = 128) -> np.ndarray:
    """Sylvester H_n = H_2 (x) ... (x) H_2, entries +-1 (natural order)."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard128() -> np.ndarray:
    return hadamard(128)


def gemv_reference(stream, rows: int, cols: int, x: np.ndarray, seed: int, tile: int = 128):
    """Matrix-vector product with the decoded [rows][cols] matrix (tiles of `tile` values along
    cols), in binary64, by the plain definition: W_hat = D H yhat / tile per tile, y = W_hat x.
    Also returns, per row, B_r = sum over the row's tiles of sum_i |yhat_i| * ||x_tile||_1, the
    scale of the rounding error of any binary32 evaluation that rotates x per tile."""
    n = rows * cols
    yh = decode_coords(stream, n).reshape(rows, cols // tile, tile)
    d = signs(seed, tile).astype(np.float64)
    h = hadamard(tile)
    w = (yh @ h.T) * d / float(tile)    # row-major tiles: w[r, j, :] = D H yhat[r, j, :] / tile
    xf = np.asarray(x, dtype=np.float64).reshape(cols // tile, tile)
    y = np.einsum("rji,ji->r", w, xf)
    bound = np.einsum("rji,j->r", np.abs(yh), np.abs(xf).sum(axis=1))
    return y, bound


def haar_gaussians(seed: int) -> np.ndarray:
    g = np.zeros(128 * 128, dtype=np.float64)
    lib().hqo_haar_gaussians(seed, _p(g))
    return g.reshape(128, 128)


def haar_matrix(seed: int) -> np.ndarray:
    """The per-layer Haar-uniform rotation Q (128 x 128, binary64): G = Q R, diag(R) > 0."""
    q = np.zeros(128 * 128, dtype=np.float64)
    lib().hqo_haar_matrix(seed, _p(q))
    return q.reshape(128, 128)


def rotate_reference(x, q: np.ndarray, transpose: bool = False) -> np.ndarray:
    """y_v = Q x_v (or Q^T x_v) for every 128-value vector v of x, binary64."""
    xv = np.asarray(x, dtype=np.float64).reshape(-1, 128)
    m = q.T if transpose else q
    return (xv @ m.T).reshape(-1)


# ---------------------------------------------------------------------------------------------
# SRFT fixed-rate KV codec ("When quantization is free" summary, Methodology 1-3), srft_oracle.c


def srft_twiddle(n: int, k: int):
    cs = np.zeros(2, dtype=np.float32)
    lib().hqo_srft_twiddle(n, k, _p(cs))
    return float(cs[0]), float(cs[1])


def _lam(lam):
    if lam is None:
        return None, None
    a = np.ascontiguousarray(lam, dtype=np.float32)
    assert a.size == 128
    return a, _p(a)


def srft_forward(x, seed: int, lam=None) -> np.ndarray:
    """v = SRFT(x) / lambda of one 128-value vector, binary32."""
    xa = np.ascontiguousarray(x, dtype=np.float32)
    v = np.zeros(128, dtype=np.float32)
    la, lp = _lam(lam)
    assert lib().hqo_srft_forward(_p(xa), seed, lp, _p(v)) == 0
    return v


def srft_inverse(y, seed: int) -> np.ndarray:
    ya = np.ascontiguousarray(y, dtype=np.float32)
    x = np.zeros(128, dtype=np.float32)
    lib().hqo_srft_inverse(_p(ya), seed, _p(x))
    return x


def srft_encode(x, seed: int, bits: int = 4, lam=None):
    """(codes uint8 [vectors][64 or 128], scales uint16 binary16 bits [vectors][16]) of a bf16 (uint16
    bits) or float32 array."""
    xa = np.ascontiguousarray(x).reshape(-1)
    dtype = 1 if xa.dtype == np.uint16 else 0
    if dtype == 0:
        xa = xa.astype(np.float32)
    n = xa.size
    nv = n // 128
    codes = np.zeros((nv, 64 if bits == 4 else 128), dtype=np.uint8)
    scales = np.zeros((nv, 16), dtype=np.uint16)
    la, lp = _lam(lam)
    rc = lib().hqo_srft_encode(_p(xa), dtype, n, seed, lp, bits, _p(codes), _p(scales))
    assert rc == 0, rc
    return codes, scales


def srft_decode(codes, scales, n: int, seed: int, bits: int = 4, lam=None, out_dtype: str = "bf16"):
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.zeros(n, dtype=np.uint16 if out_dtype == "bf16" else np.float32)
    la, lp = _lam(lam)
    rc = lib().hqo_srft_decode(_p(c), _p(s), n, seed, lp, bits, _p(out), 1 if out_dtype == "bf16" else 0)
    assert rc == 0, rc
    return out


def decode_status(stream, n: int) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(max(n, 1), dtype=np.float32)
    return int(lib().hqo_decode(_p(s), s.size, n, _p(out), 0))
