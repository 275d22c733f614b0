"""CPU checks of the C-ABI library: it loads, exports every entry point include/hq.h declares, and
rejects bad arguments on the host before any device call."""
import ctypes
import os
import re

import pytest

import kv_quantization_tile_amd as hq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(hq_[a-z_]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(hq.EXPORTS), names
    L = hq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert hq.hq_version() == (1 << 16) | 1


def test_strerror_codes():
    for code in range(-9, 1):
        assert hq.strerror(code) != "unknown status"
    assert hq.strerror(-99) == "unknown status"


def test_sizes_match_oracle_layout(orc):
    for tile in (64, 128, 256):
        for n in (0, 256, 256 * 33, 128 * 65 * 2, 128 * 458752):
            for lat in ("z", "d4", "e8", "a2"):
                for k in (0, 1, 3, 15):
                    fo, uo, F = orc.layout(n, orc.LATTICES[lat], k, tile)
                    assert hq.hq_stream_fixed_bytes(n, lat, k, tile) == uo
    L = hq.lib()
    out = ctypes.c_uint64(0)
    assert L.hq_stream_fixed_bytes(256, 2, 4, 32, ctypes.byref(out)) == hq.HQ_ERR_UNSUPPORTED
    assert L.hq_stream_fixed_bytes(64, 2, 4, 128, ctypes.byref(out)) == hq.HQ_ERR_INVALID_ARG  # n % tile
    rate = 2 * 16 * 32 * 8 + 16 * 256 + 256  # two rate passes (16 sets of 32 64-bit counters), 16 copies of the published centre, the done count
    assert hq.hq_workspace_size(0) == 4096 + rate + 256
    assert hq.hq_workspace_size(128 * 64 * 100) == 4096 + rate + ((8 * 101 + 255) // 256) * 256
    # the allocation-free encode's static array is the workspace of its largest call (2^30 values)
    assert hq.hq_workspace_size(1 << 30) == 1_065_472


def _encode_rc(params, n=128, ws_bytes=1 << 20, x=1 << 20, out=1 << 20, ws=1 << 21):
    info = hq.HqInfo()
    nb = ctypes.c_uint64(0)
    return hq.lib().hq_encode(ctypes.c_void_p(x), 1, n, ctypes.byref(params), ctypes.c_void_p(out), 1 << 20,
                              ctypes.byref(nb), ctypes.byref(info), ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(tile=32), hq.HQ_ERR_UNSUPPORTED),
    (dict(tile=512), hq.HQ_ERR_UNSUPPORTED),
    (dict(lattice=4), hq.HQ_ERR_INVALID_ARG),
    (dict(rice_k=16), hq.HQ_ERR_INVALID_ARG),
    (dict(step=-2.0), hq.HQ_ERR_INVALID_ARG),          # -1 alone is a valid sentinel
    (dict(step=float("nan")), hq.HQ_ERR_INVALID_ARG),
    (dict(step=1e-6), hq.HQ_ERR_INVALID_ARG),
    (dict(step=1e6), hq.HQ_ERR_INVALID_ARG),
    (dict(target_bps=1.0), hq.HQ_ERR_RATE),          # below E8's floor of 1.125
    (dict(lattice="a2", target_bps=1.4), hq.HQ_ERR_RATE),  # below A2's floor of 1.5 (coset bits)
    (dict(target_bps=13.0), hq.HQ_ERR_RATE),
    (dict(dither=True, lattice="z", target_bps=0.5), hq.HQ_ERR_RATE),
    (dict(dither=2), hq.HQ_ERR_INVALID_ARG),            # dither option bits without the dither
    (dict(dither=4), hq.HQ_ERR_INVALID_ARG),
    (dict(dither=6), hq.HQ_ERR_INVALID_ARG),
    (dict(dither=8), hq.HQ_ERR_INVALID_ARG),
])
def test_encode_rejects_bad_params_on_host(kw, code):
    base = dict(lattice="e8", target_bps=4.0)
    base.update(kw)
    tile = base.pop("tile", 128)
    p = hq.make_params(**base, tile=tile)
    assert _encode_rc(p) == code


def test_encode_rejects_bad_buffers_on_host():
    p = hq.make_params("e8", 4.0)
    assert _encode_rc(p, n=100) == hq.HQ_ERR_INVALID_ARG           # n % 128
    assert _encode_rc(p, n=64) == hq.HQ_ERR_INVALID_ARG            # n % 128 (tile 128)
    assert _encode_rc(hq.make_params("e8", 4.0, tile=256), n=128) == hq.HQ_ERR_INVALID_ARG  # n % 256
    assert _encode_rc(p, ws_bytes=16) == hq.HQ_ERR_INVALID_ARG       # workspace too small
    assert _encode_rc(p, ws=0) == hq.HQ_ERR_INVALID_ARG              # null workspace
    assert _encode_rc(p, x=0) == hq.HQ_ERR_INVALID_ARG               # null input
    assert _encode_rc(p, out=0) == hq.HQ_ERR_INVALID_ARG             # null output
    assert _encode_rc(p, out=(1 << 20) + 4) == hq.HQ_ERR_INVALID_ARG  # misaligned output


def test_rate_rejects_workspace_step_sentinel_on_host():
    # step == -1 means "take the operating point from the workspace": meaningless for rate control
    p = hq.make_params("e8", 4.0, step=-1.0)
    assert hq.lib().hq_rate(ctypes.c_void_p(1 << 20), 1, 128, ctypes.byref(p), None, ctypes.c_void_p(1 << 21),
                            1 << 20, None) == hq.HQ_ERR_INVALID_ARG


def test_rate_rejects_misaligned_buffers_on_host():
    # the rate passes read the input with 16-byte loads and the workspace is 256-byte aligned
    p = hq.make_params("e8", 4.0)
    L = hq.lib()
    assert L.hq_rate(ctypes.c_void_p((1 << 20) + 8), 1, 128, ctypes.byref(p), None, ctypes.c_void_p(1 << 21),
                     1 << 20, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_rate(ctypes.c_void_p(1 << 20), 1, 128, ctypes.byref(p), None, ctypes.c_void_p((1 << 21) + 64),
                     1 << 20, None) == hq.HQ_ERR_INVALID_ARG


def test_decode_and_codes_reject_bad_args_on_host():
    L = hq.lib()
    assert L.hq_decode(ctypes.c_void_p(1 << 20), 4096, ctypes.c_void_p(1 << 20), 1, 100,
                       ctypes.c_void_p(1 << 21), 8192, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_decode(ctypes.c_void_p(1 << 20), 4096, ctypes.c_void_p(1 << 20), 7, 128,
                       ctypes.c_void_p(1 << 21), 8192, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_decode(None, 4096, ctypes.c_void_p(1 << 20), 1, 128, ctypes.c_void_p(1 << 21), 8192,
                       None) == hq.HQ_ERR_INVALID_ARG
    p = hq.make_params("e8", 4.0)  # step 0: the diagnostic codes call needs a fixed step
    assert L.hq_codes(ctypes.c_void_p(1 << 20), 1, 128, ctypes.byref(p), ctypes.c_void_p(1 << 20),
                      ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), 8192, None) == hq.HQ_ERR_INVALID_ARG
    p = hq.make_params("e8", step=0.3)
    assert L.hq_codes(ctypes.c_void_p(1 << 20), 1, 128, ctypes.byref(p), ctypes.c_void_p(1 << 20),
                      ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), 4096, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_workspace_size(100, None, ctypes.byref(ctypes.c_size_t())) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_status(None, None) == hq.HQ_ERR_INVALID_ARG


def test_product_package_does_not_import_oracle():
    src = open(os.path.join(ROOT, "kv_quantization_tile_amd", "__init__.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    for f in os.listdir(os.path.join(ROOT, "kv_quantization_tile_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "kv_quantization_tile_amd", "csrc", f)).read().lower(), f


def test_gemv_rejects_bad_args_on_host():
    L = hq.lib()
    sz = ctypes.c_size_t(0)
    assert L.hq_gemv_workspace_size(4, 100, ctypes.byref(sz)) == hq.HQ_ERR_INVALID_ARG   # cols % 64
    assert L.hq_gemv_workspace_size(4, 1024, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_gemv_workspace_size(4, 1024, ctypes.byref(sz)) == hq.HQ_OK
    assert sz.value == 4096 + 4096 + 256  # header, 1024 rotated values, 64 partials of 64-value tiles
    ws, big = ctypes.c_void_p(1 << 21), 1 << 20
    args = dict(s=ctypes.c_void_p(1 << 20), rows=4, cols=1024, x=ctypes.c_void_p(1 << 22), dt=0,
                y=ctypes.c_void_p(1 << 23), ws=ws, wsb=big)

    def call(**kw):
        a = {**args, **kw}
        return L.hq_gemv(a["s"], 4096, a["rows"], a["cols"], a["x"], a["dt"], a["y"], a["ws"], a["wsb"], None)
    assert call(cols=1000) == hq.HQ_ERR_INVALID_ARG
    assert call(dt=5) == hq.HQ_ERR_INVALID_ARG
    assert call(s=None) == hq.HQ_ERR_INVALID_ARG
    assert call(x=None) == hq.HQ_ERR_INVALID_ARG
    assert call(y=None) == hq.HQ_ERR_INVALID_ARG
    assert call(wsb=16) == hq.HQ_ERR_INVALID_ARG
    assert call(x=ctypes.c_void_p((1 << 22) + 4)) == hq.HQ_ERR_INVALID_ARG  # misaligned activation


def test_srft_rejects_bad_args_on_host():
    L = hq.lib()
    P = ctypes.c_void_p
    ok = P(1 << 20)
    lam_bad = (ctypes.c_float * 128)(*([1.0] * 127 + [-1.0]))
    lam_nan = (ctypes.c_float * 128)(*([1.0] * 127 + [float("nan")]))
    E = hq.HQ_ERR_INVALID_ARG
    assert L.hq_srft_encode(ok, 1, 100, 0, None, 4, ok, ok, None) == E           # n % 128
    assert L.hq_srft_encode(ok, 2, 128, 0, None, 4, ok, ok, None) == E           # dtype
    assert L.hq_srft_encode(ok, 1, 128, 0, None, 5, ok, ok, None) == E           # bits
    assert L.hq_srft_encode(None, 1, 128, 0, None, 4, ok, ok, None) == E         # null
    assert L.hq_srft_encode(P((1 << 20) + 8), 1, 128, 0, None, 4, ok, ok, None) == E  # alignment
    assert L.hq_srft_encode(ok, 1, 128, 0, lam_bad, 4, ok, ok, None) == E        # lambda <= 0
    assert L.hq_srft_encode(ok, 1, 128, 0, lam_nan, 4, ok, ok, None) == E        # lambda NaN
    assert L.hq_srft_encode(ok, 1, 0, 0, None, 4, None, None, None) == hq.HQ_OK  # empty: nothing to do
    assert L.hq_srft_decode(ok, ok, 100, 0, None, 4, ok, 1, None) == E
    assert L.hq_srft_decode(ok, ok, 128, 0, None, 8, ok, 3, None) == E           # out dtype
    assert L.hq_srft_decode(ok, None, 128, 0, None, 4, ok, 1, None) == E
    assert L.hq_srft_decode(ok, ok, 128, 0, lam_bad, 4, ok, 1, None) == E
    assert L.hq_srft_decode(None, None, 0, 0, None, 4, None, 1, None) == hq.HQ_OK


def test_codes_rejects_misaligned_buffers_on_host():
    L = hq.lib()
    p = hq.make_params("e8", step=0.3)
    ok, ws = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    for x, codes, scales in (((1 << 20) + 8, 1 << 20, 1 << 20), (1 << 20, (1 << 20) + 4, 1 << 20),
                             (1 << 20, 1 << 20, (1 << 20) + 1)):
        assert L.hq_codes(ctypes.c_void_p(x), 1, 128, ctypes.byref(p), ctypes.c_void_p(codes),
                          ctypes.c_void_p(scales), ws, 8192, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_codes(ok, 1, 128, ctypes.byref(p), ok, ok, ctypes.c_void_p((1 << 21) + 64), 8192,
                      None) == hq.HQ_ERR_INVALID_ARG


def test_noalloc_rejects_sizes_beyond_its_static_workspace_on_host():
    """hq_encode_noalloc checks n against its static workspace's maximum before any device call."""
    p = hq.make_params("e8", 4.0)
    nb = ctypes.c_uint64(0)
    rc = hq.lib().hq_encode_noalloc(ctypes.c_void_p(1 << 20), hq.HQ_BF16, (1 << 30) + 128, ctypes.byref(p),
                                    ctypes.c_void_p(1 << 21), 1 << 20, ctypes.byref(nb), None, None)
    assert rc == hq.HQ_ERR_SCRATCH
    bad = hq.make_params("e8", 4.0, tile=32)
    rc = hq.lib().hq_encode_noalloc(ctypes.c_void_p(1 << 20), hq.HQ_BF16, 1024, ctypes.byref(bad),
                                    ctypes.c_void_p(1 << 21), 1 << 20, ctypes.byref(nb), None, None)
    assert rc == hq.HQ_ERR_UNSUPPORTED
