"""hq_encode_noalloc: the encode whose workspace is the library's static device array, for callers
that cannot allocate.  Checked through the C ABI against hq_encode (the existing entry point, with a
workspace the caller allocates) on consecutive calls, the later ones smaller, and against the
oracle."""
import ctypes

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()


def noalloc(x, params, cap, blocking=True):
    """One hq_encode_noalloc call; returns (rc, stream bytes on the host, info)."""
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    nb = ctypes.c_uint64(0)
    info = hq.HqInfo()
    dt = hq.HQ_BF16 if x.dtype == torch.bfloat16 else hq.HQ_F32
    rc = hq.lib().hq_encode_noalloc(ctypes.c_void_p(x.data_ptr()), dt, x.numel(), ctypes.byref(params),
                                    ctypes.c_void_p(out.data_ptr()), cap,
                                    ctypes.byref(nb) if blocking else None,
                                    ctypes.byref(info) if blocking else None, None)
    torch.cuda.synchronize()
    if not blocking:
        size = hq.header_fields(out[:128].cpu().numpy())["total_bytes"]
        return rc, out[:size].cpu().numpy(), None
    return rc, out[:nb.value].cpu().numpy(), info.as_dict()


def test_noalloc_equals_hq_encode_on_consecutive_calls(orc):
    # 1: the weight slice with rate control; 2: a smaller slice at a fixed point; 3: a still smaller
    # dithered KV block at the point call 2 left (step = -1); 4: asynchronous, smaller again
    w1 = synth.weight(rows=1024)
    w2 = synth.weight(rows=200)
    kv = synth.kv(5, 1, heads=1, tokens=700)
    seed = synth.kv_seed(5, 1)
    calls = [(w1, hq.make_params("e8", 4.0), True),
             (w2, hq.make_params("d4", 0.0, step=0.21, rice_k=2), True),
             (kv, hq.make_params("d4", 0.0, seed=seed, dither=True, step=-1.0), True),
             (w2[:37], hq.make_params("e8", 3.0, seed=4, dither=True), False)]
    for i, (xh, p, blocking) in enumerate(calls):
        say(f"case: hq_encode_noalloc call {i + 1}, {xh.size} values, blocking={blocking}")
        x = dev(xh)
        if p.step > 0:
            cap = hq.hq_encode_bound(xh.size, p.lattice, p.step, p.rice_k, p.dither)
        elif p.step == -1.0:
            cap = hq.hq_encode_bound(xh.size, p.lattice, 0.21, 2, p.dither)
        else:
            cap = 4 * xh.size + 65536   # rate control: far above any stream at these targets
        rc, got, info = noalloc(x, p, cap, blocking)
        assert rc == hq.HQ_OK, hq.strerror(rc)
        # the existing entry point, same params; step=-1 there takes the point of its own workspace,
        # so the reference for call 3 is the fixed point that call 2 set
        ref_step = 0.21 if p.step == -1.0 else p.step
        ref_k = 2 if p.step == -1.0 else p.rice_k
        lat = {0: "z", 1: "d4", 2: "e8", 3: "a2"}[p.lattice]
        ref, ref_info = hq.hq_encode(x, lat, p.target_bps, seed=p.seed, dither=p.dither, step=ref_step,
                                     rice_k=ref_k)
        ref = ref.cpu().numpy()
        assert got.size == ref.size and np.array_equal(got, ref), i
        if blocking:
            assert info["bytes"] == ref_info["bytes"] and info["step"] == ref_info["step"]
            assert info["rice_k"] == ref_info["rice_k"]
        s_orc, _ = orc.encode(xh, p.lattice, p.target_bps, seed=p.seed, dither=p.dither, step=ref_step,
                              rice_k=ref_k)
        assert np.array_equal(got, s_orc), i


def test_noalloc_capacity_and_limits():
    say("case: hq_encode_noalloc capacity retry and size limit")
    w = synth.weight(rows=64)
    x = dev(w)
    p = hq.make_params("e8", 4.0)
    rc, _, _ = noalloc(x, p, 2048)
    assert rc == hq.HQ_ERR_CAPACITY
    ref, _ = hq.hq_encode(x, "e8", 4.0)
    rc, got, _ = noalloc(x, p, ref.numel())
    assert rc == hq.HQ_OK and np.array_equal(got, ref.cpu().numpy())
    # above the static workspace's maximum: rejected on the host before any device work
    big = ctypes.c_uint64(0)
    rc = hq.lib().hq_encode_noalloc(ctypes.c_void_p(x.data_ptr()), hq.HQ_BF16, (1 << 30) + 128, ctypes.byref(p),
                                    ctypes.c_void_p(x.data_ptr()), 16, ctypes.byref(big), None, None)
    assert rc == hq.HQ_ERR_SCRATCH
    assert "allocation-free" in hq.strerror(rc)
