"""Rate control's workgroups wait on one another (pass B's on pass A's solve, published by workgroup
0), and every wait has a fallback that computes the awaited value itself, which keeps results
right in any case but costs milliseconds.  These tests guard the normal path: a call with rate
control must not reach a fallback when the launch needs more workgroups than the GPU holds at once
(tiles of 256 values: 2048 rate workgroups) or when other streams' kernels hold the CUs.  A call
takes about 0.1-0.2 ms normally and several milliseconds on a fallback; the bound is 5 ms, and
hq_fallbacks must report none for the workspace's last call."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
hq = pytest.importorskip("kv_quantization_tile_amd")

pytestmark = pytest.mark.gpu

BOUND_MS = 5.0


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()


def say(msg):
    print(msg, flush=True)


def timed_encodes(x, tile, reps=4, stream=None):
    """Asynchronous encodes with rate control, each between events on its stream: times in ms."""
    s = stream or torch.cuda.current_stream()
    n = x.numel()
    out = torch.empty(hq.capacity_estimate(n, "e8", 4.0, tile=tile) * 2, dtype=torch.uint8, device="cuda")
    ws = hq.workspace(n)
    times = []
    with torch.cuda.stream(s):
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            hq.hq_encode(x, "e8", 4.0, tile=tile, out=out, ws=ws, stream=s, blocking=False)
            e1.record(s)
            times.append((e0, e1))
    return times, ws


@pytest.mark.parametrize("tile", [64, 128, 256])
def test_rate_control_takes_its_normal_path(tile):
    say(f"case: rate control time, weight 14336x4096, tiles of {tile}")
    x = dev(synth.weight())
    times, ws = timed_encodes(x, tile)
    torch.cuda.synchronize()
    assert hq.hq_status(ws) == hq.HQ_OK
    assert hq.hq_fallbacks(ws) == 0  # the last call: no wait ran out of its budget
    ms = [a.elapsed_time(b) for a, b in times[1:]]
    assert max(ms) < BOUND_MS, ms


def test_rate_control_beside_other_streams():
    """Three streams, each encoding and decoding its own KV call ([8][32768][128], E8 with dither at
    2 bits per value) over and over, as a serving loop would: one stream's rate control runs while
    the others' encode and decode kernels hold the CUs."""
    say("case: rate control time, KV encode + decode on three streams at once")
    xs = [dev(synth.kv(layer, 0)) for layer in range(3)]
    streams = [torch.cuda.Stream() for _ in range(3)]  # default priority
    n = xs[0].numel()
    cap = hq.capacity_estimate(n, "e8", 2.0) * 2
    bufs = [(torch.empty(cap, dtype=torch.uint8, device="cuda"), torch.empty(n, dtype=torch.bfloat16, device="cuda"),
             hq.workspace(n), hq.workspace(0)) for _ in range(3)]
    torch.cuda.synchronize()
    marks = []
    for it in range(6):
        for i, (x, s, (out, y, ws, wsd)) in enumerate(zip(xs, streams, bufs)):
            with torch.cuda.stream(s):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                hq.hq_encode(x, "e8", 2.0, seed=synth.kv_seed(i, 0), dither=True, out=out, ws=ws, stream=s,
                             blocking=False)
                e1.record(s)
                hq.hq_decode(out, n, out=y, ws=wsd, stream=s, check=False)
                if it > 0:
                    marks.append((e0, e1))
    torch.cuda.synchronize()
    for out, y, ws, wsd in bufs:
        assert hq.hq_status(ws) == hq.HQ_OK and hq.hq_status(wsd) == hq.HQ_OK
        assert hq.hq_fallbacks(ws) == 0
    ms = [a.elapsed_time(b) for a, b in marks]
    assert max(ms) < BOUND_MS, ms
