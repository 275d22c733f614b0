"""Benchmark of the codec's hot path on one MI355X.

A step is one pass of the whole path over the workload: rate control (two sample passes), encode
(RHT, lattice, strip, Rice, look-back scan, packing) and decode (unpack, inverse RHT, bf16 store).
The default workload is the 14336 x 4096 bf16 MLP-weight tensor, E8 at 4 bits per value, no dither;
the default run also times one (layer, K) call of the KV cache, [8][32768][128] bf16, E8 + dither at
2 bps, reported under extra.kv (--config kv makes that call the headline).

Printed: one JSON line.  value = bf16 input bytes / (encode + decode time), GB/s; roofline: the
dominant kernel's algorithmic bytes per launch over its event-timed duration, against MI355X's
8 TB/s HBM peak; cpu_baseline: the CPU oracle on the same tensor on all host threads (and on one);
extra.parity: the run's stream, decode and integer codes against the oracle's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # binary32 VALU operations per second, packed forms unused
METRIC = "encode+decode GB/s of bf16 input (RHT+E8+Rice) and % of HBM peak, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", choices=["weight", "kv", "sweep", "tiles", "model", "kv_all", "gemv", "kv_haar",
                                         "srft"],
                    default="weight",
                    help="weight / kv: one tensor, the headline line; sweep: Z, A2, D4 and E8 on the weight; "
                         "tiles: E8 on the weight with tiles of 64, 128 and 256 values; "
                         "model: the 224 linear weights of an 8B-shaped decoder, one at a time; kv_all: "
                         "the 64 (layer, K|V) calls of the KV cache; gemv: fused decode + matrix-vector "
                         "product on the weight's stream; kv_haar: one KV call with the full per-layer "
                         "Haar rotation before encode and after decode; srft: the SRFT fixed-rate codec "
                         "(int4, or int8 with --bps 8) on the KV call")
    ap.add_argument("--bps", type=float, default=None)
    ap.add_argument("--dither-flags", type=int, default=1, choices=[1, 3, 5, 7],
                    help="kv: dither options (+2: 7-round Philox draw, +4: 24-bit draw)")
    ap.add_argument("--streams", type=int, default=3,
                    help="model / kv_all: streams the resident tensors are issued on, round-robin")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv", action="store_true",
                    help="default run: skip the KV calls (E8 + dither at 2 and 3 bits per value) timed beside the weight")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 256 MiB (known traffic), for scaling "
                         "the HBM byte counters of a profiler run")
    return ap.parse_args()


def copy_calibration(steps: int):
    """A plain copy of known size: 256 MiB read + 256 MiB written per launch.  A counter run over it
    gives the factor between the profiler's FETCH_SIZE / WRITE_SIZE readings and true HBM bytes."""
    import torch
    nbytes = 256 << 20
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                           "launches": steps}}), flush=True)


def measured_copy_gbs(torch, reps: int = 20) -> float:
    """Device-to-device copy of 1 GiB (read + written bytes over event time): the HBM bandwidth a
    plain streaming kernel reaches here, the second denominator beside the 8 TB/s spec."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: the model name, and its family, model and stepping
    numbers (some hosts report only a generic model name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping", "cpu MHz") and k not in fields:
                    fields[k] = v
            elif fields:
                break  # the first processor's block is enough
    except OSError:
        pass
    if not fields:
        return "unknown"
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    mhz = f", {float(fields['cpu MHz']):.0f} MHz" if "cpu MHz" in fields else ""
    return f"{fields.get('model name', 'unknown')} ({ids}{mhz})"


def workload(cfg: str, bps, dither_flags: int = 1):
    import synth
    if cfg == "weight":
        x = synth.weight()
        tb = 4.0 if bps is None else bps
        return x, dict(workload=f"mlp weight 14336x4096 bf16, E8 {tb:g} bps, no dither",
                       shape=[14336, 4096], lattice="e8", target_bps=tb, dither=False, seed=0,
                       profile=f"weight_14336x4096_e8_{tb:g}bps"), 0
    x = synth.kv(0, 0)
    tb = 2.0 if bps is None else bps
    opts = {1: "", 3: " (7-round Philox draw)", 5: " (24-bit draw)", 7: " (24-bit draw, 7-round Philox)"}
    suffix = "" if dither_flags == 1 else f"_flags{dither_flags}"
    return x, dict(workload=f"kv cache layer 0 K [8][32768][128] bf16, E8 + dither{opts[dither_flags]} {tb:g} bps",
                   shape=[8, 32768, 128], lattice="e8", target_bps=tb, dither=dither_flags,
                   seed=synth.kv_seed(0, 0), profile=f"kv_8x32768x128_e8_dither_{tb:g}bps{suffix}"), synth.kv_seed(0, 0)


CODEC_SOURCES = ("csrc/hq_kernels.hip", "csrc/hq_device.h", "csrc/hq_internal.h")
ROTATE_SOURCES = ("csrc/hq_rotate.hip",)
SRFT_SOURCES = ("csrc/hq_srft.hip", "csrc/hq_device.h")


def kernel_source_hash(sources=CODEC_SOURCES) -> str:
    """Hash of the kernels' sources and the compile flags: counter summaries taken under another
    hash describe other code."""
    import hashlib
    from kv_quantization_tile_amd.build import FLAGS
    pkg = os.path.join(ROOT, "kv_quantization_tile_amd")
    src = b"".join(open(os.path.join(pkg, f), "rb").read() for f in sources) + json.dumps(FLAGS).encode()
    return hashlib.sha256(src).hexdigest()[:16]


def profiled_traffic(profile_stem: str, kernel_prefix: str, sources=CODEC_SOURCES, namespace: str = "hq::"):
    """HBM bytes per dispatch of the named kernel, from the committed FETCH_SIZE / WRITE_SIZE summary
    of this workload (copy-calibrated); None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", profile_stem + "_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    blob = text.split("```json", 1)[-1].split("```", 1)[0]
    data = json.loads(blob)
    if data.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    for name, rec in data["kernels"].items():
        if name.startswith(namespace + kernel_prefix):
            return int(rec["traffic_bytes"])
    return None


def time_call(hq, torch, x, lat, tb, seed, dither, steps, warmup, out=None, ws=None, ws_dec=None, y=None, tile=128):
    """Events around encode (with rate control) and decode of one device tensor (steps timed,
    warmup untimed).  Returns per-step means (ms), the stream header and the decoded tensor."""
    dev = x.device
    n = x.numel()
    if out is None:
        s_ref, _ = hq.hq_encode(x, lat, tb, seed=seed, dither=dither, tile=tile)
        out = torch.empty(int(s_ref.numel() * 1.05) + 65536, dtype=torch.uint8, device=dev)
        del s_ref
    ws = hq.workspace(n, dev) if ws is None else ws
    ws_dec = hq.workspace(0, dev) if ws_dec is None else ws_dec
    y = torch.empty(n, dtype=torch.bfloat16, device=dev) if y is None else y
    stream = torch.cuda.current_stream()

    def one():
        hq.hq_encode(x, lat, tb, seed=seed, dither=dither, out=out, ws=ws, blocking=False, tile=tile)
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(stream)
        hq.hq_decode(out, n, out=y, ws=ws_dec, check=False)
        return e1

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        hq.hq_encode(x, lat, tb, seed=seed, dither=dither, out=out, ws=ws, blocking=False, tile=tile)
        hq.hq_decode(out, n, out=y, ws=ws_dec, check=False)
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    ev = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        e1 = one()
        e2 = torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        ev.append((e0, e1, e2))
    torch.cuda.synchronize()
    st, st2 = hq.hq_status(ws), hq.hq_status(ws_dec)
    assert st == 0 and st2 == 0, (st, st2)
    r = {"encode_ms": float(np.mean([a.elapsed_time(b) for a, b, _ in ev])),
         "decode_ms": float(np.mean([b.elapsed_time(c) for _, b, c in ev])),
         "step_ms": step_ms}
    return r, hq.header_fields(out[:128].cpu().numpy()), y


def profiled_valu(profile_stem: str, kernel_prefix: str, sources=CODEC_SOURCES, namespace: str = "hq::"):
    """VALU wave-instructions per dispatch of the named kernel (SQ_INSTS_VALU) from the committed
    counter summary of this workload; None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", profile_stem + "_instruction_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if "```json" not in text:
        return None
    data = json.loads(text.split("```json", 1)[-1].split("```", 1)[0])
    if data.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    for name, rec in data["kernels"].items():
        if name.startswith(namespace + kernel_prefix):
            return float(rec["valu"])
    return None


def streamed_pass(hq, torch, items, xs, nstreams, warmup):
    """All tensors resident: tensor i's encode (with rate control) and decode go to stream
    i mod nstreams, each stream with its own workspaces and buffers, so one tensor's latency-bound
    rate passes overlap another's encode and decode.  Events bracket the whole pass; afterwards
    every workspace's status must be clean."""
    dev = xs[0].device
    nmax = max(x.numel() for x in xs)
    cap = 0
    for (name, make, lat, tb, seed, dither, *rest), x in zip(items, xs):
        tile = rest[0] if rest else 128
        cap = max(cap, hq.capacity_estimate(x.numel(), lat, tb, tile=tile))
    streams = [torch.cuda.Stream(device=dev) for _ in range(nstreams)]   # default priority
    bufs = [dict(out=torch.empty(cap, dtype=torch.uint8, device=dev),
                 y=torch.empty(nmax, dtype=torch.bfloat16, device=dev),
                 ws=hq.workspace(nmax, dev), wsd=hq.workspace(0, dev)) for _ in range(nstreams)]

    def issue():
        for i, ((name, make, lat, tb, seed, dither, *rest), x) in enumerate(zip(items, xs)):
            tile = rest[0] if rest else 128
            st, b = streams[i % nstreams], bufs[i % nstreams]
            n = x.numel()
            hq.hq_encode(x, lat, tb, seed=seed, dither=dither, out=b["out"], ws=b["ws"], blocking=False,
                         tile=tile, stream=st)
            hq.hq_decode(b["out"], n, out=b["y"][:n], ws=b["wsd"], check=False, stream=st)

    cur = torch.cuda.current_stream()
    for _ in range(max(warmup, 1)):
        issue()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(cur)
    for st in streams:
        st.wait_event(t0)
    issue()
    for st in streams:
        e = torch.cuda.Event()
        e.record(st)
        cur.wait_event(e)
    t1.record(cur)
    torch.cuda.synchronize()
    for b, st in zip(bufs, streams):
        assert hq.hq_status(b["ws"], st) == 0 and hq.hq_status(b["wsd"], st) == 0
    return {"ms": t0.elapsed_time(t1)}


def series(args):
    """Many tensors or lattices, one JSON line: value = total bf16 input bytes over the summed step
    times; per-item figures in extra."""
    import torch

    import kv_quantization_tile_amd as hq
    dev = torch.device("cuda:0")
    items = []
    if args.config == "sweep":
        import synth
        xw = torch.from_numpy(synth.weight().reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
        tb = 4.0 if args.bps is None else args.bps
        for lat in ("z", "a2", "d4", "e8"):
            items.append((lat, lambda: xw, lat, tb, 0, False))
        workload = f"lattice sweep on the mlp weight 14336x4096 bf16 at {tb:g} bps: Z, A2, D4, E8, no dither"
        steps, warmup = args.steps, args.warmup
    elif args.config == "tiles":
        import synth
        xw = torch.from_numpy(synth.weight().reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
        tb = 4.0 if args.bps is None else args.bps
        for tl in (64, 128, 256):
            items.append((f"tile{tl}", lambda: xw, "e8", tb, 0, False, tl))
        workload = (f"tile-length sweep on the mlp weight 14336x4096 bf16, E8 {tb:g} bps, no dither: tiles of "
                    f"64, 128 and 256 values")
        steps, warmup = args.steps, args.warmup
    elif args.config == "model":
        import synth
        tb = 4.0 if args.bps is None else args.bps

        def gen(i, shape):
            def f():
                g = torch.Generator(device=dev)
                g.manual_seed(1000 + i)
                return (torch.randn(shape, generator=g, device=dev) * 0.02).to(torch.bfloat16).reshape(-1)
            return f
        for i, (name, shape) in enumerate(synth.model_shapes()):
            items.append((name, gen(i, shape), "e8", tb, i, False))
        workload = (f"224 linear weights of an 8B-shaped decoder (32 x q,k,v,o,gate,up,down) N(0, 0.02^2) bf16, "
                    f"drawn on the GPU one at a time, E8 {tb:g} bps, no dither")
        steps, warmup = 1, 1
    else:  # kv_all
        tb = 2.0 if args.bps is None else args.bps

        def gen(layer, is_v):
            def f():
                g = torch.Generator(device=dev)
                g.manual_seed(2_000_003 + layer * 2 + is_v)
                x = torch.randn((8, 32768, 128), generator=g, device=dev)
                if not is_v:
                    gc = torch.Generator(device=dev)
                    gc.manual_seed(7919 + layer)
                    for h in range(8):
                        ch = torch.randperm(128, generator=gc, device=dev)[:4]
                        x[h, :, ch] *= 10.0
                return x.to(torch.bfloat16).reshape(-1)
            return f
        for layer in range(32):
            for is_v in (0, 1):
                items.append((f"l{layer}.{'v' if is_v else 'k'}", gen(layer, is_v), "e8", tb,
                              (layer << 1) | is_v, True))
        workload = (f"KV cache, 32 layers x K|V calls of [8][32768][128] bf16 N(0,1) (4 K channels per head x10), "
                    f"drawn on the GPU one call at a time, E8 + dither {tb:g} bps, per-layer seed (l<<1)|isV")
        steps, warmup = 1, 1
    total_in = 0
    tot = {"encode_ms": 0.0, "decode_ms": 0.0, "step_ms": 0.0}
    per = {}
    worst_rate_err = 0.0
    enc_alg = 0
    resident = args.config in ("model", "kv_all")   # every tensor stays in HBM for the streamed pass
    kept = []
    for name, make, lat, tb, seed, dither, *rest in items:
        tile = rest[0] if rest else 128
        x = make()
        if resident:
            kept.append(x)
        n = x.numel()
        r, hdr, y = time_call(hq, torch, x, lat, tb, seed, dither, steps, warmup, tile=tile)
        for k in tot:
            tot[k] += r[k]
        total_in += 2 * n
        enc_alg += 2 * n + hdr["total_bytes"]
        rate_err = abs(hdr["payload_bits"] / n - tb)
        worst_rate_err = max(worst_rate_err, rate_err)
        if args.config in ("sweep", "tiles"):
            xf = x.float()
            nmse = float(((y.float() - xf) ** 2).sum() / (xf ** 2).sum())
            per[name] = {"payload_bps": round(hdr["payload_bits"] / n, 5),
                         "total_bps": round(8 * hdr["total_bytes"] / n, 5), "nmse": nmse,
                         "gbs": round(2 * n / (r["step_ms"] * 1e-3) / 1e9, 2),
                         **{k: round(v, 5) for k, v in r.items()}}
        del x, y
    value = total_in / (tot["step_ms"] * 1e-3) / 1e9
    enc_gbs = enc_alg / (tot["encode_ms"] * 1e-3) / 1e9
    streamed = None
    if resident:
        seq_value = value
        streamed = streamed_pass(hq, torch, items, kept, args.streams, args.warmup)
        value = total_in / (streamed["ms"] * 1e-3) / 1e9
        workload += (f"; all tensors resident in HBM, issued round-robin on {args.streams} streams "
                     f"(each tensor's encode and decode on one stream)")
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(streamed["ms"] if streamed else tot["step_ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload, "items": len(items), "input_bytes": total_in},
        "roofline": {"bound": "hbm", "achieved": round(enc_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(enc_gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "rate passes + encode_kernel",
                     "alg_bytes_per_launch": enc_alg // len(items), "launch_ms": round(tot["encode_ms"] / len(items), 5)},
        "extra": {**{k: round(v, 4) for k, v in tot.items()}, "worst_payload_rate_error_bps": round(worst_rate_err, 5),
                  **({"streamed_ms": round(streamed["ms"], 4), "streams": args.streams,
                      "one_at_a_time_value_gbs": round(seq_value, 2),
                      "one_at_a_time_note": "sum of per-tensor step times, each tensor timed alone"}
                     if streamed else {}),
                  **({("per_tile" if args.config == "tiles" else "per_lattice"): per} if per else {})},
    }
    print(json.dumps(result), flush=True)


def gemv_bench(args):
    """Fused decode + matrix-vector product on the 14336 x 4096 weight's E8 stream, next to torch's
    bf16 matrix-vector product on the uncompressed weight and to decode followed by that product."""
    import torch

    import kv_quantization_tile_amd as hq
    import synth
    dev = torch.device("cuda:0")
    rows, cols = 14336, 4096
    tb = 4.0 if args.bps is None else args.bps
    w = torch.from_numpy(synth.weight().reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
    x = torch.from_numpy(synth.gaussian(cols, seed=31)).to(dev)
    s, info = hq.hq_encode(w, "e8", tb)
    nbytes = s.numel()
    ws = torch.empty(hq.hq_gemv_workspace_size(rows, cols), dtype=torch.uint8, device=dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    wd = torch.empty(rows * cols, dtype=torch.bfloat16, device=dev)
    ws_dec = hq.workspace(0, dev)
    w2, xb = w.view(rows, cols), x.to(torch.bfloat16)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    fused_ms = timed(lambda: hq.hq_gemv(s, rows, cols, x, y=y, ws=ws, check=False))
    assert hq.hq_status(ws) == 0
    bf16_ms = timed(lambda: torch.mv(w2, xb))
    dec_mv_ms = timed(lambda: (hq.hq_decode(s, rows * cols, out=wd, ws=ws_dec, check=False),
                               torch.mv(wd.view(rows, cols), xb)))
    alg = nbytes + 4 * cols + 4 * rows
    achieved = alg / (fused_ms * 1e-3) / 1e9
    result = {
        "metric": "fused decode + matrix-vector product: bf16-equivalent weight GB/s, 1 GPU",
        "value": round(2 * rows * cols / (fused_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(fused_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"mlp weight 14336x4096 bf16 as an E8 {tb:g} bps stream ({nbytes} B), "
                               f"activation N(0,1) fp32 [4096]", "stream_bytes": nbytes,
                   "payload_bps": round(info["payload_bps"], 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "hq_gemv (all launches)",
                     "alg_bytes_per_launch": alg, "launch_ms": round(fused_ms, 5)},
        "extra": {"torch_bf16_mv_ms": round(bf16_ms, 5), "decode_then_torch_mv_ms": round(dec_mv_ms, 5),
                  "fused_vs_bf16": round(bf16_ms / fused_ms, 3), "fused_vs_decode_then_mv": round(dec_mv_ms / fused_ms, 3)},
    }
    print(json.dumps(result), flush=True)


def kv_haar_bench(args):
    """One KV call ([8][32768][128] bf16, E8 + dither) with the per-layer Haar-uniform rotation:
    rotate (MFMA), rate control, encode, decode, rotate back; the rotation kernel's roofline."""
    import torch

    import kv_quantization_tile_amd as hq
    import synth
    dev = torch.device("cuda:0")
    tb = 2.0 if args.bps is None else args.bps
    layer, is_v = 0, 0
    x_host = synth.kv(layer, is_v)
    n = x_host.size
    seed = synth.kv_seed(layer, is_v)
    x = torch.from_numpy(x_host.reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(hq.hq_haar_matrix(layer)).to(dev)
    xr = hq.hq_rotate(x, q)
    s_ref, _ = hq.hq_encode(xr, "e8", tb, seed=seed, dither=True)
    out = torch.empty(int(s_ref.numel() * 1.05) + 65536, dtype=torch.uint8, device=dev)
    ws, ws_dec = hq.workspace(n, dev), hq.workspace(0, dev)
    yr, y = torch.empty_like(x), torch.empty_like(x)

    def step(ev):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        hq.hq_rotate(x, q, out=xr)
        rec(1)
        hq.hq_encode(xr, "e8", tb, seed=seed, dither=True, out=out, ws=ws, blocking=False)
        rec(2)
        hq.hq_decode(out, n, out=yr, ws=ws_dec, check=False)
        rec(3)
        hq.hq_rotate(yr, q, transpose=True, out=y)
        rec(4)

    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()
    # timed region: steps back to back, events only at its ends; then a breakdown loop
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(None)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    assert hq.hq_status(ws) == 0 and hq.hq_status(ws_dec) == 0
    m = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))
    codec_enc_ms, dec_ms, back_ms = m(1, 2), m(2, 3), m(3, 4)

    # the rotation kernel alone, launched back to back over four buffer pairs (512 MiB touched per
    # round, twice what the on-package cache holds) so every launch reads and writes HBM
    nb = 4
    xs = [x.clone() for _ in range(nb)]
    ys = [torch.empty_like(x) for _ in range(nb)]
    for i in range(nb):
        hq.hq_rotate(xs[i], q, out=ys[i])
    torch.cuda.synchronize()
    rounds = max(args.steps, 4)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(rounds * nb)]
    for r in range(rounds):
        for i in range(nb):
            pairs[r * nb + i][0].record()
            hq.hq_rotate(xs[i], q, out=ys[i])
            pairs[r * nb + i][1].record()
    torch.cuda.synchronize()
    rot_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    assert torch.equal(ys[0], xr)
    del xs, ys
    rot_alg = 4 * n  # bf16 in + bf16 out
    achieved = rot_alg / (rot_ms * 1e-3) / 1e9
    xf, yf = x.float(), y.float()
    nmse = float(((yf - xf) ** 2).sum() / (xf ** 2).sum())
    result = {
        "metric": METRIC + " (KV path with the full per-layer rotation)", "value": round(2 * n / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"kv cache layer 0 K [8][32768][128] bf16, Haar rotation (seed 0) + E8 + dither "
                               f"{tb:g} bps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic("rotate_kv_8x32768x128_bf16", "rotate_kernel", ROTATE_SOURCES,
                                                 "hq_rot::"),
                     "kernel": "rotate_kernel",
                     "alg_bytes_per_launch": rot_alg, "launch_ms": round(rot_ms, 5)},
        "extra": {"rotate_ms": round(rot_ms, 5), "rate_and_encode_ms": round(codec_enc_ms, 5),
                  "decode_ms": round(dec_ms, 5), "rotate_back_ms": round(back_ms, 5), "nmse": nmse},
    }
    print(json.dumps(result), flush=True)




def srft_ops_per_vector(bits: int):
    """Binary32 operations of the SRFT codec's definition per 128-value vector (each add, multiply,
    division, abs-max, rounding, clamp, conversion counted once; products by the exact twiddles 1 and
    -+i not counted).  Returns (encode, decode)."""
    fft = 6 * 32 * 4 + 98 * 6          # 384 complex adds; 98 products by non-trivial twiddles
    unpack = 2 + 63 * 12                # E, G, W^k (-i G), E + ...
    enc = 128 + fft + unpack + 128 + 128 + 16 * 3 + 128 * 4 + 128  # signs, multipliers, abs-max,
    # scale (division, binary16 rounding, reciprocal), codes (multiply, rint, clamp, convert), finiteness
    dec = 128 * 3 + 16 + (4 + 63 * 12) + fft + 128 * 3 + 128       # dequantise, unpack, FFT, output
    return enc, dec


def srft_bench(args):
    """The SRFT fixed-rate codec (sign, FFT, Hermitian pack, per-group int4 / int8) on one KV call
    [8][32768][128] bf16: encode + decode per step, per-launch events, the dominant kernel's ALU
    roofline, the oracle on the whole tensor as the CPU baseline and parity of codes and decode."""
    import torch

    import kv_quantization_tile_amd as hq
    import synth
    bits = 4 if args.bps is None else int(args.bps)
    if bits not in (4, 8):
        raise SystemExit("--config srft takes --bps 4 or 8")
    dev = torch.device("cuda:0")
    x_host = synth.kv(0, 0)
    n = x_host.size
    nv = n // 128
    seed = synth.kv_seed(0, 0)
    x = torch.from_numpy(x_host.reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
    codes = torch.empty((nv, 64 if bits == 4 else 128), dtype=torch.uint8, device=dev)
    scales = torch.empty((nv, 16), dtype=torch.int16, device=dev)
    y = torch.empty_like(x)

    def step(ev):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        hq.hq_srft_encode(x, seed=seed, bits=bits, codes=codes, scales=scales)
        rec(1)
        rec(2)
        hq.hq_srft_decode(codes, scales, n, seed=seed, bits=bits, out=y)
        rec(3)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    # timed region: steps back to back, events only at its ends; then a breakdown loop
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(None)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ops_enc, ops_dec = srft_ops_per_vector(bits)
    code_bytes = nv * (64 if bits == 4 else 128) + nv * 32
    if enc_ms >= dec_ms:
        dom, ms, ops, hbm = "srft_encode_kernel", enc_ms, ops_enc * nv, 2 * n + code_bytes
    else:
        dom, ms, ops, hbm = "srft_decode_kernel", dec_ms, ops_dec * nv, 2 * n + code_bytes
    tops = ops / (ms * 1e-3) / 1e12
    xf = x.float()
    nmse = float(((y.float() - xf) ** 2).sum() / (xf ** 2).sum())
    traffic = profiled_traffic(f"srft_kv_8x32768x128_int{bits}", dom, SRFT_SOURCES, "hq_srft::")
    result = {
        "metric": "encode+decode GB/s of bf16 input (SRFT fixed-rate codec), 1 GPU", "value": round(2 * n / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"kv cache layer 0 K [8][32768][128] bf16, SRFT int{bits} + 16 binary16 group "
                               f"scales per vector"},
        "roofline": {"bound": "alu", "achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TFLOP/s",
                     "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": traffic, "kernel": dom,
                     "alg_ops_per_launch": ops, "launch_ms": round(ms, 5),
                     "hbm_gbs": round(hbm / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "extra": {"encode_ms": round(enc_ms, 5), "decode_ms": round(dec_ms, 5), "nmse": nmse,
                  "bits_per_value": (64 if bits == 4 else 128) * 8 / 128 + 16 * 16 / 128,
                  "ops_per_vector_encode": ops_enc, "ops_per_vector_decode": ops_dec},
    }
    if not args.no_cpu_baseline or not args.no_parity:
        import oracle
        if not os.path.exists(os.path.join(ROOT, "oracle", "libhq_oracle.so")):
            oracle.build()
        # the whole workload, repeated until about 10 s of host time have been spent (at most 8 times)
        reps, t_enc, t_dec = 0, 0.0, 0.0
        while True:
            t1h = time.perf_counter()
            c_orc, s_orc = oracle.srft_encode(x_host, seed, bits)
            t2h = time.perf_counter()
            y_orc = oracle.srft_decode(c_orc, s_orc, n, seed, bits)
            t3h = time.perf_counter()
            reps, t_enc, t_dec = reps + 1, t_enc + (t2h - t1h), t_dec + (t3h - t2h)
            if args.no_cpu_baseline or t_enc + t_dec >= 10.0 or reps >= 8:
                break
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {"value": round(reps * 2 * n / (t_enc + t_dec) / 1e9, 4), "unit": "GB/s",
                                      "cores": 1, "kind": "oracle",
                                      "sample": f"the whole workload ({n} values), {reps} times one encode + one "
                                                f"bf16 decode, single host thread: encode {t_enc / reps:.2f} s, "
                                                f"decode {t_dec / reps:.2f} s each"}
        if not args.no_parity:
            result["extra"]["parity_codes_equal"] = bool(np.array_equal(codes.cpu().numpy(), c_orc))
            result["extra"]["parity_scales_equal"] = bool(
                np.array_equal(scales.cpu().numpy().view(np.uint16), s_orc))
            result["extra"]["parity_decoded_equal"] = bool(
                np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), y_orc))
    print(json.dumps(result), flush=True)


def measure(hq, torch, x_host, cfg, seed, K, W):
    """Times K steps (after W warm-up steps) of one workload and breaks the step down.  Returns the
    parts of the JSON line: value, ms_per_step, config additions, roofline and extra, plus the
    device buffers the parity report reads."""
    profile_stem = cfg.pop("profile")
    n = x_host.size
    dev = torch.device("cuda:0")
    x = torch.from_numpy(x_host.reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
    lat, tb, dither = cfg["lattice"], cfg["target_bps"], cfg["dither"]

    # one blocking encode gives the operating point; the output buffer is the worst-case bound there
    s_ref, info = hq.hq_encode(x, lat, tb, seed=seed, dither=dither)
    cap = hq.hq_encode_bound(n, lat, info["step"], info["rice_k"], dither)
    del s_ref
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    ws = hq.workspace(n, dev)
    ws_dec = hq.workspace(0, dev)
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # one step = hq_encode with rate control (init, two sample passes, the solve, the encode kernel)
    # and hq_decode (header check, decode kernel)
    def encode():
        hq.hq_encode(x, lat, tb, seed=seed, dither=dither, out=out, ws=ws, blocking=False)

    def decode():
        hq.hq_decode(out, n, out=y, ws=ws_dec, check=False)

    # the encode kernel alone, for its roofline: an asynchronous hq_rate leaves the operating point
    # in the workspace, and hq_encode at that point (step=-1) launches the reset and the encode kernel
    def rate():
        hq.hq_rate(x, lat, tb, seed=seed, dither=dither, ws=ws, blocking=False)

    def encode_at_point():
        hq.hq_encode(x, lat, tb, seed=seed, dither=dither, step=-1.0, out=out, ws=ws, blocking=False)

    for _ in range(W):
        encode(); decode()
        rate(); encode_at_point()
    torch.cuda.synchronize()

    # the timed region: K steps back to back, events only at its two ends (an event recorded
    # between two kernels delays the second by several microseconds)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(K):
        encode()
        decode()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = t_start.elapsed_time(t_end) / K
    st, st2 = hq.hq_status(ws), hq.hq_status(ws_dec)
    assert st == 0 and st2 == 0, (st, st2)
    fallbacks = hq.hq_fallbacks(ws)  # the last timed encode: waits that ran out of their budget
    g_step = out[:128].clone()

    # breakdown (separate loops): encode with rate control, decode; rate control, the encode kernel
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        encode()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    enc_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]))
    dec_ms = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]))
    ek = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ek[i][0].record(stream)
        rate()
        ek[i][1].record(stream)
        encode_at_point()
        ek[i][2].record(stream)
    torch.cuda.synchronize()
    assert hq.hq_status(ws) == 0
    rate_ms = float(np.mean([ek[i][0].elapsed_time(ek[i][1]) for i in range(K)]))
    enc_kernel_ms = float(np.mean([ek[i][1].elapsed_time(ek[i][2]) for i in range(K)]))
    assert torch.equal(out[:128], g_step), "hq_rate + hq_encode(step=-1) differs from hq_encode"

    hdr = hq.header_fields(out[:128].cpu().numpy())
    total_bytes = hdr["total_bytes"]
    input_bytes = 2 * n
    value = input_bytes / (step_ms * 1e-3) / 1e9
    # algorithmic bytes: encode reads the input and writes the stream; decode reads the stream and
    # writes bf16 values
    alg_step = 2 * (input_bytes + total_bytes)
    # dominant kernel: encode_kernel (timed with its one-lane reset launch) or decode_kernel (timed
    # with its one-lane header check launch); both figures are therefore slightly conservative
    dec_alg = total_bytes + input_bytes
    enc_alg = input_bytes + total_bytes
    if dec_ms >= enc_kernel_ms:
        dom, dom_ms, dom_bytes = "decode_kernel", dec_ms, dec_alg
    else:
        dom, dom_ms, dom_bytes = "encode_kernel", enc_kernel_ms, enc_alg
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = profiled_traffic(profile_stem, dom)
    # the kernel's binding resource is the vector ALU: its measured VALU instructions (64 lanes
    # each) over the same launch time, against 256 CUs x 64 lanes x 2.4 GHz
    valu = profiled_valu(profile_stem, dom)
    valu_issue = None
    if valu is not None:
        tops = valu * 64 / (dom_ms * 1e-3) / 1e12
        valu_issue = {"achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2), "unit": "T lane-ops/s",
                      "frac": round(tops / VALU_PEAK_TOPS, 4), "lane_ops_per_value": round(valu * 64 / n, 2),
                      "source": "SQ_INSTS_VALU per dispatch x 64, from the committed counter summary"}
    r = {
        "value": value, "ms_per_step": step_ms,
        "config": {**cfg, "n_values": n, "stream_bytes": total_bytes,
                   "payload_bps": round(hdr["payload_bits"] / n, 5),
                   "side_bps": round((8 * total_bytes - hdr["payload_bits"]) / n, 5),
                   "total_bps": round(8 * total_bytes / n, 5),
                   "step": float(np.array([hdr["step_bits"]], dtype=np.uint32).view(np.float32)[0]),
                   "rice_k": hdr["k"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                     "alg_bytes_per_launch": dom_bytes, "launch_ms": round(dom_ms, 5), "valu_issue": valu_issue},
        "extra": {"encode_with_rate_control_ms": round(enc_ms, 5), "decode_ms": round(dec_ms, 5),
                  "encode_kernel_ms": round(enc_kernel_ms, 5), "hq_rate_alone_ms": round(rate_ms, 5),
                  "encode_kernel_gbs": round(enc_alg / (enc_kernel_ms * 1e-3) / 1e9, 1),
                  "decode_kernel_gbs": round(dec_alg / (dec_ms * 1e-3) / 1e9, 1),
                  "step_alg_bytes": alg_step,
                  "step_hbm_gbs": round(alg_step / (step_ms * 1e-3) / 1e9, 1),
                  "step_hbm_frac": round(alg_step / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "host_wall_ms_per_step": round(wall / K * 1e3, 5),
                  "fallbacks_last_timed_encode": fallbacks},
        "_dev": dict(x=x, out=out, y=y, total_bytes=total_bytes, step=float(info["step"]), k=int(info["rice_k"])),
    }
    return r


def parity_report(hq, torch, oracle, x_host, cfg, seed, dev_bufs):
    """The GPU results of the timed run against the oracle on the same tensor: stream bytes, decoded
    bf16 values, integer lattice codes (mismatching octets, and how many of them lie within 1e-5 of
    a Voronoi boundary), and the largest per-tile relative error of the fp32 decode,
    max_i |x_gpu - x_oracle| / max_i |x_oracle|.  Returns the report and the oracle's timings."""
    lat, tb, dither = cfg["lattice"], cfg["target_bps"], cfg["dither"]
    n = x_host.size
    L = oracle.LATTICES[lat]
    t1 = time.perf_counter()
    s_orc, info_orc = oracle.encode(x_host, L, tb, seed=seed, dither=dither)
    t2 = time.perf_counter()
    y_orc_b = oracle.decode(s_orc, n, out_dtype="bf16")
    t3 = time.perf_counter()
    g = dev_bufs["out"][:dev_bufs["total_bytes"]].cpu().numpy()
    rep = {"stream_bytes_equal": bool(g.size == s_orc.size and np.array_equal(g, s_orc)),
           "decoded_bf16_equal": bool(np.array_equal(
               dev_bufs["y"].view(torch.int16).cpu().numpy().view(np.uint16), y_orc_b)),
           "step_and_k_equal": bool(info_orc["step"] == dev_bufs["step"] and info_orc["k"] == dev_bufs["k"])}
    # integer codes at the operating point
    step = dev_bufs["step"]
    c_orc, sc_orc = oracle.quantize(x_host, L, step, seed=seed, dither=dither)
    c_gpu, sc_gpu = hq.hq_codes(dev_bufs["x"], step, lat, seed=seed, dither=dither)
    c_gpu = c_gpu.cpu().numpy()
    bad = np.nonzero((c_gpu.reshape(-1, 8) != c_orc.reshape(-1, 8)).any(axis=1))[0]
    attributed = 0
    if bad.size:
        v = oracle.lattice_inputs(x_host, L, step, seed, dither).reshape(-1, 8).astype(np.float64)
        half = 0.5 if lat in ("e8", "a2") else 1.0
        wm = np.tile([1.0, 3.0], 4) if lat == "a2" else np.ones(8)
        for i in bad[:100000]:
            cg, co = c_gpu.reshape(-1, 8)[i] * half, c_orc.reshape(-1, 8)[i] * half
            dist = abs((wm * (v[i] - cg) ** 2).sum() - (wm * (v[i] - co) ** 2).sum()) / (
                2 * np.sqrt((wm * (cg - co) ** 2).sum()))
            attributed += int(dist <= 1e-5)
    rep["octets"] = int(n // 8)
    rep["code_mismatch_octets"] = int(bad.size)
    rep["code_mismatch_boundary_attributed"] = attributed
    rep["scales_equal"] = bool(np.array_equal(sc_gpu.cpu().numpy().view(np.uint16), sc_orc))
    # fp32 decode, per-tile relative error
    y32 = hq.hq_decode(dev_bufs["out"][:dev_bufs["total_bytes"]], n, out_dtype=torch.float32).cpu().numpy()
    y_orc = oracle.decode(s_orc, n).reshape(-1, 128)
    err = np.abs(y32.reshape(-1, 128).astype(np.float64) - y_orc).max(axis=1)
    mag = np.abs(y_orc).max(axis=1).astype(np.float64)
    rel = np.where(mag > 0, err / np.where(mag > 0, mag, 1.0), np.where(err > 0, np.inf, 0.0))
    rep["max_tile_rel_decode_err_f32"] = float(rel.max())
    rep["payload_bps_error"] = round(abs(info_orc["payload_bps"] - tb), 5)
    return rep, {"encode_s": t2 - t1, "decode_s": t3 - t2, "stream": s_orc, "info": info_orc}


def host_threads() -> int:
    """The host CPUs this process may use (its affinity mask), at most 16: the CPU share of one GPU
    on the machines this runs on."""
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:
        c = os.cpu_count() or 1
    return max(1, min(c, 16))


def cpu_baseline_all_cores(oracle, x_host, cfg, seed, orc_times, threads):
    """The oracle, unchanged and single-threaded per call, on all host threads: rate control once on
    the whole tensor, then the tensor split into `threads` slices of whole 8192-value chunks, each
    encoded (at the operating point rate control chose) and decoded to bf16 by one thread (ctypes
    releases the interpreter lock during the oracle's C calls, and the oracle holds no global
    state).  Repeated until about 2 s of wall time (at most 8 times)."""
    from concurrent.futures import ThreadPoolExecutor
    lat, tb, dither = cfg["lattice"], cfg["target_bps"], cfg["dither"]
    L = oracle.LATTICES[lat]
    flat = x_host.reshape(-1)
    n = flat.size
    chunks = (n + 8191) // 8192
    bounds = [min(n, (chunks * i // threads) * 8192) for i in range(threads + 1)]
    slices = [flat[bounds[i]:bounds[i + 1]] for i in range(threads) if bounds[i + 1] > bounds[i]]

    def work(part, step, k):
        s, _ = oracle.encode(part, L, 0.0, seed=seed, dither=dither, step=step, rice_k=k)
        oracle.decode(s, part.size, out_dtype="bf16")
        return part.size

    reps, wall = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as pool:
        while True:
            t0 = time.perf_counter()
            step, _, k = oracle.rate(x_host, L, tb, seed=seed, dither=dither)
            done = sum(pool.map(lambda p: work(p, step, k), slices))
            wall += time.perf_counter() - t0
            reps += 1
            assert done == n
            if wall >= 2.0 or reps >= 8:
                break
    one = 2 * n / (orc_times["encode_s"] + orc_times["decode_s"]) / 1e9
    return {"value": round(reps * 2 * n / wall / 1e9, 4), "unit": "GB/s", "cores": len(slices), "kind": "oracle",
            "sample": f"the whole workload ({n} values), {reps} times: the oracle's rate control on one thread, "
                      f"then {len(slices)} slices of whole 8192-value chunks encoded at that operating point and "
                      f"decoded to bf16, one slice per host thread; mean wall {wall / reps:.3f} s per pass",
            "one_thread_gbs": round(one, 4),
            "one_thread_sample": f"one encode with rate control ({orc_times['encode_s']:.2f} s) and one bf16 decode "
                                 f"({orc_times['decode_s']:.2f} s) of the whole workload on one thread",
            "cpu": cpu_model(), "host_cpus_visible": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "tiles shard across GPUs without communication, see the design notes", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    if args.config in ("sweep", "tiles", "model", "kv_all"):
        series(args)
        return
    if args.config == "gemv":
        gemv_bench(args)
        return
    if args.config == "kv_haar":
        kv_haar_bench(args)
        return
    if args.config == "srft":
        srft_bench(args)
        return
    import torch

    import kv_quantization_tile_amd as hq

    # the headline workload (the weight by default), and, in the default run, one KV call beside it
    # at 2 and at 3 bits per value
    x_host, cfg, seed = workload(args.config, args.bps, args.dither_flags)
    K = args.steps
    r = measure(hq, torch, x_host, cfg, seed, K, args.warmup)
    seconds = []
    if args.config == "weight" and args.bps is None and not args.no_kv:
        for key, bps in (("kv", None), ("kv_3bps", 3.0)):
            xk, cfgk, seedk = workload("kv", bps, 1)
            seconds.append((key, xk, cfgk, seedk, measure(hq, torch, xk, cfgk, seedk, K, args.warmup)))

    result = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": r["config"],
        "roofline": r["roofline"],
        "extra": r["extra"],
    }
    copy_gbs = measured_copy_gbs(torch)
    result["roofline"]["measured_copy_gbs"] = round(copy_gbs, 1)
    result["roofline"]["frac_of_measured_copy"] = round(r["roofline"]["achieved"] / copy_gbs, 4)
    for key, xk, cfgk, seedk, rk in seconds:
        result["extra"][key] = {"workload": rk["config"]["workload"], "value_gbs": round(rk["value"], 2),
                                "ms_per_step": round(rk["ms_per_step"], 5), "config": rk["config"],
                                "roofline": {**rk["roofline"], "measured_copy_gbs": round(copy_gbs, 1)},
                                **rk["extra"]}

    if not args.no_cpu_baseline or not args.no_parity:
        import oracle
        if not os.path.exists(os.path.join(ROOT, "oracle", "libhq_oracle.so")):
            oracle.build()
        rep, times = parity_report(hq, torch, oracle, x_host, r["config"], seed, r["_dev"])
        if not args.no_parity:
            result["extra"]["parity"] = rep
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline_all_cores(oracle, x_host, r["config"], seed, times,
                                                            host_threads())
        for key, xk, cfgk, seedk, rk in seconds:
            repk, tk = parity_report(hq, torch, oracle, xk, rk["config"], seedk, rk["_dev"])
            if not args.no_parity:
                result["extra"][key]["parity"] = repk
            result["extra"][key]["cpu_oracle_one_thread_gbs"] = round(
                2 * xk.size / (tk["encode_s"] + tk["decode_s"]) / 1e9, 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
