"""Benchmark of the codec's hot path on one MI355X.

A step is one pass of the whole path over the workload: rate control (two sample passes), encode
(RHT, lattice, strip, Rice, look-back scan, packing) and decode (unpack, inverse RHT, bf16 store).
The default workload is the 14336 x 4096 bf16 MLP-weight tensor, E8 at 4 bits per value, no dither;
--config kv times one (layer, K) call of the KV cache, [8][32768][128] bf16, E8 + dither at 2 bps.

Printed: one JSON line.  value = bf16 input bytes / (encode + decode time), GB/s; roofline: the
dominant kernel's algorithmic bytes per launch over its event-timed duration, against MI355X's
8 TB/s HBM peak; cpu_baseline: the CPU oracle on the same tensor, one host thread.
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
METRIC = "encode+decode GB/s of bf16 input (RHT+E8+Rice) and % of HBM peak, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", choices=["weight", "kv"], default="weight")
    ap.add_argument("--bps", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def workload(cfg: str, bps):
    import synth
    if cfg == "weight":
        x = synth.weight()
        tb = 4.0 if bps is None else bps
        return x, dict(workload=f"mlp weight 14336x4096 bf16, E8 {tb:g} bps, no dither",
                       shape=[14336, 4096], lattice="e8", target_bps=tb, dither=False, seed=0,
                       profile=f"weight_14336x4096_e8_{tb:g}bps"), 0
    x = synth.kv(0, 0)
    tb = 2.0 if bps is None else bps
    return x, dict(workload=f"kv cache layer 0 K [8][32768][128] bf16, E8 + dither {tb:g} bps",
                   shape=[8, 32768, 128], lattice="e8", target_bps=tb, dither=True,
                   seed=synth.kv_seed(0, 0), profile=f"kv_8x32768x128_e8_dither_{tb:g}bps"), synth.kv_seed(0, 0)


def kernel_source_hash() -> str:
    import hashlib
    pkg = os.path.join(ROOT, "kv_quantization_tile_amd")
    src = b"".join(open(os.path.join(pkg, f), "rb").read() for f in
                   ("csrc/hq_kernels.hip", "csrc/hq_device.h", "csrc/hq_internal.h", "build.py"))
    return hashlib.sha256(src).hexdigest()[:16]


def profiled_traffic(profile_stem: str, kernel_prefix: str):
    """HBM bytes per dispatch of the named kernel, from the committed FETCH_SIZE / WRITE_SIZE summary
    of this workload (copy-calibrated); None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", profile_stem + "_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    blob = text.split("```json", 1)[-1].split("```", 1)[0]
    data = json.loads(blob)
    if data.get("source_sha256_16") != kernel_source_hash():
        return None
    for name, rec in data["kernels"].items():
        if name.startswith("hq::" + kernel_prefix):
            return int(rec["traffic_bytes"])
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "tiles shard across GPUs without communication, see the design notes", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    import torch

    import kv_quantization_tile_amd as hq

    x_host, cfg, seed = workload(args.config, args.bps)
    profile_stem = cfg.pop("profile")
    n = x_host.size
    dev = torch.device("cuda:0")
    x = torch.from_numpy(x_host.reshape(-1).view(np.int16)).view(torch.bfloat16).to(dev)
    lat, tb, dither = cfg["lattice"], cfg["target_bps"], cfg["dither"]

    # one blocking encode sizes the buffers and gives the operating point
    s_ref, info = hq.hq_encode(x, lat, tb, seed=seed, dither=dither)
    cap = int(s_ref.numel() * 1.05) + 65536
    out = torch.empty(cap, dtype=torch.uint8, device=dev)
    ws = hq.workspace(n, dev)
    ws_dec = hq.workspace(0, dev)
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # one step = rate control, encode and decode; the encode is issued as an asynchronous hq_rate
    # followed by hq_encode at the operating point it chose (exactly the kernels of one hq_encode
    # with rate control), so that events can bracket the encode kernel alone
    def rate():
        hq.hq_rate(x, lat, tb, seed=seed, dither=dither, ws=ws, blocking=False)

    def encode():
        hq.hq_encode(x, lat, tb, seed=seed, dither=dither, step=-1.0, out=out, ws=ws, blocking=False)

    def decode():
        hq.hq_decode(out, n, out=y, ws=ws_dec, check=False)

    for _ in range(args.warmup):
        rate(); encode(); decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        rate()
        ev[i][1].record(stream)
        encode()
        ev[i][2].record(stream)
        decode()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rate_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]))
    enc_ms = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]))
    dec_ms = float(np.mean([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]))
    step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][3]) for i in range(K)]))
    st = hq.hq_status(ws)
    st2 = hq.hq_status(ws_dec)
    assert st == 0 and st2 == 0, (st, st2)

    hdr = hq.header_fields(out[:128].cpu().numpy())
    total_bytes = hdr["total_bytes"]
    input_bytes = 2 * n
    value = input_bytes / (step_ms * 1e-3) / 1e9
    # algorithmic bytes: encode reads the input and writes the stream; decode reads the stream and
    # writes bf16 values
    alg_step = 2 * (input_bytes + total_bytes)
    # dominant kernel: encode_kernel (timed alone) or decode_kernel (timed with its 1-lane header
    # check launch, which makes the decode figure slightly conservative)
    dec_alg = total_bytes + input_bytes
    enc_alg = input_bytes + total_bytes
    if dec_ms >= enc_ms:
        dom, dom_ms, dom_bytes = "decode_kernel", dec_ms, dec_alg
    else:
        dom, dom_ms, dom_bytes = "encode_kernel", enc_ms, enc_alg
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = profiled_traffic(profile_stem, dom)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {**cfg, "n_values": n, "stream_bytes": total_bytes,
                   "payload_bps": round(hdr["payload_bits"] / n, 5),
                   "total_bps": round(8 * total_bytes / n, 5),
                   "step": float(np.array([hdr["step_bits"]], dtype=np.uint32).view(np.float32)[0]),
                   "rice_k": hdr["k"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                     "alg_bytes_per_launch": dom_bytes, "launch_ms": round(dom_ms, 5)},
        "extra": {"rate_control_ms": round(rate_ms, 5), "encode_ms": round(enc_ms, 5),
                  "decode_ms": round(dec_ms, 5),
                  "encode_kernel_gbs": round(enc_alg / (enc_ms * 1e-3) / 1e9, 1),
                  "decode_kernel_gbs": round(dec_alg / (dec_ms * 1e-3) / 1e9, 1),
                  "step_alg_bytes": alg_step,
                  "step_hbm_gbs": round(alg_step / (step_ms * 1e-3) / 1e9, 1),
                  "step_hbm_frac": round(alg_step / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "host_wall_ms_per_step": round(wall / K * 1e3, 5)},
    }

    if not args.no_cpu_baseline or not args.no_parity:
        import oracle
        if not os.path.exists(os.path.join(ROOT, "oracle", "libhq_oracle.so")):
            oracle.build()
        t1 = time.perf_counter()
        s_orc, info_orc = oracle.encode(x_host, oracle.LATTICES[lat], tb, seed=seed, dither=dither)
        t2 = time.perf_counter()
        y_orc = oracle.decode(s_orc, n, out_dtype="bf16")
        t3 = time.perf_counter()
        cpu_gbs = input_bytes / (t3 - t1) / 1e9
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                      "sample": f"the whole workload ({n} values), one encode (with rate "
                                                f"control) + one bf16 decode, single host thread: "
                                                f"encode {t2 - t1:.2f} s, decode {t3 - t2:.2f} s"}
        if not args.no_parity:
            g = out[:total_bytes].cpu().numpy()
            same_stream = bool(g.size == s_orc.size and np.array_equal(g, s_orc))
            same_out = bool(np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), y_orc))
            result["extra"]["parity_stream_bytes_equal"] = same_stream
            result["extra"]["parity_decoded_equal"] = same_out
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
