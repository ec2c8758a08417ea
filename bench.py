"""Benchmark of the GRINQH decode-stage VMM on one MI355X.

One step = one decode-stage VMM of one linear layer at batch 1: precision
assignment from |x| and calibrated thresholds, active-row selection, bit-plane
streaming, reconstruction, dequantisation, fp32 accumulation and the split-K
reduction (the fused ``grinqh_decode_vmm`` launch).  Inputs are resident in
HBM before timing starts; every step reads a different copy of the layer
(planes, scales, zeros, x) so that the working set (>= 512 MB) cannot sit in
the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is the achieved bandwidth over algorithmic
bytes (sum_i b_i N_pad / 8 plane bytes + 4 N bytes of fp16 scale and zero per
active group + 2 K bytes of x) per step, in GB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROT_BYTES = 512 << 20

WORKLOADS = {
    # name: (K, N, config, matrix, P key, levels)
    "llama3-8b-gate-4096x14336-avg3": (4096, 14336, 2, 4, 3, "5"),
    "llama3-8b-gate-4096x14336-avg2": (4096, 14336, 2, 4, 2, "5"),
    "llama3-8b-gate-4096x14336-avg4": (4096, 14336, 2, 4, 4, "5"),
    "attn-proj-4096x4096-avg2": (4096, 4096, 1, 0, 2, "5"),
    "attn-proj-4096x4096-avg3": (4096, 4096, 1, 0, 3, "5"),
    "attn-proj-4096x4096-avg4": (4096, 4096, 1, 0, 4, "5"),
    "attn-proj-4096x4096-avg8": (4096, 4096, 1, 0, 8, "5"),
}
DEFAULT = "llama3-8b-gate-4096x14336-avg3"
SWEEP = ["attn-proj-4096x4096-avg2", "attn-proj-4096x4096-avg3", "attn-proj-4096x4096-avg4",
         "attn-proj-4096x4096-avg8", "llama3-8b-gate-4096x14336-avg2", "llama3-8b-gate-4096x14336-avg4"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _P(key, levels):
    import synthetic
    return (synthetic.P_LEVELS_5 if levels == "5" else synthetic.P_LEVELS_4)[key], \
        (synthetic.LEVELS_5 if levels == "5" else synthetic.LEVELS_4)


class Prepared:
    """A layer resident on the GPU in R rotated copies, thresholds calibrated on the GPU."""

    def __init__(self, name, mode="decode"):
        import torch
        import synthetic
        import decode_stage_gemv_amd as grq
        K, N, cfg, mat, pkey, lv = WORKLOADS[name]
        self.name, self.K, self.N = name, K, N
        self.P, self.levels = _P(pkey, lv)
        t0 = time.time()
        lay = synthetic.make_layer(K, N, config=cfg, matrix=mat, n_test=1)
        dev = torch.device("cuda:0")
        planes = grq.pack(torch.from_numpy(lay.codes).to(dev))
        scales = torch.from_numpy(lay.scales).to(dev)
        zeros = torch.from_numpy(lay.zeros).to(dev)
        calib = torch.from_numpy(lay.calib).to(dev)
        th_dev = grq.calibrate(calib, self.P)
        self.thresholds = [float(v) for v in th_dev.cpu().numpy()]
        per_copy = planes.numel() + 2 * scales.numel() * 2 + 2 * K
        self.R = max(1, -(-ROT_BYTES // per_copy))
        xs = synthetic.make_activations(K, self.R, config=cfg, matrix=mat)
        self.copies = []
        for r in range(self.R):
            self.copies.append((planes.clone(), scales.clone(), zeros.clone(),
                                torch.from_numpy(xs[r]).to(dev)))
        del planes
        self.ws = grq.make_workspace(K, N)
        self.y = torch.empty(N, dtype=torch.float32, device=dev)
        self.mode = mode
        self.ybufs = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(2)]
        # algorithmic bytes of each copy's step, from the GPU's own assignment
        self.bytes = []
        self.avg_bits = []
        Np = (N + 31) // 32 * 32
        G = (K + 127) // 128
        for (_, _, _, x) in self.copies:
            bits, _, _ = grq.assign_bits(x, self.thresholds, self.levels)
            b = bits.to(torch.int64)
            pad = torch.zeros(G * 128 - K, dtype=torch.int64, device=dev)
            active_groups = int((torch.cat([b, pad]).view(G, 128).amax(dim=1) > 0).sum().item())
            self.bytes.append(int(b.sum().item()) * Np // 8 + 4 * N * active_groups + 2 * K)
            self.avg_bits.append(float(b.sum().item()) / K)
        self.host_x = xs
        self.host_layer = lay
        torch.cuda.synchronize()
        log(f"prepared {name}: R={self.R} copies, avg bits {np.mean(self.avg_bits):.3f}, "
            f"{np.mean(self.bytes) / 1e6:.2f} MB/step, setup {time.time() - t0:.1f}s")

    def step(self, k):
        import decode_stage_gemv_amd as grq
        planes, scales, zeros, x = self.copies[k % self.R]
        if self.mode == "accumulate":
            # decode-loop ping-pong: add into one buffer, clear the other for the next step
            grq.decode_vmm_accumulate(planes, scales, zeros, x, self.K, self.N, self.thresholds,
                                      self.levels, self.ybufs[k % 2], self.ybufs[(k + 1) % 2])
        else:
            grq.decode_vmm(planes, scales, zeros, x, self.K, self.N, self.thresholds, self.levels,
                           self.ws, out=self.y)

    def run(self, steps, warmup, graph=True):
        """Time `steps` back-to-back steps; returns (ms per step, bytes per step).

        With graph=True the steps are captured once into a HIP graph and the
        timed region is one replay (no host launch overhead between steps).
        Events are recorded on the stream the kernels run on.
        """
        import torch
        for k in range(warmup):
            self.step(k)
        torch.cuda.synchronize()
        if graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for k in range(steps):
                        self.step(k)
                g.replay()                      # warm replay
                s.synchronize()
                start = torch.cuda.Event(enable_timing=True)
                stop = torch.cuda.Event(enable_timing=True)
                start.record(s)
                g.replay()
                stop.record(s)
                s.synchronize()
            ms = start.elapsed_time(stop) / steps
        else:
            stream = torch.cuda.current_stream()
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for k in range(steps):
                self.step(k)
            stop.record(stream)
            torch.cuda.synchronize()
            ms = start.elapsed_time(stop) / steps
        step_bytes = float(np.mean([self.bytes[k % self.R] for k in range(steps)]))
        return ms, step_bytes


def copy_probe(nbytes=512 << 20, reps=20):
    """A plain device-to-device copy of known size: reads nbytes, writes nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"copy_probe": {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms,
                                     "GB_s_read_plus_write": gbs}}), flush=True)


def cpu_baseline(prep, budget_s=15.0):
    """The oracle's decode step (assign, select, fp64 VMM) on the host cores."""
    import oracle
    lay = prep.host_layer
    th = np.asarray(prep.thresholds, np.float32)
    n, t_total, bytes_total = 0, 0.0, 0.0
    while t_total < budget_s and n < 50:
        x = prep.host_x[n % prep.R]
        t0 = time.perf_counter()
        oracle.decode_step(lay.codes, lay.scales, lay.zeros, x, th, prep.levels)
        t_total += time.perf_counter() - t0
        bytes_total += prep.bytes[n % prep.R]
        n += 1
    cores = len(os.sched_getaffinity(0))
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_vmm": t_total / n * 1e6,
            "sample": f"{n} full decode steps of {prep.name} (assign + select + fp64 VMM), "
                      f"{t_total:.1f}s of host time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--sweep", action="store_true", help="also time the bit-width sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step from the host")
    ap.add_argument("--mode", choices=["decode", "accumulate"], default="decode",
                    help="decode: grinqh_decode_vmm (deterministic split-K); "
                         "accumulate: grinqh_decode_vmm_accumulate (fp32 atomics, ping-pong outputs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 512 MiB device copy (reference for bandwidth and counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode VMM path here is single-GPU "
              "(multi-GPU sharding is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    prep = Prepared(args.workload, args.mode)
    ms, step_bytes = prep.run(args.steps, args.warmup, graph=not args.no_graph)
    if args.no_graph:
        log("host-launched steps (no graph): includes Python and ctypes launch overhead")
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"{args.workload}: {ms * 1e3:.2f} us/VMM, {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")

    sweep = {}
    if args.sweep:
        for name in SWEEP:
            p = Prepared(name, args.mode)
            m, b = p.run(args.steps, args.warmup)
            sweep[name] = {"us_per_vmm": m * 1e3, "GB_s": b / (m * 1e-3) / 1e9,
                           "frac_of_peak": b / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "avg_bits": float(np.mean(p.avg_bits)), "bytes": b}
            log(f"{name}: {m * 1e3:.2f} us/VMM, {sweep[name]['GB_s']:.1f} GB/s")
            del p
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(prep)
    out = {
        "metric": "µs per VMM and achieved HBM GB/s (% of peak) at avg 2/3/4/8 bits, batch 1",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_vmm": ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8 planes, fp16 x/scale/zero, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, RTN 8-bit, log-normal x with 1% outlier channels)",
        "config": {"workload": args.workload, "entry_point": "grinqh_decode_vmm" if args.mode == "decode" else "grinqh_decode_vmm_accumulate", "K": prep.K, "N": prep.N,
                   "avg_bits": float(np.mean(prep.avg_bits)), "bytes_per_step": step_bytes,
                   "rotated_copies": prep.R, "thresholds": prep.thresholds, "levels": list(prep.levels)},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "cpu_baseline": cpu,
    }
    if sweep:
        out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
