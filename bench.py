"""Benchmark of the GRINQH decode-stage VMM on one MI355X.

One step = one decode-stage VMM of one linear layer at batch 1: precision
assignment from |x| and calibrated thresholds, active-row selection, bit-plane
streaming, reconstruction, dequantisation and fp32 accumulation, in one
launch.  The default entry point is ``grinqh_decode_vmm_accumulate`` used the
way a decode loop uses it: each step adds x W into an output buffer that the
previous step zeroed, and zeroes the other one for the next step (ping-pong),
so every step produces a complete y = x W.  ``--mode decode`` times
``grinqh_decode_vmm`` (deterministic split-K reduction) instead, and
``--mode list`` the two-launch form (``grinqh_assign_bits`` then
``grinqh_vmm`` over the explicit active list); the default run reports all
three.

Inputs are resident in HBM before timing starts; every step reads a different
copy of the layer (planes, scales, zeros, x) so that the working set (>= 512
MB) cannot sit in the 256 MB Infinity Cache.  Steps are captured once in a HIP
graph and replayed; the time per step comes from HIP events recorded on the
stream the kernels run on, around one replay.

Prints one JSON line.  ``value`` is the achieved bandwidth over algorithmic
bytes (sum_i b_i N_pad / 8 plane bytes + 4 N bytes of fp16 scale and zero per
active group + 2 K bytes of x) per step, in GB/s.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
ROT_BYTES = 512 << 20
MAX_COPIES = 128     # rotated copies of one layer at most (4096 x 4096 at avg 2 needs 114)

# name: (K, N, config, matrix, P key, level set); level sets "b6" and "b4"
# belong to stores of 6-bit and 4-bit codes (the others to 8-bit codes)
WORKLOADS = {
    "llama3-8b-gate-4096x14336-avg3": (4096, 14336, 2, 4, 3, "5"),
    "llama3-8b-gate-4096x14336-avg2": (4096, 14336, 2, 4, 2, "5"),
    "llama3-8b-gate-4096x14336-avg4": (4096, 14336, 2, 4, 4, "5"),
    "llama3-8b-gate-4096x14336-avg8": (4096, 14336, 2, 4, 8, "5"),
    "llama3-8b-down-14336x4096-avg3": (14336, 4096, 2, 6, 3, "5"),
    "attn-proj-4096x4096-avg2": (4096, 4096, 1, 0, 2, "5"),
    "attn-proj-4096x4096-avg3": (4096, 4096, 1, 0, 3, "5"),
    "attn-proj-4096x4096-avg4": (4096, 4096, 1, 0, 4, "5"),
    "attn-proj-4096x4096-avg8": (4096, 4096, 1, 0, 8, "5"),
}
for _b in ("0.5", "1", "2", "3", "4", "6", "8"):
    WORKLOADS[f"llama3-70b-gate-8192x28672-avg{_b}"] = (8192, 28672, 4, 0, float(_b), "4")
    WORKLOADS[f"llama3-70b-down-28672x8192-avg{_b}"] = (28672, 8192, 4, 1, float(_b), "4")
# smaller maximum widths: effective 3 and 4 bits under b_max = 6 and an
# effective 2 and 3 bits under b_max = 4 (Table 7 runs 4-of-6 and 3-of-4)
for _b in (3, 4):
    WORKLOADS[f"llama3-8b-gate-4096x14336-bmax6-avg{_b}"] = (4096, 14336, 2, 4, _b, "b6")
    WORKLOADS[f"llama3-70b-gate-8192x28672-bmax6-avg{_b}"] = (8192, 28672, 4, 0, _b, "b6")
for _b in (2, 3):
    WORKLOADS[f"llama3-8b-gate-4096x14336-bmax4-avg{_b}"] = (4096, 14336, 2, 4, _b, "b4")
    WORKLOADS[f"llama3-70b-gate-8192x28672-bmax4-avg{_b}"] = (8192, 28672, 4, 0, _b, "b4")
DEFAULT = "llama3-8b-gate-4096x14336-avg3"
SWEEP = ([f"attn-proj-4096x4096-avg{b}" for b in (2, 3, 4, 8)]
         + [f"llama3-8b-gate-4096x14336-avg{b}" for b in (2, 3, 4, 8)]
         + [f"llama3-70b-gate-8192x28672-avg{b}" for b in ("0.5", "1", "2", "3", "4", "6", "8")])
SWEEP_BMAX = ([f"llama3-8b-gate-4096x14336-bmax6-avg{b}" for b in (3, 4)]
              + [f"llama3-8b-gate-4096x14336-bmax4-avg{b}" for b in (2, 3)]
              + [f"llama3-70b-gate-8192x28672-bmax6-avg{b}" for b in (3, 4)]
              + [f"llama3-70b-gate-8192x28672-bmax4-avg{b}" for b in (2, 3)])
# workloads whose layer is also timed at two other widths for the marginal bandwidth
MARGINAL_PAIRS = {"llama3-8b-gate-4096x14336-avg3": ("llama3-8b-gate-4096x14336-avg2",
                                                     "llama3-8b-gate-4096x14336-avg8")}
ENTRY = {"accumulate": "grinqh_decode_vmm_accumulate", "decode": "grinqh_decode_vmm",
         "list": "grinqh_assign_bits+grinqh_vmm"}
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "vmm_traffic_*.md")
KERNEL_SOURCES = ("decode_stage_gemv_amd/csrc/vmm.hip", "decode_stage_gemv_amd/csrc/bitplane.hpp",
                  "decode_stage_gemv_amd/csrc/common.hpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _P(key, levels):
    import synthetic
    table, lv = {"5": (synthetic.P_LEVELS_5, synthetic.LEVELS_5),
                 "4": (synthetic.P_LEVELS_4, synthetic.LEVELS_4),
                 "b6": (synthetic.P_BMAX6, synthetic.LEVELS_BMAX6),
                 "b4": (synthetic.P_BMAX4, synthetic.LEVELS_BMAX4)}[levels]
    return table[key], lv


def bmax_of(levels):
    """Code width of the store a level set belongs to."""
    return {"b6": 6, "b4": 4}.get(levels, 8)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, mode):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    The summary states the kernel-source hash it was taken with; a summary of
    older kernel sources does not count."""
    want = kernel_source_hash()
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        text = open(path).read()
        m_w = re.search(r"^workload:\s*(\S+)", text, re.M)
        m_m = re.search(r"^entry point:\s*(\S+)", text, re.M)
        m_h = re.search(r"^kernel sources sha256:\s*([0-9a-f]{64})", text, re.M)
        m_t = re.search(r"^traffic bytes per launch:\s*([0-9.]+)", text, re.M)
        if not (m_w and m_m and m_h and m_t):
            continue
        if m_w.group(1) == workload and m_m.group(1) == ENTRY[mode] and m_h.group(1) == want:
            return float(m_t.group(1))
    return None


class Layer:
    """One synthetic layer packed on the GPU, in R rotated copies.

    Copies are added on demand (`ensure`): a workload needs enough copies
    that one cycle through them reads at least ROT_BYTES of data (the bytes
    its steps actually read, not the size of the store), so no copy can
    still sit in the 256 MB Infinity Cache when its turn comes again."""

    def __init__(self, K, N, cfg, mat, b_max=8):
        import torch
        import synthetic
        import decode_stage_gemv_amd as grq
        t0 = time.time()
        self.K, self.N, self.cfg, self.mat, self.b_max = K, N, cfg, mat, b_max
        lay = synthetic.make_layer(K, N, config=cfg, matrix=mat, n_test=1, b_max=b_max)
        dev = torch.device("cuda:0")
        planes = grq.pack(torch.from_numpy(lay.codes).to(dev), b_max=b_max)
        scales = torch.from_numpy(lay.scales).to(dev)
        zeros = torch.from_numpy(lay.zeros).to(dev)
        self.calib = torch.from_numpy(lay.calib).to(dev)
        # one activation vector per possible copy, drawn once (copy r uses row r)
        self.xs_host = synthetic.make_activations(K, MAX_COPIES, config=cfg, matrix=mat)
        self.copies = [(planes, scales, zeros, torch.from_numpy(self.xs_host[0]).to(dev))]
        self.host = lay
        self.np_cols = int(grq.lib().grinqh_planes_bytes(1, N, 8))
        torch.cuda.synchronize()
        log(f"layer {K}x{N} (b_max {b_max}): setup {time.time() - t0:.1f}s")

    @property
    def R(self):
        return len(self.copies)

    def ensure(self, R):
        """Grow to at least R copies (planes, scales, zeros, and a fresh x each)."""
        import torch
        if R <= self.R:
            return
        if R > MAX_COPIES:
            raise ValueError(f"{R} rotated copies requested, at most {MAX_COPIES}")
        dev = torch.device("cuda:0")
        planes, scales, zeros, _ = self.copies[0]
        for r in range(self.R, R):
            self.copies.append((planes.clone(), scales.clone(), zeros.clone(),
                                torch.from_numpy(self.xs_host[r]).to(dev)))
        torch.cuda.synchronize()
        log(f"layer {self.K}x{self.N}: {self.R} rotated copies")


def rotation_copies(bytes_per_step):
    """Copies needed so that one cycle reads at least ROT_BYTES (twice the
    256 MB Infinity Cache) of the bytes the steps actually read."""
    return max(2, -(-ROT_BYTES // max(int(bytes_per_step), 1)))


_SCRUB = {}


def scrub_init():
    """Allocate and fill the scrub buffer once, long before any timed region
    (the fill leaves dirty lines in the Infinity Cache; their write-back must
    not land inside a measurement)."""
    import torch
    if "buf" not in _SCRUB:
        _SCRUB["buf"] = torch.ones(ROT_BYTES // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()


def scrub_cache():
    """Read 512 MiB (twice the 256 MB Infinity Cache) so that nothing a timed
    region reads is still cached from an earlier pass over the same copies.
    A read, not a write: evicting clean lines costs nothing later, while
    written lines would be written back during the next timed region."""
    scrub_init()
    _SCRUB["sum"] = _SCRUB["buf"].sum()


class Prepared:
    """A workload: a layer, thresholds calibrated on the GPU for its level mix."""

    def __init__(self, name, mode="accumulate", layer=None):
        import torch
        import decode_stage_gemv_amd as grq
        K, N, cfg, mat, pkey, lv = WORKLOADS[name]
        self.name, self.K, self.N, self.mode = name, K, N, mode
        self.P, self.levels = _P(pkey, lv)
        self.b_max = bmax_of(lv)
        self.layer = layer if layer is not None else Layer(K, N, cfg, mat, self.b_max)
        assert self.layer.b_max == self.b_max
        self.thresholds = [float(v) for v in grq.calibrate(self.layer.calib, self.P).cpu().numpy()]
        # size the rotation by the bytes a step of this workload reads
        b0, _ = algorithmic_bytes(self.layer.copies[0][3], K, N, self.thresholds, self.levels, self.layer.np_cols)
        self.layer.ensure(rotation_copies(0.9 * b0))
        self.R = self.layer.R
        dev = torch.device("cuda:0")
        self.ws = grq.make_workspace(K, N)
        self.y = torch.empty(N, dtype=torch.float32, device=dev)
        # the two-launch form: assignment buffers
        self.bits = torch.empty(K, dtype=torch.uint8, device=dev)
        self.idx = torch.empty(K, dtype=torch.int32, device=dev)
        self.nact = torch.empty(1, dtype=torch.int32, device=dev)
        self.ybufs = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(2)]
        # algorithmic bytes of each copy's step, from the GPU's own assignment
        self.bytes, self.avg_bits = [], []
        for (_, _, _, x) in self.layer.copies:
            nb, avg = algorithmic_bytes(x, K, N, self.thresholds, self.levels, self.layer.np_cols)
            self.bytes.append(nb)
            self.avg_bits.append(avg)
        torch.cuda.synchronize()
        self.touched_per_cycle = float(np.sum(self.bytes))
        log(f"prepared {name} ({ENTRY[mode]}): avg bits {np.mean(self.avg_bits):.3f}, "
            f"{np.mean(self.bytes) / 1e6:.2f} MB/step, {self.R} copies, "
            f"{self.touched_per_cycle / 1e6:.0f} MB read per rotation cycle")

    def step(self, k):
        import decode_stage_gemv_amd as grq
        planes, scales, zeros, x = self.layer.copies[k % self.R]
        if self.mode == "accumulate":
            # decode-loop ping-pong: add into one buffer, clear the other for the next step
            grq.decode_vmm_accumulate(planes, scales, zeros, x, self.K, self.N, self.thresholds,
                                      self.levels, self.ybufs[k % 2], self.ybufs[(k + 1) % 2],
                                      b_max=self.b_max)
        elif self.mode == "decode":
            grq.decode_vmm(planes, scales, zeros, x, self.K, self.N, self.thresholds, self.levels,
                           self.ws, out=self.y, b_max=self.b_max)
        else:
            # assignment and compaction, then the VMM over the explicit list
            grq.assign_bits(x, self.thresholds, self.levels, self.bits, self.idx, self.nact)
            grq.vmm(planes, scales, zeros, x, self.bits, self.idx, self.nact, self.K, self.N, self.ws,
                    out=self.y, b_max=self.b_max)

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
                # The cache scrub (about 100 us of device work) runs first on
                # the same stream, and the start event and the replay are
                # queued behind it: the start is stamped when the scrub
                # ends, with the replay already queued, so the timed region
                # holds the K steps and no wait for the host's submission.
                scrub_cache()
                start.record(s)
                g.replay()
                stop.record(s)
                s.synchronize()
            ms = start.elapsed_time(stop) / steps
        else:
            stream = torch.cuda.current_stream()
            scrub_cache()
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


def algorithmic_bytes(x, K, N, thresholds, levels, np_cols):
    """Bytes one VMM must read for activation x: the planes of the widths the
    GPU's own assignment gives, a scale and a zero per column of every group
    with an active row, and x.  Also returns the average width."""
    import torch
    import decode_stage_gemv_amd as grq
    bits, _, _ = grq.assign_bits(x, thresholds, levels)
    b = bits.to(torch.int64)
    G = (K + 127) // 128
    pad = torch.zeros(G * 128 - K, dtype=torch.int64, device=b.device)
    active_groups = int((torch.cat([b, pad]).view(G, 128).amax(dim=1) > 0).sum().item())
    total = int(b.sum().item())
    return total * np_cols // 8 + 4 * N * active_groups + 2 * K, total / K


class Stack:
    """One token's pass through the 36-layer Qwen3-8B linear stack: 252
    matrices (q, k, v, o, gate, up, down per layer) packed at 8 bits and
    resident together (6.95 GB of planes), calibrated for an average of 3
    bits over levels {0,2,3,4,8}.

    fused=False: one VMM per matrix, each with its own activation and
    thresholds (252 launches per token).  grouped=True: the same per-matrix
    VMMs, with the matrices that sit at one position of the layer (q, k and
    v; gate and up) issued as one grouped launch (144 launches per token;
    every matrix keeps its own store, activation and thresholds, and the
    launches keep the layer order).  fused=True: the matrices that read
    the same input in the model are packed side by side by columns, q|k|v
    and gate|up, and share one activation and one set of thresholds (the
    thresholds depend only on the input's calibration vectors), so a layer
    takes 4 VMMs (144 launches per token); the weights are the same draws.

    keep_cols > 0 keeps, per VMM, that many seeded columns (plus the first
    and last) of the codes, scales and zeros on the host for parity checks."""

    GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def __init__(self, keep_cols=0, fused=False, progress=True, grouped=False):
        import torch
        import synthetic
        import decode_stage_gemv_amd as grq
        t0 = time.time()
        dev = torch.device("cuda:0")
        if fused and grouped:
            raise ValueError("the fused stack has no separate matrices to group")
        self.fused = fused
        self.P, self.levels = synthetic.P_LEVELS_5[3], synthetic.LEVELS_5
        listing = synthetic.qwen3_stack()
        # launch groups: positions in self.mats issued together
        self.groups = None
        if grouped:
            gid = {name: g for g, grp in enumerate(self.GROUPS) for name in grp}
            self.groups = []
            for j, (_, layer, name, _, _) in enumerate(listing):
                if self.groups and self.groups[-1][0] == (layer, gid[name]):
                    self.groups[-1][1].append(j)
                else:
                    self.groups.append(((layer, gid[name]), [j]))
            self.groups = [g for _, g in self.groups]
        if fused:
            by = {(layer, name): (idx, K, N) for idx, layer, name, K, N in listing}
            units = [[(by[(layer, n)][0], n) + by[(layer, n)][1:] for n in grp]
                     for layer in range(synthetic.QWEN3_8B_LAYERS) for grp in self.GROUPS]
        else:
            units = [[(idx, name, K, N)] for idx, _, name, K, N in listing]
        self.mats = []
        for u, unit in enumerate(units):
            idx0, K = unit[0][0], unit[0][2]
            parts = [synthetic.device_weights(K, N, synthetic.STACK_CONFIG, idx, dev) for idx, _, _, N in unit]
            codes, scales, zeros = (torch.cat([p[i] for p in parts], dim=1) if len(parts) > 1 else parts[0][i]
                                    for i in range(3))
            del parts
            N = codes.shape[1]
            planes = grq.pack(codes)
            m = {"idx": idx0, "name": "|".join(n for _, n, _, _ in unit), "K": K, "N": N,
                 "planes": planes, "scales": scales, "zeros": zeros}
            if keep_cols:
                r = np.random.default_rng([synthetic.STACK_CONFIG, idx0, 9 + len(unit)])
                cols = np.unique(np.concatenate([r.choice(N, keep_cols, replace=False), [0, N - 1]]))
                ct = torch.from_numpy(cols).to(dev)
                m["cols"] = cols
                m["host"] = tuple(t.index_select(1, ct).cpu().numpy() for t in (codes, scales, zeros))
            del codes
            calib = torch.from_numpy(synthetic.make_calibration(K, synthetic.STACK_CONFIG, idx0)).to(dev)
            m["thresholds"] = [float(v) for v in grq.calibrate(calib, self.P).cpu().numpy()]
            m["x_host"] = synthetic.make_activations(K, 1, synthetic.STACK_CONFIG, idx0)[0]
            m["x"] = torch.from_numpy(m["x_host"]).to(dev)
            self.mats.append(m)
            if progress and u % 36 == 35:
                log(f"stack: {u + 1} of {len(units)} VMMs packed ({time.time() - t0:.1f}s)")
        self.ys = [[torch.zeros(m["N"], dtype=torch.float32, device=dev) for m in self.mats] for _ in range(2)]
        self.plane_bytes = sum(m["planes"].numel() for m in self.mats)
        torch.cuda.synchronize()
        log(f"stack{' (fused projections)' if fused else (' (grouped launches)' if grouped else '')}: "
            f"{len(self.mats)} VMMs in {self.launches} launches per token, "
            f"{self.plane_bytes / 1e9:.2f} GB of planes resident, setup {time.time() - t0:.1f}s")

    @property
    def launches(self):
        return len(self.groups) if self.groups is not None else len(self.mats)

    def token(self, t):
        """One token's VMMs (decode-loop form: add into output set t % 2,
        clear set (t + 1) % 2 for the next token)."""
        import decode_stage_gemv_amd as grq
        ya, yb = self.ys[t % 2], self.ys[(t + 1) % 2]
        if self.groups is not None:
            for grp in self.groups:
                ms = [self.mats[j] for j in grp]
                grq.decode_vmm_accumulate_group(
                    [(m["planes"], m["scales"], m["zeros"], m["x"], m["N"], m["thresholds"], self.levels,
                      ya[j], yb[j]) for j, m in zip(grp, ms)], ms[0]["K"])
            return
        for j, m in enumerate(self.mats):
            grq.decode_vmm_accumulate(m["planes"], m["scales"], m["zeros"], m["x"], m["K"], m["N"],
                                      m["thresholds"], self.levels, ya[j], yb[j])

    def bytes_per_token(self):
        import decode_stage_gemv_amd as grq
        total, bits = 0, 0.0
        for m in self.mats:
            np_cols = int(grq.lib().grinqh_planes_bytes(1, m["N"], 8))
            b, avg = algorithmic_bytes(m["x"], m["K"], m["N"], m["thresholds"], self.levels, np_cols)
            total += b
            bits += avg * m["K"] * m["N"]
        return total, bits / sum(m["K"] * m["N"] for m in self.mats)


def stack_bench(fused=False, tokens=4, warmup=2, grouped=False):
    """Time per token of the Qwen3-8B stack: `tokens` passes captured in one
    HIP graph, timed over one replay with events on the capture stream."""
    import torch
    st = Stack(fused=fused, grouped=grouped)
    nbytes, avg_bits = st.bytes_per_token()
    for t in range(warmup):
        st.token(t)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for t in range(tokens):
                st.token(t)
        g.replay()
        s.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(s)
        g.replay()
        stop.record(s)
        s.synchronize()
    us = start.elapsed_time(stop) * 1e3 / tokens
    gbs = nbytes / (us * 1e-6) / 1e9
    n = len(st.mats)
    form = ("fused projections: q|k|v and gate|up packed side by side, sharing x and thresholds" if fused else
            ("one VMM per matrix, fresh x per VMM; q,k,v and gate,up of a layer in one grouped launch each"
             if grouped else "one VMM per matrix, fresh x per VMM"))
    out = {"model": "qwen3-8b linear stack (36 layers x q,k,v,o,gate,up,down)", "form": form,
           "vmms_per_token": n, "launches_per_token": st.launches,
           "entry_point": "grinqh_decode_vmm_accumulate_group" if grouped else ENTRY["accumulate"],
           "avg_bits": avg_bits,
           "plane_bytes_resident": st.plane_bytes, "bytes_per_token": nbytes, "us_per_token": us,
           "us_per_vmm": us / n, "GB_s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "tokens_timed": tokens}
    log(f"stack{' fused' if fused else (' grouped' if grouped else '')}: {us:.1f} us per token "
        f"({us / n:.2f} us per VMM, {n} VMMs, {st.launches} launches), "
        f"{nbytes / 1e9:.3f} GB per token, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak), "
        f"avg bits {avg_bits:.3f}")
    del st, g
    torch.cuda.empty_cache()
    return out


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak


def _graph_time(fn, steps, warmup):
    """Microseconds per call of fn over one HIP-graph replay of `steps` calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                fn()
        g.replay()
        s.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        scrub_cache()   # queued ahead of the start event, as in Prepared.run
        start.record(s)
        g.replay()
        stop.record(s)
        s.synchronize()
    return start.elapsed_time(stop) * 1e3 / steps


def prefill_bench(layer, M, steps=20, warmup=3, dense_reference=True):
    """Dense prefill of M tokens through grinqh_prefill (every row at b_max).

    Reports TFLOP/s over 2 M K N flops against the dense fp16 matrix-core peak.
    For context it also times torch.matmul on the same weights dequantised to
    a dense fp16 matrix (a plain library GEMM that reads 2 bytes per weight;
    not part of this library's path)."""
    import torch
    import synthetic
    import decode_stage_gemv_amd as grq
    K, N = layer.K, layer.N
    X = torch.from_numpy(synthetic.make_activations(K, M, config=layer.cfg, matrix=layer.mat)).cuda()
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    state = {"k": 0}

    def step():
        planes, scales, zeros, _ = layer.copies[state["k"] % layer.R]
        state["k"] += 1
        grq.prefill(planes, scales, zeros, X, K, N, out=Y, b_max=layer.b_max)

    us = _graph_time(step, steps, warmup)
    flops = 2.0 * M * K * N
    out = {"tokens": M, "K": K, "N": N, "b_max": layer.b_max, "us": us, "TFLOP_s": flops / (us * 1e-6) / 1e12}
    out["frac_of_mfma_f16_peak"] = out["TFLOP_s"] / MFMA_F16_PEAK_TFLOPS
    # the two-launch path: unpack the store once into fp16 fragments, then a
    # dense GEMM; both timed, the unpack's cost is amortised over M tokens
    dense = grq.unpack_dense(layer.copies[0][0], layer.copies[0][1], layer.copies[0][2], K, N, b_max=layer.b_max)

    def unpack_step():
        planes, scales, zeros, _ = layer.copies[state["k"] % layer.R]
        state["k"] += 1
        grq.unpack_dense(planes, scales, zeros, K, N, out=dense, b_max=layer.b_max)

    us_u = _graph_time(unpack_step, steps, warmup)
    us_g = _graph_time(lambda: grq.dense_gemm(X, dense, K, N, out=Y), steps, warmup)
    out["unpacked"] = {"unpack_us": us_u, "gemm_us": us_g, "total_us": us_u + us_g,
                       "gemm_TFLOP_s": flops / (us_g * 1e-6) / 1e12,
                       "TFLOP_s": flops / ((us_u + us_g) * 1e-6) / 1e12}
    del dense
    log(f"unpacked prefill: unpack {us_u:.1f} us + dense GEMM {us_g:.1f} us "
        f"({out['unpacked']['gemm_TFLOP_s']:.0f} TFLOP/s GEMM alone)")
    if dense_reference:
        lay = layer.host
        g = np.arange(K) // 128
        W = torch.from_numpy(lay.codes).cuda().to(torch.float32)
        W.mul_(torch.from_numpy(lay.scales).cuda().to(torch.float32)[g]).add_(
            torch.from_numpy(lay.zeros).cuda().to(torch.float32)[g])
        W16 = W.to(torch.float16)
        del W
        Yd = torch.empty((M, N), dtype=torch.float16, device="cuda")
        us_d = _graph_time(lambda: torch.matmul(X, W16, out=Yd), steps, warmup)
        out["dense_fp16_matmul_us"] = us_d
        out["dense_fp16_matmul_TFLOP_s"] = flops / (us_d * 1e-6) / 1e12
        del W16, Yd
    log(f"prefill {M}x{K}x{N} (b_max {layer.b_max}): {us:.1f} us, {out['TFLOP_s']:.0f} TFLOP/s "
        f"({out['frac_of_mfma_f16_peak']:.1%} of fp16 MFMA peak)"
        + (f"; dense fp16 torch.matmul {out['dense_fp16_matmul_us']:.1f} us" if dense_reference else ""))
    return out


def lut_bench(name, steps=100, warmup=10):
    """grinqh_decode_vmm_lut on the workload's shape with nested synthetic
    tables (one per output column and width), decode-loop ping-pong outputs,
    rotated copies of planes, tables and x so the working set exceeds the
    Infinity Cache.  Algorithmic bytes per step: the planes the rows' widths
    select, the tables of the levels in use (N 2^b fp16 entries per width)
    and x."""
    import torch
    import synthetic
    import decode_stage_gemv_amd as grq
    K, N, cfg, mat, pkey, lv = WORKLOADS[name]
    P, levels = _P(pkey, lv)
    b_max = bmax_of(lv)
    t_setup = time.time()
    codes, tables = synthetic.make_lut_weights(K, N, config=cfg, matrix=mat, b_max=b_max)
    dev = torch.device("cuda:0")
    planes = grq.pack(torch.from_numpy(codes).to(dev), b_max=b_max)
    lut = torch.from_numpy(synthetic.lut_flat(tables, N, b_max)).to(dev)
    calib = torch.from_numpy(synthetic.make_calibration(K, config=cfg, matrix=mat)).to(dev)
    th = [float(v) for v in grq.calibrate(calib, P).cpu().numpy()]
    xs = synthetic.make_activations(K, MAX_COPIES, config=cfg, matrix=mat)
    used = sorted(set(int(v) for v in levels if v > 0))
    lut_bytes = sum(N * (1 << b) * 2 for b in used)
    np_cols = int(grq.lib().grinqh_planes_bytes(1, N, 8))

    def nbytes(x):
        bits, _, _ = grq.assign_bits(x, th, levels)
        return int(bits.to(torch.int64).sum().item()) * np_cols // 8 + lut_bytes + 2 * K

    # rotation sized by the bytes a step reads (planes of its widths, tables, x)
    R = rotation_copies(0.9 * nbytes(torch.from_numpy(xs[0]).to(dev)))
    copies = [(planes if r == 0 else planes.clone(), lut if r == 0 else lut.clone(),
               torch.from_numpy(xs[r]).to(dev)) for r in range(R)]
    ybufs = [torch.zeros(N, dtype=torch.float32, device=dev) for _ in range(2)]
    step_bytes = [nbytes(x) for (_, _, x) in copies]
    state = {"k": 0}

    def step():
        k = state["k"]
        state["k"] += 1
        pl, lt, x = copies[k % R]
        grq.decode_vmm_lut(pl, lt, x, K, N, th, levels, ybufs[k % 2], ybufs[(k + 1) % 2], b_max=b_max)

    log(f"lut layer {K}x{N} (b_max {b_max}): R={R} copies ({sum(step_bytes) / 1e6:.0f} MB read per cycle), "
        f"setup {time.time() - t_setup:.1f}s")
    us = _graph_time(step, steps, warmup)
    b = float(np.mean([step_bytes[k % R] for k in range(steps)]))
    out = {"workload": name, "entry_point": "grinqh_decode_vmm_lut", "us_per_vmm": us,
           "GB_s": b / (us * 1e-6) / 1e9, "bytes_per_step": b, "table_bytes_per_step": lut_bytes,
           "rotated_copies": R, "touched_bytes_per_cycle": float(sum(step_bytes))}
    out["frac_of_peak"] = out["GB_s"] / HBM_PEAK_GBS
    log(f"{name} grinqh_decode_vmm_lut: {us:.2f} us/VMM, {out['GB_s']:.1f} GB/s ({out['frac_of_peak']:.1%})")
    return out


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
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms, "GB_s_read_plus_write": gbs,
            "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}


def cpu_baseline(prep, budget_s=15.0):
    """The oracle's decode step (assign, select, fp64 VMM) on the host cores,
    over whole steps of the same workload until about budget_s of host time."""
    import oracle
    lay = prep.layer.host
    th = np.asarray(prep.thresholds, np.float32)
    n, t_total, bytes_total = 0, 0.0, 0.0
    while t_total < budget_s and n < 200:
        x = prep.layer.xs_host[n % prep.R]
        t0 = time.perf_counter()
        oracle.decode_step(lay.codes, lay.scales, lay.zeros, x, th, prep.levels, b_max=prep.b_max)
        t_total += time.perf_counter() - t0
        bytes_total += prep.bytes[n % prep.R]
        n += 1
    cores = len(os.sched_getaffinity(0))
    try:                      # threads NumPy's BLAS ran the fp64 products on
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = min(cores, max(blas)) if blas else cores
    except ImportError:
        threads = cores
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_vmm": t_total / n * 1e6,
            "sample": f"{n} whole decode steps of {prep.name} (assign + select + fp64 VMM, "
                      f"numpy), {t_total:.1f}s of host time"}


def linear_fit(points):
    """Least squares us = a + bytes / BW over (bytes, us) points."""
    b = np.array([p[0] for p in points], np.float64)
    t = np.array([p[1] for p in points], np.float64)
    A = np.stack([np.ones_like(b), b], axis=1)
    (a, slope), *_ = np.linalg.lstsq(A, t, rcond=None)
    pred = a + slope * b
    r2 = 1.0 - float(np.sum((t - pred) ** 2)) / max(float(np.sum((t - t.mean()) ** 2)), 1e-30)
    return {"intercept_us": float(a), "bw_eff_GB_s": float(1e-3 / slope) if slope > 0 else None, "r2": r2}


TIMELINE_PHASES = {
    "accumulate": [(0, "start"), (1, "widths known"), (2, "buckets counted"), (3, "record tables written"),
                   (4, "first three records issued"), (5, "waves reduced"), (6, "atomics issued"),
                   (7, "atomics acknowledged")],
    "decode": [(0, "start"), (1, "widths known"), (2, "buckets counted"), (3, "record tables written"),
               (4, "first three records issued"), (5, "waves reduced"),
               (6, "column words added, y written where last (up to 64 splits); partial row acknowledged (more)"),
               (7, "tile sum written (last workgroup of a tile; more than 64 splits)")],
}


def _timeline_summary(stamps, mask, phases):
    """Percentiles (0, 10, 50, 90, 100) over the launch's workgroups of each
    stamp, in microseconds after the first workgroup started (100 MHz clock)."""
    import decode_stage_gemv_amd as grq
    st = stamps.reshape(grq.TIMELINE_WORKGROUPS, grq.TIMELINE_SLOTS)[mask].astype(np.int64)
    t0 = st[:, 0].min()

    def pct(v):
        return [round(float(np.percentile(v, q)), 2) for q in (0, 10, 50, 90, 100)]

    out = {}
    for slot, label in phases:
        col = st[:, slot]
        valid = col >= t0      # a slot a workgroup did not record this launch holds an older value
        if valid.any():
            out[label] = pct((col[valid] - t0) / 100.0)
    waves = st[:, 8:8 + 16]
    ok = waves >= t0
    if ok.any():
        first = np.where(ok, waves, np.iinfo(np.int64).max).min(axis=1)
        last = np.where(ok, waves, np.iinfo(np.int64).min).max(axis=1)
        out["records done (first wave)"] = pct((first - t0) / 100.0)
        out["records done (last wave)"] = pct((last - t0) / 100.0)
    return out


def timeline_bench(name, mode, steps, warmup):
    """Where a launch's time goes, from the timeline build's clock stamps: one
    launch after host-launched warm-up steps, and the last step of a HIP-graph
    replay of `steps` steps (each step on a different rotated copy, as in the
    timed runs)."""
    import torch
    import decode_stage_gemv_amd as grq
    prep = Prepared(name, mode)
    for k in range(max(warmup, 2 * prep.R)):
        prep.step(k)
    torch.cuda.synchronize()
    s1 = grq.timeline_read()
    prep.step(0)
    torch.cuda.synchronize()
    s2 = grq.timeline_read()
    # the launch's workgroups are the ones whose start stamp changed
    mask = s2.reshape(-1, grq.TIMELINE_SLOTS)[:, 0] != s1.reshape(-1, grq.TIMELINE_SLOTS)[:, 0]
    res = {"workload": name, "entry_point": ENTRY[mode], "workgroups": int(mask.sum()),
           "units": "us after the first workgroup started; percentiles 0/10/50/90/100 over workgroups",
           "host_launch": _timeline_summary(s2, mask, TIMELINE_PHASES[mode])}
    ms, _ = prep.run(steps, 0, graph=True)
    s3 = grq.timeline_read()
    res["graph_replay"] = _timeline_summary(s3, mask, TIMELINE_PHASES[mode])
    res["graph_replay_us_per_step"] = ms * 1e3
    for form in ("host_launch", "graph_replay"):
        for label, v in res[form].items():
            log(f"timeline {name} {form}: {label:40s} {v}")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-sweep", dest="sweep", action="store_false",
                    help="skip the bit-width sweep (4096^2 and 4096x14336 at avg 2/3/4/8, 70B gate at 0.5..8 bits)")
    ap.add_argument("--sweep-bmax", action="store_true",
                    help="also time stores of 6-bit and 4-bit codes (4096x14336 and 70B gate)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step from the host")
    ap.add_argument("--mode", choices=sorted(ENTRY), default="accumulate",
                    help="accumulate: grinqh_decode_vmm_accumulate (ping-pong outputs); "
                         "decode: grinqh_decode_vmm (deterministic split-K); "
                         "list: grinqh_assign_bits then grinqh_vmm (two launches)")
    ap.add_argument("--only", action="store_true", help="time only the chosen entry point")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 512 MiB device copy (reference for bandwidth and counters)")
    ap.add_argument("--prefill-tokens", type=int, default=2048,
                    help="tokens of the dense prefill timed on the same layer (0: skip)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the dense prefill of the chosen workload's layer")
    ap.add_argument("--no-lut", action="store_true",
                    help="skip the table-reconstruction leg (grinqh_decode_vmm_lut)")
    ap.add_argument("--lut-only", action="store_true", help="time only grinqh_decode_vmm_lut")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the Qwen3-8B stack leg (252 VMMs per token, 6.95 GB of planes)")
    ap.add_argument("--stack-only", action="store_true", help="time only the Qwen3-8B stack")
    ap.add_argument("--timeline", action="store_true",
                    help="load the timeline build (libgrinqh_timeline.so, `python -m decode_stage_gemv_amd.build "
                         "--timeline`) and report where a launch of the chosen workload and mode spends its time")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this decode VMM path runs on a single GPU "
              "(sharding across GPUs is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.timeline:
        import decode_stage_gemv_amd as grq
        grq.use_library(grq.TIMELINE_LIB_PATH)
        scrub_init()
        mode = args.mode if args.mode in TIMELINE_PHASES else "accumulate"
        print(json.dumps({"timeline": timeline_bench(args.workload, mode, min(args.steps, 100),
                                                     args.warmup)}), flush=True)
        return
    scrub_init()
    if args.copy_probe:
        print(json.dumps({"copy_probe": copy_probe()}), flush=True)
        return
    if args.stack_only:
        print(json.dumps({"stack": stack_bench(), "stack_grouped": stack_bench(grouped=True),
                          "stack_fused": stack_bench(fused=True)}), flush=True)
        return
    if args.lut_only:
        print(json.dumps({"lut": lut_bench(args.workload, min(args.steps, 100), min(args.warmup, 10))}), flush=True)
        return
    if args.prefill_only:
        K, N, cfg, mat, _, lv = WORKLOADS[args.workload]
        res = prefill_bench(Layer(K, N, cfg, mat, bmax_of(lv)), args.prefill_tokens or 2048,
                            steps=min(args.steps, 20), warmup=min(args.warmup, 3), dense_reference=False)
        print(json.dumps({"prefill": res}), flush=True)
        return
    prep = Prepared(args.workload, args.mode)
    ms, step_bytes = prep.run(args.steps, args.warmup, graph=not args.no_graph)
    if args.no_graph:
        log("host-launched steps (no graph): includes Python and ctypes launch overhead")
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"{args.workload} {ENTRY[args.mode]}: {ms * 1e3:.2f} us/VMM, {gbs:.1f} GB/s "
        f"({gbs / HBM_PEAK_GBS:.1%} of HBM peak)")

    others = {}
    if not args.only:
        for mode in sorted(ENTRY):
            if mode == args.mode:
                continue
            p = Prepared(args.workload, mode, layer=prep.layer)
            m, b = p.run(args.steps, args.warmup, graph=not args.no_graph)
            others[ENTRY[mode]] = {"us_per_vmm": m * 1e3, "GB_s": b / (m * 1e-3) / 1e9}
            log(f"{args.workload} {ENTRY[mode]}: {m * 1e3:.2f} us/VMM, {others[ENTRY[mode]]['GB_s']:.1f} GB/s")
            del p

    # the metric's sweep: 4096 x 4096 and 4096 x 14336 at avg 2/3/4/8 bits and
    # the 70B gate at 0.5..8 bits (the headline layer is reused, not redrawn)
    sweep = {}
    names = [] if args.only else (SWEEP if args.sweep else []) + (SWEEP_BMAX if args.sweep_bmax else [])
    if names:
        layers = {(prep.K, prep.N, prep.layer.cfg, prep.layer.mat, prep.b_max): prep.layer}
        for name in names:
            K, N, cfg, mat, _, lv = WORKLOADS[name]
            key = (K, N, cfg, mat, bmax_of(lv))
            if key not in layers:
                for k in [k for k in layers if layers[k] is not prep.layer]:
                    del layers[k]
                torch.cuda.empty_cache()
                layers[key] = Layer(K, N, cfg, mat, bmax_of(lv))
            if name == args.workload:
                m, b, p = ms, step_bytes, prep
            else:
                p = Prepared(name, args.mode, layer=layers[key])
                m, b = p.run(min(args.steps, 100), args.warmup, graph=not args.no_graph)
            sweep[name] = {"us_per_vmm": m * 1e3, "GB_s": b / (m * 1e-3) / 1e9,
                           "frac_of_peak": b / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "avg_bits": float(np.mean(p.avg_bits)), "bytes": b,
                           "rotated_copies": p.R, "touched_bytes_per_cycle": p.touched_per_cycle}
            log(f"{name}: {m * 1e3:.2f} us/VMM, {sweep[name]['GB_s']:.1f} GB/s "
                f"({sweep[name]['frac_of_peak']:.1%}), avg bits {sweep[name]['avg_bits']:.2f}")
            if p is not prep:
                del p
        layers.clear()
        torch.cuda.empty_cache()
        fit_pts = [(v["bytes"], v["us_per_vmm"]) for k, v in sweep.items() if k.startswith("llama3-70b-gate-8192x28672-avg")]
        if len(fit_pts) >= 3:
            sweep["linear_fit_70b_gate"] = linear_fit(fit_pts)
            log(f"70B gate linear fit: {sweep['linear_fit_70b_gate']}")
        all_pts = [(v["bytes"], v["us_per_vmm"]) for k, v in sweep.items() if k in SWEEP]
        if len(all_pts) >= 3:
            # one line over every shape of the sweep (4096^2, 4096x14336, 70B gate)
            sweep["linear_fit_all_shapes"] = linear_fit(all_pts)
            log(f"linear fit over all swept shapes: {sweep['linear_fit_all_shapes']}")

    # marginal bandwidth: the same layer at two widths; the difference in
    # bytes over the difference in time is what streaming a byte costs once
    # the fixed per-launch cost (dispatch, dependent latencies) is paid
    marginal = None
    pair = MARGINAL_PAIRS.get(args.workload)
    if pair and all(n in sweep for n in pair):
        (n_lo, n_hi) = pair
        t_lo, b_lo = sweep[n_lo]["us_per_vmm"], sweep[n_lo]["bytes"]
        t_hi, b_hi = sweep[n_hi]["us_per_vmm"], sweep[n_hi]["bytes"]
        bw = (b_hi - b_lo) / ((t_hi - t_lo) * 1e-6) / 1e9 if t_hi > t_lo else None
        marginal = {"low": {"workload": n_lo, "us_per_vmm": t_lo, "bytes": b_lo},
                    "high": {"workload": n_hi, "us_per_vmm": t_hi, "bytes": b_hi},
                    "GB_s": bw, "frac_of_peak": bw / HBM_PEAK_GBS if bw else None,
                    "fixed_us": t_lo - b_lo / (bw * 1e3) if bw else None}
        if bw:
            log(f"marginal bandwidth ({n_lo} -> {n_hi}): {bw:.0f} GB/s ({bw / HBM_PEAK_GBS:.1%} of peak), "
                f"fixed part {marginal['fixed_us']:.2f} us")

    prefill = None
    if args.prefill_tokens > 0 and not args.only:
        prefill = prefill_bench(prep.layer, args.prefill_tokens)
    lut = None
    if not args.no_lut and not args.only:
        lut = lut_bench(args.workload, min(args.steps, 100), min(args.warmup, 10))

    stack = stack_grouped = stack_fused = None
    if not args.no_stack and not args.only:
        stack = stack_bench()
        stack_grouped = stack_bench(grouped=True)
        stack_fused = stack_bench(fused=True)

    copy = copy_probe()
    log(f"copy probe: {copy['GB_s_read_plus_write']:.0f} GB/s read + write "
        f"({copy['frac_of_hbm_peak']:.1%} of the 8 TB/s peak); the VMM reaches {gbs / copy['GB_s_read_plus_write']:.1%} of it")
    cpu = None if args.no_cpu_baseline else cpu_baseline(prep)
    traffic = measured_traffic(args.workload, args.mode)
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
        "dtype": "f32",
        "data": f"synthetic (seeded N(0,0.02) weights, RTN {prep.b_max}-bit codes, log-normal |x| "
                "with 1% outlier channels)",
        "config": {"workload": args.workload, "entry_point": ENTRY[args.mode], "K": prep.K, "N": prep.N,
                   "b_max": prep.b_max,
                   "avg_bits": float(np.mean(prep.avg_bits)), "bytes_per_step": step_bytes,
                   "rotated_copies": prep.R, "touched_bytes_per_cycle": prep.touched_per_cycle,
                   "cache_scrub_read_bytes_before_timing": ROT_BYTES, "graph_replay": not args.no_graph,
                   "arithmetic": "fp16 x times codes (as fp16 subnormals) into fp32 accumulators, fp32 dequant",
                   "thresholds": prep.thresholds, "levels": list(prep.levels)},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
    }
    out["copy_probe"] = dict(copy, vmm_frac_of_copy=gbs / copy["GB_s_read_plus_write"])
    if marginal:
        out["marginal"] = marginal
    if others:
        out["other_entry_points"] = others
    if sweep:
        out["sweep"] = sweep
    if prefill:
        out["prefill"] = prefill
    if lut:
        out["lut"] = lut
    if stack:
        out["stack"] = stack
        out["stack_grouped"] = stack_grouped
        out["stack_fused"] = stack_fused
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
