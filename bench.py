#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one pass of the whole hot path over the b=32, t=4096 decode
workloads: grouped-query decode (64 query / 8 KV heads, d=128, s=1), absorbed
MLA decode (h=128, k=512, p=64) at s=1, and at s=4 draft tokens, launched
back to back on one stream. A call is its tile kernel, plus the log-sum-exp
combine where sequences are split over several blocks (MLA s=1). Inputs are
seeded synthetic bf16 N(0,1) tensors, resident in HBM
before timing. Every part rotates over enough copies of its inputs that the
copies together exceed 512 MB (twice the 256 MB last-level cache), so no call
finds its inputs cached by the previous call of the same part.

Prints ONE JSON line: value = algorithmic TFLOP/s of the step (closed-form
FLOPs / wall time per step over the K timed steps, which have no marker
between calls), plus
  parts      per-call times from HIP events at every call boundary over a
             pass of the K steps (marked_us; each marker adds a dispatch
             gap) and less the mean gap (us);
  timing     per part, the median per-launch time of 5 batches of 20 launches,
             with and without input rotation;
  ceilings   the HBM read rate and the bf16 MFMA rate this GPU attains (probe
             kernels: a streaming read, a register-only MFMA loop), and the
             rate of a vendor-library GEMM;
  roofline   the dominant call placed on the MI355X roofline, with `traffic`
             = HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
             of this same invocation (child processes, before this process
             touches the GPU), scaled by what the counters read for a 1 GiB
             device copy;
  parity     every output row of every part against the fp64 oracle;
  sweep      the MLA s-sweep s = 1..32 and where it crosses the ridge;
  ragged     the ragged long-context MLA workload (b=64, lengths U{1024..32768});
  variants   MQA (hkv = 1) and MHA (hkv = hq) at d=128, t=4096, with their
             measured arithmetic intensity against the closed forms;
  cpu_baseline the fp64 oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-traffic] [--no-extras]
    python bench.py --crossover | --split | --projections | --gqa-long | --cu-scaling   (separate studies)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import shutil
import statistics
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as wl  # noqa: E402
from decode_attention_bf16_amd import binding  # noqa: E402
from decode_attention_bf16_amd import costmodel as cm  # noqa: E402

PEAK_TFLOPS = cm.MI355X_BF16_FLOPS / 1e12
PEAK_GBS = cm.MI355X_HBM_BYTES_PER_S / 1e9
RIDGE = cm.MI355X_BF16_FLOPS / cm.MI355X_HBM_BYTES_PER_S
CSRC = os.path.join(ROOT, "decode_attention_bf16_amd", "csrc")
ROTATE_BYTES = 512 << 20   # rotation copies of a part's inputs together exceed this
BATCHES, LAUNCHES = 5, 20  # the protocol's batches of launches
CALIB_BYTES = 1 << 30      # device copy that calibrates the HBM counters
METRIC = "decode-attn TFLOP/s + HBM TB/s (% of MI355X roofline), b=32 t=4096, s=1 and s=4"
OUT_TOL, LSE_TOL = 1e-2, 1e-3


def kernel_source_hash() -> str:
    """sha256 prefix of the decode library's sources (csrc/ without the ceiling probes' own file)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name == "read_probe.hip":
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _input_bytes(tensors):
    return sum(t.numel() * t.element_size() for t in tensors)


class Part:
    """One decode call of the step: `copies` input sets resident on the GPU (set 0 is the seeded
    workload, the others drawn on the GPU from seeded generators), preallocated outputs and workspace."""

    def __init__(self, name, kind, shape, dev, path=0, copies=None, on_gpu_only=False):
        self.name, self.kind, self.shape, self.path = name, kind, shape, path
        if kind == "mla":
            self.cost = cm.mla_absorbed(shape.b, shape.h, shape.s, shape.t_max, shape.k, shape.p)
            nbytes = binding.mla_decode_workspace_size(shape.b, shape.s, shape.h, shape.k, shape.p, shape.t_max)
            oshape, lshape = (shape.b, shape.s, shape.h, shape.k), (shape.b, shape.s, shape.h)
        else:
            self.cost = cm.gqa(shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max)
            nbytes = binding.gqa_decode_workspace_size(shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max, 0,
                                                       path)
            oshape, lshape = (shape.b, shape.s, shape.hq, shape.d), (shape.b, shape.s, shape.hq)
        if on_gpu_only:
            self.cpu = None
            first = self._draw(dev, 0)
        else:
            self.cpu = wl.make_mla(shape) if kind == "mla" else wl.make_gqa(shape)
            first = tuple(t.to(dev) for t in self.cpu)
        if shape.ragged is not None:
            sl = (self.cpu[3] if self.cpu is not None else first[3].cpu()).tolist()
            self.cost = (cm.mla_absorbed_ragged(sl, shape.h, shape.s, shape.k, shape.p, shape.t_max)
                         if kind == "mla" else cm.gqa_ragged(sl, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max))
        n = copies if copies is not None else max(1, math.ceil(ROTATE_BYTES / _input_bytes(first[:3])))
        self.inputs = [first] + [self._draw(dev, i) for i in range(1, n)]
        self.out = torch.empty(oshape, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(lshape, dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.bound = "mfma" if self.cost.ai > RIDGE else "hbm"
        self.t_min = cm.roofline_time(self.cost)

    def _draw(self, dev, i):
        """Input set i drawn on the GPU: same shapes, N(0,1) bf16, the workload's lengths."""
        g = torch.Generator(device=dev).manual_seed(7919 * (i + 1) + self.shape.seed)
        sh = self.shape
        r = lambda *s: torch.randn(s, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)  # noqa: E731
        if self.cpu is not None:
            sl = self.cpu[3].to(dev)
        else:  # full-length sequences (every workload drawn only on the GPU is one)
            sl = torch.full((sh.b,), sh.t_max, dtype=torch.int32, device=dev)
        if self.kind == "mla":
            return (r(sh.b, sh.s, sh.h, sh.k), r(sh.b, sh.s, sh.h, sh.p), r(sh.b, sh.t_max, sh.k + sh.p), sl)
        return (r(sh.b, sh.s, sh.hq, sh.d), r(sh.b, sh.t_max, sh.hkv, sh.d), r(sh.b, sh.t_max, sh.hkv, sh.d), sl)

    @property
    def copies(self):
        return len(self.inputs)

    def __call__(self, i=0):
        x = self.inputs[i % len(self.inputs)]
        if self.kind == "mla":
            binding.mla_decode(*x, self.shape.scale, out=self.out, lse=self.lse, workspace=self.ws)
        else:
            binding.gqa_decode(*x, self.shape.scale, path=self.path, out=self.out, lse=self.lse, workspace=self.ws)

    def roofline(self, sec):
        if self.bound == "mfma":
            a = self.cost.flops / sec / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / PEAK_TFLOPS, 4)}
        a = self.cost.bytes / sec / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(a / PEAK_GBS, 4)}

    def summary(self, sec):
        return {"us": round(sec * 1e6, 2), "tflops": round(self.cost.flops / sec / 1e12, 2),
                "tbs": round(self.cost.bytes / sec / 1e12, 3), "ai": round(self.cost.ai, 1), "bound": self.bound,
                "t_min_us": round(self.t_min * 1e6, 2), "roofline_frac": round(self.t_min / sec, 4)}


def time_steps(parts, steps, warmup):
    """W untimed warmup steps, then exactly K timed steps (step k uses input copy k of every part), bracketed by
    device synchronisation and one HIP event at each end, with nothing between the calls. Returns (wall seconds
    per step, HIP-event seconds per step)."""
    stream = torch.cuda.current_stream()
    for k in range(warmup):
        for p in parts:
            p(k)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for k in range(steps):
        for p in parts:
            p(k)
    b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, a.elapsed_time(b) / 1e3 / steps


def time_calls(parts, steps):
    """Per-call breakdown of the step with markers: the same K steps once more with one HIP event on the
    library's stream at every boundary between consecutive calls, so a call's time is the difference of
    the events either side of it. A marker between two calls delays the next dispatch by a few
    microseconds (the queue waits for the marker's completion), so each call's time here includes one such
    gap and the calls add up to more than the unmarked step of time_steps."""
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps * len(parts) + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    i = 0
    for k in range(steps):
        for p in parts:
            p(k)
            i += 1
            evs[i].record(stream)
    torch.cuda.synchronize()
    per = {p.name: 0.0 for p in parts}
    i = 0
    for k in range(steps):
        for p in parts:
            per[p.name] += evs[i].elapsed_time(evs[i + 1]) / 1e3
            i += 1
    return {n: v / steps for n, v in per.items()}


def time_batches(part, rotate=True, batches=BATCHES, launches=LAUNCHES, warmup=3):
    """Per-launch seconds of `batches` batches of `launches` back-to-back calls (HIP events around each
    batch), rotating over the part's input copies or repeating copy 0. Returns (median, all)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        part(i if rotate else 0)
    res = []
    for bi in range(batches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(launches):
            part(bi * launches + i if rotate else 0)
        b.record(stream)
        b.synchronize()
        res.append(a.elapsed_time(b) / 1e3 / launches)
    return statistics.median(res), res


def read_ceiling(dev, reps=10):
    """HBM bytes per second of one streaming read of 1 GiB: the read-rate probe library built beside the
    decode library (non-temporal 16-byte loads, grid-stride), best of three launch shapes; two buffers
    alternate so that no launch finds its bytes in the last-level cache."""
    import ctypes
    lib = _probe_lib()
    nbytes = 1 << 30
    bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device=dev) for i in range(2)]
    shapes = ((256, 8), (512, 4), (1024, 2))  # blocks of 256 threads, loads in flight per thread
    sink = torch.empty(max(b for b, _ in shapes) * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for blocks, unroll in shapes:
        def run(i):
            rc = lib.da_probe_read(ctypes.c_void_p(bufs[i % 2].data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                   blocks, unroll, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("read probe launch failed: HIP error %d" % rc)
        for i in range(3):
            run(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) / 1e3))
    del bufs, sink
    torch.cuda.empty_cache()
    return best


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(binding.__file__)), "libda_read_probe.so"))
    lib.da_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.da_probe_read.restype = ctypes.c_int
    lib.da_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.da_probe_mfma.restype = ctypes.c_int
    return lib


def mfma_ceiling(dev, reps=5, iters=4000):
    """bf16 FLOP/s of the probe library's MFMA loop: four waves per SIMD, each running four independent
    chains of 32x32x16 MFMAs on register operands (no memory traffic), i.e. the matrix rate at the clock
    the chip sustains under a full matrix load."""
    import ctypes
    lib = _probe_lib()
    blocks = 4 * torch.cuda.get_device_properties(dev).multi_processor_count  # 4 waves per block
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        rc = lib.da_probe_mfma(blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("MFMA probe launch failed: HIP error %d" % rc)
    for _ in range(2):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    flops = float(blocks) * 4 * iters * 4 * 32768 * reps
    del sink
    return flops / (e0.elapsed_time(e1) / 1e3)


def gemm_ceiling(dev, reps=20, n=12288):
    """bf16 FLOP/s of an n^3 GEMM through the vendor library: the matrix rate this GPU sustains for a plain
    product (a reference point, not the decode path)."""
    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    rate = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) / 1e3)
    del x, y
    torch.cuda.empty_cache()
    return rate


def measured_ceilings(dev, reps=20):
    """What this GPU attains, as reference points for the ridge (not the decode path): HBM bytes per
    second of a 1 GiB device-to-device copy (read + write), and bf16 FLOP/s of a 12288^3 GEMM through
    the vendor library."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * a.numel() * reps / (e0.elapsed_time(e1) / 1e3)
    del a, b
    torch.cuda.empty_cache()
    return copy, gemm_ceiling(dev, reps)


# ------------------------------------------------------------------ parity and the CPU baseline
def oracle_of(part):
    """The fp64 oracle's result for every row of the part's seeded workload (input copy 0), and the
    oracle's wall time and multiply-add count."""
    import oracle
    oracle.build(force=False)
    t0 = time.perf_counter()
    fn = oracle.mla if part.kind == "mla" else oracle.gqa
    o, l, macs = fn(*part.cpu, part.shape.scale, return_macs=True)
    return o, l, macs, time.perf_counter() - t0


def parity_of(part, ref_o, ref_l):
    """max |out - out_ref| / max |out_ref| and max |lse - lse_ref| over every row (copy 0's outputs)."""
    import numpy as np
    part(0)
    torch.cuda.synchronize()
    o = part.out.float().cpu().numpy().astype(np.float64).reshape(ref_o.shape)
    l = part.lse.cpu().numpy().astype(np.float64).reshape(ref_l.shape)
    full = ~np.isneginf(ref_l)
    dout = float(np.abs(o[full] - ref_o[full]).max() / np.abs(ref_o[full]).max()) if full.any() else 0.0
    dlse = float(np.abs(l[full] - ref_l[full]).max()) if full.any() else 0.0
    empty_ok = bool(np.all(np.isneginf(l[~full])) and np.all(o[~full] == 0))
    return {"rows": int(ref_l.size), "max_dout_rel": float("%.3e" % dout), "max_dlse": float("%.3e" % dlse),
            "pass": bool(dout <= OUT_TOL and dlse <= LSE_TOL and empty_ok and np.isfinite(o).all())}


# ------------------------------------------------------------------ HBM traffic from the counters
PROBE_PARTS = ("gqa", "mla_s1", "mla_s4", "gqa_mqa", "gqa_mha")


def probe_part(name, dev):
    shapes = {"gqa": ("gqa", wl.GQA_LAYER), "mla_s1": ("mla", wl.MLA_DSV3), "mla_s4": ("mla", wl.MLA_MTP4),
              "gqa_mqa": ("gqa", wl.GQA_MQA), "gqa_mha": ("gqa", wl.GQA_MHA)}
    kind, shape = shapes[name]
    return Part(name, kind, shape, dev, copies=1, on_gpu_only=True)


def counter_probe():
    """Child-process body under rocprofv3: two calls of each probed part in order, then one 1 GiB device
    copy (the counters' calibration), nothing else on the library's kernels."""
    dev = torch.device("cuda:0")
    binding.load_library()
    for name in PROBE_PARTS:
        p = probe_part(name, dev)
        torch.cuda.synchronize()
        p(0)
        p(0)
        torch.cuda.synchronize()
        del p
        torch.cuda.empty_cache()
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe_parts": PROBE_PARTS}), flush=True)


def _read_counter_csv(outdir):
    """[(dispatch id, kernel name, summed counter value)] in dispatch order."""
    files = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    rows = {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                did = int(r.get("Dispatch_Id") or r.get("Dispatch_ID") or 0)
                name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
                val = float(r.get("Counter_Value") or 0.0)
                ent = rows.setdefault(did, [name, 0.0])
                ent[1] += val
    return [(d, n, v) for d, (n, v) in sorted(rows.items())]


def measure_traffic():
    """HBM bytes per call of each probed part, from one FETCH_SIZE run and one WRITE_SIZE run of the counter
    probe, each scaled by what the same counter reads for the 1 GiB copy. Runs before this process uses
    the GPU. Returns (dict or None, note)."""
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None, "rocprofv3 not found"
    env = dict(os.environ, TMPDIR="/tmp")
    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        outdir = tempfile.mkdtemp(prefix="da_pmc_", dir="/tmp")
        cmd = [prof, "--pmc", ctr, "--output-format", "csv", "-d", outdir, "-o", "pmc", "--", sys.executable,
               os.path.abspath(__file__), "--counter-probe"]
        try:
            r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                               timeout=240)
        except subprocess.TimeoutExpired:
            return None, "%s run timed out" % ctr
        disp = _read_counter_csv(outdir)
        shutil.rmtree(outdir, ignore_errors=True)
        if r.returncode != 0 and not disp:
            return None, "%s run failed (rc %d): %s" % (ctr, r.returncode, r.stdout.decode()[-300:])
        mine = lambda n: re.search(r"(^|[^A-Za-z0-9_:])da::", n) is not None  # noqa: E731 (not cuda::)
        lib = [(n, v) for _, n, v in disp if mine(n)]
        calib = [v for _, n, v in disp if not mine(n)]
        if not lib or not calib or calib[-1] <= 0:
            return None, "%s: no library or calibration dispatches in the counter output" % ctr
        scale = CALIB_BYTES / (calib[-1] * 1024.0)  # the copy reads (writes) exactly CALIB_BYTES
        calls = []  # each call: a tile kernel and the combine kernel that follows it
        for n, v in lib:
            if "combine" in n and calls:
                calls[-1] += v
            else:
                calls.append(v)
        if len(calls) != 2 * len(PROBE_PARTS):
            return None, "%s: %d library calls in the counter output, expected %d" % (ctr, len(calls),
                                                                                    2 * len(PROBE_PARTS))
        for i, name in enumerate(PROBE_PARTS):
            kib = 0.5 * (calls[2 * i] + calls[2 * i + 1])
            per.setdefault(name, {})[ctr] = {"kib_per_call": round(kib, 1), "scale": round(scale, 4),
                                              "bytes_per_call": kib * 1024.0 * scale}
    res = {}
    for name, d in per.items():
        res[name] = {"bytes_per_call": round(d["FETCH_SIZE"]["bytes_per_call"] + d["WRITE_SIZE"]["bytes_per_call"]),
                     "fetch_kib": d["FETCH_SIZE"]["kib_per_call"], "fetch_scale": d["FETCH_SIZE"]["scale"],
                     "write_kib": d["WRITE_SIZE"]["kib_per_call"], "write_scale": d["WRITE_SIZE"]["scale"]}
    return res, "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, over two calls per part (mean), scaled by the counters' " \
                "reading for a 1 GiB device copy"


# ------------------------------------------------------------------ the extra keys of the default line
def sweep_key(dev):
    """MLA s-sweep at the DeepSeek-V3-like shapes with rotating inputs, and the ridge crossing."""
    rows, us = [], {}
    for s in wl.MTP_SWEEP:
        p = Part("mla_s%d" % s, "mla", wl.mla_mtp(s), dev, on_gpu_only=True)
        sec, _ = time_batches(p)
        us[s] = (sec * 1e6, p.cost.flops / sec / 1e12)
        rows.append(dict({"s": s}, **p.summary(sec)))
        del p
        torch.cuda.empty_cache()
    bw, fl = measured_ceilings(dev)
    rd = read_ceiling(dev)
    mf = mfma_ceiling(dev)
    sh = wl.mla_mtp(1)
    best = max(tf for _, tf in us.values()) * 1e12
    cross = lambda f, b: round(cm.mla_ridge_crossing_s(sh.h, sh.k, sh.p, sh.t_max, peak_flops=f, bw=b), 3)  # noqa
    summary = {"spec_ridge_flop_per_byte": round(RIDGE, 1),
               "spec_crossing_s": cross(cm.MI355X_BF16_FLOPS, cm.MI355X_HBM_BYTES_PER_S),
               "measured_copy_tbs": round(bw / 1e12, 3), "measured_gemm_tflops": round(fl / 1e12, 1),
               "measured_ridge_flop_per_byte": round(fl / bw, 1), "measured_crossing_s": cross(fl, bw),
               "measured_read_tbs": round(rd / 1e12, 3), "read_ridge_flop_per_byte": round(fl / rd, 1),
               "read_crossing_s": cross(fl, rd),
               "measured_mfma_tflops": round(mf / 1e12, 1), "mfma_read_ridge_flop_per_byte": round(mf / rd, 1),
               "mfma_read_crossing_s": cross(mf, rd),
               "kernel_best_tflops": round(best / 1e12, 1), "kernel_crossing_s": cross(best, bw),
               "time_vs_s1": {str(s): round(t / us[1][0], 3) for s, (t, _) in sorted(us.items())}}
    return {"workload": "mla_mtp (b=32, h=128, k=512, p=64, t=4096, s drafts; rotating inputs, median of %d x %d)"
                        % (BATCHES, LAUNCHES), "points": rows, "ridge": summary}


def ragged_key(dev, want_parity):
    p = Part("mla_ragged", "mla", wl.MLA_RAGGED, dev, copies=1)
    sec, _ = time_batches(p, rotate=False)
    res = {"workload": "mla_ragged (b=64, s=1, h=128, k=512, p=64, seqlens U{1024..32768}, seed 4; "
                       "1.25 GB read per call, median of %d x %d)" % (BATCHES, LAUNCHES)}
    res.update(p.summary(sec))
    if want_parity:
        o, l, _, _ = oracle_of(p)
        res["parity"] = parity_of(p, o, l)
    del p
    torch.cuda.empty_cache()
    return res


def variants_key(dev, traffic, want_parity):
    """MQA and MHA at the layer's geometry: time, roofline, and the measured intensity (algorithmic FLOPs
    over counted HBM bytes) against the closed forms (MQA: hq; MHA: 1)."""
    res = {}
    for name, shape, closed in (("gqa_mqa", wl.GQA_MQA, "hq = %d" % wl.GQA_MQA.hq),
                                ("gqa_mha", wl.GQA_MHA, "1")):
        p = Part(name, "gqa", shape, dev)
        sec, _ = time_batches(p)
        ent = {"workload": "b=%d s=%d hq=%d hkv=%d d=%d t=%d, %d rotating copies"
                           % (shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max, p.copies)}
        ent.update(p.summary(sec))
        ent["ai_kv_only_closed_form"] = closed
        if traffic and name in traffic:
            ent["traffic"] = traffic[name]["bytes_per_call"]
            ent["measured_ai"] = round(p.cost.flops / traffic[name]["bytes_per_call"], 2)
        if want_parity:
            o, l, _, _ = oracle_of(p)
            ent["parity"] = parity_of(p, o, l)
        res[name] = ent
        del p
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ separate studies
class UnabsorbedPart:
    """One un-absorbed (per-head K/V) MLA decode call at the DeepSeek-V3-like shapes with s drafts. The
    decompressed K [b,t,h,192] and V [b,t,h,128] (10.7 GB at b=32, t=4096) are drawn on the GPU from a
    seeded generator and shared by every s."""

    kv = None

    def __init__(self, s, dev, b=32, h=128, t=4096):
        self.name, self.s = "mla_unabsorbed_s%d" % s, s
        if UnabsorbedPart.kv is None:
            g = torch.Generator(device=dev).manual_seed(7)
            UnabsorbedPart.kv = (torch.randn((b, t, h, 192), generator=g, device=dev, dtype=torch.bfloat16),
                                 torch.randn((b, t, h, 128), generator=g, device=dev, dtype=torch.bfloat16),
                                 torch.full((b,), t, dtype=torch.int32, device=dev))
        g = torch.Generator(device=dev).manual_seed(100 + s)
        self.q = torch.randn((b, s, h, 192), generator=g, device=dev, dtype=torch.bfloat16)
        self.scale = 1.0 / math.sqrt(192)
        self.out = torch.empty((b, s, h, 128), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
        nbytes = binding.mla_decode_unabsorbed_workspace_size(b, s, h, 192, 128, t)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.cost = cm.mla_unabsorbed(b, h, s, t, 128, 64)

    def __call__(self, i=0):
        k, v, sl = UnabsorbedPart.kv
        binding.mla_decode_unabsorbed(self.q, k, v, sl, self.scale, out=self.out, lse=self.lse, workspace=self.ws)


class ProjectionPart:
    """One per-head projection call at the DeepSeek-V3-like shapes (h=128, d=128, k=512): the query
    absorption or the output decompression for b*s query tokens."""

    def __init__(self, kind, s, dev, b=32, h=128, d=128, k=512):
        self.name, self.kind = "%s_s%d" % (kind, s), kind
        g = torch.Generator(device=dev).manual_seed(11 + s)
        if kind == "absorb":
            self.a = torch.randn((b, s, h, d), generator=g, device=dev, dtype=torch.bfloat16)
            self.w = torch.randn((h, k, d), generator=g, device=dev, dtype=torch.bfloat16)
            self.out = torch.empty((b, s, h, k), dtype=torch.bfloat16, device=dev)
        else:
            self.a = torch.randn((b, s, h, k), generator=g, device=dev, dtype=torch.bfloat16)
            self.w = torch.randn((h, d, k), generator=g, device=dev, dtype=torch.bfloat16)
            self.out = torch.empty((b, s, h, d), dtype=torch.bfloat16, device=dev)
        m = b * s
        self.flops = 2.0 * m * h * d * k
        self.bytes = 2.0 * (h * d * k + m * h * d + m * h * k)  # weights once, input and output rows

    def __call__(self, i=0):
        if self.kind == "absorb":
            binding.mla_absorb_queries(self.a, self.w, out=self.out)
        else:
            binding.mla_decompress_output(self.a, self.w, out=self.out)


class SplitPart:
    """One split-cache MLA decode call (b=32, h=128, t=4096 = o latent + n decompressed rows, s drafts),
    inputs drawn on the GPU from a seeded generator."""

    def __init__(self, s, n, dev, b=32, h=128, t=4096):
        self.name, self.s, self.n = "split_s%d_n%d" % (s, n), s, n
        o = t - n
        g = torch.Generator(device=dev).manual_seed(900 + n)
        r = lambda *shape: torch.randn(shape, generator=g, device=dev, dtype=torch.bfloat16)  # noqa: E731
        self.args = (r(b, s, h, 128), r(b, s, h, 64), r(h, 512, 128), r(h, 128, 512), r(b, max(o, 1), 576),
                     torch.full((b,), o, dtype=torch.int32, device=dev), r(b, n, h, 192), r(b, n, h, 128),
                     torch.full((b,), n, dtype=torch.int32, device=dev))
        self.scale = 1.0 / math.sqrt(192)
        self.out = torch.empty((b, s, h, 128), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
        nbytes = binding.mla_decode_split_cache_workspace_size(b, s, h, max(o, 1), n, 0)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.cost = cm.mla_split_latent(b, h, s, o, n, 128, 512, 64)

    def __call__(self, i=0):
        binding.mla_decode_split_cache(*self.args, self.scale, out=self.out, lse=self.lse, workspace=self.ws)


def studies(args, dev):
    if args.crossover:
        first = None
        for s in wl.MTP_SWEEP + (48, 64):
            pa = Part("mla_s%d" % s, "mla", wl.mla_mtp(s), dev, on_gpu_only=True)
            pu = UnabsorbedPart(s, dev)
            ta, _ = time_batches(pa)
            tu, _ = time_batches(pu, rotate=False)
            if first is None and tu < ta:
                first = s
            print(json.dumps({"crossover": "mla absorbed vs un-absorbed (b=32, h=128, t=4096, k=512, p=64, d=128)",
                              "s": s, "absorbed_us": round(ta * 1e6, 2), "unabsorbed_us": round(tu * 1e6, 2),
                              "absorbed_tflops": round(pa.cost.flops / ta / 1e12, 2),
                              "unabsorbed_tflops": round(pu.cost.flops / tu / 1e12, 2),
                              "unabsorbed_tbs": round(pu.cost.bytes / tu / 1e12, 3),
                              "unabsorbed_roofline_frac": round(cm.roofline_time(pu.cost) / tu, 4),
                              "faster": "unabsorbed" if tu < ta else "absorbed"}), flush=True)
            del pa, pu
        print(json.dumps({"crossover_s": first, "note": "smallest s of the sweep at which the un-absorbed kernel "
                          "is faster (null: none up to s=64)"}), flush=True)
    elif args.split:
        s = 16
        pa = Part("absorbed_s%d" % s, "mla", wl.mla_mtp(s), dev, on_gpu_only=True)
        ta, _ = time_batches(pa)
        print(json.dumps({"split": "absorbed only (n=0)", "s": s, "us": round(ta * 1e6, 2)}), flush=True)
        del pa
        for n in (64, 256, 1024, 2048, 4096):
            p = SplitPart(s, n, dev)
            sec, _ = time_batches(p, rotate=False)
            t_min = cm.roofline_time(p.cost)
            print(json.dumps({"split": "latent o + decompressed n (b=32, h=128, t=4096)", "s": s, "o": 4096 - n,
                              "n": n, "us": round(sec * 1e6, 2), "tflops": round(p.cost.flops / sec / 1e12, 2),
                              "tbs": round(p.cost.bytes / sec / 1e12, 3), "ai": round(p.cost.ai, 1),
                              "t_min_us": round(t_min * 1e6, 2), "roofline_frac": round(t_min / sec, 4)}),
                  flush=True)
            del p
            torch.cuda.empty_cache()
    elif args.cu_scaling:
        # the K/V stream (GQA token-group kernel, 0.54 GB per call) on 32..256 blocks, one per CU
        for blocks in (32, 64, 128, 256):
            b = blocks // 8
            shape = wl.GQAShape(b=b, s=1, hq=64, hkv=8, d=128, t_max=4096 * 32 // b, scale=1.0 / math.sqrt(128),
                                seed=12)
            p = Part("gqa_%dblocks" % blocks, "gqa", shape, dev, copies=1, on_gpu_only=True)

            def call(i=0, p=p):
                binding.gqa_decode(*p.inputs[0], shape.scale, out=p.out, lse=p.lse, null_workspace=True)
            sec, _ = time_batches(call, rotate=False)
            print(json.dumps({"cu_scaling": "GQA K/V stream, one block per (sequence, KV head), 0.54 GB per call",
                              "blocks": blocks, "b": b, "t": shape.t_max, "us": round(sec * 1e6, 2),
                              "tbs": round(p.cost.bytes / sec / 1e12, 3),
                              "gbs_per_block": round(p.cost.bytes / sec / 1e9 / blocks, 1)}), flush=True)
            del p
            torch.cuda.empty_cache()
    elif args.projections:
        for s in (1, 4, 32):
            for kind in ("absorb", "decompress"):
                p = ProjectionPart(kind, s, dev)
                sec, _ = time_batches(p, rotate=False)
                t_min = max(p.flops / cm.MI355X_BF16_FLOPS, p.bytes / cm.MI355X_HBM_BYTES_PER_S)
                print(json.dumps({"projection": kind, "b": 32, "s": s, "h": 128, "d": 128, "k": 512,
                                  "us": round(sec * 1e6, 2), "tflops": round(p.flops / sec / 1e12, 2),
                                  "tbs": round(p.bytes / sec / 1e12, 3), "ai": round(p.flops / p.bytes, 1),
                                  "t_min_us": round(t_min * 1e6, 2), "roofline_frac": round(t_min / sec, 4)}),
                      flush=True)
                del p
    elif args.gqa_long:
        for path in (2, 1):
            p = Part("gqa_long", "gqa", wl.GQA_LONG, dev, path=path, copies=1)
            sec, _ = time_batches(p, rotate=False)
            print(json.dumps(dict({"workload": "gqa_long (b=1, s=1, hq=24, hkv=4, d=256, t=262144, seed 6)",
                                   "kernel": "mfma" if path == 2 else "valu"}, **p.summary(sec))), flush=True)
            del p
    elif args.sweep:
        print(json.dumps(sweep_key(dev)), flush=True)
    elif args.ragged:
        print(json.dumps(ragged_key(dev, want_parity=False)), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle: no cpu_baseline, no parity")
    ap.add_argument("--no-traffic", action="store_true", help="skip the rocprofv3 counter runs (traffic: null)")
    ap.add_argument("--no-extras", action="store_true", help="only the step: no sweep, ragged or variants keys")
    ap.add_argument("--only", default="", help="comma list of step parts to run (gqa,mla_s1,mla_s4)")
    ap.add_argument("--gqa-path", type=int, default=0, help="GQA kernel: 0 auto, 1 VALU dot, 2 MFMA")
    ap.add_argument("--counter-probe", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--sweep", action="store_true", help="only the MLA s-sweep key")
    ap.add_argument("--ragged", action="store_true", help="only the ragged long-context MLA key")
    ap.add_argument("--crossover", action="store_true",
                    help="absorbed vs un-absorbed MLA decode over the s-sweep (b=32, h=128, t=4096)")
    ap.add_argument("--split", action="store_true",
                    help="split latent/decompressed cache at s=16 over n (b=32, h=128, t=4096)")
    ap.add_argument("--projections", action="store_true",
                    help="per-head query absorption and output decompression (b=32, h=128, d=128, k=512)")
    ap.add_argument("--cu-scaling", action="store_true",
                    help="HBM rate of the K/V stream on 32..256 blocks (one per CU), 0.54 GB per call")
    ap.add_argument("--gqa-long", action="store_true",
                    help="only the long-context GQA workload (t=262144, hq=24, hkv=4, d=256), both kernels")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (the decode kernels shard by "
              "batch or KV head with no communication; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    if args.counter_probe:
        counter_probe()
        return
    only_study = (args.crossover or args.split or args.projections or args.gqa_long or args.sweep or args.ragged
                  or args.cu_scaling)
    traffic, traffic_note = (None, "not measured (--no-traffic)")
    if not only_study and not args.no_traffic:
        # the counter runs happen before this process touches the GPU
        traffic, traffic_note = measure_traffic()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    binding.load_library()
    if only_study:
        studies(args, dev)
        return

    parts = [Part("gqa", "gqa", wl.GQA_LAYER, dev, args.gqa_path), Part("mla_s1", "mla", wl.MLA_DSV3, dev),
             Part("mla_s4", "mla", wl.MLA_MTP4, dev)]
    if args.only:
        keep = set(args.only.split(","))
        parts = [p for p in parts if p.name in keep]
    # the protocol's batches first: they also bring the GPU to its steady clock before the timed steps
    timing = {}
    for p in parts:
        rot, rot_all = time_batches(p, rotate=True)
        same, same_all = time_batches(p, rotate=False)
        timing[p.name] = {"rotating_median_us": round(rot * 1e6, 2), "same_input_median_us": round(same * 1e6, 2),
                          "rotating_batches_us": [round(x * 1e6, 2) for x in rot_all],
                          "same_input_batches_us": [round(x * 1e6, 2) for x in same_all]}
    # the per-call breakdown first (the marked pass), then the W warmup and the K timed steps, which are
    # thus the last calls of the run
    marked = time_calls(parts, args.steps)
    wall, ev_step = time_steps(parts, args.steps, args.warmup)
    # a call's time inside the step: its marked time less the mean gap one marker adds, i.e. the marked
    # pass's excess over the unmarked step spread evenly over the calls (the kernel trace shows equal gaps)
    gap = max(0.0, (sum(marked.values()) - ev_step) / len(parts))
    per = {n: v - gap for n, v in marked.items()}
    read_bw = read_ceiling(dev)
    mfma_fl = mfma_ceiling(dev)
    gemm_fl = gemm_ceiling(dev)

    flops = sum(p.cost.flops for p in parts)
    byts = sum(p.cost.bytes for p in parts)
    dom = max(parts, key=lambda p: per[p.name])
    roof = dom.roofline(per[dom.name])
    measured = mfma_fl / 1e12 if roof["bound"] == "mfma" else read_bw / 1e9
    roof["measured_peak"] = round(measured, 1)
    roof["frac_of_measured"] = round(roof["achieved"] / measured, 4)
    roof["traffic"] = traffic[dom.name]["bytes_per_call"] if traffic and dom.name in traffic else None
    roof["kernel"] = dom.name + (" (one call inside the step from HIP events at the call boundaries over K steps, "
                                 "less the mean marker gap; the call is the tile kernel alone at this shape)")
    part_info = {}
    for p in parts:
        part_info[p.name] = dict(p.summary(per[p.name]), copies=p.copies, marked_us=round(marked[p.name] * 1e6, 2))
        if p.bound == "hbm":
            part_info[p.name]["of_measured_read"] = round(p.cost.bytes / per[p.name] / read_bw, 4)
        else:
            part_info[p.name]["of_measured_mfma"] = round(p.cost.flops / per[p.name] / mfma_fl, 4)
            part_info[p.name]["of_measured_gemm"] = round(p.cost.flops / per[p.name] / gemm_fl, 4)
        if traffic and p.name in traffic:
            part_info[p.name]["traffic"] = traffic[p.name]["bytes_per_call"]
            part_info[p.name]["traffic_over_algorithmic"] = round(traffic[p.name]["bytes_per_call"] / p.cost.bytes, 3)
            part_info[p.name]["measured_ai"] = round(p.cost.flops / traffic[p.name]["bytes_per_call"], 1)
    res = {
        "metric": METRIC,
        "value": round(flops / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "event_ms_per_step": round(ev_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "+".join(p.name for p in parts) + " (b=32, t=4096: gqa hq=64 hkv=8 d=128 s=1; "
                               "mla h=128 k=512 p=64 s=1 and s=4)",
                   "global_batch": 32, "seq_len": 4096, "parallelism": "single-gpu"},
        "hbm_tbs": round(byts / wall / 1e12, 3),
        "step_roofline_frac": round(sum(p.t_min for p in parts) / wall, 4),
        "roofline": roof,
        "ceilings": {"measured_read_tbs": round(read_bw / 1e12, 3), "spec_hbm_tbs": PEAK_GBS / 1e3,
                     "measured_mfma_tflops": round(mfma_fl / 1e12, 1),
                     "measured_gemm_tflops": round(gemm_fl / 1e12, 1), "spec_bf16_tflops": PEAK_TFLOPS,
                     "note": "measured_read: one streaming read of 1 GiB by the read probe, best of three launch "
                             "shapes; measured_mfma: the probe's register-only loop of 32x32x16 bf16 MFMAs on every "
                             "SIMD; measured_gemm: a 12288^3 bf16 GEMM through the vendor library; a part's "
                             "of_measured_* = its algorithmic rate over them; roofline.measured_peak is the read "
                             "or MFMA-loop rate"},
        "parts": part_info,
        "parts_note": ("marked_us: HIP events at every call boundary over a pass of K steps, each marker adding a "
                       "dispatch gap; us: marked_us less the mean gap (the marked pass's excess over the unmarked "
                       "timed step, %.2f us, spread evenly over the calls)" % (gap * 1e6)),
        "timing": dict(timing, protocol="per-launch time, median of %d batches of %d launches; rotating = each "
                                        "launch takes the next of the part's input copies (together > 512 MB)"
                                        % (BATCHES, LAUNCHES)),
        "traffic_note": traffic_note,
        "traffic_detail": traffic,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu:
        import oracle
        par, tot_macs, tot_sec = {}, 0, 0.0
        for p in parts:
            o, l, macs, sec = oracle_of(p)
            tot_macs += macs
            tot_sec += sec
            par[p.name] = parity_of(p, o, l)
        res["parity"] = par
        res["cpu_baseline"] = {"value": round(2.0 * tot_macs / tot_sec / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": "fp64 oracle on every query row of the step's three workloads "
                                         "(%.1f GFLOP, %.1f s)" % (2.0 * tot_macs / 1e9, tot_sec)}
    if not args.no_extras:
        del parts
        torch.cuda.empty_cache()
        res["sweep"] = sweep_key(dev)
        res["ragged"] = ragged_key(dev, want_parity=not args.no_cpu)
        res["variants"] = variants_key(dev, traffic, want_parity=not args.no_cpu)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
