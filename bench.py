#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one pass of the whole hot path over the b=32, t=4096 decode
workloads: grouped-query decode (64 query / 8 KV heads, d=128, s=1), absorbed
MLA decode (h=128, k=512, p=64) at s=1, and at s=4 draft tokens. Each call runs
the device planner, the tile kernel and the log-sum-exp combine. Inputs are
seeded synthetic bf16 N(0,1) tensors, resident in HBM before timing; the three
workloads together stream ~840 MB per step, so no input stays in the 256 MB
last-level cache between its uses.

Prints ONE JSON line: value = algorithmic TFLOP/s of the step (closed-form
FLOPs / wall time per step), plus per-part kernel times from HIP events, the
roofline placement of the dominant call and the fp64 CPU oracle timed on a
sample of the same rows.

    python bench.py [--steps K] [--warmup W] [--cpu-sample F] [--no-cpu]
    python bench.py --sweep          # s-sweep of MLA (one JSON line per s, for the ridge crossing)
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import sys
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class Part:
    """One decode call of the step, with preallocated outputs and workspace."""

    def __init__(self, name, kind, shape, dev, path=0):
        self.name, self.kind, self.shape, self.path = name, kind, shape, path
        if kind == "mla":
            cpu = wl.make_mla(shape)
            self.cost = cm.mla_absorbed(shape.b, shape.h, shape.s, shape.t_max, shape.k, shape.p)
            self.flops_masked = cm.mla_absorbed_ragged(cpu[3].tolist(), shape.h, shape.s, shape.k, shape.p,
                                                       shape.t_max, masked=True).flops
            nbytes = binding.mla_decode_workspace_size(shape.b, shape.s, shape.h, shape.k, shape.p, shape.t_max)
            self.out = torch.empty((shape.b, shape.s, shape.h, shape.k), dtype=torch.bfloat16, device=dev)
            self.lse = torch.empty((shape.b, shape.s, shape.h), dtype=torch.float32, device=dev)
        else:
            cpu = wl.make_gqa(shape)
            self.cost = cm.gqa(shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max)
            self.flops_masked = cm.gqa_ragged(cpu[3].tolist(), shape.s, shape.hq, shape.hkv, shape.d, shape.t_max,
                                              masked=True).flops
            nbytes = binding.gqa_decode_workspace_size(shape.b, shape.s, shape.hq, shape.hkv, shape.d, shape.t_max, 0,
                                                       self.path)
            self.out = torch.empty((shape.b, shape.s, shape.hq, shape.d), dtype=torch.bfloat16, device=dev)
            self.lse = torch.empty((shape.b, shape.s, shape.hq), dtype=torch.float32, device=dev)
        self.cpu = cpu
        self.gpu = [t.to(dev) for t in cpu]
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.bound = "mfma" if self.cost.ai > RIDGE else "hbm"
        self.t_min = cm.roofline_time(self.cost)

    def __call__(self):
        if self.kind == "mla":
            binding.mla_decode(*self.gpu, self.shape.scale, out=self.out, lse=self.lse, workspace=self.ws)
        else:
            binding.gqa_decode(*self.gpu, self.shape.scale, path=self.path, out=self.out, lse=self.lse,
                               workspace=self.ws)

    def roofline(self, sec):
        if self.bound == "mfma":
            a = self.cost.flops / sec / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / PEAK_TFLOPS, 4)}
        a = self.cost.bytes / sec / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_GBS, "unit": "GB/s", "frac": round(a / PEAK_GBS, 4)}


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

    def __call__(self):
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

    def __call__(self):
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

    def __call__(self):
        binding.mla_decode_split_cache(*self.args, self.scale, out=self.out, lse=self.lse, workspace=self.ws)


def time_parts(parts, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for p in parts:
            p()
    torch.cuda.synchronize()
    evs = {p.name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(steps)] for p in parts}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        for p in parts:
            a, b = evs[p.name][k]
            a.record(stream)
            p()
            b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = {p.name: sum(a.elapsed_time(b) for a, b in evs[p.name]) / steps / 1e3 for p in parts}
    return wall, per


def measured_ceilings(dev, reps=20):
    """What this GPU attains, as reference points for the ridge (not the decode path): HBM bytes per
    second of a 1 GiB device-to-device copy (read + write), and bf16 FLOP/s of a 12288^3 GEMM through
    the vendor library."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    n = 12288
    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    res = {}
    for name, fn, work in (("copy", lambda: b.copy_(a), 2.0 * a.numel()),
                           ("gemm", lambda: torch.matmul(x, y), 2.0 * n ** 3)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = work * reps / (e0.elapsed_time(e1) / 1e3)
    del a, b, x, y
    torch.cuda.empty_cache()
    return res["copy"], res["gemm"]


def ridge_summary(us, dev):
    """Where the MLA s-sweep crosses the ridge: analytic s* at the published ceilings, at the ceilings
    measured here, and at this kernel's own best matrix rate; plus the time of each s relative to s=1
    (flat below the crossing, proportional to s above it)."""
    sh = wl.mla_mtp(1)
    bw, fl = measured_ceilings(dev)
    best = max(tf for _, tf in us.values()) * 1e12
    cross = lambda f, b: round(cm.mla_ridge_crossing_s(sh.h, sh.k, sh.p, sh.t_max, peak_flops=f, bw=b), 3)
    return {"sweep_summary": "mla_mtp ridge crossing (b=32, h=128, k=512, p=64, t=4096)",
            "spec_ridge_flop_per_byte": round(RIDGE, 1),
            "spec_crossing_s": cross(cm.MI355X_BF16_FLOPS, cm.MI355X_HBM_BYTES_PER_S),
            "measured_copy_tbs": round(bw / 1e12, 3), "measured_gemm_tflops": round(fl / 1e12, 1),
            "measured_ridge_flop_per_byte": round(fl / bw, 1), "measured_crossing_s": cross(fl, bw),
            "kernel_best_tflops": round(best / 1e12, 1), "kernel_crossing_s": cross(best, bw),
            "time_vs_s1": {str(s): round(t / us[1][0], 3) for s, (t, _) in sorted(us.items())}}


def cpu_baseline(parts, fraction):
    import oracle
    oracle.build(force=False)
    tot_flops = 0.0
    t0 = time.perf_counter()
    for p in parts:
        n = max(1, int(p.shape.rows * fraction))
        rows = wl.sample_rows(p.shape.rows, n, p.shape.seed).numpy()
        if p.kind == "mla":
            _, _, macs = oracle.mla(*p.cpu, p.shape.scale, rows=rows, return_macs=True)
        else:
            _, _, macs = oracle.gqa(*p.cpu, p.shape.scale, rows=rows, return_macs=True)
        tot_flops += 2.0 * macs
    dt = time.perf_counter() - t0
    return {"value": round(tot_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "fp64 oracle on a seeded %.0f%% sample of the query rows of each of the step's three "
                      "workloads (%.1f GFLOP, %.1f s)" % (100 * fraction, tot_flops / 1e9, dt)}


def load_traffic(name):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample", type=float, default=1.0,
                    help="fraction of each workload's query rows the fp64 oracle baseline computes")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="s-sweep of MLA (one JSON line per s)")
    ap.add_argument("--ragged", action="store_true", help="only the ragged long-context MLA workload")
    ap.add_argument("--crossover", action="store_true",
                    help="absorbed vs un-absorbed MLA decode over the s-sweep (b=32, h=128, t=4096)")
    ap.add_argument("--split", action="store_true",
                    help="split latent/decompressed cache at s=16 over n (b=32, h=128, t=4096)")
    ap.add_argument("--projections", action="store_true",
                    help="per-head query absorption and output decompression (b=32, h=128, d=128, k=512)")
    ap.add_argument("--gqa-long", action="store_true",
                    help="only the long-context GQA workload (t=262144, hq=24, hkv=4, d=256), both kernels")
    ap.add_argument("--only", default="", help="comma list of parts to run (gqa,mla_s1,mla_s4)")
    ap.add_argument("--gqa-path", type=int, default=0, help="GQA kernel: 0 auto, 1 VALU dot, 2 MFMA")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (the decode kernels shard by "
              "batch or KV head with no communication; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    binding.load_library()

    if args.ragged:
        p = Part("mla_ragged", "mla", wl.MLA_RAGGED, dev)
        wall, per = time_parts([p], args.steps, args.warmup)
        sec = per[p.name]
        c = cm.mla_absorbed_ragged(p.cpu[3].tolist(), p.shape.h, p.shape.s, p.shape.k, p.shape.p, p.shape.t_max,
                                   masked=False)
        t_min = cm.roofline_time(c)
        print(json.dumps({"workload": "mla_ragged (b=64, s=1, h=128, k=512, p=64, seqlens U{1024..32768}, seed 4)",
                          "us": round(sec * 1e6, 2), "tflops": round(c.flops / sec / 1e12, 2),
                          "tbs": round(c.bytes / sec / 1e12, 3), "ai": round(c.ai, 1),
                          "bound": "mfma" if c.ai > RIDGE else "hbm", "t_min_us": round(t_min * 1e6, 2),
                          "roofline_frac": round(t_min / sec, 4)}), flush=True)
        return

    if args.crossover:
        first = None
        for s in wl.MTP_SWEEP + (48, 64):
            pa = Part("mla_s%d" % s, "mla", wl.mla_mtp(s), dev)
            pu = UnabsorbedPart(s, dev)
            _, per = time_parts([pa, pu], args.steps, args.warmup)
            ta, tu = per[pa.name], per[pu.name]
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
        return

    if args.split:
        s = 16
        pa = Part("absorbed_s%d" % s, "mla", wl.mla_mtp(s), dev)
        _, per = time_parts([pa], args.steps, args.warmup)
        print(json.dumps({"split": "absorbed only (n=0)", "s": s, "us": round(per[pa.name] * 1e6, 2)}), flush=True)
        del pa
        for n in (64, 256, 1024, 2048, 4096):
            p = SplitPart(s, n, dev)
            _, per = time_parts([p], args.steps, args.warmup)
            sec = per[p.name]
            t_min = cm.roofline_time(p.cost)
            print(json.dumps({"split": "latent o + decompressed n (b=32, h=128, t=4096)", "s": s, "o": 4096 - n,
                              "n": n, "us": round(sec * 1e6, 2), "tflops": round(p.cost.flops / sec / 1e12, 2),
                              "tbs": round(p.cost.bytes / sec / 1e12, 3), "ai": round(p.cost.ai, 1),
                              "t_min_us": round(t_min * 1e6, 2), "roofline_frac": round(t_min / sec, 4)}),
                  flush=True)
            del p
            torch.cuda.empty_cache()
        return

    if args.projections:
        for s in (1, 4, 32):
            for kind in ("absorb", "decompress"):
                p = ProjectionPart(kind, s, dev)
                _, per = time_parts([p], args.steps, args.warmup)
                sec = per[p.name]
                t_min = max(p.flops / cm.MI355X_BF16_FLOPS, p.bytes / cm.MI355X_HBM_BYTES_PER_S)
                print(json.dumps({"projection": kind, "b": 32, "s": s, "h": 128, "d": 128, "k": 512,
                                  "us": round(sec * 1e6, 2), "tflops": round(p.flops / sec / 1e12, 2),
                                  "tbs": round(p.bytes / sec / 1e12, 3), "ai": round(p.flops / p.bytes, 1),
                                  "t_min_us": round(t_min * 1e6, 2), "roofline_frac": round(t_min / sec, 4)}),
                      flush=True)
                del p
        return

    if args.gqa_long:
        for path in (2, 1):
            p = Part("gqa_long", "gqa", wl.GQA_LONG, dev, path=path)
            wall, per = time_parts([p], args.steps, args.warmup)
            sec = per[p.name]
            c = p.cost
            print(json.dumps({"workload": "gqa_long (b=1, s=1, hq=24, hkv=4, d=256, t=262144, seed 6)",
                              "kernel": "mfma" if path == 2 else "valu",
                              "us": round(sec * 1e6, 2), "tflops": round(c.flops / sec / 1e12, 3),
                              "tbs": round(c.bytes / sec / 1e12, 3), "ai": round(c.ai, 1), "bound": p.bound,
                              "t_min_us": round(p.t_min * 1e6, 2), "roofline_frac": round(p.t_min / sec, 4)}),
                  flush=True)
            del p
        return

    if args.sweep:
        us = {}
        for s in wl.MTP_SWEEP:
            p = Part("mla_s%d" % s, "mla", wl.mla_mtp(s), dev)
            wall, per = time_parts([p], args.steps, args.warmup)
            sec = per[p.name]
            us[s] = (sec * 1e6, p.cost.flops / sec / 1e12)
            print(json.dumps({"sweep": "mla_mtp", "s": s, "us": round(sec * 1e6, 2),
                              "tflops": round(p.cost.flops / sec / 1e12, 2),
                              "tbs": round(p.cost.bytes / sec / 1e12, 3), "ai": round(p.cost.ai, 1),
                              "bound": p.bound, "t_min_us": round(p.t_min * 1e6, 2),
                              "roofline_frac": round(p.t_min / sec, 4)}), flush=True)
            del p
            torch.cuda.empty_cache()
        print(json.dumps(ridge_summary(us, dev)), flush=True)
        return

    parts = [Part("gqa", "gqa", wl.GQA_LAYER, dev, args.gqa_path), Part("mla_s1", "mla", wl.MLA_DSV3, dev),
             Part("mla_s4", "mla", wl.MLA_MTP4, dev)]
    if args.only:
        keep = set(args.only.split(","))
        parts = [p for p in parts if p.name in keep]
    wall, per = time_parts(parts, args.steps, args.warmup)

    flops = sum(p.cost.flops for p in parts)
    byts = sum(p.cost.bytes for p in parts)
    dom = max(parts, key=lambda p: per[p.name])
    roof = dom.roofline(per[dom.name])
    traffic = load_traffic(dom.name)
    roof["traffic"] = traffic
    roof["kernel"] = dom.name
    part_info = {}
    for p in parts:
        sec = per[p.name]
        part_info[p.name] = {"us": round(sec * 1e6, 2), "tflops": round(p.cost.flops / sec / 1e12, 2),
                             "tbs": round(p.cost.bytes / sec / 1e12, 3), "ai": round(p.cost.ai, 1),
                             "bound": p.bound, "t_min_us": round(p.t_min * 1e6, 2),
                             "roofline_frac": round(p.t_min / sec, 4),
                             "masked_tflops": round(p.flops_masked / sec / 1e12, 2)}
    res = {
        "metric": "decode-attn TFLOP/s + HBM TB/s (% of MI355X roofline), b=32 t=4096, s=1 and s=4",
        "value": round(flops / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
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
        "parts": part_info,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(parts, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
