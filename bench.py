#!/usr/bin/env python3
"""Benchmark of the scalar affine scan on one MI355X.

One step = the whole scalar hot path over one batch: scan_fwd then scan_bwd
(fp32, layout [B, C, T], B=8, C=1536, T=4096, h0 per row) -- the kernel-level
"forward + backward combined" measurement of the associative-scan-triton
README's benchmark shape. Inputs are seeded synthetic tensors resident in HBM
before the timed region starts.

Printed: one JSON line.
- `value`: algorithmic throughput of the step in GB/s over K back-to-back
  timed steps (32 bytes per element: g, x read and h written by the forward;
  g, h, dy read and dx, dg written by the backward).
- `roofline`: the dominant kernel (the backward), from HIP-event durations of
  its launches inside the timed region (event pairs on every fifth step, so
  their cost stays out of most of the timed steps).
- `protocol`: the README's timing protocol ("performance": device events with
  the cache cleared between repetitions): for every measurement below, each
  repetition is preceded by a 1 GiB write to a scratch buffer (outside the
  timed interval, larger than the L2 caches and the 256 MB Infinity Cache),
  timed alone with HIP events on the launch stream, after as many untimed
  flushed warm-up repetitions; median, p10 and p90 are reported, with
  elements/s, GB/s and the fraction of the 8 TB/s peak.
- `ceilings`: the practical bandwidth for each kernel's exact bytes and
  read:write mix, from the library's streaming kernel (mscan_stream_ceiling).
- `cpu_baseline` (headline) and `cpu_oracle` (every other workload): the fp64
  oracle on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--T 4096] [--reps R]
                    [--no-sweep] [--no-workloads] [--no-cpu-baseline] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "GB/s & % HBM peak, scalar scan fwd/fwd+bwd B=8 C=1536 T=4K–64K"
BYTES_FWD, BYTES_BWD = 12, 20  # algorithmic bytes per element, fp32
# Kernel-level forward+backward times the associative-scan-triton README reports
# for this workload (B=8, C=1536) on an H100 80GB, per T ("performance",
# kernel-level table; other hardware, context only).
PAGE_FWDBWD_MS = {128: 0.027, 256: 0.043, 512: 0.077, 1024: 0.161, 2048: 0.306, 4096: 0.602,
                  8192: 1.186, 16384: 2.322, 32768: 4.602, 65536: 9.212}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scalar_B8_C1536_T4096.json")
FLUSH_BYTES = 1 << 30


def source_sha():
    """Hash of everything that decides the kernels' code: every source under
    csrc/, the public header and the build script (which holds the flags)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "associative_scan_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".cpp", ".h")))
    files += [os.path.join(ROOT, "include", "mscan.h"), os.path.join(ROOT, "associative_scan_amd", "build.py")]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--T", type=int, default=4096)
    p.add_argument("--reps", type=int, default=50, help="timed repetitions per protocol measurement")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-workloads", action="store_true", help="skip the packed, log-space and matrix workloads")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also launch one plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


EV_EVERY = 5  # steps between per-launch event pairs in the timed region


class Protocol:
    """Per-repetition timing with the caches flushed between repetitions."""

    def __init__(self, torch, dev, stream, reps):
        self.torch, self.stream, self.reps = torch, stream, reps
        self.flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.n_flush = 0

    def flush(self):
        self.n_flush += 1
        self.flush_buf.fill_(float(self.n_flush & 7))

    def time(self, fn, reps=None):
        torch = self.torch
        reps = reps or self.reps
        # warm-up: as many untimed repetitions, each behind its flush, as are
        # timed (the first few dozen calls on freshly allocated tensors run
        # up to 10% slower than the steady state)
        for _ in range(reps):
            self.flush()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in evs:
            self.flush()
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        q = lambda f: ms[min(len(ms) - 1, int(round(f * (len(ms) - 1))))]
        return {"median_ms": q(0.5), "p10_ms": q(0.1), "p90_ms": q(0.9), "reps": reps}


def _rate(t, nbytes, units, unit):
    """Throughput entry from a Protocol.time result (median; p10/p90 time)."""
    med = t["median_ms"] * 1e-3
    gbps = nbytes / med / 1e9
    return {"ms": round(t["median_ms"], 5), "p10_ms": round(t["p10_ms"], 5), "p90_ms": round(t["p90_ms"], 5),
            "reps": t["reps"], "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            f"{unit}_per_s": round(units / med, 1), "bytes": nbytes}


def ceiling(m, torch, dev, proto, nsrc, ndst, n_floats):
    """GB/s of the streaming kernel moving nsrc reads + ndst writes of n floats."""
    n = (n_floats + 3) // 4 * 4
    src = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(nsrc)]
    dst = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(ndst)]
    t = proto.time(lambda: m.stream_ceiling(src, dst))
    nbytes = (nsrc + ndst) * 4 * n
    del src, dst
    torch.cuda.empty_cache()
    return {"mix": f"{nsrc}r:{ndst}w", "gbps": round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1),
            "ms": round(t["median_ms"], 5), "bytes": nbytes}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(rows would shard across GPUs with no communication). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import associative_scan_amd as m
    import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, C, T = 8, 1536, args.T
    n = B * C * T

    # ---- inputs (seeded, resident in HBM) --------------------------------
    d = gen.dense(B, C, T)
    g = torch.from_numpy(d["g"]).to(dev)
    x = torch.from_numpy(d["x"]).to(dev)
    h0 = torch.from_numpy(d["h0"]).to(dev)
    dy = torch.from_numpy(d["dy"]).to(dev)
    host = d
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        h = m.scan_fwd(g, x, h0=h0)
        if ev is not None:
            ev[1].record(stream)
        dx, dg, dh0 = m.scan_bwd(g, h, dy, h0=h0)
        if ev is not None:
            ev[2].record(stream)
        return h, dx, dg, dh0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed region: K steps back to back ----------------------------
    # Per-launch HIP events (the roofline's kernel durations) are recorded on
    # every EV_EVERY-th step: each record drains the queue and costs a few
    # microseconds, which on every step would add ~4% to the whole-step time.
    inst = [i for i in range(args.steps) if i % EV_EVERY == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in inst}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        out = step(evs.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs.values()]
    fwd_avg, bwd_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    gbps = (BYTES_FWD + BYTES_BWD) * n / (ms_step * 1e-3) / 1e9
    bwd_gbps = BYTES_BWD * n / (bwd_avg * 1e-3) / 1e9
    fwd_gbps = BYTES_FWD * n / (fwd_avg * 1e-3) / 1e9
    del out

    # ---- the protocol: flushed repetitions, median / p10 / p90 -------------
    proto = Protocol(torch, dev, stream, args.reps)
    hcur = m.scan_fwd(g, x, h0=h0)
    protocol = {
        "flush_bytes_between_reps": FLUSH_BYTES,
        "headline": {
            "fwd": _rate(proto.time(lambda: m.scan_fwd(g, x, h0=h0)), BYTES_FWD * n, n, "elements"),
            "bwd": _rate(proto.time(lambda: m.scan_bwd(g, hcur, dy, h0=h0)), BYTES_BWD * n, n, "elements"),
            "fwd_bwd": _rate(proto.time(lambda: step()), (BYTES_FWD + BYTES_BWD) * n, n, "elements"),
        },
    }
    del hcur
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.empty_cache()
    ceilings = {"headline_fwd": ceiling(m, torch, dev, proto, 2, 1, n),
                "headline_bwd": ceiling(m, torch, dev, proto, 3, 2, n)}

    # ---- T sweep (forward and forward+backward), on-device random inputs ---
    sweep = []
    if not args.no_sweep:
        del g, x, dy
        torch.cuda.empty_cache()
        gen_t = torch.Generator(device=dev)
        gen_t.manual_seed(1234)
        for Ts in (128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
            ns = B * C * Ts
            gs = torch.rand((B, C, Ts), device=dev, generator=gen_t)
            xs = torch.randn((B, C, Ts), device=dev, generator=gen_t)
            dys = torch.randn((B, C, Ts), device=dev, generator=gen_t)

            def run(bwd):
                hs = m.scan_fwd(gs, xs, h0=h0)
                if bwd:
                    m.scan_bwd(gs, hs, dys, h0=h0)

            res = {"T": Ts, "elements": ns}
            for name, bwd, nb in (("fwd", False, BYTES_FWD), ("fwd_bwd", True, BYTES_FWD + BYTES_BWD)):
                res[name] = _rate(proto.time(lambda: run(bwd)), nb * ns, ns, "elements")
            if Ts in PAGE_FWDBWD_MS:
                res["page_h100_fwd_bwd_ms"] = PAGE_FWDBWD_MS[Ts]
            sweep.append(res)
            del gs, xs, dys
            torch.cuda.empty_cache()

    # ---- the other workloads of the scan family (performance only) -----------
    workloads = {}
    if not args.no_workloads:
        workloads = other_workloads(m, gen, torch, dev, proto, np)

    # ---- CPU baseline: the fp64 oracle on the host ----------------------------
    cpu = cpu_oracle = None
    if not args.no_cpu_baseline:
        import oracle
        nrows = B * C
        gs, xs = host["g"].reshape(-1, T), host["x"].reshape(-1, T)
        dys, h0s = host["dy"].reshape(-1, T), host["h0"].reshape(-1)
        times = []
        t_budget = time.time()
        # the whole workload, repeated for about 10 s of host time (at least 3 runs)
        while len(times) < 3 or (time.time() - t_budget < 10.0 and len(times) < 200):
            t0 = time.perf_counter()
            hr = oracle.scan_fwd(gs, xs, h0=h0s)
            oracle.scan_bwd(gs, hr, dys, h0=h0s)
            times.append(time.perf_counter() - t0)
            del hr
        t_med = float(np.median(times))
        cpu = {"value": round((BYTES_FWD + BYTES_BWD) * nrows * T / t_med / 1e9, 3), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"the full workload ({nrows} rows x T={T}), forward+backward, median of {len(times)} runs "
                         f"({t_med * 1e3:.1f} ms each, {sum(times):.1f} s total), fp64 C oracle with OpenMP over rows, "
                         "fp64 conversion of inputs included"}
        del host, gs, xs, dys
        cpu_oracle = oracle_workloads(oracle, gen, np)

    # ---- HBM traffic from committed rocprofv3 counter runs -------------------
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha") == source_sha() and tr.get("T") == T:
            traffic = tr["bwd_bytes_per_launch"]

    rec = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGE_FWDBWD_MS[T] / ms_step, 3) if T in PAGE_FWDBWD_MS else None,
        "vs_baseline_ref": (f"H100 80GB kernel-level fwd+bwd {PAGE_FWDBWD_MS[T]} ms for the same workload "
                            "(associative-scan-triton README); other hardware, context only")
        if T in PAGE_FWDBWD_MS else None,
        "dtype": "f32",
        "data": "synthetic (seeded: g~U(0,1), x~N(0,1), h0~N(0,1), dy~N(0,1))",
        "config": {"workload": f"scalar scan forward+backward, B={B} C={C} T={T}, fp32, layout [B,C,T], h0 per row",
                   "B": B, "C": C, "T": T, "elements": n, "bytes_per_step": (BYTES_FWD + BYTES_BWD) * n},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "elements_per_s": round(n / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "scan_bwd (k_scalar<float, bwd>)",
                     "achieved": round(bwd_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": BYTES_BWD * n, "avg_launch_ms": round(bwd_avg, 5),
                     "launches_timed": len(bwd_ms)},
        "kernels": {"scan_fwd": {"avg_launch_ms": round(fwd_avg, 5), "gbps": round(fwd_gbps, 1),
                                 "frac": round(fwd_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": BYTES_FWD * n},
                    "scan_bwd": {"avg_launch_ms": round(bwd_avg, 5), "gbps": round(bwd_gbps, 1),
                                 "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": BYTES_BWD * n}},
        "protocol": protocol,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "cpu_oracle": cpu_oracle,
        "sweep": sweep,
        "workloads": workloads,
        "kernel_source_sha": source_sha(),
    }
    print(json.dumps(rec), flush=True)


def other_workloads(m, gen, torch, dev, proto, np):
    """Packed bidirectional bf16, log-space and matrix-affine workloads at their
    full shapes, each with the streaming ceiling for its read:write mix. Inputs
    are drawn on the device with the workloads' distributions (values do not
    affect the timing); parity of the same shapes is checked by the GPU tests."""
    out = {}
    gt = torch.Generator(device=dev)
    gt.manual_seed(2024)

    # packed variable-length, two branches in opposite directions, bf16 inputs
    C, Tt = 1536, 65536
    L = gen.varlen_lengths(np.random.default_rng(3), 16, Tt, 8192)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(L)]), dtype=torch.int32, device=dev)
    br = []
    for _ in range(2):
        g = torch.sigmoid(torch.randn((C, Tt), device=dev, generator=gt) + 2.0)
        g[:, torch.rand(Tt, device=dev, generator=gt) < 1.0 / 1024] = 0.0
        br.append((g.to(torch.bfloat16), torch.randn((C, Tt), device=dev, generator=gt).to(torch.bfloat16)))
    dy = torch.randn((C, Tt), device=dev, generator=gt)
    n = C * Tt

    def vf():
        return [m.scan_fwd(b[0], b[1], cu_seqlens=cu, reverse=(i == 1)) for i, b in enumerate(br)]

    def vfb():
        hs = vf()
        for i, b in enumerate(br):
            m.scan_bwd(b[0], hs[i], dy, cu_seqlens=cu, reverse=(i == 1), need_dh0=False)

    h_one = m.scan_fwd(br[0][0], br[0][1], cu_seqlens=cu)
    out["varlen_bidir_bf16"] = {
        "workload": "C=1536, 65536 packed tokens in 16 sequences, bf16 g and x, fp32 h, two branches (causal + reverse)",
        "fwd": _rate(proto.time(vf), 2 * 8 * n, 2 * n, "elements"),
        "fwd_one_branch": _rate(proto.time(lambda: m.scan_fwd(br[0][0], br[0][1], cu_seqlens=cu)), 8 * n, n,
                                "elements"),
        "bwd_one_branch": _rate(proto.time(lambda: m.scan_bwd(br[0][0], h_one, dy, cu_seqlens=cu, need_dh0=False)),
                                18 * n, n, "elements"),
        "fwd_bwd": _rate(proto.time(vfb), 2 * (8 + 18) * n, 2 * n, "elements")}
    del br, h_one
    torch.cuda.empty_cache()
    # bytes of one branch: forward 4 B read : 4 B written per element; backward 10 : 8
    out["varlen_bidir_bf16"]["ceilings"] = {"fwd": ceiling(m, torch, dev, proto, 1, 1, n),
                                            "bwd": ceiling(m, torch, dev, proto, 4, 3, (18 * n) // 28)}

    # the same packed workload given gate logits z ~ N(2, 1) (bf16; resets z = -inf):
    # g = sigmoid(z) is computed inside the scan kernels
    bz = []
    for _ in range(2):
        z = torch.randn((C, Tt), device=dev, generator=gt) + 2.0
        z[:, torch.rand(Tt, device=dev, generator=gt) < 1.0 / 1024] = float("-inf")
        bz.append((z.to(torch.bfloat16), torch.randn((C, Tt), device=dev, generator=gt).to(torch.bfloat16)))

    def zf():
        return [m.scan_fwd_gated(b[0], b[1], cu_seqlens=cu, reverse=(i == 1)) for i, b in enumerate(bz)]

    def zfb():
        hs = zf()
        for i, b in enumerate(bz):
            m.scan_bwd_gated(b[0], hs[i], dy, cu_seqlens=cu, reverse=(i == 1), need_dh0=False)

    out["varlen_bidir_bf16_logits"] = {
        "workload": "the packed bidirectional workload with bf16 gate logits, g = sigmoid(z) fused into the scan",
        "fwd": _rate(proto.time(zf), 2 * 8 * n, 2 * n, "elements"),
        "fwd_bwd": _rate(proto.time(zfb), 2 * (8 + 18) * n, 2 * n, "elements")}
    del bz, dy
    torch.cuda.empty_cache()

    # log space
    B, D, T = 8, 1024, 8192
    la = -torch.nn.functional.softplus(torch.randn((B, D, T), device=dev, generator=gt))
    lb = torch.randn((B, D, T), device=dev, generator=gt)
    n = B * D * T
    dyl = torch.randn((B, D, T), device=dev, generator=gt)
    hl = m.scan_log_fwd(la, lb)

    def lfb():
        h_ = m.scan_log_fwd(la, lb)
        m.scan_log_bwd(la, lb, h_, dyl, need_dh0=False)

    out["logspace"] = {"workload": "B=8 D=1024 T=8192 fp32, log_a = -softplus(N(0,1)), log_b ~ N(0,1), dy ~ N(0,1)",
                       "fwd": _rate(proto.time(lambda: m.scan_log_fwd(la, lb)), 12 * n, n, "elements"),
                       "bwd": _rate(proto.time(lambda: m.scan_log_bwd(la, lb, hl, dyl, need_dh0=False)),
                                    24 * n, n, "elements"),
                       "fwd_bwd": _rate(proto.time(lfb), 36 * n, n, "elements")}
    del la, hl
    # the same workload given the gate logits: log_a = -softplus(z) fused into the scan
    zl = torch.randn((B, D, T), device=dev, generator=gt)
    hz = m.scan_log_fwd_gated(zl, lb)

    def zlfb():
        h_ = m.scan_log_fwd_gated(zl, lb)
        m.scan_log_bwd_gated(zl, lb, h_, dyl, need_dh0=False)

    out["logspace_logits"] = {"workload": "B=8 D=1024 T=8192 fp32, logits z ~ N(0,1) with log_a = -softplus(z) fused",
                              "fwd": _rate(proto.time(lambda: m.scan_log_fwd_gated(zl, lb)), 12 * n, n, "elements"),
                              "bwd": _rate(proto.time(lambda: m.scan_log_bwd_gated(zl, lb, hz, dyl, need_dh0=False)),
                                           24 * n, n, "elements"),
                              "fwd_bwd": _rate(proto.time(zlfb), 36 * n, n, "elements")}
    del zl, hz, lb, dyl
    torch.cuda.empty_cache()
    out["logspace"]["ceilings"] = {"fwd": ceiling(m, torch, dev, proto, 2, 1, n),
                                   "bwd": ceiling(m, torch, dev, proto, 4, 2, n)}

    # matrix-affine: rotations (k=2, v=1) and scaled orthogonal blocks (k=4, v=4
    # over 8 x 512 blocks, T=8192; k=16, v=16 over 8 x 64 blocks, T=4096)
    for name, k, v in (("matrix_rot2", 2, 1), ("matrix_orth4", 4, 4), ("matrix_orth16", 16, 16)):
        R, T = (8 * 64, 4096) if k == 16 else (8 * 512, 8192)
        if k == 2:
            rr = 0.5 + 0.5 * torch.rand((R, T), device=dev, generator=gt)
            th = (torch.rand((R, T), device=dev, generator=gt) * 2 - 1) * np.pi
            A = torch.stack([torch.stack([rr * th.cos(), -rr * th.sin()], -1),
                             torch.stack([rr * th.sin(), rr * th.cos()], -1)], -2)
            del rr, th
        else:
            A = torch.randn((R, T, k, k), device=dev, generator=gt)
            for j in range(k):  # Gram-Schmidt on the columns
                for i in range(j):
                    A[..., :, j] -= (A[..., :, i] * A[..., :, j]).sum(-1, keepdim=True) * A[..., :, i]
                A[..., :, j] /= A[..., :, j].norm(dim=-1, keepdim=True)
            A *= 0.9
        A[torch.rand((R, T), device=dev, generator=gt) < 1.0 / 2048] = 0.0
        Bm = torch.randn((R, T, k, v), device=dev, generator=gt)
        dyk = torch.randn((R, T, k, v), device=dev, generator=gt)
        h = m.matrix_affine_scan_fwd(A, Bm)
        fb, bb = 4 * (k * k + 2 * k * v), 4 * (2 * k * k + 3 * k * v)
        steps = R * T
        out[name] = {"workload": f"B=8 x {R // 8} state blocks, T={T}, k={k} v={v}, fp32, resets 1/2048",
                     "fwd": _rate(proto.time(lambda: m.matrix_affine_scan_fwd(A, Bm)), fb * steps, steps,
                                  "steps"),
                     "bwd": _rate(proto.time(lambda: m.matrix_affine_scan_bwd(A, h, dyk, need_dh0=False)),
                                  bb * steps, steps, "steps")}
        del A, Bm, dyk, h
        torch.cuda.empty_cache()
        # forward reads k^2 + kv and writes kv floats per step; backward reads
        # k^2 + 2kv and writes k^2 + kv; the ceiling streams the same bytes in
        # the nearest supported mix of whole arrays
        kk, kv = k * k, k * v
        fwd_mix = (2, 1) if kk == kv else (3, 1)
        bwd_mix = (3, 2) if kk == kv else (4, 3)
        out[name]["ceilings"] = {
            "fwd": ceiling(m, torch, dev, proto, *fwd_mix, (fb * steps) // (4 * sum(fwd_mix))),
            "bwd": ceiling(m, torch, dev, proto, *bwd_mix, (bb * steps) // (4 * sum(bwd_mix)))}
    return out


def _oracle_time(fn, np, max_runs=3, budget_s=3.0):
    """Median wall time of fn() over up to max_runs runs (stopping once the
    runs so far exceed budget_s), and the number of runs."""
    ts = []
    t_all = time.perf_counter()
    while len(ts) < max_runs:
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s:
            break
    return float(np.median(ts)), len(ts)


def oracle_workloads(oracle, gen, np):
    """The fp64 oracle timed on the host on every workload the parity tests
    use: full tensors where they fit a few seconds of host time, else a stated
    subset of rows at full length. Throughput is algorithmic bytes (the GPU
    kernels' fp32 / bf16 byte counts) over wall time, fp64 conversion of the
    inputs included."""
    res = {}
    threads = oracle.num_threads()

    def entry(t, runs, nbytes, units, unit, rows_used, rows_total, what):
        return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", f"{unit}_per_s": round(units / t, 1),
                "ms": round(t * 1e3, 2), "runs": runs, "rows_used": rows_used, "rows_total": rows_total,
                "cores": threads, "sample": what}

    # quick start (C=4, T=128), forward + backward
    q = gen.quickstart()
    t, r = _oracle_time(lambda: oracle.scan_bwd(q["g"], oracle.scan_fwd(q["g"], q["x"]), q["dy"]), np, 50, 1.0)
    res["quickstart_C4_T128"] = entry(t, r, 32 * 4 * 128, 4 * 128, "elements", 4, 4, "full, forward+backward")

    # dense B=8 C=1536, T = 128 .. 8192, forward + backward, all rows
    for T in (128, 512, 2048, 8192):
        d = gen.dense(8, 1536, T)
        gs, xs, dys, h0s = (d["g"].reshape(-1, T), d["x"].reshape(-1, T), d["dy"].reshape(-1, T),
                            d["h0"].reshape(-1))
        t, r = _oracle_time(lambda: oracle.scan_bwd(gs, oracle.scan_fwd(gs, xs, h0=h0s), dys, h0=h0s), np)
        ne = 12288 * T
        res[f"dense_T{T}"] = entry(t, r, 32 * ne, ne, "elements", 12288, 12288, "full, forward+backward")
        del d, gs, xs, dys, h0s

    # packed bidirectional (bf16 values widened exactly), both branches forward
    vb = gen.varlen_bidir()
    cu = vb["cu_seqlens"]
    t, r = _oracle_time(lambda: [oracle.scan_fwd(vb[b]["g"], vb[b]["x"], cu_seqlens=cu, reverse=vb[b]["reverse"])
                                 for b in ("fwd", "bwd")], np, 2)
    ne = 1536 * 65536
    res["varlen_bidir_bf16"] = entry(t, r, 2 * 8 * ne, 2 * ne, "elements", 1536, 1536,
                                     "full, forward of both branches")
    del vb

    # log space B=8 D=1024 T=8192, forward
    ls = gen.logspace()
    la, lb = ls["log_a"].reshape(-1, 8192), ls["log_b"].reshape(-1, 8192)
    t, r = _oracle_time(lambda: oracle.scan_log_fwd(la, lb), np, 2)
    ne = 8192 * 8192
    res["logspace"] = entry(t, r, 12 * ne, ne, "elements", 8192, 8192, "full, forward")
    del ls, la, lb

    # matrix 2x1 rotations, forward + reverse adjoint, all 4096 rows
    mr = gen.matrix_rot2()
    t, r = _oracle_time(lambda: oracle.matrix_affine_scan_bwd(mr["A"], oracle.matrix_affine_scan_fwd(mr["A"], mr["B"]),
                                                              mr["dy"]), np, 2)
    ns = 4096 * 8192
    res["matrix_rot2"] = entry(t, r, (4 * (4 + 4) + 4 * (8 + 6)) * ns, ns, "steps", 4096, 4096,
                               "full, forward+backward")
    del mr

    # matrix 4x4: 256 of the 4096 rows (every 16th) at full T=8192 (the full
    # workload would need ~20 GB of fp64 host arrays), forward+backward
    rows = np.arange(0, 4096, 16)
    mo = gen.matrix_orth4(rows=rows)
    t, r = _oracle_time(lambda: oracle.matrix_affine_scan_bwd(mo["A"], oracle.matrix_affine_scan_fwd(mo["A"], mo["B"]),
                                                              mo["dy"]), np, 2)
    ns = len(rows) * 8192
    res["matrix_orth4"] = entry(t, r, (4 * (16 + 32) + 4 * (32 + 48)) * ns, ns, "steps", len(rows), 4096,
                                "256 rows (every 16th) at full T, forward+backward")
    del mo
    return res


if __name__ == "__main__":
    main()
