#!/usr/bin/env python3
"""Throughput of the fused 2D Neighborhood Attention forward pass on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--pass forward|backward]

One step = one full forward pass (neighbourhood map, QK + bias, softmax, AV,
store) over one batch of the workload, on inputs already resident in HBM.
With --pass backward, one step is one backward pass instead (dq, dk, dv and
the bias gradient from q, k, v, the bias table and dout).
The default workload is the NAT-Tiny stage-1 layer: B=64, heads=2, 56x56,
D=32, k=7, d=1, bf16 (fp32 accumulation), seeded synthetic N(0,1) data.

To keep the 256 MB Infinity Cache from serving the inputs, the timed steps
rotate through enough input/output replicas to touch >= 1 GiB.  The K timed
launches are captured once in a HIP graph and replayed (launch overhead off
the host); wall time brackets the replay with device synchronisations, and
HIP events recorded on the same stream give the per-launch kernel time used
for the roofline figure.  After the replay, 100 eager steps are timed one by
one with their own HIP events (median, p10, p90 in per_launch_us).  The
default fused forward also times the unfused three-kernel path the same way
(the "unfused" object), and the float64 oracle runs on the host CPUs
(cpu_baseline: every CPU of the process's affinity mask, at most 16, the CPU
share of a one-GPU job on the GPU host; the count used and the host's are
both recorded) and on one (cpu_baseline_1core).  The default run also times
the DiNAT stage-1 (56x56, d=8) and stage-2 (28x28, d=4) layers the same way,
each a sub-object of "workloads" with its own roofline and cpu_baseline
(--also selects them).

Every pass checks a sample of its outputs against the oracle; the run exits
with status 3 (after printing its line) when an error exceeds the stated
tolerance: 1e-5 for fp32, 2e-2 for bf16/fp16, 2e-5 for the log-sum-exp.

Prints ONE JSON line (rank 0).  --gpus N > 1 is refused: this library's
benchmark runs on a single GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from vision_transformer_local_amd import inputs as I  # noqa: E402
from vision_transformer_local_amd import na2d  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
WORKLOADS = {
    "nat_tiny_s1": I.NAT_TINY_S1,
    "dinat_s1_d8": I.DINAT_S1_D8,
    "dinat_s2_d4": I.DINAT_S2_D4,
    "sweep_56": I.NAT_TINY_SWEEP[0], "sweep_28": I.NAT_TINY_SWEEP[1],
    "sweep_14": I.NAT_TINY_SWEEP[2], "sweep_7": I.NAT_TINY_SWEEP[3],
    "det_k7_d1_bf16": I.DETECTION[0], "det_k7_d1_f16": I.DETECTION[1],
    "det_k7_d8_bf16": I.DETECTION[2], "det_k7_d8_f16": I.DETECTION[3],
    "det_k13_d1_bf16": I.DETECTION[4], "det_k13_d1_f16": I.DETECTION[5],
    "det_k13_d8_bf16": I.DETECTION[6], "det_k13_d8_f16": I.DETECTION[7],
    "tiny_f32": I.TINY,
    "dinat_s1_d8_pad48": I.DINAT_S1_D8_PAD48,
}
BLOCK_WORKLOADS = {
    "block_56": I.BLOCK_SWEEP[0], "block_28": I.BLOCK_SWEEP[1],
    "block_14": I.BLOCK_SWEEP[2], "block_7": I.BLOCK_SWEEP[3],
}
# Kernel sources per measured family: a committed counter summary is used
# only while the sources of its family are unchanged.
_CSRC = "vision_transformer_local_amd/csrc/"
_SHARED = [_CSRC + "na2d_mfma_common.h", _CSRC + "na2d_internal.h"]
_FORWARD = [_CSRC + f for f in (
    "na2d_mfma.hip", "na2d_stream.hip", "na2d_dense.hip", "na2d_scalar.hip")] + _SHARED
SOURCE_FAMILIES = {
    "forward": _FORWARD,
    "block": [_CSRC + "na2d_linear.hip", _CSRC + "na2d_block.hip"] + _FORWARD,
    "backward": [_CSRC + "na2d_backward.hip", _CSRC + "na2d_backward_mfma.hip"] + _SHARED,
}


def elem_size(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def algorithmic_bytes(p) -> int:
    """Bytes the method itself must move: q, k, v read once, out written once,
    plus the bias table."""
    s = elem_size(p.dtype)
    side = 2 * p.kernel_size - 1
    return 4 * p.D * s * p.n_query_heads + p.heads * side * side * s


def backward_algorithmic_bytes(p) -> int:
    """Bytes the backward pass must move: q, k, v and dout read once, dq, dk
    and dv written once, the bias table read and its fp32 gradient written."""
    s = elem_size(p.dtype)
    side = 2 * p.kernel_size - 1
    return 7 * p.D * s * p.n_query_heads + p.heads * side * side * (s + 4)


def kernel_source_hash(which: str = "forward") -> str:
    h = hashlib.sha256()
    for rel in SOURCE_FAMILIES[which]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when none exists for this kernel source."""
    fn = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (path, workload))
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    family = path if path in ("backward", "block") else "forward"
    if rec.get("kernel_source_hash") != kernel_source_hash(family):
        return None  # kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(p, cpu_inputs, budget_s=10.0, min_runs=3, max_runs=500, backward=False,
                 pads=None, threads=None):
    """The float64 oracle on the host cores (all of them, or `threads`):
    whole-workload passes repeated until about budget_s seconds of CPU work,
    median pass time.  pads: the (pad_k, pad_v) of a padded forward."""
    import oracle
    threads = threads or oracle.default_threads()
    arrs = [t.to(torch.float64).numpy() for t in cpu_inputs]
    fn = oracle.backward if backward else oracle.forward
    if pads is not None:
        pk, pv = (t.to(torch.float64).numpy() for t in pads)

        def fn(q, k, v, rpb, ks, d, threads):
            return oracle.forward_padded(q, k, v, rpb, pk, pv, ks, d, threads=threads)
    times = []
    start = time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - start < budget_s
                                    and len(times) < max_runs):
        t0 = time.perf_counter()
        fn(*arrs, p.kernel_size, p.dilation, threads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": p.n_query_heads / t, "unit": "queries*heads/s", "cores": threads,
            "host_cpus": oracle.host_cpus(), "kind": "oracle",
            "threads_rule": "every CPU of the process's affinity mask, at most %d (a one-GPU "
                            "job's CPU share on the GPU host)" % oracle.MAX_THREADS,
            "sample": "whole workload (%d query-heads) run %d times in %.1f s, median pass, "
                      "float64" % (p.n_query_heads, len(times), time.perf_counter() - start)}


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Read+write GB/s of a plain device copy (torch) of nbytes: the
    bandwidth a simple streaming kernel attains on this GPU."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps / 1e3
    del src, dst
    return 2 * nbytes / t / 1e9


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="nat_tiny_s1",
                    choices=sorted(WORKLOADS) + sorted(BLOCK_WORKLOADS))
    ap.add_argument("--path", default="fused", choices=["fused", "tiled", "fma", "unfused"],
                    help="fused: the library's choice; tiled: the block-tiled matrix-core "
                         "kernel only; fma: the per-lane fp32 kernel; unfused: the three "
                         "kernels of the decomposition the pages show")
    ap.add_argument("--pass", dest="which", default="forward",
                    choices=["forward", "backward", "block"],
                    help="forward: the operator; backward: its gradients; block: the "
                         "attention block (projection -> NA -> projection) on the "
                         "block_* workloads")
    ap.add_argument("--padded", action="store_true",
                    help="forward through na2d_forward_padded (maps smaller than k*d are "
                         "padded with per-head pad vectors, attended and cropped)")
    ap.add_argument("--layout", default="dense", choices=["dense", "channels_last"],
                    help="forward I/O layout: dense [B, heads, H, W, D], or channels-last "
                         "[B, H, W, heads*D] through na2d_forward_strided")
    ap.add_argument("--lse", action="store_true",
                    help="forward through na2d_forward_lse (also writes each query's fp32 "
                         "log-sum-exp)")
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-launch", type=int, default=100,
                    help="eager steps timed one by one after the timed region (0: none)")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused path beside the fused forward")
    ap.add_argument("--no-copy-reference", action="store_true",
                    help="skip the device-copy bandwidth measurement")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--also", default="dinat_s1_d8,dinat_s2_d4",
                    help="further forward workloads timed in the same run (plain fused "
                         "forward only), each a sub-object of the JSON line under "
                         "'workloads'; empty: none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (each (batch, "
              "head) plane is independent, so more GPUs would each run this same kernel "
              "on their share of the batch)." % args.gpus, file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the factor that turns those counters into bytes.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": max(1, args.steps)}))
        return 0
    L = na2d.lib()
    if args.which == "block":
        return bench_block(args, dev, L)
    p = WORKLOADS[args.workload]
    if args.which == "backward":
        return bench_backward(args, p, dev, L)

    rec, ok = bench_forward(args, args.workload, dev, L, main_line=True)
    if rec is None:
        return 2
    plain = (args.path == "fused" and args.layout == "dense" and not args.padded
             and not args.lse)
    extras = [w for w in args.also.split(",") if w and w != args.workload] if plain else []
    for w in extras:
        if w not in WORKLOADS:
            print("--also: unknown workload %s" % w, file=sys.stderr)
            return 2
        sub, sub_ok = bench_forward(args, w, dev, L, main_line=False)
        rec.setdefault("workloads", {})[w] = sub
        ok = ok and sub_ok
    print(json.dumps(rec), flush=True)
    if not ok:
        print("sample error above the stated tolerance (%s)" % json.dumps(TOLERANCE),
              file=sys.stderr)
        return 3
    return 0


# Accuracy the library promises against the float64 oracle (absolute, on the
# same rounded inputs): the bench's own sample check fails the run above it.
TOLERANCE = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2, "lse": 2e-5}


def bench_forward(args, workload, dev, L, main_line=True):
    """One workload of the forward pass: the timed steps, the sample check
    against the oracle, the roofline figures and (unless switched off) the
    oracle's own rate.  Returns (record, sample within tolerance); the record
    of an extra workload (main_line False) carries no run-wide fields."""
    p = WORKLOADS[workload]
    cpu = I.make_inputs(p, seed=0)
    q0, k0, v0, rpb0 = cpu
    dt_code = {"f32": 0, "bf16": 1, "f16": 2}[p.dtype]
    algo = {"fused": 0, "fma": 1, "tiled": 3}.get(args.path, 0)
    B, heads, H, W, D = p.shape
    ks, dil = p.kernel_size, p.dilation
    cl = args.layout == "channels_last"
    if (cl or args.padded) and args.path != "fused":
        print("--layout channels_last and --padded take the fused path only", file=sys.stderr)
        return None, False
    if cl and args.padded:
        print("--padded takes the dense layout", file=sys.stderr)
        return None, False
    if args.lse and (cl or args.padded or args.path != "fused"):
        print("--lse takes the fused path on the dense layout", file=sys.stderr)
        return None, False
    span = p.kernel_size * p.dilation
    if not args.padded and (p.H < span or p.W < span):
        print("workload %s needs --padded (map below kernel*dilation)" % workload,
              file=sys.stderr)
        return None, False
    tbytes = q0.numel() * q0.element_size()
    attn_bytes = p.n_query_heads * p.kernel_size ** 2 * 4 if args.path == "unfused" else 0
    per_replica = 4 * tbytes + attn_bytes
    R = max(2, math.ceil(args.rotate_bytes / per_replica))
    rpb = rpb0.to(dev)
    reps = []

    def relayout(t):
        # [B, heads, H, W, D] -> channels-last [B, H, W, heads*D], viewed per head
        x = t.permute(0, 2, 3, 1, 4).reshape(t.shape[0], t.shape[2], t.shape[3], -1)
        return na2d.heads_view(x.contiguous().to(dev), t.shape[1])

    for _ in range(R):
        if cl:
            q, k, v = (relayout(t) for t in (q0, k0, v0))
            out = na2d.heads_view(torch.empty((B, H, W, heads * D), dtype=q.dtype, device=dev),
                                  heads)
        else:
            q, k, v = (t.to(dev) for t in (q0, k0, v0))
            out = torch.empty_like(q)
        attn = (torch.empty(p.shape[:4] + (p.kernel_size ** 2,), dtype=torch.float32,
                            device=dev) if args.path == "unfused" else None)
        if args.lse:  # the per-query log-sum-exp output rides in the attn slot
            attn = torch.empty(p.shape[:4], dtype=torch.float32, device=dev)
        reps.append((q, k, v, out, attn))

    gen = torch.Generator("cpu").manual_seed(500)
    pad_k, pad_v = (torch.randn(heads, D, generator=gen).to(q0.dtype).to(dev) for _ in range(2))
    si = (ctypes.c_int64 * 4)(*reps[0][0].stride()[:4])
    so = (ctypes.c_int64 * 4)(*reps[0][3].stride()[:4])

    def launch(i, stream):
        q, k, v, out, attn = reps[i % R]
        st = ctypes.c_void_p(stream)
        if args.path == "unfused":
            r = L.na2d_qkrpb(q.data_ptr(), k.data_ptr(), rpb.data_ptr(), attn.data_ptr(),
                             B, heads, H, W, D, ks, dil, dt_code, st)
            r = r or L.na2d_softmax(attn.data_ptr(), attn.data_ptr(), B, heads, H, W, ks, st)
            r = r or L.na2d_av(attn.data_ptr(), v.data_ptr(), out.data_ptr(),
                               B, heads, H, W, D, ks, dil, dt_code, st)
        elif args.padded:
            r = L.na2d_forward_padded(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                      pad_k.data_ptr(), pad_v.data_ptr(), out.data_ptr(), B,
                                      heads, H, W, D, ks, dil, dt_code, st)
        elif args.lse:
            r = L.na2d_forward_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                   out.data_ptr(), attn.data_ptr(), B, heads, H, W, D, ks, dil,
                                   dt_code, st)
        elif cl:
            r = L.na2d_forward_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                       out.data_ptr(), B, heads, H, W, D, ks, dil, si, so,
                                       dt_code, st)
        else:
            r = L.na2d_forward_algo(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                    out.data_ptr(), B, heads, H, W, D, ks, dil, dt_code,
                                    algo, st)
        if r != 0:
            raise RuntimeError("launch failed: " + na2d.na2d_status_string(r))

    ms_per_step, kernel_ms, per_launch = time_steps(args, launch, dev)
    K = args.steps

    # sanity: a sample of the first replica's output against the oracle
    import numpy as np
    import oracle
    idx = np.random.default_rng(0).choice(p.n_query_heads, size=min(4096, p.n_query_heads),
                                          replace=False)
    if args.padded:
        ref = oracle.forward_padded(q0, k0, v0, rpb0, pad_k.cpu(), pad_v.cpu(), ks,
                                    dil).reshape(-1, D)[idx]
    else:
        r = oracle.forward(q0, k0, v0, rpb0, ks, dil, idx=idx, lse=args.lse)
        ref = r["out"]
    got = reps[0][3].contiguous().reshape(-1, D)[torch.from_numpy(idx).to(dev)]
    got = got.double().cpu().numpy()
    max_err = float(np.abs(got - ref).max())
    ok = max_err <= TOLERANCE[p.dtype]
    lse_err = None
    if args.lse:
        gl = reps[0][4].reshape(-1)[torch.from_numpy(idx).to(dev)].double().cpu().numpy()
        lse_err = float(np.abs(gl - r["lse"]).max())
        ok = ok and lse_err <= TOLERANCE["lse"]
    del reps
    torch.cuda.empty_cache()

    value = p.n_query_heads / (ms_per_step / 1e3)
    abytes = algorithmic_bytes(p)
    if args.path == "unfused":
        abytes += 4 * p.n_query_heads * p.kernel_size ** 2 * 4  # fp32 attn w, r, w, r
    if args.lse:
        abytes += 4 * p.n_query_heads  # the fp32 log-sum-exp written
    achieved = abytes / (kernel_ms / 1e3) / 1e9
    traffic = measured_traffic(workload,
                               "strided" if cl else ("padded" if args.padded else
                                                     ("lse" if args.lse else args.path)))
    config = {"workload": "%s: %s" % (workload, p.describe()),
              "B": B, "heads": heads, "H": H, "W": W, "D": D,
              "kernel_size": ks, "dilation": dil, "path": args.path,
              "layout": args.layout, "padded": args.padded, "lse": args.lse,
              "timing": args.mode, "replicas": R}
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    if main_line:
        rec = {
            "metric": "NA2D fwd queries*heads/s (+ achieved HBM GB/s as % of MI355X peak)",
            "value": value,
            "unit": "queries*heads/s",
            "n_gpus": 1,
            "steps": K,
            "warmup": args.warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": p.dtype,
            "data": "synthetic (seeded N(0,1) q/k/v, 0.02*N(0,1) bias)",
            "config": config,
        }
    else:
        rec = {"value": value, "unit": "queries*heads/s", "ms_per_step": ms_per_step,
               "dtype": p.dtype, "config": config}
    rec.update({
        "roofline": roofline,
        "kernel_ms": kernel_ms,
        "per_launch_us": per_launch,
        "algorithmic_bytes_per_step": abytes,
        "sample_max_abs_err": max_err,
        "sample_within_tolerance": ok,
        "kernel_source_hash": kernel_source_hash(),
    })
    if args.lse:
        rec["sample_max_abs_err_lse"] = lse_err
    if (main_line and args.path == "fused" and not (cl or args.padded or args.lse)
            and not args.no_unfused):
        rec["unfused"] = unfused_beside(args, p, dev, L, cpu)
    if main_line and not args.no_copy_reference:
        copy_gbs = copy_bandwidth(dev)
        rec["copy_reference"] = {"copy_gbs": copy_gbs, "achieved_over_copy": achieved / copy_gbs,
                                 "what": "torch device copy of 1 GiB, read+write bytes"}
    if not args.no_cpu_baseline:
        pads = (pad_k.cpu(), pad_v.cpu()) if args.padded else None
        rec["cpu_baseline"] = cpu_baseline(p, cpu, pads=pads)
        if main_line:
            rec["cpu_baseline_1core"] = cpu_baseline(p, cpu, pads=pads, threads=1,
                                                     budget_s=8.0)
    return rec, ok


def unfused_beside(args, p, dev, L, cpu):
    """The unfused three-kernel path (scores + bias, softmax, weighted sum of
    values through an fp32 [.., k*k] tensor) on the same workload and inputs,
    timed with the same protocol, for the comparison beside the fused one."""
    q0, k0, v0, rpb0 = cpu
    B, heads, H, W, D = p.shape
    ks, dil = p.kernel_size, p.dilation
    dt_code = {"f32": 0, "bf16": 1, "f16": 2}[p.dtype]
    tbytes = q0.numel() * q0.element_size()
    attn_bytes = p.n_query_heads * ks * ks * 4
    R = max(2, math.ceil(args.rotate_bytes / (4 * tbytes + attn_bytes)))
    rpb = rpb0.to(dev)
    reps = [tuple(t.to(dev) for t in (q0, k0, v0)) +
            (torch.empty_like(q0, device=dev),
             torch.empty(p.shape[:4] + (ks * ks,), dtype=torch.float32, device=dev))
            for _ in range(R)]

    def launch(i, stream):
        q, k, v, out, attn = reps[i % R]
        st = ctypes.c_void_p(stream)
        r = L.na2d_qkrpb(q.data_ptr(), k.data_ptr(), rpb.data_ptr(), attn.data_ptr(),
                         B, heads, H, W, D, ks, dil, dt_code, st)
        r = r or L.na2d_softmax(attn.data_ptr(), attn.data_ptr(), B, heads, H, W, ks, st)
        r = r or L.na2d_av(attn.data_ptr(), v.data_ptr(), out.data_ptr(),
                           B, heads, H, W, D, ks, dil, dt_code, st)
        if r != 0:
            raise RuntimeError("launch failed: " + na2d.na2d_status_string(r))

    ms_per_step, kernel_ms, per_launch = time_steps(args, launch, dev)
    abytes = algorithmic_bytes(p) + 4 * attn_bytes  # fp32 attn written, read, written, read
    achieved = abytes / (kernel_ms / 1e3) / 1e9
    del reps
    torch.cuda.empty_cache()
    return {"path": "unfused (qkrpb -> softmax -> av, three launches)",
            "value": p.n_query_heads / (ms_per_step / 1e3), "unit": "queries*heads/s",
            "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, "per_launch_us": per_launch,
            "achieved_gbs": achieved, "frac": achieved / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": abytes, "replicas": R}


def per_launch_us(launch, stream, n=100, warm=10):
    """Eager launches, each bracketed by its own pair of HIP events on the
    launch stream: median, p10 and p90 of the n durations in microseconds
    (steps rotate through the replicas as in the timed region)."""
    import numpy as np
    for i in range(warm):
        launch(i, stream.cuda_stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        launch(warm + i, stream.cuda_stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90)), "n": n,
            "what": "HIP events around each of %d eager steps after %d warm-up steps" % (n, warm)}


def time_steps(args, launch, dev):
    """Warm up, capture K launches in a graph (or not), time them: returns
    (wall ms per step, event ms per step, per-launch statistics)."""
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        launch(i, stream.cuda_stream)
    torch.cuda.synchronize()
    K = args.steps
    graph = None
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                cap = torch.cuda.current_stream(dev).cuda_stream
                for i in range(K):
                    launch(i, cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            launch(i, stream.cuda_stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del graph
    per_launch = per_launch_us(launch, stream, n=args.per_launch) if args.per_launch > 0 else None
    return (t1 - t0) * 1e3 / K, ev0.elapsed_time(ev1) / K, per_launch


def block_algorithmic_bytes(p) -> int:
    """Bytes the block itself must move: x read and y written once, the
    weights, biases and bias table read once."""
    s = elem_size(p.dtype)
    side = 2 * p.kernel_size - 1
    M = p.B * p.H * p.W
    return (2 * M * p.C + 4 * p.C * p.C + 4 * p.C + p.heads * side * side) * s


def na2d_block_fused(p):
    """Whether the library's automatic plan runs this block as one kernel
    (mirrors the fused kernel's coverage: bf16/fp16, C = 64 in 2 heads,
    k in {3, 5, 7}, no dilation, no padding)."""
    return (p.dtype in ("bf16", "f16") and p.C == 64 and p.heads == 2 and
            p.kernel_size in (3, 5, 7) and p.dilation == 1 and
            min(p.H, p.W) >= p.kernel_size)


def bench_block(args, dev, L):
    """One step = the attention block (three launches) over the workload."""
    import numpy as np
    if args.workload not in BLOCK_WORKLOADS:
        print("--pass block takes a block_* workload", file=sys.stderr)
        return 2
    p = BLOCK_WORKLOADS[args.workload]
    cpu = I.make_block_inputs(p, seed=0)
    x0, w_qkv, b_qkv, rpb, w_out, b_out = cpu
    B, H, W, C = x0.shape
    ks, dil = p.kernel_size, p.dilation
    params = [t.to(dev) for t in (w_qkv, b_qkv, rpb, w_out, b_out)]
    wsb = na2d.na2d_block_workspace_size(B, H, W, C, p.heads, x0.dtype)
    xbytes = x0.numel() * x0.element_size()
    R = max(2, math.ceil(args.rotate_bytes / (2 * xbytes + wsb)))
    reps = [(x0.to(dev), torch.empty_like(x0, device=dev),
             torch.empty(wsb, dtype=torch.uint8, device=dev)) for _ in range(R)]
    dt_code = {"f32": 0, "bf16": 1, "f16": 2}[p.dtype]
    wq, bq, rp, wo, bo = params

    # --path fused: the library's choice (one fused kernel where it applies);
    # --path unfused: the three launches
    plan = na2d.BLOCK_UNFUSED if args.path == "unfused" else na2d.BLOCK_AUTO

    def launch(i, stream):
        x, y, ws = reps[i % R]
        r = L.na2d_block_forward_path(x.data_ptr(), wq.data_ptr(), bq.data_ptr(), rp.data_ptr(),
                                      wo.data_ptr(), bo.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                      wsb, B, H, W, C, p.heads, ks, dil, dt_code, plan,
                                      ctypes.c_void_p(stream))
        if r != 0:
            raise RuntimeError("launch failed: " + na2d.na2d_status_string(r))

    ms_per_step, kernel_ms, per_launch = time_steps(args, launch, dev)

    # sanity: a sample of pixels of the first replica against the oracle
    import oracle
    idx = np.random.default_rng(0).choice(B * H * W, size=min(2048, B * H * W), replace=False)
    dt = x0.dtype
    ref = oracle.block_forward(
        x0, w_qkv, b_qkv, rpb, w_out, b_out, p.heads, ks, dil,
        stored=lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).double().numpy())
    got = reps[0][1].reshape(-1, C)[torch.from_numpy(idx).to(dev)].double().cpu().numpy()
    refs = ref.reshape(-1, C)[idx]
    max_err = float(np.abs(got - refs).max())
    # the block's bound: the operator's tolerance plus one rounding of y
    ulp = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -23}[p.dtype]
    ok = float((np.abs(got - refs) - ulp * np.abs(refs)).max()) <= TOLERANCE[p.dtype]

    abytes = block_algorithmic_bytes(p)
    achieved = abytes / (kernel_ms / 1e3) / 1e9
    M = B * H * W
    rec = {
        "metric": "NA block pixels/s (+ achieved HBM GB/s as % of MI355X peak)",
        "value": M / (ms_per_step / 1e3),
        "unit": "pixels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) features, N(0,1/C) weights, 0.5*N(0,1) biases)",
        "config": {"workload": "%s block: %s" % (args.workload, p.describe()),
                   "B": B, "H": H, "W": W, "C": C, "heads": p.heads, "kernel_size": ks,
                   "dilation": dil, "path": "block_unfused" if plan == na2d.BLOCK_UNFUSED else
                   ("block_fused" if na2d_block_fused(p) else "block_unfused"),
                   "timing": args.mode, "replicas": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.workload, "block")},
        "kernel_ms": kernel_ms,
        "per_launch_us": per_launch,
        "algorithmic_bytes_per_step": abytes,
        "sample_max_abs_err": max_err,
        "sample_within_tolerance": ok,
        "kernel_source_hash": kernel_source_hash("block"),
    }
    print(json.dumps(rec), flush=True)
    if not ok:
        print("sample error above the stated tolerance", file=sys.stderr)
        return 3
    return 0


def bench_backward(args, p, dev, L):
    """One step = one backward pass (three kernel launches) over the workload."""
    import numpy as np
    B, heads, H, W, D = p.shape
    ks, dil = p.kernel_size, p.dilation
    q0, k0, v0, rpb0 = I.make_inputs(p, seed=0)
    gen = torch.Generator("cpu").manual_seed(1000)
    d0 = torch.randn(q0.shape, generator=gen, dtype=torch.float32).to(q0.dtype)
    tbytes = q0.numel() * q0.element_size()
    wsb = na2d.na2d_backward_workspace_size(B, heads, H, W, D, ks, dil, True)
    R = max(2, math.ceil(args.rotate_bytes / (7 * tbytes + wsb)))
    rpb = rpb0.to(dev)
    side = 2 * ks - 1
    drpb = torch.empty((heads, side, side), dtype=torch.float32, device=dev)
    reps = []
    for _ in range(R):
        ins = [t.to(dev) for t in (q0, k0, v0, d0)]
        outs = [torch.empty_like(ins[0]) for _ in range(3)]
        reps.append((ins, outs, torch.empty(wsb, dtype=torch.uint8, device=dev)))
    dt_code = {"f32": 0, "bf16": 1, "f16": 2}[p.dtype]

    def launch(i, stream):
        (q, k, v, dout), (dq, dk, dv), ws = reps[i % R]
        r = L.na2d_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            drpb.data_ptr(), ws.data_ptr(), wsb, B, heads, H, W, D, ks, dil,
                            dt_code, ctypes.c_void_p(stream))
        if r != 0:
            raise RuntimeError("launch failed: " + na2d.na2d_status_string(r))

    ms_per_step, kernel_ms, per_launch = time_steps(args, launch, dev)

    # sanity: the first replica's gradients against the oracle (skipped on the
    # largest maps, where the parity tests cover them)
    max_err, ok = None, True
    if p.n_query_heads * ks * ks <= 64 * 2 * 56 * 56 * 49:
        import oracle
        ref = oracle.backward(q0, k0, v0, rpb0, d0, ks, dil)
        got = [t.double().cpu().numpy() for t in reps[0][1]]
        got.append(drpb.double().cpu().numpy())
        names = ("dq", "dk", "dv", "drpb")
        max_err = max(float(np.abs(g - ref[n]).max()) for g, n in zip(got, names))
        # per element |gpu - oracle| <= r |oracle| + a rms(oracle): one
        # rounding of each gradient to its type plus fp32 accumulation (the
        # bias gradient is fp32 whatever the data type)
        for g, n in zip(got, names):
            r_, a_ = BACKWARD_TOLERANCE["f32" if n == "drpb" else p.dtype]
            rms = float(np.sqrt(np.mean(ref[n] ** 2))) or 1.0
            ok = ok and float((np.abs(g - ref[n]) - r_ * np.abs(ref[n])).max()) <= a_ * rms

    abytes = backward_algorithmic_bytes(p)
    achieved = abytes / (kernel_ms / 1e3) / 1e9
    rec = {
        "metric": "NA2D bwd queries*heads/s (+ achieved HBM GB/s as % of MI355X peak)",
        "value": p.n_query_heads / (ms_per_step / 1e3),
        "unit": "queries*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v/dout, 0.02*N(0,1) bias)",
        "config": {"workload": "%s backward: %s" % (args.workload, p.describe()),
                   "B": B, "heads": heads, "H": H, "W": W, "D": D,
                   "kernel_size": ks, "dilation": dil, "path": "backward",
                   "timing": args.mode, "replicas": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.workload, "backward")},
        "kernel_ms": kernel_ms,
        "per_launch_us": per_launch,
        "algorithmic_bytes_per_step": abytes,
        "sample_max_abs_err": max_err,
        "sample_within_tolerance": ok,
        "kernel_source_hash": kernel_source_hash("backward"),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(p, (q0, k0, v0, rpb0, d0), backward=True)
    print(json.dumps(rec), flush=True)
    if not ok:
        print("gradient error above the stated tolerance", file=sys.stderr)
        return 3
    return 0


# (relative, absolute-over-rms) bounds of the backward pass per data type
BACKWARD_TOLERANCE = {"bf16": (2.0 ** -8, 1e-3), "f16": (2.0 ** -10, 3e-4), "f32": (1e-5, 1e-5)}


if __name__ == "__main__":
    sys.exit(main())
