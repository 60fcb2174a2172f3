"""Benchmark of the MI355X FlashAttention forward library.

One step = one ``fa_forward`` call over the prefill workload the metric is
quoted on (B=1, H=32, Nq=Nk=2048, D=128, bf16, non-causal), inputs already
resident in HBM. The metric's second half, split-KV decode bandwidth, is
measured in the same run on the decode workload (B=16, H=32, one query,
Nk=32768, D=128, 64 splits) and reported under "decode". The backward pass
(recompute from the saved LSE) is timed on the prefill workload and reported
under "backward". Prints ONE JSON line.

Timing: W untimed warm-up steps plus untimed steps until half a second of GPU
work has run (the engine clock ramps up under load), then K steps between two
HIP events recorded on the stream the kernels are launched on (torch's current
stream, which is the stream handed to the library), synchronised on both
sides.

Algorithmic counts (not the implementation's):
  prefill FLOPs = 4*B*H*Nq*Nk*D (halved when causal)
  bytes         = Q, K, V read once + O written once (+ LSE, fp32)
  backward FLOPs = 10*B*H*Nq*Nk*D (S, dP, dV, dQ, dK: five products; halved
                   when causal), the recompute of S counted
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s & % bf16 MFMA peak (prefill); decode GB/s & % HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "flashattention_online_softmax_forward_amd", "csrc")


def _code_only(text):
    """Source text without comments, trailing blanks or empty lines, so that a
    comment edit leaves the digest of a kernel's code unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name, digest):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    in profiles/<name>.md, or None when absent or taken on other kernel source."""
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None
    return float(m_b.group(1))


def workload_counts(w):
    flops = 4.0 * w.B * w.H * w.Nq * w.Nk * w.D * (0.5 if w.causal else 1.0)
    elem = 4 if w.dtype.is_floating_point and w.dtype.itemsize == 4 else 2
    bytes_ = elem * w.B * w.H * (2 * w.Nq * w.D + 2 * w.Nk * w.D) + 4 * w.B * w.H * w.Nq
    return flops, bytes_


def time_steps(fn, steps, warmup, torch, settle_s=0.5):
    """W warm-up calls, then keep calling (untimed) until ``settle_s`` seconds
    of GPU work have run, so the engine clock has ramped up before the timed
    region; then K timed calls between two events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(w, q, k, v, budget_s):
    """The fp64 oracle as it stands, on the host, over whole heads of the same
    workload until about ``budget_s`` seconds of work are done."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as orc

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    flops_head = 4.0 * w.Nq * w.Nk * w.D * (0.5 if w.causal else 1.0)
    done, t_total, passes = 0, 0.0, 0
    widened = {}
    # Whole heads in order, over and over (the workload is one pass) until the
    # budget is spent; only the oracle call itself is timed.
    while t_total < budget_s:
        for (b, h) in heads:
            if (b, h) not in widened:
                widened[(b, h)] = tuple(x[b, h].float().cpu().numpy().astype(np.float64)[None, None]
                                        for x in (q, k, v))
            qh, kh, vh = widened[(b, h)]
            t0 = time.perf_counter()
            orc.attention(qh, kh, vh, w.scale, w.causal)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": flops_head * done / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} head computations ({done / len(heads):.2f} passes over the {len(heads)} heads) of "
                  f"{w.name}, fp64 two-pass, every row, {t_total:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_b1_h32_n2048_d128")
    ap.add_argument("--decode-workload", default="decode_b16_h32_kv32768_d128_s64")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--backward-workload", default=None, help="default: --workload")
    ap.add_argument("--backward-steps", type=int, default=50)
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many bytes "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on a single GPU; there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import flashattention_online_softmax_forward_amd as fa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ms = time_steps(lambda: dst.copy_(src), args.steps, args.warmup, torch)
        print(json.dumps({"copy_bytes": n * 4, "ms": ms, "GB/s": 2 * n * 4 / ms / 1e6}))
        return

    w = synth.WORKLOADS[args.workload]
    q, k, v = synth.make_workload(w, seed=0, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    if w.is_decode:
        raise SystemExit("--workload names a prefill workload; decode is reported under 'decode'")
    if w.dtype == torch.float32:
        step = lambda: fa.fa_forward_f32(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse)  # noqa: E731
        peak, dtype, kname = PEAK_FP32_TFLOPS, "f32", "fwd_f32_kernel"
        files = ["fa_fwd_f32.hip", "fa_device.h", "fa_internal.h"]
    else:
        step = lambda: fa.fa_forward(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse)  # noqa: E731
        peak, dtype, kname = PEAK_BF16_TFLOPS, "bf16", "fwd_mfma_kernel"
        files = ["fa_fwd_mfma.hip", "fa_device.h", "fa_internal.h"]
    ms = time_steps(step, args.steps, args.warmup, torch)
    flops, _ = workload_counts(w)
    tflops = flops / (ms * 1e-3) / 1e12
    digest = kernel_source_digest(files)
    traffic = measured_traffic(f"{kname}_{w.name}", digest)

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) inputs)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "scale": w.scale},
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic,
                     "kernel_source_digest": digest},
    }

    if not args.no_decode:
        dw = synth.WORKLOADS[args.decode_workload]
        dq, dk, dv = synth.make_workload(dw, seed=0, device="cuda")
        dout = torch.empty_like(dq)
        dlse = torch.empty((dw.B, dw.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_decode_workspace_bytes(dw.B, dw.H, dw.D, dw.num_splits), dtype=torch.uint8,
                         device="cuda")
        dstep = lambda: fa.fa_decode_splitkv(dq, dk, dv, dw.num_splits, scale=dw.scale, workspace=ws,  # noqa: E731
                                             out=dout, lse=dlse)
        dms = time_steps(dstep, args.decode_steps, args.warmup, torch)
        _, dbytes = workload_counts(dw)
        gbs = dbytes / (dms * 1e-3) / 1e9
        ddigest = kernel_source_digest(["fa_decode.hip", "fa_device.h", "fa_internal.h"])
        result["decode"] = {
            "workload": dw.name, "ms_per_call": round(dms, 6), "value": round(gbs, 2), "unit": "GB/s",
            "algorithmic_bytes": dbytes, "num_splits": dw.num_splits,
            "roofline": {"kernel": "decode_partial_kernel + decode_combine_kernel", "bound": "hbm",
                         "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(f"decode_partial_kernel_{dw.name}", ddigest),
                         "kernel_source_digest": ddigest},
        }
        del dq, dk, dv, ws

    if not args.no_backward:
        bw = synth.WORKLOADS[args.backward_workload or args.workload]
        if bw.dtype != torch.bfloat16 or bw.is_decode:
            raise SystemExit("the backward pass is bf16 prefill only")
        bq, bk, bv = synth.make_workload(bw, seed=0, device="cuda")
        bdo = synth.make_do(bw.B, bw.H, bw.Nq, bw.D, bw.dtype, seed=0, device="cuda")
        bo, blse = fa.fa_forward(bq, bk, bv, causal=bw.causal, scale=bw.scale)
        grads = tuple(torch.empty_like(t) for t in (bq, bk, bv))
        bws = torch.empty(max(16, fa.fa_backward_workspace_bytes(bw.B, bw.H, bw.Nq)), dtype=torch.uint8,
                          device="cuda")
        bstep = lambda: fa.fa_backward(bq, bk, bv, bo, bdo, blse, causal=bw.causal, scale=bw.scale,  # noqa: E731
                                       workspace=bws, dq=grads[0], dk=grads[1], dv=grads[2])
        bms = time_steps(bstep, args.backward_steps, args.warmup, torch)
        fwd_flops, _ = workload_counts(bw)
        btf = 2.5 * fwd_flops / (bms * 1e-3) / 1e12
        bdigest = kernel_source_digest(["fa_bwd.hip", "fa_device.h", "fa_internal.h"])
        result["backward"] = {
            "workload": bw.name, "ms_per_call": round(bms, 6), "value": round(btf, 3), "unit": "TFLOP/s",
            "algorithmic_flops": 2.5 * fwd_flops,
            "roofline": {"kernel": "bwd_dq_kernel + bwd_dkdv_kernel", "bound": "mfma",
                         "achieved": round(btf, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(btf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(f"bwd_kernels_{bw.name}", bdigest),
                         "kernel_source_digest": bdigest},
        }
        del bq, bk, bv, bdo, bo, grads, bws

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
