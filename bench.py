"""Benchmark of the MI355X FlashAttention library: one JSON line.

The headline step is one ``fa_forward`` call over the prefill workload the
metric is quoted on (B=1, H=32, Nq=Nk=2048, D=128, bf16, non-causal), inputs
already resident in HBM. Every other workload the method is checked on is
timed in the same run, each as a leg of its own with its roofline and an
oracle baseline beside it:
  c1        single head, fp32 [1,1,256,64] (its calls queued ahead: see time_steps)
  c3        causal prefill [4,32,4096,128], Q and K x3
  c4        causal prefill [1,16,16000,64] with a ragged tail
  long      non-causal prefill [1,32,16384,128] (beyond the five workloads:
            the long-sequence end of the non-causal D = 128 regime)
  decode    split-KV decode B=16, H=32, Nk=32768, D=128, 64 splits (two kernels)
  backward  the backward pass with recompute on the headline workload

Timing: W untimed warm-up calls plus untimed calls until half a second of GPU
work has run (the engine clock ramps up under load), then K calls between two
HIP events recorded on the stream the kernels are launched on (torch's
current stream, which is the stream handed to the library), synchronised on
both sides.

Algorithmic counts (not the implementation's):
  forward FLOPs  = 4*B*H*Nq*Nk*D, halved when causal
  forward bytes  = Q, K, V read once + O written once (+ LSE, fp32)
  decode bytes   = K, V read once + q read and O written once (+ LSE)
  backward FLOPs = 10*B*H*Nq*Nk*D (S, dP, dV, dQ, dK: five products; halved
                   when causal), the recompute of S counted

Each leg's ``roofline`` carries ``traffic`` (HBM bytes per launch) and, for
the MFMA kernels, ``mfma_busy`` (the fraction of SIMD cycles in which the
matrix core was busy) read from the rocprofv3 summary of that kernel and
workload under profiles/, and only while the kernel's source still has the
digest recorded there; otherwise they are null.

``cpu_baseline`` (each leg): the fp64 oracle as it stands, on the host, on a
bounded sample of the leg's own inputs. Samples are independent units (a
block of query rows of one head; one head for decode and the backward), run
by one thread per core of the process's affinity mask (at most 16), each with
a single-threaded BLAS, until the leg's time budget is spent. The rate is the
algorithmic work of the completed units over the wall time of the run.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s & % bf16 MFMA peak (prefill); decode GB/s & % HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "flashattention_online_softmax_forward_amd", "csrc")
MAX_BASELINE_THREADS = 16
# Spin before a queued-ahead timed region: ~10 ms at the 2.4 GHz peak clock,
# several times the host's cost of submitting a leg's calls.
QUEUE_AHEAD_CYCLES = 24_000_000

HEADLINE = "prefill_b1_h32_n2048_d128"
# leg -> (workload, what is timed)
LEGS = {
    "c1": ("single_head_f32_256x64", "forward"),
    "c3": ("causal_b4_h32_n4096_d128_qkx3", "forward"),
    "c4": ("causal_b1_h16_n16000_d64", "forward"),
    "long": ("prefill_b1_h32_n16384_d128", "forward"),
    "decode": ("decode_b16_h32_kv32768_d128_s64", "decode"),
    "backward": (HEADLINE, "backward"),
}
FWD_FILES = ["fa_fwd_mfma.hip", "fa_fwd_mfma16.hip", "fa_device.h", "fa_internal.h"]
F32_FILES = ["fa_fwd_f32.hip", "fa_device.h", "fa_internal.h"]
DEC_FILES = ["fa_decode.hip", "fa_device.h", "fa_internal.h"]
BWD_FILES = ["fa_bwd.hip", "fa_device.h", "fa_internal.h"]


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


def profile_value(name, key, digest):
    """``key: value`` recorded in profiles/<name>.md from rocprofv3 counter
    runs, or None when absent or taken on other kernel source."""
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_v = re.search(r"^" + re.escape(key) + r":\s*([0-9.eE+-]+)\s*$", text, flags=re.M)
    if not m_src or not m_v or m_src.group(1) != digest:
        return None
    return float(m_v.group(1))


def measured_traffic(name, digest):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) of profiles/<name>.md."""
    return profile_value(name, "hbm_bytes_per_launch", digest)


def workload_counts(w):
    flops = 4.0 * w.B * w.H * w.Nq * w.Nk * w.D * (0.5 if w.causal else 1.0)
    elem = 4 if w.dtype.is_floating_point and w.dtype.itemsize == 4 else 2
    bytes_ = elem * w.B * w.H * (2 * w.Nq * w.D + 2 * w.Nk * w.D) + 4 * w.B * w.H * w.Nq
    return flops, bytes_


def time_steps(fn, steps, warmup, torch, settle_s=0.5, queue_ahead=False):
    """W warm-up calls, then keep calling (untimed) until ``settle_s`` seconds
    of GPU work have run, so the engine clock has ramped up before the timed
    region; then K timed calls between two events on the launch stream.

    ``queue_ahead``: for kernels shorter than the host's cost of one call, a
    short spin kernel goes first on the stream, so that all K calls are
    queued before the first of them starts and the GPU runs them back to
    back (otherwise the events would time the host's submission rate)."""
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
    if queue_ahead:
        torch.cuda._sleep(QUEUE_AHEAD_CYCLES)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


# ---------------------------------------------------------------- oracle baseline

def baseline_threads():
    return max(1, min(len(os.sched_getaffinity(0)), MAX_BASELINE_THREADS))


def run_units(units, budget_s, threads):
    """Run ``units`` (callables returning their algorithmic work) round robin
    on ``threads`` threads until ``budget_s`` seconds have passed; a unit that
    has started is finished. Returns (completed units, total work, wall s)."""
    lock = threading.Lock()
    state = {"next": 0, "done": 0, "work": 0.0}
    t0 = time.perf_counter()
    deadline = t0 + budget_s

    def worker():
        while time.perf_counter() < deadline:
            with lock:
                i = state["next"]
                state["next"] += 1
            w = units[i % len(units)]()
            with lock:
                state["done"] += 1
                state["work"] += w
    pool = [threading.Thread(target=worker) for _ in range(threads)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    return state["done"], state["work"], time.perf_counter() - t0


def _widen(t, np):
    return t.float().cpu().numpy().astype(np.float64)


def cpu_baseline(kind, w, tensors, budget_s, max_bytes=4 << 30):
    """The fp64 oracle as it stands on a bounded sample of one leg's inputs.

    kind "forward": units of up to 512 query rows of one head, through
    ``attention_rows``; work = 4 D sum_i (keys row i may see), in FLOP.
    kind "decode": one head per unit, through ``decode``; work = the head's
    algorithmic bytes. kind "backward": one head per unit, through
    ``attention_backward_head``; work = 10 Nq Nk D FLOP (halved causal).
    At most ``max_bytes`` of widened fp64 inputs are prepared (heads in
    order); the units cycle over them until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention as orc

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head = 8 * sum(t[0, 0].numel() for t in tensors)
    heads = heads[:max(1, min(len(heads), max_bytes // per_head))]
    # Widened before the clock starts: the oracle is timed, not the copies.
    wide = {bh: tuple(_widen(t[bh[0], bh[1]], np) for t in tensors) for bh in heads}

    units = []
    if kind == "forward":
        rows_per_unit = min(w.Nq, 512)
        for bh in heads:
            for r0 in range(0, w.Nq, rows_per_unit):
                rows = np.arange(r0, min(w.Nq, r0 + rows_per_unit))
                seen = np.minimum(rows + 1, w.Nk) if w.causal else np.full(rows.shape, w.Nk)
                work = 4.0 * w.D * float(seen.sum())

                def unit(bh=bh, rows=rows, work=work):
                    q, k, v = wide[bh]
                    orc.attention_rows(q[rows], rows, k, v, w.scale, w.causal, nq=w.Nq)
                    return work
                units.append(unit)
        unit_desc, unit_name, scale_to = f"{rows_per_unit}-row blocks", "TFLOP/s", 1e12
    elif kind == "decode":
        work = 2.0 * (2 * w.Nk * w.D + 2 * w.D) + 4.0
        for bh in heads:
            def unit(bh=bh):
                q, k, v = wide[bh]
                orc.decode(q[None, None], k[None, None], v[None, None], w.scale)
                return work
            units.append(unit)
        unit_desc, unit_name, scale_to = "heads", "GB/s", 1e9
    else:
        work = 10.0 * w.Nq * w.Nk * w.D * (0.5 if w.causal else 1.0)
        for bh in heads:
            def unit(bh=bh):
                q, k, v, do = wide[bh]
                orc.attention_backward_head(q, k, v, do, w.scale, w.causal)
                return work
            units.append(unit)
        unit_desc, unit_name, scale_to = "heads", "TFLOP/s", 1e12

    threads = baseline_threads()
    with threadpool_limits(limits=1):
        done, total, wall = run_units(units, budget_s, threads)
    return {
        "value": total / wall / scale_to,
        "unit": unit_name,
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} units ({unit_desc}, cycling over {len(units)} units of the first {len(heads)} of "
                  f"{w.B * w.H} heads) of {w.name}, fp64 two-pass oracle, {wall:.1f} s wall on {threads} threads "
                  f"(one per core of the affinity mask, single-threaded BLAS each)",
    }


# ---------------------------------------------------------------- legs

def roofline(kernel, bound, achieved, peak, unit, profile, digest, mfma):
    r = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": measured_traffic(profile, digest),
         "kernel_source_digest": digest}
    if mfma:
        r["mfma_busy"] = profile_value(profile, "mfma_busy", digest)
    return r


def forward_leg(fa, synth, torch, w, steps, warmup):
    q, k, v = synth.make_workload(w, seed=0, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    if w.dtype == torch.float32:
        step = lambda: fa.fa_forward_f32(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse)  # noqa: E731
        kname, peak, files, dtype = "fwd_f32_kernel", PEAK_FP32_TFLOPS, F32_FILES, "f32"
    else:
        step = lambda: fa.fa_forward(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse)  # noqa: E731
        # D = 128 runs the 16x16x32 kernel, D = 64 the 32x32x16 one
        kname = "fwd_mfma16_kernel" if w.D == 128 else "fwd_mfma_kernel"
        peak, files, dtype = PEAK_BF16_TFLOPS, FWD_FILES, "bf16"
    # The single-head fp32 kernel (~15 us) is shorter than one call's host
    # cost; its calls are queued ahead so the events time the kernels.
    ms = time_steps(step, steps, warmup, torch, queue_ahead=w.dtype == torch.float32)
    flops, bytes_ = workload_counts(w)
    tflops = flops / (ms * 1e-3) / 1e12
    digest = kernel_source_digest(files)
    leg = {
        "workload": w.name, "dtype": dtype, "ms_per_call": round(ms, 6), "value": round(tflops, 3),
        "unit": "TFLOP/s", "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
        "config": {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D, "causal": w.causal,
                   "qk_mul": w.qk_mul, "scale": w.scale},
        "roofline": roofline(kname, "mfma" if dtype == "bf16" else "alu", tflops, peak, "TFLOP/s",
                             f"{kname}_{w.name}", digest, dtype == "bf16"),
    }
    return leg, (q, k, v)


def decode_leg(fa, synth, torch, w, steps, warmup):
    q, k, v = synth.make_workload(w, seed=0, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.H, w.D, w.num_splits), dtype=torch.uint8, device="cuda")
    step = lambda: fa.fa_decode_splitkv(q, k, v, w.num_splits, scale=w.scale, workspace=ws,  # noqa: E731
                                        out=out, lse=lse)
    ms = time_steps(step, steps, warmup, torch)
    _, bytes_ = workload_counts(w)
    gbs = bytes_ / (ms * 1e-3) / 1e9
    digest = kernel_source_digest(DEC_FILES)
    leg = {
        "workload": w.name, "ms_per_call": round(ms, 6), "value": round(gbs, 2), "unit": "GB/s",
        "algorithmic_bytes": bytes_, "num_splits": w.num_splits,
        "roofline": roofline("decode_partial_kernel + decode_combine_kernel", "hbm", gbs, PEAK_HBM_GBS, "GB/s",
                             f"decode_partial_kernel_{w.name}", digest, False),
    }
    return leg, (q, k, v)


def backward_leg(fa, synth, torch, w, steps, warmup):
    if w.dtype != torch.bfloat16 or w.is_decode:
        raise SystemExit("the backward leg is bf16 prefill only")
    q, k, v = synth.make_workload(w, seed=0, device="cuda")
    do = synth.make_do(w.B, w.H, w.Nq, w.D, w.dtype, seed=0, device="cuda")
    o, lse = fa.fa_forward(q, k, v, causal=w.causal, scale=w.scale)
    grads = tuple(torch.empty_like(t) for t in (q, k, v))
    ws = torch.empty(max(16, fa.fa_backward_workspace_bytes(w.B, w.H, w.Nq)), dtype=torch.uint8, device="cuda")
    step = lambda: fa.fa_backward(q, k, v, o, do, lse, causal=w.causal, scale=w.scale,  # noqa: E731
                                  workspace=ws, dq=grads[0], dk=grads[1], dv=grads[2])
    ms = time_steps(step, steps, warmup, torch)
    fwd_flops, _ = workload_counts(w)
    flops = 2.5 * fwd_flops
    tf = flops / (ms * 1e-3) / 1e12
    digest = kernel_source_digest(BWD_FILES)
    leg = {
        "workload": w.name, "ms_per_call": round(ms, 6), "value": round(tf, 3), "unit": "TFLOP/s",
        "algorithmic_flops": flops,
        # the two kernels: dQ (and D), then dK/dV
        "roofline": roofline("bwd_dq16_kernel + bwd_dkdv16_kernel", "mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                             f"bwd_kernels_{w.name}", digest, True),
    }
    return leg, (q, k, v, do)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed calls of the headline step")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--leg-steps", type=int, default=50, help="timed calls of every other leg")
    ap.add_argument("--legs", default=",".join(LEGS), help="comma-separated subset of: " + ", ".join(LEGS))
    ap.add_argument("--workload", default=HEADLINE, help="headline workload (a prefill workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work, headline leg")
    ap.add_argument("--leg-cpu-budget", type=float, default=5.0, help="seconds of oracle work, other legs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many bytes "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on a single GPU; there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.legs.split(",") if x]
    for x in legs:
        if x not in LEGS:
            raise SystemExit(f"unknown leg {x!r}; choose from {', '.join(LEGS)}")

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
    if w.is_decode or w.dtype != torch.bfloat16:
        raise SystemExit("--workload names the bf16 prefill workload of the headline step")
    head, head_inputs = forward_leg(fa, synth, torch, w, args.steps, args.warmup)
    print(f"[bench] {w.name}: {head['ms_per_call']:.6f} ms, {head['value']:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) inputs)",
        "config": dict(workload=w.name, **head["config"]),
        "roofline": head["roofline"],
    }

    run = {"forward": forward_leg, "decode": decode_leg, "backward": backward_leg}
    leg_inputs = {}
    for name in legs:
        wname, kind = LEGS[name]
        lw = synth.WORKLOADS[wname]
        leg, inputs = run[kind](fa, synth, torch, lw, args.leg_steps, args.warmup)
        print(f"[bench] {name} {lw.name}: {leg['ms_per_call']:.6f} ms, {leg['value']} {leg['unit']}",
              file=sys.stderr, flush=True)
        result[name] = leg
        if not args.no_cpu_baseline:
            leg_inputs[name] = (kind, lw, inputs)
        del inputs

    # The oracle runs after every GPU leg, on the host, each leg on its own
    # inputs (only the heads it samples are copied back).
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline("forward", w, head_inputs, args.cpu_budget)
        for name, (kind, lw, inputs) in leg_inputs.items():
            result[name]["cpu_baseline"] = cpu_baseline(kind, lw, inputs, args.leg_cpu_budget)
            print(f"[bench] {name} oracle: {result[name]['cpu_baseline']['value']:.4g} "
                  f"{result[name]['cpu_baseline']['unit']}", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
