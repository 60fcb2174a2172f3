"""Host-side accounting of bench.py, on the CPU: the algorithmic FLOP and byte
counts the roofline figures divide by, the digest that ties a profile's HBM
counters to the kernel source they were taken on, and the lookup of those
counters."""

import importlib.util
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_workload_counts(bench):
    # 4 B H Nq Nk D FLOPs (two products of 2 N^2 D each), halved under the causal mask.
    flops, _ = bench.workload_counts(synth.WORKLOADS["prefill_b1_h32_n2048_d128"])
    assert flops == 4 * 32 * 2048 * 2048 * 128
    flops, _ = bench.workload_counts(synth.WORKLOADS["causal_b4_h32_n4096_d128_qkx3"])
    assert flops == 2 * 4 * 32 * 4096 * 4096 * 128
    # Decode reads K and V (bf16) and q once, and writes O and LSE.
    _, nbytes = bench.workload_counts(synth.WORKLOADS["decode_b16_h32_kv32768_d128_s64"])
    kv = 2 * 16 * 32 * 32768 * 128 * 2
    assert kv <= nbytes <= kv + 16 * 32 * (128 * 2 * 2 + 4)


def test_code_only_ignores_comments(bench):
    a = "// header\nint f(int x) {  // trailing\n\n    /* block\n       comment */\n    return x + 1;\n}\n"
    b = "int f(int x) {\n    return x + 1;\n}"
    c = "int f(int x) {\n    return x + 2;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(b) != bench._code_only(c)


def test_profile_traffic_lookup(bench):
    found = 0
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        m_d = re.search(r"^kernel_source_digest:\s*([0-9a-f]+)$", text, re.M)
        m_b = re.search(r"^hbm_bytes_per_launch:\s*(\d+)$", text, re.M)
        if not (m_d and m_b):
            continue
        found += 1
        stem = name[:-len(".md")]
        assert bench.measured_traffic(stem, m_d.group(1)) == float(m_b.group(1))
        assert bench.measured_traffic(stem, "0" * 16) is None
    assert found >= 3
    assert bench.measured_traffic("no_such_kernel_no_such_workload", "0" * 16) is None


def test_profile_value_is_digest_gated(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "k_w.md").write_text("# x\n\nkernel_source_digest: 00ff\nhbm_bytes_per_launch: 123\n"
                                     "mfma_busy: 0.5125\n")
    assert bench.profile_value("k_w", "mfma_busy", "00ff") == 0.5125
    assert bench.profile_value("k_w", "hbm_bytes_per_launch", "00ff") == 123.0
    assert bench.profile_value("k_w", "mfma_busy", "00fe") is None
    assert bench.profile_value("k_w", "no_such_key", "00ff") is None


def test_run_units_counts_only_completed_work(bench):
    calls = []

    def unit():
        calls.append(1)
        return 2.5
    done, work, wall = bench.run_units([unit, unit, unit], 0.05, 3)
    assert done == len(calls) >= 3
    assert work == 2.5 * done
    assert wall >= 0.05


@pytest.mark.parametrize("kind,name", [("forward", "single_head_f32_256x64"),
                                       ("forward", "causal_b1_h16_n16000_d64"),
                                       ("decode", "decode_b16_h32_kv32768_d128_s64"),
                                       ("backward", "prefill_b1_h32_n2048_d128")])
def test_cpu_baseline_on_small_stand_ins(bench, kind, name):
    """The oracle baseline runs on CPU tensors of a workload's layout (shrunk so
    the test is quick) and reports a positive rate, its unit and its cores."""
    import dataclasses

    w = synth.WORKLOADS[name]
    small = dataclasses.replace(w, B=1, H=2, Nq=min(w.Nq, 64), Nk=min(w.Nk, 100))
    q, k, v = synth.make_workload(small, seed=0)
    tensors = (q, k, v) if kind != "backward" else (q, k, v, synth.make_do(1, 2, small.Nq, small.D, small.dtype))
    r = bench.cpu_baseline(kind, small, tensors, 0.2)
    assert r["value"] > 0 and r["kind"] == "oracle"
    assert r["unit"] == ("GB/s" if kind == "decode" else "TFLOP/s")
    assert 1 <= r["cores"] <= bench.MAX_BASELINE_THREADS
    assert r["cores"] <= len(os.sched_getaffinity(0))
