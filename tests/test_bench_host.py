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
