"""The C-ABI library on the CPU: it loads, exports every function include/fa.h
declares, and rejects bad arguments before anything is enqueued. No call here
reaches a kernel launch."""

import ctypes
import os
import re
import subprocess

import pytest

from flashattention_online_softmax_forward_amd import _lib
from flashattention_online_softmax_forward_amd.build import LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

INVALID, UNSUPPORTED = 1, 2
FAKE = 0x10000          # 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_api():
    assert declared_functions() == sorted(
        ["fa_forward", "fa_forward_masked", "fa_forward_f16", "fa_forward_f16_masked",
         "fa_forward_f32", "fa_forward_f32_masked", "fa_rope", "fa_rope_workspace_bytes", "fa_forward_rope",
         "fa_decode_workspace_bytes", "fa_decode_splitkv", "fa_decode_splitkv_masked",
         "fa_decode_splitkv_f16", "fa_decode_splitkv_f16_masked", "fa_decode_splitkv_noalloc",
         "fa_backward_workspace_bytes", "fa_backward", "fa_backward_masked", "fa_backward_f16",
         "fa_backward_f16_masked", "fa_status_string"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert name in _lib.PROTOTYPES, f"{name} has no ctypes prototype"
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_string(code).decode().startswith(name)
    assert lib.fa_status_string(99).decode().startswith("FA_ERR_UNKNOWN")


def fwd(lib, fn="fa_forward", Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, L=None,
        B=1, H=1, Nq=16, Nk=16, D=128, scale=0.125, causal=0):
    return getattr(lib, fn)(Q, K, V, O, L, B, H, Nq, Nk, D, scale, causal, None)


@pytest.mark.parametrize("fn", ["fa_forward", "fa_forward_f16", "fa_forward_f32"])
def test_forward_rejects_bad_arguments(lib, fn):
    assert fwd(lib, fn, Q=None) == INVALID
    assert fwd(lib, fn, O=None) == INVALID
    assert fwd(lib, fn, K=FAKE + 8) == INVALID                       # misaligned
    assert fwd(lib, fn, L=FAKE + 0x400002) == INVALID                # misaligned LSE
    assert fwd(lib, fn, B=-1) == INVALID
    assert fwd(lib, fn, Nk=0) == INVALID
    assert fwd(lib, fn, Nk=-3) == INVALID
    assert fwd(lib, fn, scale=0.0) == INVALID
    assert fwd(lib, fn, scale=-0.5) == INVALID
    assert fwd(lib, fn, scale=float("inf")) == INVALID
    assert fwd(lib, fn, scale=float("nan")) == INVALID
    assert fwd(lib, fn, D=96) == UNSUPPORTED
    assert fwd(lib, fn, D=256) == UNSUPPORTED
    assert fwd(lib, fn, O=FAKE) == INVALID                           # O aliases Q
    assert fwd(lib, fn, O=FAKE + 0x100000 + 64) == INVALID           # O overlaps K
    assert fwd(lib, fn, B=65536, H=65536, Nq=1024) == UNSUPPORTED    # grid too large
    assert fwd(lib, fn, causal=3) == INVALID                          # no such alignment
    assert fwd(lib, fn, causal=-1) == INVALID


@pytest.mark.parametrize("fn", ["fa_forward_masked", "fa_forward_f16_masked", "fa_forward_f32_masked"])
def test_masked_forward_rejects_bad_kv_lens(lib, fn):
    def call(lens, **kw):
        a = dict(Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, L=None, B=2, H=1, Nq=16,
                 Nk=16, D=64, scale=0.125, causal=2)
        a.update(kw)
        return getattr(lib, fn)(a["Q"], a["K"], a["V"], a["O"], a["L"], lens, a["B"], a["H"], a["Nq"], a["Nk"],
                                a["D"], a["scale"], a["causal"], None)
    assert call(FAKE + 0x400002) == INVALID                           # misaligned kv_lens
    assert call(FAKE + 0x300000) == INVALID                           # kv_lens inside O
    assert call(FAKE + 0x500000, L=FAKE + 0x500000) == INVALID        # kv_lens inside LSE
    assert call(FAKE + 0x400000, causal=5) == INVALID
    assert call(FAKE + 0x400000, B=0) == 0                            # nothing to do


@pytest.mark.parametrize("fn", ["fa_forward", "fa_forward_f16", "fa_forward_f32"])
def test_forward_empty_problem_is_a_noop(lib, fn):
    # nothing to compute: returns before any pointer is looked at or any launch
    assert fwd(lib, fn, Q=None, K=None, V=None, O=None, B=0) == 0
    assert fwd(lib, fn, Q=None, K=None, V=None, O=None, H=0) == 0
    assert fwd(lib, fn, Q=None, K=None, V=None, O=None, Nq=0) == 0


def test_decode_workspace_bytes(lib):
    assert lib.fa_decode_workspace_bytes(16, 32, 128, 64) == 16 * 32 * 64 * 130 * 4
    assert lib.fa_decode_workspace_bytes(2, 3, 64, 5) == 2 * 3 * 5 * 66 * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 96, 4) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 128, 0) == 0
    assert lib.fa_decode_workspace_bytes(-1, 1, 128, 4) == 0


def dec(lib, Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, L=None, W=FAKE + 0x400000,
        wbytes=None, B=2, H=2, Nk=100, D=128, scale=0.1, S=4):
    if wbytes is None:
        wbytes = B * H * S * (D + 2) * 4 if B >= 0 and H >= 0 and S > 0 else 0
    return lib.fa_decode_splitkv(Q, K, V, O, L, W, wbytes, B, H, Nk, D, scale, S, None)


def test_decode_rejects_bad_arguments(lib):
    assert dec(lib, W=None) == INVALID
    assert dec(lib, wbytes=2 * 2 * 4 * 130 * 4 - 4) == INVALID       # workspace one float short
    assert dec(lib, S=0) == INVALID
    assert dec(lib, Nk=0) == INVALID
    assert dec(lib, scale=0.0) == INVALID
    assert dec(lib, D=80) == UNSUPPORTED
    assert dec(lib, W=FAKE + 0x400004) == INVALID                    # misaligned workspace
    assert dec(lib, W=FAKE + 0x100000) == INVALID                    # workspace overlaps K
    assert dec(lib, B=0, Q=None, K=None, V=None, O=None, W=None) == 0


def test_decode_noalloc_rejects_bad_arguments_before_any_hip_call(lib):
    """Everything checked here returns before the scratch's address is looked
    up, so it runs without a GPU."""
    def nd(Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, B=2, H=2, Nk=100, D=128, scale=0.1,
           S=4):
        return lib.fa_decode_splitkv_noalloc(Q, K, V, O, None, B, H, Nk, D, scale, S, None)
    cap = 32 << 20
    assert nd(B=64, H=64, S=cap // (64 * 64 * 130 * 4) + 1) == UNSUPPORTED   # partials exceed the scratch
    assert nd(B=1 << 20, H=1 << 10, S=64) == UNSUPPORTED
    assert nd(S=0) == INVALID
    assert nd(Q=None) == INVALID
    assert nd(Nk=0) == INVALID
    assert nd(scale=float("nan")) == INVALID
    assert nd(D=96) == UNSUPPORTED
    assert nd(B=0, Q=None, K=None, V=None, O=None) == 0


def test_backward_workspace_bytes(lib):
    assert lib.fa_backward_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 4
    assert lib.fa_backward_workspace_bytes(1, 32, 2048) == 32 * 2048 * 4
    assert lib.fa_backward_workspace_bytes(-1, 1, 4) == 0


def bwd(lib, Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, dO=FAKE + 0x400000,
        L=FAKE + 0x500000, dQ=FAKE + 0x600000, dK=FAKE + 0x700000, dV=FAKE + 0x800000, W=FAKE + 0x900000,
        wbytes=None, B=2, H=2, Nq=100, Nk=100, D=128, scale=0.1, causal=0):
    if wbytes is None:
        wbytes = max(B * H * Nq * 4, 0)
    return lib.fa_backward(Q, K, V, O, dO, L, dQ, dK, dV, W, wbytes, B, H, Nq, Nk, D, scale, causal, None)


def test_backward_rejects_bad_arguments(lib):
    for name in ("Q", "K", "V", "O", "dO", "L", "dQ", "dK", "dV", "W"):
        assert bwd(lib, **{name: None}) == INVALID, name
    assert bwd(lib, dO=FAKE + 0x400008) == INVALID                   # misaligned
    assert bwd(lib, L=FAKE + 0x500002) == INVALID                    # misaligned LSE
    assert bwd(lib, wbytes=2 * 2 * 100 * 4 - 4) == INVALID           # workspace one float short
    assert bwd(lib, Nk=0) == INVALID
    assert bwd(lib, Nq=-1) == INVALID
    assert bwd(lib, scale=float("nan")) == INVALID
    assert bwd(lib, D=96) == UNSUPPORTED
    assert bwd(lib, dQ=FAKE) == INVALID                              # dQ aliases Q
    assert bwd(lib, dK=FAKE + 0x500000) == INVALID                   # dK overlaps LSE
    assert bwd(lib, dV=FAKE + 0x700000 + 64) == INVALID              # dV overlaps dK
    assert bwd(lib, W=FAKE + 0x600000) == INVALID                    # workspace overlaps dQ
    assert bwd(lib, B=65536, H=65536, Nq=1024) == UNSUPPORTED        # grid too large
    assert bwd(lib, causal=3) == INVALID
    # nothing to compute: returns before any pointer is looked at
    none = dict(Q=None, K=None, V=None, O=None, dO=None, L=None, dQ=None, dK=None, dV=None, W=None)
    assert bwd(lib, B=0, **none) == 0
    assert bwd(lib, Nq=0, Nk=0, **none) == 0
    # Nq = 0 < Nk zeroes dK, dV: those two must be valid
    assert bwd(lib, Nq=0, dK=None) == INVALID
    assert bwd(lib, Nq=0, dV=FAKE + 0x700000) == INVALID             # dV aliases dK


def test_masked_backward_and_decode_reject_bad_kv_lens(lib):
    def bm(lens, **kw):
        a = dict(Q=FAKE, K=FAKE + 0x100000, V=FAKE + 0x200000, O=FAKE + 0x300000, dO=FAKE + 0x400000,
                 L=FAKE + 0x500000, dQ=FAKE + 0x600000, dK=FAKE + 0x700000, dV=FAKE + 0x800000, W=FAKE + 0x900000,
                 B=2, H=2, Nq=100, Nk=100, D=128, scale=0.1, causal=2)
        a.update(kw)
        return lib.fa_backward_masked(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["L"], lens, a["dQ"], a["dK"],
                                      a["dV"], a["W"], a["B"] * a["H"] * a["Nq"] * 4, a["B"], a["H"], a["Nq"],
                                      a["Nk"], a["D"], a["scale"], a["causal"], None)
    assert bm(FAKE + 0xA00002) == INVALID                             # misaligned
    assert bm(FAKE + 0x700000 + 16) == INVALID                        # inside dK
    assert bm(FAKE + 0x900000) == INVALID                             # inside the workspace
    assert bm(FAKE + 0xA00000, causal=4) == INVALID

    def dm(lens, W=FAKE + 0x400000):
        return lib.fa_decode_splitkv_masked(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, None, lens,
                                            W, 2 * 2 * 4 * 130 * 4, 2, 2, 100, 128, 0.1, 4, None)
    assert dm(FAKE + 0x500002) == INVALID                             # misaligned
    assert dm(FAKE + 0x400000 + 64) == INVALID                        # inside the workspace
    assert dm(FAKE + 0x300000) == INVALID                             # inside O


def test_rope_rejects_bad_arguments(lib):
    def rope(X=FAKE, Y=FAKE + 0x100000, C=FAKE + 0x200000, S=FAKE + 0x300000, n_pos=64, style=0, dtype=0, B=1,
             H=2, N=64, D=128):
        return lib.fa_rope(X, Y, C, S, n_pos, style, dtype, B, H, N, D, None)
    assert rope(style=2) == INVALID
    assert rope(dtype=3) == INVALID
    assert rope(D=96) == UNSUPPORTED
    assert rope(n_pos=63) == INVALID                                  # table shorter than N
    assert rope(C=FAKE + 0x200004) == INVALID                         # misaligned table
    assert rope(Y=FAKE + 0x40) == INVALID                             # partial overlap with X
    assert rope(Y=FAKE + 0x200000) == INVALID                         # Y over the cos table
    assert rope(X=None) == INVALID
    assert rope(N=0, X=None, Y=None, C=None, S=None) == 0
    assert lib.fa_rope_workspace_bytes(2, 3, 100, 64) == 2 * 3 * 100 * 64 * 2


def test_forward_rope_rejects_bad_arguments(lib):
    def fr(W=FAKE + 0x600000, wbytes=1 * 2 * 64 * 128 * 2, n_pos=64, C=FAKE + 0x400000, S=FAKE + 0x500000,
           style=0, dtype=0, causal=0, Nq=64, Nk=64):
        return lib.fa_forward_rope(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, None, None, C, S,
                                   n_pos, style, dtype, W, wbytes, 1, 2, Nq, Nk, 128, 0.1, causal, None)
    assert fr(wbytes=100) == INVALID                                  # workspace too small
    assert fr(W=None) == INVALID
    assert fr(W=FAKE + 0x100000) == INVALID                           # workspace over K
    assert fr(n_pos=63) == INVALID
    assert fr(Nk=80, n_pos=70) == INVALID
    assert fr(style=5) == INVALID
    assert fr(dtype=2) == INVALID
    assert fr(causal=7) == INVALID
    assert fr(C=None) == INVALID


def test_python_binding_refuses_cpu_tensors(lib):
    import torch

    import flashattention_online_softmax_forward_amd as fa

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ROCm GPU"):
        fa.fa_forward(q, q, q)
    with pytest.raises(ValueError, match="ROCm GPU"):
        fa.fa_decode_splitkv(q[:, :, :1], q, q, num_splits=2)
    with pytest.raises(ValueError, match="ROCm GPU"):
        fa.fa_backward(q, q, q, q, q, torch.zeros(1, 1, 4))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "flashattention_online_softmax_forward_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_python_binding_checks_caller_buffers_before_the_device(lib):
    """A caller-supplied out / lse of the wrong shape, or a non-contiguous
    workspace, is refused before the device is looked at, so on the CPU that
    error is the one raised, and no call reaches the library. (A workspace
    that is too small is refused by the library itself, from the byte count
    it is given: see the decode and backward tests above.)"""
    import torch

    import flashattention_online_softmax_forward_amd as fa

    bf = torch.bfloat16
    q = torch.zeros(2, 3, 8, 64, dtype=bf)
    kv = torch.zeros(2, 3, 16, 64, dtype=bf)
    lse = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fa_forward(q, kv, kv, out=torch.zeros(2, 3, 7, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_forward(q, kv, kv, lse=torch.zeros(2, 3, 4))

    q1 = torch.zeros(2, 3, 1, 64, dtype=bf)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fa_decode_splitkv(q1, kv, kv, num_splits=4, out=torch.zeros(1, 3, 1, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_decode_splitkv(q1, kv, kv, num_splits=4, lse=torch.zeros(2, 2))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_decode_splitkv(q1, kv, kv, num_splits=4, lse=torch.zeros(2, 3, 1))
    need = fa.fa_decode_workspace_bytes(2, 3, 64, 4)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_decode_splitkv(q1, kv, kv, num_splits=4, workspace=torch.zeros(2 * need, dtype=torch.uint8)[::2])

    cos = torch.zeros(16, 32)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fa_forward_rope(q, kv, kv, cos, cos, out=torch.zeros(2, 3, 8, 128, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_forward_rope(q, kv, kv, cos, cos, lse=torch.zeros(2, 3, 16))
    need = fa.fa_rope_workspace_bytes(2, 3, 16, 64)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_forward_rope(q, kv, kv, cos, cos, workspace=torch.zeros(2 * need, dtype=torch.uint8)[::2])

    with pytest.raises(ValueError, match="dk must have shape"):
        fa.fa_backward(q, kv, kv, q, q, lse, dk=torch.zeros(2, 3, 8, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fa_backward(q, kv, kv, q, q, torch.zeros(2, 3, 16))
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_backward(q, kv, kv, q, q, lse, workspace=torch.zeros(64, dtype=torch.uint8)[::2])

    # Right shapes everywhere: the device check is what refuses them.
    with pytest.raises(ValueError, match="ROCm GPU"):
        fa.fa_decode_splitkv(q1, kv, kv, num_splits=4, out=torch.zeros_like(q1), lse=torch.zeros(2, 3))
    with pytest.raises(ValueError, match="ROCm GPU"):
        fa.fa_forward_rope(q, kv, kv, cos, cos, out=torch.zeros_like(q), lse=lse)
