"""Seeded synthetic inputs shared by the tests, ``smoke()`` and the bench.

This module holds no attention arithmetic: it only draws i.i.d. standard
normal tensors (the distribution the ML-compiler chapter's harness draws its
Q, K and V from, section 11.8 and its ``__main__``) and names the workloads.
Both the HIP path and the oracle receive exactly the tensors produced here;
the oracle widens the same bf16/fp32 values to fp64.

Recipe: each tensor has its own ``torch.Generator`` seeded with
``seed * 1_000_003 + tensor_id`` (Q = 0, K = 1, V = 2, the
output gradient dO = 3) on the device the tensor
will live on. Values are drawn in fp32, multiplied in fp32 by the workload's
factor (3 for Q and K of the rescale-stress workload), then rounded to the
storage dtype by torch's round-to-nearest-even cast. Large tensors are drawn in
slabs along the first axis so the fp32 staging buffer stays small; the slab
order is fixed, so a given (seed, shape, device) always gives the same values.
"""

from __future__ import annotations

import dataclasses
import math

import torch

Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    dtype: torch.dtype
    causal: bool = False
    qk_mul: float = 1.0
    num_splits: int = 0          # > 0: single-token split-KV decode

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def is_decode(self) -> bool:
        return self.num_splits > 0


# The workloads the method is measured and checked on.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f32_256x64", 1, 1, 256, 256, 64, torch.float32),
        Workload("prefill_b1_h32_n2048_d128", 1, 32, 2048, 2048, 128, torch.bfloat16),
        Workload("causal_b4_h32_n4096_d128_qkx3", 4, 32, 4096, 4096, 128, torch.bfloat16,
                 causal=True, qk_mul=3.0),
        Workload("causal_b1_h16_n16000_d64", 1, 16, 16000, 16000, 64, torch.bfloat16, causal=True),
        Workload("decode_b16_h32_kv32768_d128_s64", 16, 32, 1, 32768, 128, torch.bfloat16,
                 num_splits=64),
        # Beyond the five: a long non-causal prefill, the long-sequence end of
        # the non-causal D = 128 prefill regime (the forward rate grows with N
        # as each workgroup's Q load and O store are spread over more tiles).
        Workload("prefill_b1_h32_n16384_d128", 1, 32, 16384, 16384, 128, torch.bfloat16),
    ]
}


def normal(shape, dtype, seed: int, tensor_id: int, device="cpu", mul: float = 1.0,
           slab_elems: int = 1 << 28) -> torch.Tensor:
    """i.i.d. N(0, 1) * mul drawn in fp32 and rounded to ``dtype``."""
    shape = tuple(int(s) for s in shape)
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tensor_id)
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel() == 0:
        return out
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(-1, 1)
    rows_per_slab = max(1, slab_elems // max(1, flat.shape[1]))
    for r0 in range(0, flat.shape[0], rows_per_slab):
        r1 = min(flat.shape[0], r0 + rows_per_slab)
        z = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        if mul != 1.0:
            z.mul_(mul)
        flat[r0:r1].copy_(z)
    return out


def make_qkv(B, H, Nq, Nk, D, dtype, seed: int = 0, device="cpu", qk_mul: float = 1.0):
    """Q [B,H,Nq,D], K and V [B,H,Nk,D], contiguous, on ``device``."""
    q = normal((B, H, Nq, D), dtype, seed, Q_ID, device, qk_mul)
    k = normal((B, H, Nk, D), dtype, seed, K_ID, device, qk_mul)
    v = normal((B, H, Nk, D), dtype, seed, V_ID, device)
    return q, k, v


def make_workload(w: Workload, seed: int = 0, device="cpu"):
    return make_qkv(w.B, w.H, w.Nq, w.Nk, w.D, w.dtype, seed, device, w.qk_mul)


def make_do(B, H, Nq, D, dtype, seed: int = 0, device="cpu"):
    """Output gradient dO [B,H,Nq,D] ~ N(0, 1) for the backward pass."""
    return normal((B, H, Nq, D), dtype, seed, DO_ID, device)


def rope_tables(n_pos: int, D: int, base: float = 10000.0, device="cpu"):
    """RoPE cos/sin tables, fp32 [n_pos, D/2]: angle of position p and pair i
    is p * base^(-2i/D), the usual frequency schedule (the tables are inputs
    of the rotation; the method does not fix them)."""
    inv = base ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2.0 / D)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return (torch.cos(ang).to(torch.float32).to(device).contiguous(),
            torch.sin(ang).to(torch.float32).to(device).contiguous())
