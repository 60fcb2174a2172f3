"""Worst-case error bounds of the bf16 backward kernels' gradients, used by
the GPU parity tests (and checked for sensitivity on the CPU).

The kernels receive the bf16 O and fp32 LSE of the library's own forward pass,
as a training step would; the oracle differentiates the exact definition. No
tolerance for the gradients is given by the workload definition, so every
element gets a worst-case bound derived from the kernels' arithmetic.
Notation: u = 2^-8, the unit roundoff of bf16 round-to-nearest-even (8
significant bits); g(n) = n 2^-24, the bound of an fp32 sum of n exact
products relative to the sum of their magnitudes.

* P carries a relative error eps[i,j] = expm1(eL[i] + eS[i,j]) + 2^-16:
  eL is the forward's LSE error on row i (measured against the oracle), eS =
  scale g(D) (|Q| |K|^T) the fp32 error of S, and 2^-16 covers the fp32
  rounding of the exponent's argument and the hardware exp2.
* dV = P^T dO with P rounded to bf16 (u), fp32 sums over Nq queries, output
  rounded (u):
      |err dV| <= ((2u + g(Nq)) P + eps P)^T |dO|.
* dS = P (dP - D) is formed in fp32 and rounded to bf16 (u); dP and D are fp32
  sums of D exact products (g(D)), and D is taken from the forward's bf16 O
  rather than the exact O, which moves it by dD = sum_d dO (O_bf16 - O).
  With E1 = P |dP - D| and E2 = P (|dD| + g(D) (|dO| |V|^T + rowsum |dO||O|)):
      |err dS| <= (u + eps) E1 + (1 + 2u) E2,
  and dQ = scale dS K (fp32 sums over Nk keys, output rounded, u):
      |err dQ| <= scale ([(2u + g(Nk) + eps) E1 + (1 + 2u) E2] |K|),
      |err dK| <= scale ([(2u + g(Nq) + eps) E1 + (1 + 2u) E2]^T |Q|).
Second-order terms are covered by a factor 1.01, and 1e-6 absolute covers
exp2 underflow and fp32 rounding next to zero. Rows with one or two
visible keys come close to these bounds (the roundings of dS and of the output
can both be near u there); the printed err/bound ratio shows the margin.
"""

from __future__ import annotations

import numpy as np

from oracle import attention as orc

U = 2.0 ** -8
ABS = 1e-6


def g(n):
    return n * 2.0 ** -24


def bounds_head(q, k, v, do, o_gpu, lse_err, scale, causal, kv_len=None, u=U, tiny=2.0 ** -134):
    """Per-element error bounds (dQ, dK, dV) of one head, from the module
    docstring's derivation. Inputs are fp64 arrays of the 16-bit values;
    lse_err [Nq] is the forward's LSE error (0 on rows with no key). u is the
    unit roundoff of the element type (2^-8 bf16, 2^-11 fp16) and tiny half
    its subnormal spacing (2^-134 bf16, 2^-25 fp16): a P or dS value below the
    smallest normal is rounded with that absolute error instead of u
    relative, which adds tiny * sum |dO| to dV and scale * tiny * sum |K|
    (|Q|) to dQ (dK)."""
    U = u
    nq, D = q.shape
    nk = k.shape[0]
    p = orc.softmax_weights(q, k, scale, causal, kv_len)
    eps = np.expm1(lse_err[:, None] + scale * g(D) * (np.abs(q) @ np.abs(k).T)) + 2.0 ** -16
    dp = do @ v.T
    d_exact = (p * dp).sum(axis=1, keepdims=True)
    d_gpu = (do * o_gpu).sum(axis=1, keepdims=True)
    e1 = p * np.abs(dp - d_exact)
    e2 = p * (np.abs(d_gpu - d_exact)
              + g(D) * (np.abs(do) @ np.abs(v).T + (np.abs(do) * np.abs(o_gpu)).sum(axis=1, keepdims=True)))
    bv = ((2 * U + g(nq)) * p + eps * p).T @ np.abs(do)
    bq = scale * (((2 * U + g(nk) + eps) * e1 + (1 + 2 * U) * e2) @ np.abs(k))
    bk = scale * (((2 * U + g(nq) + eps) * e1 + (1 + 2 * U) * e2).T @ np.abs(q))
    bv = bv + tiny * np.abs(do).sum(axis=0)[None, :]
    bq = bq + scale * tiny * np.abs(k).sum(axis=0)[None, :]
    bk = bk + scale * tiny * np.abs(q).sum(axis=0)[None, :]
    return 1.01 * bq + ABS, 1.01 * bk + ABS, 1.01 * bv + ABS
