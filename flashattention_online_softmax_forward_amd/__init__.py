"""MI355X (gfx950) FlashAttention forward: thin Python binding of include/fa.h.

Each function marshals torch tensors into the C ABI of ``libfa_mi355x.so`` and
nothing else: every step of the computation runs in the library's HIP kernels.
torch supplies device memory and the current stream. Tensors are [B, H, N, D]
contiguous on a ROCm device; outputs are allocated here with torch when the
caller does not pass them. There is no CPU fallback: without the built library
or a GPU tensor these functions raise.

``causal`` is False / 0 (no mask), True / 1 / "top_left" (key j <= query i) or
2 / "bottom_right" (key j <= i + Lk - Nq). ``kv_lens`` (optional int32 [B] on
the device) gives each batch entry's real key count; keys past it are padding.
Rows that may attend no key come back as O = 0, LSE = -inf.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib

CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT = 0, 1, 2
ROPE_HALF, ROPE_PAIRS = 0, 1
_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20   # FA_DECODE_NOALLOC_SCRATCH_BYTES of include/fa.h

__all__ = [
    "CAUSAL_NONE",
    "CAUSAL_TOP_LEFT",
    "CAUSAL_BOTTOM_RIGHT",
    "fa_forward",
    "fa_forward_f16",
    "fa_forward_rope",
    "fa_rope",
    "fa_rope_workspace_bytes",
    "ROPE_HALF",
    "ROPE_PAIRS",
    "fa_forward_f32",
    "fa_decode_splitkv",
    "fa_decode_workspace_bytes",
    "fa_decode_splitkv_noalloc",
    "DECODE_NOALLOC_SCRATCH_BYTES",
    "fa_backward",
    "fa_backward_workspace_bytes",
    "fa_status_string",
    "FAError",
]

FAError = _lib.FAError


def fa_status_string(code: int) -> str:
    return _lib.status_string(code)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_layout(name: str, t, dtype: torch.dtype, shape=None, ndim: int = 4) -> None:
    """Type, dtype, rank, exact shape (when given) and contiguity; device-free,
    so a wrong-shaped tensor is refused before anything else is looked at."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    elif t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D [B, H, N, D] (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_devices(ref: torch.Tensor, **tensors) -> None:
    """Every tensor on the one ROCm device of ``ref``; None entries are skipped."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must live on a ROCm GPU (got {ref.device}); there is no CPU path")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} must live on {ref.device} (got {t.device})")


def _check_workspace(workspace) -> int:
    """A contiguous tensor; returns its size in bytes, which the library
    compares with what the call needs (FA_ERR_INVALID_ARG when short)."""
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous torch.Tensor")
    return workspace.numel() * workspace.element_size()


def _causal_mode(causal) -> int:
    if isinstance(causal, str):
        names = {"none": CAUSAL_NONE, "top_left": CAUSAL_TOP_LEFT, "bottom_right": CAUSAL_BOTTOM_RIGHT}
        if causal not in names:
            raise ValueError(f"causal must be one of {sorted(names)} (got {causal!r})")
        return names[causal]
    mode = int(causal)
    if mode not in (CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT):
        raise ValueError(f"causal must be 0, 1 or 2 (got {causal!r})")
    return mode


def _check_kv_lens(kv_lens, B):
    if kv_lens is None:
        return None
    if not isinstance(kv_lens, torch.Tensor) or kv_lens.dtype != torch.int32 or kv_lens.dim() != 1 \
            or kv_lens.shape[0] != B or not kv_lens.is_contiguous():
        raise ValueError(f"kv_lens must be a contiguous int32 tensor of shape [{B}]")
    return kv_lens


def _check_qkv(q, k, v, dtype):
    """q [B,H,Nq,D], k and v [B,H,Nk,D] of one dtype; returns (B, H, Nq, Nk, D)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_layout(name, t, dtype)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, D) or tuple(v.shape) != (B, H, Nk, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, H, Nq, Nk, D


def _forward(fn_name, dtype, q, k, v, causal, scale, out, lse, want_lse, kv_lens=None):
    B, H, Nq, Nk, D = _check_qkv(q, k, v, dtype)
    if out is not None:
        _check_layout("out", out, dtype, q.shape)
    if lse is not None:
        _check_layout("lse", lse, torch.float32, (B, H, Nq))
    kv_lens = _check_kv_lens(kv_lens, B)
    mode = _causal_mode(causal)
    _check_devices(q, k=k, v=v, out=out, lse=lse, kv_lens=kv_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    lse_p = lse.data_ptr() if lse is not None else None
    if kv_lens is None:
        code = getattr(lib, fn_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p,
                                     B, H, Nq, Nk, D, float(scale), mode, _stream(q))
    else:
        fn_name += "_masked"
        code = getattr(lib, fn_name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p,
                                     kv_lens.data_ptr(), B, H, Nq, Nk, D, float(scale), mode, _stream(q))
    _lib.check(code, fn_name)
    return out, lse


def fa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=False,
               scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True,
               kv_lens: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bf16 forward: returns (O bf16 [B,H,Nq,D], LSE fp32 [B,H,Nq] or None)."""
    return _forward("fa_forward", torch.bfloat16, q, k, v, causal, scale, out, lse, want_lse, kv_lens)


def fa_forward_f16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=False,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   kv_lens: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fp16 forward: returns (O fp16 [B,H,Nq,D], LSE fp32 [B,H,Nq] or None)."""
    return _forward("fa_forward_f16", torch.float16, q, k, v, causal, scale, out, lse, want_lse, kv_lens)


def fa_forward_f32(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=False,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   kv_lens: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fp32 forward: returns (O fp32 [B,H,Nq,D], LSE fp32 [B,H,Nq] or None)."""
    return _forward("fa_forward_f32", torch.float32, q, k, v, causal, scale, out, lse, want_lse, kv_lens)


def fa_decode_workspace_bytes(B: int, H: int, D: int, num_splits: int) -> int:
    return int(_lib.load().fa_decode_workspace_bytes(B, H, D, num_splits))


def _check_decode(q, k, v, out, lse, kv_lens):
    """Shapes of a decode call (device-free); returns (B, H, Nk, D)."""
    if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
        raise TypeError(f"q must be a bfloat16 or float16 tensor (got {getattr(q, 'dtype', type(q))})")
    B, H, one, Nk, D = _check_qkv(q, k, v, q.dtype)
    if one != 1:
        raise ValueError("decode takes exactly one query token per (batch, head)")
    if out is not None:
        _check_layout("out", out, q.dtype, q.shape)
    if lse is not None:
        _check_layout("lse", lse, torch.float32, (B, H))
    _check_kv_lens(kv_lens, B)
    return B, H, Nk, D


def fa_decode_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_splits: int,
                      scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      want_lse: bool = True, kv_lens: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode of one query token: q [B,H,1,D], k/v [B,H,Nk,D], bf16 or
    fp16 (of which the first kv_lens[b] keys are real, when given).
    Returns (O [B,H,1,D] in the input type, LSE fp32 [B,H] or None).
    ``workspace`` is a device tensor of at least
    fa_decode_workspace_bytes(B,H,D,num_splits) bytes; one is allocated when
    not given."""
    B, H, Nk, D = _check_decode(q, k, v, out, lse, kv_lens)
    need = fa_decode_workspace_bytes(B, H, D, num_splits)
    ws_bytes = _check_workspace(workspace) if workspace is not None else None
    _check_devices(q, k=k, v=v, out=out, lse=lse, kv_lens=kv_lens, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel()
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    lse_p = lse.data_ptr() if lse is not None else None
    lib = _lib.load()
    name = "fa_decode_splitkv" + ("_f16" if q.dtype == torch.float16 else "")
    if kv_lens is None:
        code = getattr(lib, name)(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p, workspace.data_ptr(), ws_bytes,
            B, H, Nk, D, float(scale), int(num_splits), _stream(q))
    else:
        name += "_masked"
        code = getattr(lib, name)(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_p, kv_lens.data_ptr(),
            workspace.data_ptr(), ws_bytes, B, H, Nk, D, float(scale), int(num_splits), _stream(q))
    _lib.check(code, name)
    return out, lse


def fa_decode_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_splits: int,
                              out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bf16 split-KV decode that allocates nothing: the partial states live in
    the library's fixed per-GPU scratch (DECODE_NOALLOC_SCRATCH_BYTES), so the
    caller passes the outputs, ``out`` [B,H,1,D] and optionally ``lse`` fp32
    [B,H]. Calls that may overlap in time on one GPU share that scratch and
    must be serialised by the caller. Returns (out, lse)."""
    if not isinstance(q, torch.Tensor) or q.dtype != torch.bfloat16:
        raise TypeError(f"q must be a bfloat16 tensor (got {getattr(q, 'dtype', type(q))})")
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    B, H, Nk, D = _check_decode(q, k, v, out, lse, None)
    _check_devices(q, k=k, v=v, out=out, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code = _lib.load().fa_decode_splitkv_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, H, Nk, D, float(scale), int(num_splits), _stream(q))
    _lib.check(code, "fa_decode_splitkv_noalloc")
    return out, lse


def fa_backward_workspace_bytes(B: int, H: int, Nq: int) -> int:
    return int(_lib.load().fa_backward_workspace_bytes(B, H, Nq))


def fa_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                do: torch.Tensor, lse: torch.Tensor, causal=False,
                scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                dv: Optional[torch.Tensor] = None, kv_lens: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward with recompute, bf16 or fp16: q, o, do [B,H,Nq,D], k, v
    [B,H,Nk,D], lse fp32 [B,H,Nq] (the forward's, same scale, causal and
    kv_lens). Returns (dQ, dK, dV) in the input type with the shapes of q, k,
    v. ``workspace`` holds at least fa_backward_workspace_bytes(B,H,Nq) bytes;
    one is allocated when not given."""
    if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
        raise TypeError(f"q must be a bfloat16 or float16 tensor (got {getattr(q, 'dtype', type(q))})")
    B, H, Nq, Nk, D = _check_qkv(q, k, v, q.dtype)
    _check_layout("o", o, q.dtype, q.shape)
    _check_layout("do", do, q.dtype, q.shape)
    _check_layout("lse", lse, torch.float32, (B, H, Nq))
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_layout(name, t, q.dtype, ref.shape)
    _check_kv_lens(kv_lens, B)
    mode = _causal_mode(causal)
    need = fa_backward_workspace_bytes(B, H, Nq)
    ws_bytes = _check_workspace(workspace) if workspace is not None else None
    _check_devices(q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv, kv_lens=kv_lens, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr())
    outs = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), ws_bytes)
    lib = _lib.load()
    name = "fa_backward" + ("_f16" if q.dtype == torch.float16 else "")
    if kv_lens is None:
        code = getattr(lib, name)(*ptrs, *outs, B, H, Nq, Nk, D, float(scale), mode, _stream(q))
    else:
        name += "_masked"
        code = getattr(lib, name)(*ptrs, kv_lens.data_ptr(), *outs, B, H, Nq, Nk, D, float(scale), mode,
                                  _stream(q))
    _lib.check(code, name)
    return dq, dk, dv


def _rope_style(style) -> int:
    if isinstance(style, str):
        names = {"half": ROPE_HALF, "pairs": ROPE_PAIRS}
        if style not in names:
            raise ValueError(f"style must be one of {sorted(names)} (got {style!r})")
        return names[style]
    if int(style) not in (ROPE_HALF, ROPE_PAIRS):
        raise ValueError(f"style must be 0 (half) or 1 (pairs), got {style!r}")
    return int(style)


def _check_tables(cos, sin, D):
    """cos, sin fp32 [n_pos, D/2] of one shape (device-free); returns n_pos."""
    for name, t in (("cos", cos), ("sin", sin)):
        _check_layout(name, t, torch.float32, ndim=2)
        if t.shape[1] != D // 2:
            raise ValueError(f"{name} must be [n_pos, {D // 2}]")
    if cos.shape != sin.shape:
        raise ValueError("cos and sin must have the same shape")
    return cos.shape[0]


def fa_rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, style="half",
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotary position embedding of x [B,H,N,D] (bf16 or fp16): row n rotated by
    cos[n], sin[n] (fp32 [n_pos, D/2]). ``out`` may be ``x`` (in place)."""
    if not isinstance(x, torch.Tensor) or x.dtype not in _DTYPES:
        raise TypeError(f"x must be a bfloat16 or float16 tensor (got {getattr(x, 'dtype', type(x))})")
    _check_layout("x", x, x.dtype)
    B, H, N, D = x.shape
    n_pos = _check_tables(cos, sin, D)
    if out is not None:
        _check_layout("out", out, x.dtype, x.shape)
    st = _rope_style(style)
    _check_devices(x, cos=cos, sin=sin, out=out)
    out = torch.empty_like(x) if out is None else out
    code = _lib.load().fa_rope(x.data_ptr(), out.data_ptr(), cos.data_ptr(), sin.data_ptr(), n_pos,
                               st, _DTYPES[x.dtype], B, H, N, D, _stream(x))
    _lib.check(code, "fa_rope")
    return out


def fa_rope_workspace_bytes(B: int, H: int, Nk: int, D: int) -> int:
    return int(_lib.load().fa_rope_workspace_bytes(B, H, Nk, D))


def fa_forward_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                    style="half", causal=False, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    want_lse: bool = True, kv_lens: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward pass of rope(Q), rope(K), V (bf16 or fp16): key j at position j,
    query i at position i (i + Lk - Nq under bottom-right alignment).
    Returns (O [B,H,Nq,D] in the input type, LSE fp32 [B,H,Nq] or None)."""
    if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
        raise TypeError(f"q must be a bfloat16 or float16 tensor (got {getattr(q, 'dtype', type(q))})")
    B, H, Nq, Nk, D = _check_qkv(q, k, v, q.dtype)
    n_pos = _check_tables(cos, sin, D)
    if out is not None:
        _check_layout("out", out, q.dtype, q.shape)
    if lse is not None:
        _check_layout("lse", lse, torch.float32, (B, H, Nq))
    _check_kv_lens(kv_lens, B)
    st, mode = _rope_style(style), _causal_mode(causal)
    need = fa_rope_workspace_bytes(B, H, Nk, D)
    ws_bytes = _check_workspace(workspace) if workspace is not None else None
    _check_devices(q, k=k, v=v, cos=cos, sin=sin, out=out, lse=lse, kv_lens=kv_lens, workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel()
    code = _lib.load().fa_forward_rope(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        kv_lens.data_ptr() if kv_lens is not None else None, cos.data_ptr(), sin.data_ptr(), n_pos,
        st, _DTYPES[q.dtype], workspace.data_ptr(), ws_bytes,
        B, H, Nq, Nk, D, float(scale), mode, _stream(q))
    _lib.check(code, "fa_forward_rope")
    return out, lse
