"""Causal sliding-window attention on AMD MI355X (gfx950): thin Python binding of libswattn.so.

Every step of the computation runs in the HIP kernels behind the C ABI (include/swattn.h); this
module only checks tensor metadata, allocates outputs/workspaces with torch and passes raw device
pointers plus torch's current HIP stream.  The functions ``attn_*`` mirror the C entry points one to
one; ``attention`` (autograd) and ``KVCache`` (Engine prefill/decode) are conveniences built on them.

Operations: the windowed attention kernel of the "nanochat: GPT-2-grade LLM for <<$100" post
(web3.cnoyu.life, "Jan29" entry; list of the largest improvements, item 1) and the KV-cache Engine's
prefill and decode (followin.io walkthrough, section "Pretraining", Engine paragraph).
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import SWATTN_BF16, SWATTN_F32, check, last_error, load

__all__ = [
    "attn_abi_version", "attn_last_error", "attn_fwd", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv",
    "attn_bwd_workspace_bytes",
    "attn_prefill", "attn_kv_append", "attn_decode", "attn_decode_step",
    "attn_decode_step_noalloc",
    "attn_decode_workspace_bytes", "attn_decode_launches", "attn_fwd_varlen", "attn_bwd_varlen", "attn_fwd_qknorm",
    "attn_bwd_qknorm", "attention", "attention_varlen", "attention_qknorm", "KVCache",
    "DecodeStepGraph", "FULL", "QKNORM_EPS",
]

QKNORM_EPS = 1e-6  # default eps of the QK RMS norm (the pages do not give one)

FULL = 2 ** 31 - 1  # a window that is never smaller than the sequence: full causal attention


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _win(window, n: int) -> int:
    if window is None:
        return FULL
    window = int(window)
    if window < 1:
        raise ValueError("window must be >= 1 (None = full causal)")
    return min(window, FULL)


def attn_abi_version() -> int:
    return load().attn_abi_version()


def attn_last_error() -> str:
    return last_error()


def attn_bwd_workspace_bytes(B: int, H: int, T: int, D: int) -> int:
    return load().attn_bwd_workspace_bytes(B, H, T, D)


def attn_decode_workspace_bytes(B: int, H: int, Lcap: int, D: int) -> int:
    return load().attn_decode_workspace_bytes(B, H, Lcap, D)


def attn_decode_launches(B: int, H: int, Lcap: int, D: int, window=None) -> int:
    """Kernel launches of attn_decode / attn_decode_step at these sizes: 1 (one workgroup per
    (sequence, head)) or 2 (split-K across workgroups, then a merge kernel)."""
    rc = load().attn_decode_launches(B, H, Lcap, D, _win(window, Lcap))
    if rc < 0:
        check(rc, "attn_decode_launches")
    return rc


def attn_fwd(q, k, v, o=None, lse=None, window=None, want_lse=True):
    """Forward over [B, T, H, D] (bf16 or fp32).  Returns (o, lse[B, H, T] float32 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"q must be bfloat16 or float32 (got {dt})")
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, n, (B, T, H, D), dt)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (B, T, H, D), dt)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", (B, H, T), torch.float32)
    rc = load().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse), B, H, T,
                         D, _win(window, T), SWATTN_F32 if dt == torch.float32 else SWATTN_BF16,
                         _stream(q))
    check(rc, "attn_fwd")
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, window=None, dq=None, dk=None, dv=None, ws=None):
    """Backward (bf16).  Returns (dq, dk, dv)."""
    B, T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    _need(lse, "lse", (B, H, T), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    need = attn_bwd_workspace_bytes(B, H, T, D)
    if ws is None:
        ws = torch.empty(need, device=q.device, dtype=torch.uint8)
    rc = load().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, D,
                         _win(window, T), SWATTN_BF16, ws.data_ptr(), ws.numel() * ws.element_size(),
                         _stream(q))
    check(rc, "attn_bwd")
    return dq, dk, dv


def _bwd_ws(q, ws):
    B, T, H, D = q.shape
    need = attn_bwd_workspace_bytes(B, H, T, D)
    if ws is None:
        ws = torch.empty(need, device=q.device, dtype=torch.uint8)
    return ws, ws.numel() * ws.element_size()


def attn_bwd_dq(q, k, v, o, lse, dout, ws, window=None, dq=None):
    """First backward pass: Delta into ``ws`` (keep it for attn_bwd_dkdv) and dq."""
    B, T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    _need(lse, "lse", (B, H, T), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    _need(dq, "dq", (B, T, H, D), torch.bfloat16)
    ws, nbytes = _bwd_ws(q, ws)
    rc = load().attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), B, H, T, D, _win(window, T),
                            SWATTN_BF16, ws.data_ptr(), nbytes, _stream(q))
    check(rc, "attn_bwd_dq")
    return dq


def attn_bwd_dkdv(q, k, v, lse, dout, ws, window=None, dk=None, dv=None):
    """Second backward pass: reads Delta from ``ws`` (left by attn_bwd_dq), writes dk, dv."""
    B, T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    _need(lse, "lse", (B, H, T), torch.float32)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("dk", dk), ("dv", dv)):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    if ws is None:
        raise ValueError("attn_bwd_dkdv needs the workspace filled by attn_bwd_dq")
    _, nbytes = _bwd_ws(q, ws)
    rc = load().attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                              dout.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, D,
                              _win(window, T), SWATTN_BF16, ws.data_ptr(), nbytes, _stream(q))
    check(rc, "attn_bwd_dkdv")
    return dk, dv


def attn_prefill(q, kcache, vcache, lens, o=None, lse=None, window=None, want_lse=False):
    """Ragged prefill: q [B, Tq, H, D], caches [B, Lcap, H, D], lens int32 [B] on the device."""
    B, Tq, H, D = q.shape
    Lcap = kcache.shape[1]
    _need(q, "q", None, torch.bfloat16)
    _need(kcache, "kcache", (B, Lcap, H, D), torch.bfloat16)
    _need(vcache, "vcache", (B, Lcap, H, D), torch.bfloat16)
    _need(lens, "lens", (B,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (B, Tq, H, D), torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Tq), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", (B, H, Tq), torch.float32)
    rc = load().attn_prefill(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                             o.data_ptr(), _ptr(lse), B, H, Tq, Lcap, D, _win(window, Tq),
                             _stream(q))
    check(rc, "attn_prefill")
    return o, lse


def attn_kv_append(kcache, vcache, knew, vnew, pos):
    """kcache[b, pos[b]] = knew[b] (and v); pos int32 [B] on the device."""
    B, Lcap, H, D = kcache.shape
    _need(kcache, "kcache", None, torch.bfloat16)
    _need(vcache, "vcache", (B, Lcap, H, D), torch.bfloat16)
    _need(knew, "knew", (B, H, D), torch.bfloat16)
    _need(vnew, "vnew", (B, H, D), torch.bfloat16)
    _need(pos, "pos", (B,), torch.int32)
    rc = load().attn_kv_append(kcache.data_ptr(), vcache.data_ptr(), knew.data_ptr(),
                               vnew.data_ptr(), pos.data_ptr(), B, H, Lcap, D, _stream(kcache))
    check(rc, "attn_kv_append")


def attn_decode(q, kcache, vcache, lens, o=None, lse=None, window=None, ws=None, want_lse=False):
    """Decode: q [B, H, D], caches [B, Lcap, H, D], lens int32 [B] (including the new token)."""
    B, H, D = q.shape
    Lcap = kcache.shape[1]
    _need(q, "q", None, torch.bfloat16)
    _need(kcache, "kcache", (B, Lcap, H, D), torch.bfloat16)
    _need(vcache, "vcache", (B, Lcap, H, D), torch.bfloat16)
    _need(lens, "lens", (B,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (B, H, D), torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty((B, H), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", (B, H), torch.float32)
    need = attn_decode_workspace_bytes(B, H, Lcap, D)
    if ws is None:
        ws = torch.empty(need, device=q.device, dtype=torch.uint8)
    rc = load().attn_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), lens.data_ptr(),
                            o.data_ptr(), _ptr(lse), B, H, Lcap, D, _win(window, Lcap),
                            ws.data_ptr(), ws.numel() * ws.element_size(), _stream(q))
    check(rc, "attn_decode")
    return o, lse


def attn_decode_step(q, knew, vnew, kcache, vcache, pos, o=None, lse=None, window=None, ws=None,
                     want_lse=False):
    """Append + decode in one call: kcache[b, pos[b]] = knew[b] (and v), then q [B, H, D] attends
    to cache rows .. pos[b].  pos int32 [B] on the device counts the cached tokens before the step."""
    B, H, D = q.shape
    Lcap = kcache.shape[1]
    _need(q, "q", None, torch.bfloat16)
    _need(knew, "knew", (B, H, D), torch.bfloat16)
    _need(vnew, "vnew", (B, H, D), torch.bfloat16)
    _need(kcache, "kcache", (B, Lcap, H, D), torch.bfloat16)
    _need(vcache, "vcache", (B, Lcap, H, D), torch.bfloat16)
    _need(pos, "pos", (B,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (B, H, D), torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty((B, H), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", (B, H), torch.float32)
    need = attn_decode_workspace_bytes(B, H, Lcap, D)
    if ws is None:
        ws = torch.empty(need, device=q.device, dtype=torch.uint8)
    rc = load().attn_decode_step(q.data_ptr(), knew.data_ptr(), vnew.data_ptr(), kcache.data_ptr(),
                                 vcache.data_ptr(), pos.data_ptr(), o.data_ptr(), _ptr(lse), B, H,
                                 Lcap, D, _win(window, Lcap), ws.data_ptr(),
                                 ws.numel() * ws.element_size(), _stream(q))
    check(rc, "attn_decode_step")
    return o, lse


def attn_decode_step_noalloc(q, knew, vnew, kcache, vcache, pos, o, lse=None, window=None):
    """attn_decode_step with no workspace: the library keeps the split schedule's partial results
    in a static device array (32 MiB per GPU), so the call allocates nothing.  The output ``o``
    ([B, H, D] bf16) and the optional ``lse`` ([B, H] float32) must be given.  Calls on one GPU
    share that array and must not run concurrently."""
    B, H, D = q.shape
    Lcap = kcache.shape[1]
    _need(q, "q", None, torch.bfloat16)
    _need(knew, "knew", (B, H, D), torch.bfloat16)
    _need(vnew, "vnew", (B, H, D), torch.bfloat16)
    _need(kcache, "kcache", (B, Lcap, H, D), torch.bfloat16)
    _need(vcache, "vcache", (B, Lcap, H, D), torch.bfloat16)
    _need(pos, "pos", (B,), torch.int32)
    _need(o, "o", (B, H, D), torch.bfloat16)
    if lse is not None:
        _need(lse, "lse", (B, H), torch.float32)
    rc = load().attn_decode_step_noalloc(q.data_ptr(), knew.data_ptr(), vnew.data_ptr(),
                                         kcache.data_ptr(), vcache.data_ptr(), pos.data_ptr(),
                                         o.data_ptr(), _ptr(lse), B, H, Lcap, D,
                                         _win(window, Lcap), _stream(q))
    check(rc, "attn_decode_step_noalloc")
    return o, lse


def _cu(cu_seqlens, device):
    _need(cu_seqlens, "cu_seqlens", None, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [nseq + 1] with nseq >= 1")
    if cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be on the same device as q")
    return cu_seqlens.numel() - 1


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, o=None, lse=None, window=None,
                    want_lse=True):
    """Packed sequences: q, k, v [total, H, D] bf16, sequence s = rows cu_seqlens[s] ..
    cu_seqlens[s + 1] - 1 attending only to itself.  Returns (o, lse [H, total] or None)."""
    total, H, D = q.shape
    _need(q, "q", None, torch.bfloat16)
    _need(k, "k", (total, H, D), torch.bfloat16)
    _need(v, "v", (total, H, D), torch.bfloat16)
    nseq = _cu(cu_seqlens, q.device)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (total, H, D), torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty((H, total), device=q.device, dtype=torch.float32)
    if lse is not None:
        _need(lse, "lse", (H, total), torch.float32)
    rc = load().attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse),
                                cu_seqlens.data_ptr(), nseq, total, int(max_seqlen), H, D,
                                _win(window, int(max_seqlen)), _stream(q))
    check(rc, "attn_fwd_varlen")
    return o, lse


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, window=None, dq=None, dk=None,
                    dv=None, ws=None):
    """Backward of attn_fwd_varlen.  Returns (dq, dk, dv), each [total, H, D] bf16."""
    total, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, (total, H, D), torch.bfloat16)
    _need(lse, "lse", (H, total), torch.float32)
    nseq = _cu(cu_seqlens, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, (total, H, D), torch.bfloat16)
    need = attn_bwd_workspace_bytes(1, H, total, D)
    if ws is None:
        ws = torch.empty(need, device=q.device, dtype=torch.uint8)
    rc = load().attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), cu_seqlens.data_ptr(), nseq, total, int(max_seqlen),
                                H, D, _win(window, int(max_seqlen)), ws.data_ptr(),
                                ws.numel() * ws.element_size(), _stream(q))
    check(rc, "attn_bwd_varlen")
    return dq, dk, dv


def attn_fwd_qknorm(q, k, v, window=None, eps=QKNORM_EPS, o=None, want_lse=True):
    """Attention over RMS-normalised q and k rows ([B, T, H, D] bf16).  Returns
    (o, lse, qn, kn, rq, rk): the normalised rows and 1 / rms per row [B, H, T] feed the backward."""
    B, T, H, D = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    rq = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    rk = torch.empty_like(rq)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (B, T, H, D), torch.bfloat16)
    lse = torch.empty((B, H, T), device=q.device, dtype=torch.float32) if want_lse else None
    rc = load().attn_fwd_qknorm(q.data_ptr(), k.data_ptr(), v.data_ptr(), qn.data_ptr(),
                                kn.data_ptr(), rq.data_ptr(), rk.data_ptr(), o.data_ptr(),
                                _ptr(lse), B, H, T, D, _win(window, T), float(eps), _stream(q))
    check(rc, "attn_fwd_qknorm")
    return o, lse, qn, kn, rq, rk


def attn_bwd_qknorm(qn, kn, v, o, lse, dout, rq, rk, window=None, dq=None, dk=None, dv=None,
                    ws=None):
    """Backward of attn_fwd_qknorm: (dq, dk, dv) with respect to the raw q, k and v."""
    B, T, H, D = qn.shape
    for t, n in ((qn, "qn"), (kn, "kn"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    for t, n in ((lse, "lse"), (rq, "rq"), (rk, "rk")):
        _need(t, n, (B, H, T), torch.float32)
    dq = torch.empty_like(qn) if dq is None else dq
    dk = torch.empty_like(kn) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, (B, T, H, D), torch.bfloat16)
    need = attn_bwd_workspace_bytes(B, H, T, D)
    if ws is None:
        ws = torch.empty(need, device=qn.device, dtype=torch.uint8)
    rc = load().attn_bwd_qknorm(qn.data_ptr(), kn.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), rq.data_ptr(), rk.data_ptr(),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, D,
                                _win(window, T), ws.data_ptr(), ws.numel() * ws.element_size(),
                                _stream(qn))
    check(rc, "attn_bwd_qknorm")
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, window):
        o, lse = attn_fwd(q, k, v, window=window)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.window = window
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), window=ctx.window)
        return dq, dk, dv, None


def attention(q, k, v, window=None):
    """Differentiable windowed causal attention over [B, T, H, D] bf16 tensors."""
    return _Attention.apply(q, k, v, window)


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, window):
        o, lse = attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, window=window)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.max_seqlen, ctx.window = max_seqlen, window
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu = ctx.saved_tensors
        dq, dk, dv = attn_bwd_varlen(q, k, v, o, lse, do.contiguous(), cu, ctx.max_seqlen,
                                     window=ctx.window)
        return dq, dk, dv, None, None, None


class _AttentionQKNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, window, eps):
        o, lse, qn, kn, rq, rk = attn_fwd_qknorm(q, k, v, window=window, eps=eps)
        ctx.save_for_backward(qn, kn, v, o, lse, rq, rk)
        ctx.window = window
        return o

    @staticmethod
    def backward(ctx, do):
        qn, kn, v, o, lse, rq, rk = ctx.saved_tensors
        dq, dk, dv = attn_bwd_qknorm(qn, kn, v, o, lse, do.contiguous(), rq, rk, window=ctx.window)
        return dq, dk, dv, None, None


def attention_qknorm(q, k, v, window=None, eps=QKNORM_EPS):
    """Differentiable attention over RMS-normalised q and k ([B, T, H, D] bf16): the norm has no
    parameters; gradients flow back to the raw q and k."""
    return _AttentionQKNorm.apply(q, k, v, window, eps)


def attention_varlen(q, k, v, cu_seqlens, max_seqlen, window=None):
    """Differentiable attention over packed sequences (documents): q, k, v [total, H, D] bf16."""
    return _AttentionVarlen.apply(q, k, v, cu_seqlens, max_seqlen, window)


class KVCache:
    """Per-layer KV cache [n_layer][B, Lcap, H, D] bf16 with Engine prefill / decode.

    ``lens`` (device int32 [B]) counts the cached tokens; ``decode`` appends the new token at row
    ``lens`` and then attends with ``lens + 1`` keys.  The same ``lens`` serves every layer, so
    advance it with ``step()`` once per generated token after the last layer.

    ``max_len`` is a host-side upper bound of ``lens`` (set by ``prefill`` / ``set_lens``, advanced
    by ``step``): ``decode`` raises instead of letting a sequence run past the capacity, where the
    kernels would append nothing and return o = 0.
    """

    def __init__(self, n_layer, B, Lcap, H, D, device="cuda", windows=None):
        self.n_layer, self.B, self.Lcap, self.H, self.D = n_layer, B, Lcap, H, D
        shape = (n_layer, B, Lcap, H, D)
        self.k = torch.zeros(shape, device=device, dtype=torch.bfloat16)
        self.v = torch.zeros(shape, device=device, dtype=torch.bfloat16)
        self.lens = torch.zeros(B, device=device, dtype=torch.int32)
        self.max_len = 0
        self.windows = list(windows) if windows is not None else [None] * n_layer
        self._ws = torch.empty(attn_decode_workspace_bytes(B, H, Lcap, D), device=device,
                               dtype=torch.uint8)

    def set_lens(self, lens, max_len=None):
        """Set the cached-token counts (int32 [B]); ``max_len`` (host int) is their maximum, read
        from the device when not given."""
        self.lens.copy_(lens)
        self.max_len = int(lens.max()) if max_len is None else int(max_len)
        if self.max_len > self.Lcap:
            raise ValueError(f"a length of {self.max_len} exceeds the cache capacity {self.Lcap}")

    def prefill(self, layer, q, k, v, lens):
        """Write prompts (padded [B, Tq, H, D]) into the cache and attend causally."""
        Tq = q.shape[1]
        if Tq > self.Lcap:
            raise ValueError("prompt longer than the cache")
        self.k[layer, :, :Tq].copy_(k)
        self.v[layer, :, :Tq].copy_(v)
        self.set_lens(lens)
        o, _ = attn_prefill(q, self.k[layer], self.v[layer], self.lens,
                            window=self.windows[layer])
        return o

    def _check_room(self):
        if self.max_len >= self.Lcap:
            raise RuntimeError(f"KV cache full: a sequence holds up to {self.max_len} of "
                               f"{self.Lcap} rows, so the next token has no row to go to")

    def decode(self, layer, q, k_new, v_new, o=None):
        """Append the new token's key / value at row ``lens`` and attend (one call)."""
        self._check_room()
        o, _ = attn_decode_step(q, k_new, v_new, self.k[layer], self.v[layer], self.lens, o=o,
                                window=self.windows[layer], ws=self._ws)
        return o

    def step(self):
        self._check_room()
        self.lens.add_(1)
        self.max_len += 1


class DecodeStepGraph:
    """One generated token's attention over every layer of a ``KVCache``, captured once in a HIP
    graph (torch.cuda.CUDAGraph) and replayed per token.

    The graph reads the per-layer inputs from fixed buffers ``q``, ``k_new``, ``v_new``
    ([n_layer, B, H, D] bf16) and writes ``o`` ([n_layer, B, H, D]); it appends to the cache,
    attends, and finally advances ``cache.lens`` by one.  Fill the inputs, call ``replay()``, read
    ``o``.  Only library kernels and one elementwise add are captured (no memset nodes).
    ``replay`` raises, as ``KVCache.decode`` does, once the cache has no room for another token.
    """

    def __init__(self, cache: KVCache):
        self.cache = cache
        shape = (cache.n_layer, cache.B, cache.H, cache.D)
        dev = cache.lens.device
        self.q = torch.zeros(shape, device=dev, dtype=torch.bfloat16)
        self.k_new = torch.zeros_like(self.q)
        self.v_new = torch.zeros_like(self.q)
        self.o = torch.zeros_like(self.q)
        # one eager pass first, so every kernel is loaded before capture; pos = -1 writes nothing
        idle = torch.full_like(cache.lens, -1)
        for layer in range(cache.n_layer):
            attn_decode_step(self.q[layer], self.k_new[layer], self.v_new[layer], cache.k[layer],
                             cache.v[layer], idle, o=self.o[layer], window=cache.windows[layer],
                             ws=cache._ws)
        torch.cuda.synchronize(dev)
        # capture records the launches without running them: the host-side length bound must not
        # advance for it
        max_len = cache.max_len
        cache.max_len = 0
        self.graph = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(self.graph):
                for layer in range(cache.n_layer):
                    cache.decode(layer, self.q[layer], self.k_new[layer], self.v_new[layer],
                                 o=self.o[layer])
                cache.step()
        finally:
            cache.max_len = max_len

    def replay(self):
        self.cache._check_room()
        self.graph.replay()
        self.cache.max_len += 1
        return self.o
