"""Python face of libtwotower_attn: its C-ABI calls on torch tensors.

Argument marshalling only -- shapes, strides, device pointers and the current
stream go to the library; every step of the computation runs in its HIP
kernels. torch provides device memory and streams.

Method: Nemotron-TwoTower (arXiv 2606.26493): ``block_attn`` is Eq. (1) of
section 2.1, ``lse_merge`` combines partial attentions over disjoint parts of
Eq. (1)'s key set, ``conf_unmask`` is the ConfidenceSample step of
Algorithm 2 (section 2.2), ``kv_append`` grows a layer's context cache by a
committed block (Algorithm 1, section 2.1), ``masked_nll`` is the training
loss L_MD of Eq. (4).
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from ._lib import TT_BF16, TT_F32, BlockAttnParams, ConfUnmaskParams, KvAppendParams, MaskedNllParams, check, lib

_DT = {torch.bfloat16: TT_BF16, torch.float32: TT_F32}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must share one device")


def _ws(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} bytes < {nbytes}")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_params(Q, Kc, Vc, page_table, ctx_len, Kd=None, Vd=None, *, page_size: int, max_ctx_len: int,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, o_dtype=None,
                debug_flags: Optional[torch.Tensor] = None) -> BlockAttnParams:
    """Build the parameter struct for ``tt_block_attn`` (allocating ``out``/``lse`` if absent).

    Shapes, dtypes and layouts are checked here, before anything reaches the library, so that a
    mismatched tensor raises ValueError instead of making a kernel read out of bounds.
    ``debug_flags``: a one-element int32 tensor that turns on the library's device-side data
    checks (TT_DEBUG_* bits are ORed into it).
    """
    if Q.dim() != 4:
        raise ValueError("Q must be [B][S][Hq][head_dim]")
    B, S, Hq, D = Q.shape
    if Q.stride(3) != 1:
        raise ValueError("Q's head_dim must be contiguous")
    Hkv = Kc.shape[1] if Kc is not None else (Kd.shape[2] if Kd is not None else Hq)
    if Kc is not None:
        if Vc is None or Kc.dim() != 4 or tuple(Vc.shape) != tuple(Kc.shape):
            raise ValueError("Kc and Vc must both be [num_pages][Hkv][page_size][head_dim]")
        if Kc.shape[3] != D:
            raise ValueError(f"the cache's head_dim {Kc.shape[3]} differs from Q's {D}")
        if Kc.dtype != Q.dtype or Vc.dtype != Q.dtype:
            raise TypeError("the cache must have Q's dtype")
    if (Kd is None) != (Vd is None):
        raise ValueError("Kd and Vd go together")
    if Kd is not None:
        if tuple(Kd.shape) != (B, S, Hkv, D) or tuple(Vd.shape) != (B, S, Hkv, D):
            raise ValueError(f"Kd and Vd must be [B][S][Hkv][head_dim] = {(B, S, Hkv, D)}")
        if Kd.dtype != Q.dtype or Vd.dtype != Q.dtype:
            raise TypeError("Kd and Vd must have Q's dtype")
    if ctx_len is not None and tuple(ctx_len.shape) != (B,):
        raise ValueError("ctx_len must be [B]")
    if page_table is not None and (page_table.dim() != 2 or page_table.shape[0] < B):
        raise ValueError("page_table must be [B][max_pages]")
    if debug_flags is not None and (debug_flags.dtype != torch.int32 or debug_flags.numel() < 1):
        raise ValueError("debug_flags must be an int32 tensor")
    if o_dtype is None:
        o_dtype = Q.dtype
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=o_dtype, device=Q.device)
    elif tuple(out.shape) != (B, S, Hq, D) or out.stride(3) != 1:
        raise ValueError("out must be [B][S][Hq][head_dim] with head_dim contiguous")
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=Q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be dense float32 [B][Hq][S]")
    p = BlockAttnParams()
    p.dtype = _code(Q)
    p.o_dtype = _code(out)
    p.B, p.S, p.Hq, p.Hkv, p.head_dim = B, S, Hq, Hkv, D
    p.softmax_scale = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    p.Q = _ptr(Q)
    p.q_stride_b, p.q_stride_s, p.q_stride_h = Q.stride(0), Q.stride(1), Q.stride(2)
    if Kc is not None:
        if not (Kc.is_contiguous() and Vc.is_contiguous()):
            raise ValueError("the paged cache must be dense [num_pages][Hkv][page_size][head_dim]")
        if Kc.shape[2] != page_size:
            raise ValueError("Kc.shape[2] must equal page_size")
        p.Kctx, p.Vctx = _ptr(Kc), _ptr(Vc)
        p.num_pages = Kc.shape[0]
    p.page_size = page_size
    if page_table is not None:
        if page_table.dtype != torch.int32 or not page_table.is_contiguous():
            raise ValueError("page_table must be dense int32 [B][max_pages]")
        p.page_table = _ptr(page_table)
        p.max_pages = page_table.shape[1]
    if ctx_len is not None:
        if ctx_len.dtype != torch.int32:
            raise ValueError("ctx_len must be int32")
        p.ctx_len = _ptr(ctx_len)
    p.max_ctx_len = int(max_ctx_len)
    if Kd is not None:
        if Kd.stride() != Vd.stride() or Kd.stride(3) != 1:
            raise ValueError("Kden and Vden must share strides with head_dim contiguous")
        p.Kden, p.Vden = _ptr(Kd), _ptr(Vd)
        p.den_stride_b, p.den_stride_s, p.den_stride_h = Kd.stride(0), Kd.stride(1), Kd.stride(2)
    p.O = _ptr(out)
    p.o_stride_b, p.o_stride_s, p.o_stride_h = out.stride(0), out.stride(1), out.stride(2)
    p.LSE = _ptr(lse)
    p.debug_flags = _ptr(debug_flags)
    p._keep = (out, lse)  # keep outputs alive with the struct
    return p


def block_attn_workspace_bytes(p: BlockAttnParams) -> int:
    return int(lib().tt_block_attn_workspace_bytes(p))


def block_attn(Q, Kc, Vc, page_table, ctx_len, Kd=None, Vd=None, *, page_size: int = 16,
               max_ctx_len: Optional[int] = None, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, o_dtype=None,
               workspace: Optional[torch.Tensor] = None, debug_flags: Optional[torch.Tensor] = None):
    """Eq. (1) for one attention layer: returns (O [B][S][Hq][D], LSE [B][Hq][S] float32).

    Q [B][S][Hq][D]; Kc, Vc [num_pages][Hkv][page_size][D]; page_table [B][max_pages] int32;
    ctx_len [B] int32; Kd, Vd [B][S][Hkv][D] or None (prefix-only partial). ``max_ctx_len``
    is the host-side bound of ctx_len (read back from the device when omitted).
    """
    _need_cuda(Q, Kc, Vc, page_table, ctx_len, Kd, Vd, out, lse, workspace, debug_flags)
    if max_ctx_len is None:
        max_ctx_len = int(ctx_len.max().item()) if ctx_len is not None and ctx_len.numel() else 0
    p = attn_params(Q, Kc, Vc, page_table, ctx_len, Kd, Vd, page_size=page_size, max_ctx_len=max_ctx_len,
                    scale=scale, out=out, lse=lse, o_dtype=o_dtype, debug_flags=debug_flags)
    out, lse = p._keep
    ws = _ws(block_attn_workspace_bytes(p), Q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(lib().tt_block_attn(p, _ptr(ws), nbytes, _stream(Q)), "tt_block_attn")
    return out, lse


def lse_merge(O_parts: torch.Tensor, lse_parts: torch.Tensor, *, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, o_dtype=torch.float32):
    """Merge P partials: O_parts [P][B][S][Hq][d] f32, lse_parts [P][B][Hq][S] f32 -> (O, lse)."""
    _need_cuda(O_parts, lse_parts, out, lse)
    P, B, S, Hq, d = O_parts.shape
    if O_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials are float32")
    if not (O_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("partials must be dense")
    if tuple(lse_parts.shape) != (P, B, Hq, S):
        raise ValueError("lse_parts must be [P][B][Hq][S]")
    if out is None:
        out = torch.empty((B, S, Hq, d), dtype=o_dtype, device=O_parts.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=O_parts.device)
    if not out.is_contiguous():
        raise ValueError("out must be dense")
    check(lib().tt_lse_merge(P, _ptr(O_parts), _ptr(lse_parts), B, S, Hq, d, _ptr(out), _code(out), _ptr(lse),
                             _stream(O_parts)), "tt_lse_merge")
    return out, lse


def unmask_params(logits, mask_in, tokens, *, gamma: float, temperature: float, steps_left: int,
                  mask_out=None, conf=None, num_masked=None, uniforms=None) -> ConfUnmaskParams:
    B, S, V = logits.shape
    if logits.stride(2) != 1 or logits.stride(0) != S * logits.stride(1):
        raise ValueError("logits rows must be evenly strided with the vocabulary contiguous")
    for t, name, dt in ((mask_in, "mask_in", torch.uint8), (tokens, "tokens", torch.int32)):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != (B, S):
            raise ValueError(f"{name} must be dense {dt} [B][S]")
    if uniforms is not None and (uniforms.dtype != torch.float32 or not uniforms.is_contiguous()
                                 or tuple(uniforms.shape) != (B, S)):
        raise ValueError("uniforms must be dense float32 [B][S]")
    if mask_out is not None and (mask_out.dtype != torch.uint8 or not mask_out.is_contiguous()
                                 or tuple(mask_out.shape) != (B, S)):
        raise ValueError("mask_out must be dense uint8 [B][S]")
    if conf is not None and (conf.dtype != torch.float32 or not conf.is_contiguous()
                             or tuple(conf.shape) != (B, S)):
        raise ValueError("conf must be dense float32 [B][S]")
    if num_masked is not None and (num_masked.dtype != torch.int32 or not num_masked.is_contiguous()
                                   or tuple(num_masked.shape) != (B,)):
        raise ValueError("num_masked must be dense int32 [B]")
    p = ConfUnmaskParams()
    p.dtype = _code(logits)
    p.B, p.S, p.V = B, S, V
    p.logits = _ptr(logits)
    p.logits_stride_row = logits.stride(1)
    p.mask_in = _ptr(mask_in)
    p.mask_out = _ptr(mask_in if mask_out is None else mask_out)
    p.tokens = _ptr(tokens)
    p.gamma = float(gamma)
    p.temperature = float(temperature)
    p.steps_left = int(steps_left)
    p.conf = _ptr(conf)
    p.num_masked = _ptr(num_masked)
    p.uniforms = _ptr(uniforms)
    return p


def conf_unmask(logits, mask_in, tokens, *, gamma: float, temperature: float = 1.0, steps_left: int = 1,
                mask_out=None, conf=None, num_masked=None, uniforms=None, workspace=None):
    """One ConfidenceSample step, in place on ``tokens`` and ``mask_out`` (default: ``mask_in``).

    logits [B][S][V] bf16/f32; mask_in [B][S] uint8 (1 = masked); tokens [B][S] int32.
    Optional outputs: conf [B][S] float32 (masked rows), num_masked [B] int32.
    uniforms [B][S] float32 in [0, 1): draw each token from softmax(x / temperature)
    instead of taking the argmax (confidence = the drawn token's probability).
    Returns (tokens, mask_out).
    """
    _need_cuda(logits, mask_in, tokens, mask_out, conf, num_masked, uniforms, workspace)
    p = unmask_params(logits, mask_in, tokens, gamma=gamma, temperature=temperature, steps_left=steps_left,
                      mask_out=mask_out, conf=conf, num_masked=num_masked, uniforms=uniforms)
    ws = _ws(int(lib().tt_conf_unmask_workspace_bytes(p)), logits.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(lib().tt_conf_unmask(p, _ptr(ws), nbytes, _stream(logits)), "tt_conf_unmask")
    return tokens, (mask_in if mask_out is None else mask_out)


def conf_unmask_workspace_bytes(p: ConfUnmaskParams) -> int:
    return int(lib().tt_conf_unmask_workspace_bytes(p))


def append_params(Kc, Vc, page_table, ctx_len, Knew, Vnew, *, pool=None, pool_count=None,
                  status=None) -> KvAppendParams:
    """Build the parameter struct for ``tt_kv_append`` (allocating ``status`` if absent)."""
    num_pages, Hkv, page_size, D = Kc.shape
    B, S = Knew.shape[0], Knew.shape[1]
    if not (Kc.is_contiguous() and Vc.is_contiguous()) or Vc.shape != Kc.shape or Vc.dtype != Kc.dtype:
        raise ValueError("the paged caches must be dense and alike [num_pages][Hkv][page_size][head_dim]")
    if Knew.dtype != Kc.dtype or Vnew.dtype != Kc.dtype:
        raise TypeError("new rows must have the cache's dtype")
    if tuple(Knew.shape) != (B, S, Hkv, D) or Knew.stride() != Vnew.stride() or Knew.stride(3) != 1:
        raise ValueError("Knew and Vnew must be [B][S][Hkv][head_dim] with equal strides, head_dim contiguous")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != B:
        raise ValueError("page_table must be dense int32 [B][max_pages]")
    if ctx_len.dtype != torch.int32 or tuple(ctx_len.shape) != (B,):
        raise ValueError("ctx_len must be int32 [B]")
    if (pool is None) != (pool_count is None):
        raise ValueError("pool and pool_count go together")
    for t, name in ((pool, "pool"), (pool_count, "pool_count")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be dense int32")
    if status is None:
        status = torch.full((1,), -1, dtype=torch.int32, device=Kc.device)
    p = KvAppendParams()
    p.dtype = _code(Kc)
    p.B, p.S, p.Hkv, p.head_dim = B, S, Hkv, D
    p.Kctx, p.Vctx = _ptr(Kc), _ptr(Vc)
    p.page_size, p.num_pages, p.max_pages = page_size, num_pages, page_table.shape[1]
    p.page_table, p.ctx_len = _ptr(page_table), _ptr(ctx_len)
    p.Knew, p.Vnew = _ptr(Knew), _ptr(Vnew)
    p.new_stride_b, p.new_stride_s, p.new_stride_h = Knew.stride(0), Knew.stride(1), Knew.stride(2)
    p.pool, p.pool_count, p.status = _ptr(pool), _ptr(pool_count), _ptr(status)
    p._keep = (status,)
    return p


def kv_append(Kc, Vc, page_table, ctx_len, Knew, Vnew, *, pool=None, pool_count=None, status=None):
    """Append each sequence's S new K/V rows at its ctx_len, in place, and grow ctx_len by S.

    Kc, Vc [num_pages][Hkv][page_size][D]; page_table [B][max_pages] int32 (entries < 0 are
    filled from ``pool``); ctx_len [B] int32; Knew, Vnew [B][S][Hkv][D]; pool int32 page ids with
    pool_count a one-element int32 tensor. Returns the one-element int32 status tensor (device):
    0 appended, 1 capacity, 2 pool exhausted, 3 page id out of range (then nothing changed).
    """
    _need_cuda(Kc, Vc, page_table, ctx_len, Knew, Vnew, pool, pool_count, status)
    p = append_params(Kc, Vc, page_table, ctx_len, Knew, Vnew, pool=pool, pool_count=pool_count, status=status)
    check(lib().tt_kv_append(p, _stream(Kc)), "tt_kv_append")
    return p._keep[0]


def nll_params(logits, targets, mask, *, nll=None, loss=None, count=None) -> MaskedNllParams:
    B, S, V = logits.shape
    if logits.stride(2) != 1 or logits.stride(0) != S * logits.stride(1):
        raise ValueError("logits rows must be evenly strided with the vocabulary contiguous")
    for t, name, dt in ((targets, "targets", torch.int32), (mask, "mask", torch.uint8)):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != (B, S):
            raise ValueError(f"{name} must be dense {dt} [B][S]")
    if nll is not None and (nll.dtype != torch.float32 or not nll.is_contiguous() or tuple(nll.shape) != (B, S)):
        raise ValueError("nll must be dense float32 [B][S]")
    if loss is None:
        loss = torch.zeros(1, dtype=torch.float32, device=logits.device)
    p = MaskedNllParams()
    p.dtype = _code(logits)
    p.B, p.S, p.V = B, S, V
    p.logits, p.logits_stride_row = _ptr(logits), logits.stride(1)
    p.targets, p.mask = _ptr(targets), _ptr(mask)
    p.nll, p.loss, p.count = _ptr(nll), _ptr(loss), _ptr(count)
    p._keep = (loss,)
    return p


def masked_nll(logits, targets, mask, *, nll=None, count=None, loss=None, workspace=None):
    """L_MD of Eq. (4): mean over masked positions of logsumexp(x) - x[target]. Returns the loss as a
    one-element float32 device tensor; ``nll`` [B][S] float32 receives the per-position values and
    ``count`` (one int32) the number of masked positions, when given."""
    _need_cuda(logits, targets, mask, nll, count, loss, workspace)
    p = nll_params(logits, targets, mask, nll=nll, loss=loss, count=count)
    ws = _ws(int(lib().tt_masked_nll_workspace_bytes(p)), logits.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(lib().tt_masked_nll(p, _ptr(ws), nbytes, _stream(logits)), "tt_masked_nll")
    return p._keep[0]


def abi_version() -> int:
    return int(lib().tt_abi_version())


def status_string(code: int) -> str:
    return lib().tt_status_string(code).decode()


__all__ = ["block_attn", "lse_merge", "conf_unmask", "kv_append", "masked_nll", "attn_params", "unmask_params",
           "append_params", "nll_params",
           "block_attn_workspace_bytes", "conf_unmask_workspace_bytes", "abi_version", "status_string",
           "TT_F32", "TT_BF16", "_lib"]
