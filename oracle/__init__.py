"""ctypes wrapper of the float64 CPU oracle (``oracle/tt_oracle.c``).

Test infrastructure only: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are its only users. It shares no code with the
HIP library and never calls it.

Each function follows the Nemotron-TwoTower paper (arXiv 2606.26493):
``block_attn`` is Eq. (1) of section 2.1, ``lse_merge`` is the split of
Eq. (1)'s concatenated key set into disjoint parts, ``conf_unmask`` is the
ConfidenceSample step of Algorithm 2 (section 2.2, "Sampling"),
``kv_append`` is the cache side of Algorithm 1's context update after a
block is committed (section 2.1), ``masked_nll`` is the loss L_MD of Eq. (4)
(section 2.2).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TT_ORACLE_LIBRARY selects another build of the oracle (the sanitizer test loads one)
_LIB_PATH = os.environ.get("TT_ORACLE_LIBRARY") or os.path.join(_HERE, "libtt_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library; a path selects another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    lib.oracle_block_attn.restype = _I
    lib.oracle_block_attn.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.c_double, _P, _P, _P, _I, _I, _P, _I,
                                      _P, _I, _P, _P, _I, _P, _P, _P]
    lib.oracle_lse_merge.restype = _I
    lib.oracle_lse_merge.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    lib.oracle_conf_unmask.restype = _I
    lib.oracle_conf_unmask.argtypes = [_I, _I, _I, _I, ctypes.c_longlong, _P, _P, _P, ctypes.c_double,
                                       ctypes.c_double, _I, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_num_threads.restype = _I
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [_I]
    lib.oracle_kv_append.restype = _I
    lib.oracle_kv_append.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_masked_nll.restype = _I
    lib.oracle_masked_nll.argtypes = [_I, _I, _I, _I, ctypes.c_longlong, _P, _P, _P, _P, _P, _P]
    return lib


class use_library:
    """Context manager: route the wrappers to another build of the oracle
    (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def num_threads() -> int:
    return int(load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on."""
    load().oracle_set_num_threads(int(n))


def _raw(t: Optional[torch.Tensor]):
    """(numpy array kept alive, pointer, dtype code) of a CPU tensor, widened as-is."""
    if t is None:
        return None, None, None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        a = t.view(torch.int16).numpy().view(np.uint16)
        code = 1
    elif t.dtype == torch.float32:
        a = t.numpy()
        code = 0
    else:
        raise TypeError(f"oracle inputs are float32 or bfloat16, got {t.dtype}")
    return a, a.ctypes.data, code


def _i32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu")
        return np.ascontiguousarray(t.numpy().astype(np.int32))
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def all_rows(B: int, Hq: int, S: int) -> np.ndarray:
    """Every (b, h, s) triple, in [B][Hq][S] order."""
    b, h, s = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(S), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), s.ravel()], axis=1).astype(np.int32)


def block_attn(Q, Kc, Vc, page_table, ctx_len, Kd=None, Vd=None, *, page_size: int,
               scale: float, rows=None, max_ctx_len: Optional[int] = None):
    """Eq. (1) for the selected (b, h, s) rows (all rows when ``rows`` is None).

    Returns (O, LSE) as float64 numpy arrays: with ``rows=None`` they have the
    shapes [B][S][Hq][D] and [B][Hq][S]; otherwise [n][D] and [n].

    Out-of-range data reads as the library defines it: a prefix length clamped into
    [0, min(max_ctx_len, max_pages * page_size)] (no max_ctx_len: the table's
    capacity), a page id clamped into [0, num_pages).
    """
    B, S, Hq, D = Q.shape
    Hkv = Kc.shape[1]
    if Kc.shape[2] != page_size:
        raise ValueError("Kc's third dimension must be page_size")
    qa, qp, dt = _raw(Q)
    ka, kp, dk = _raw(Kc)
    va, vp, _ = _raw(Vc)
    kda, kdp, _ = _raw(Kd)
    vda, vdp, _ = _raw(Vd)
    if dk != dt:
        raise TypeError("Q and the cache must share a dtype")
    pt = _i32(page_table).reshape(B, -1)
    cl = _i32(ctx_len)
    cap = pt.shape[1] * int(page_size)
    len_cap = cap if max_ctx_len is None else min(int(max_ctx_len), cap)
    full = rows is None
    r = all_rows(B, Hq, S) if full else _i32(rows).reshape(-1, 3)
    n = r.shape[0]
    O = np.zeros((n, D), np.float64)
    L = np.zeros((n,), np.float64)
    rc = load().oracle_block_attn(dt, B, S, Hq, Hkv, D, float(scale), qp, kp, vp, int(page_size), int(Kc.shape[0]),
                                  pt.ctypes.data, pt.shape[1], cl.ctypes.data, len_cap, kdp, vdp, n,
                                  r.ctypes.data, O.ctypes.data, L.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_block_attn rejected its arguments")
    del qa, ka, va, kda, vda
    if full:
        O = O.reshape(B, Hq, S, D).transpose(0, 2, 1, 3).copy()
        L = L.reshape(B, Hq, S)
    return O, L


def lse_merge(O_parts, lse_parts):
    """O_parts [P][n][D], lse_parts [P][n] (float64) -> (O [n][D], lse [n])."""
    Op = np.ascontiguousarray(np.asarray(O_parts, dtype=np.float64))
    lp = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
    P, n, D = Op.shape
    O = np.zeros((n, D), np.float64)
    L = np.zeros((n,), np.float64)
    rc = load().oracle_lse_merge(P, n, D, Op.ctypes.data, lp.ctypes.data, O.ctypes.data, L.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_lse_merge rejected its arguments")
    return O, L


def conf_unmask(logits, mask, tokens, *, gamma: float, temperature: float, steps_left: int, uniforms=None):
    """One ConfidenceSample step. ``gamma`` and ``temperature`` are used as given
    (pass float32-rounded values to mirror a float32 caller). With ``uniforms``
    ([B][S] float32 in [0, 1)) each masked row's token is drawn from
    softmax(x / temperature) by inverse transform sampling instead of taken greedily.

    Returns dict(tokens, mask, conf, argmax, margin, num_masked) as numpy arrays; ``argmax``
    is the predicted token (greedy or drawn) and ``margin`` (sampling only, else None) the
    distance of u from the cumulative values bracketing the drawn token.
    """
    B, S, V = logits.shape
    la, lp, dt = _raw(logits)
    mk = np.ascontiguousarray(np.asarray(mask.cpu() if isinstance(mask, torch.Tensor) else mask,
                                         dtype=np.uint8))
    tk = _i32(tokens)
    tok_out = np.zeros((B, S), np.int32)
    mask_out = np.zeros((B, S), np.uint8)
    conf = np.zeros((B, S), np.float64)
    am = np.zeros((B, S), np.int32)
    nm = np.zeros((B,), np.int32)
    un = margin = None
    if uniforms is not None:
        un = np.ascontiguousarray(np.asarray(uniforms.cpu() if isinstance(uniforms, torch.Tensor) else uniforms,
                                             dtype=np.float32).reshape(B, S))
        margin = np.full((B, S), np.nan, np.float64)
    rc = load().oracle_conf_unmask(dt, B, S, V, V, lp, mk.ctypes.data, tk.ctypes.data, float(gamma),
                                   float(temperature), int(steps_left), None if un is None else un.ctypes.data,
                                   tok_out.ctypes.data, mask_out.ctypes.data, conf.ctypes.data, am.ctypes.data,
                                   None if margin is None else margin.ctypes.data, nm.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_conf_unmask rejected its arguments")
    del la
    return dict(tokens=tok_out, mask=mask_out, conf=conf, argmax=am, margin=margin, num_masked=nm)


def kv_append(Kc, Vc, page_table, ctx_len, Knew, Vnew, pool=None, pool_count=0):
    """Commit-time cache append (Algorithm 1, section 2.1) on CPU copies; inputs are unchanged.

    Kc, Vc [num_pages][Hkv][page_size][D] (float32 or bfloat16); page_table [B][max_pages];
    ctx_len [B]; Knew, Vnew [B][S][Hkv][D] of the cache's dtype; pool: page ids (or None) with
    pool_count of them in use. Returns dict(Kc, Vc, page_table, ctx_len, pool_count, status) with
    torch tensors for the caches and numpy arrays for the integers.
    """
    num_pages, Hkv, page_size, D = Kc.shape
    B, S = Knew.shape[0], Knew.shape[1]
    dt = Kc.dtype
    if Vc.dtype != dt or Knew.dtype != dt or Vnew.dtype != dt:
        raise TypeError("caches and new rows must share a dtype")
    esz = {torch.float32: 4, torch.bfloat16: 2}[dt]

    def raw(t):
        t = t.detach().to("cpu").contiguous().clone()
        return t, t.view(torch.uint8).numpy()

    Kt, ka = raw(Kc)
    Vt, va = raw(Vc)
    _, kn = raw(Knew)
    _, vn = raw(Vnew)
    pt = _i32(page_table).reshape(B, -1).copy()
    cl = _i32(ctx_len).copy()
    pl = _i32(pool if pool is not None else [0]).copy()
    pc = np.array([int(pool_count)], np.int32)
    rc = load().oracle_kv_append(esz, B, S, Hkv, D, page_size, num_pages, pt.shape[1], ka.ctypes.data,
                                 va.ctypes.data, pt.ctypes.data, cl.ctypes.data, kn.ctypes.data, vn.ctypes.data,
                                 pl.ctypes.data, pc.ctypes.data if pool is not None else None)
    return dict(Kc=Kt, Vc=Vt, page_table=pt, ctx_len=cl, pool_count=int(pc[0]), status=int(rc))


def masked_nll(logits, targets, mask):
    """L_MD of Eq. (4) in float64: returns dict(nll [B][S] (NaN where unmasked), loss, count)."""
    B, S, V = logits.shape
    la, lp, dt = _raw(logits)
    tg = _i32(targets).reshape(B, S)
    mk = np.ascontiguousarray(np.asarray(mask.cpu() if isinstance(mask, torch.Tensor) else mask, dtype=np.uint8))
    nll = np.full((B, S), np.nan, np.float64)
    loss = np.zeros(1, np.float64)
    cnt = np.zeros(1, np.int32)
    load().oracle_masked_nll(dt, B, S, V, V, lp, tg.ctypes.data, mk.ctypes.data, nll.ctypes.data, loss.ctypes.data,
                             cnt.ctypes.data)
    del la
    return dict(nll=nll, loss=float(loss[0]), count=int(cnt[0]))


def f32(x: float) -> float:
    """x rounded to float32, as a float32 caller hands it to the library."""
    return float(np.float32(x))
