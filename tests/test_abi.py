"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments on the host before launching anything.

No test here passes a pointer a kernel could dereference: every call is one
that validation must refuse, so these tests are safe with or without a GPU.
"""
import ctypes
import math
import subprocess

import pytest

from attention_eq_block_amd import _lib
from attention_eq_block_amd._lib import (TT_BF16, TT_F32, BlockAttnParams, ConfUnmaskParams, KvAppendParams,
                                         MaskedNllParams)

FAKE = 0x1000  # never dereferenced: every call below must fail validation first


def test_library_loads_and_reports_version():
    L = _lib.lib()
    assert L.tt_abi_version() == 3


def test_exports_every_header_function():
    names = _lib.header_functions()
    assert set(names) == {"tt_abi_version", "tt_status_string", "tt_block_attn", "tt_block_attn_workspace_bytes",
                          "tt_block_attn_noalloc",
                          "tt_lse_merge", "tt_conf_unmask", "tt_conf_unmask_workspace_bytes", "tt_kv_append",
                          "tt_masked_nll", "tt_masked_nll_workspace_bytes"}
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert not [s for s in exported if s.startswith("tt_") and s not in names], "undeclared tt_ export"


def test_status_strings():
    L = _lib.lib()
    for code, name in _lib.STATUS.items():
        assert L.tt_status_string(code).decode().startswith(name)
    assert L.tt_status_string(99) == b"unknown tt_status"


def attn_ok(**kw):
    """A parameter set that passes validation in every field except those overridden."""
    p = BlockAttnParams()
    p.dtype, p.o_dtype = TT_BF16, TT_BF16
    p.B, p.S, p.Hq, p.Hkv, p.head_dim = 2, 16, 32, 2, 128
    p.softmax_scale = 1 / math.sqrt(128)
    p.Q = p.O = p.Kctx = p.Vctx = p.page_table = p.ctx_len = p.Kden = p.Vden = FAKE
    p.q_stride_h, p.q_stride_s, p.q_stride_b = 128, 32 * 128, 16 * 32 * 128
    p.o_stride_h, p.o_stride_s, p.o_stride_b = 128, 32 * 128, 16 * 32 * 128
    p.den_stride_h, p.den_stride_s, p.den_stride_b = 128, 2 * 128, 16 * 2 * 128
    p.page_size, p.num_pages, p.max_pages, p.max_ctx_len = 16, 64, 32, 512
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def call_attn(p, ws=None, nbytes=0):
    return _lib.lib().tt_block_attn(ctypes.byref(p), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 3), (dict(dtype=TT_F32, o_dtype=TT_BF16), 3),
    (dict(S=0), 2), (dict(S=65), 2), (dict(Hq=30, Hkv=4), 2), (dict(Hkv=0), 2), (dict(B=-1), 2),
    (dict(head_dim=96), 4), (dict(head_dim=256), 4),
    (dict(softmax_scale=0.0), 6), (dict(softmax_scale=float("nan")), 6), (dict(softmax_scale=-1.0), 6),
    (dict(softmax_scale=float("inf")), 6),
    (dict(Q=None), 1), (dict(O=None), 1), (dict(Kden=None), 1), (dict(Kctx=None), 1), (dict(page_table=None), 1),
    (dict(ctx_len=None), 1),
    (dict(page_size=8), 2), (dict(page_size=24), 2), (dict(max_pages=31), 2), (dict(num_pages=0), 2),
    (dict(max_ctx_len=-3), 2),
    (dict(Q=FAKE + 8), 4), (dict(O=FAKE + 2), 4), (dict(Kctx=FAKE + 4), 4), (dict(q_stride_h=100), 4),
    (dict(den_stride_s=4), 4), (dict(o_stride_b=-8), 4),
    (dict(B=1 << 13, page_size=1024, max_ctx_len=1 << 26, max_pages=1 << 16), 2),  # 2^34 tiles
    (dict(q_stride_b=1 << 31), 4), (dict(o_stride_s=1 << 32), 4),  # strides must fit 31 bits
    (dict(B=1 << 15, max_pages=1 << 15), 4),  # page table past 2^30 entries
    # offsets inside one sequence are 32-bit byte offsets: (S-1)*stride_s + (H-1)*stride_h + d < 2^30
    (dict(q_stride_s=1 << 27), 4), (dict(o_stride_s=1 << 27), 4), (dict(den_stride_s=1 << 27), 4),
    (dict(q_stride_h=1 << 26), 4),
    (dict(q_stride_s=1 << 25, o_stride_s=1 << 25, den_stride_s=1 << 25), 5),  # within the bound: valid
])
def test_attn_validation(kw, code):
    rc = call_attn(attn_ok(**kw))
    assert rc == code, (kw, _lib.STATUS.get(rc))


def test_attn_valid_args_need_workspace():
    assert call_attn(attn_ok()) == 5
    nb = _lib.lib().tt_block_attn_workspace_bytes(ctypes.byref(attn_ok()))
    assert nb > 0
    assert call_attn(attn_ok(), None, nb) == 5


def test_attn_zero_batch_is_a_noop():
    assert call_attn(attn_ok(B=0, Q=None, O=None)) == 0


def test_attn_workspace_bytes_of_invalid_is_zero():
    assert _lib.lib().tt_block_attn_workspace_bytes(ctypes.byref(attn_ok(S=0))) == 0
    assert _lib.lib().tt_block_attn_workspace_bytes(None) == 0
    assert _lib.lib().tt_block_attn(None, None, 0, None) == 1


def test_attn_workspace_grows_with_batch():
    L = _lib.lib()
    a = L.tt_block_attn_workspace_bytes(ctypes.byref(attn_ok(B=2)))
    b = L.tt_block_attn_workspace_bytes(ctypes.byref(attn_ok(B=64)))
    assert b > a > 0


def unmask_ok(**kw):
    p = ConfUnmaskParams()
    p.dtype, p.B, p.S, p.V = TT_BF16, 4, 16, 131072
    p.logits = p.mask_in = p.mask_out = p.tokens = FAKE
    p.logits_stride_row = 131072
    p.gamma, p.temperature, p.steps_left = 0.8, 0.1, 16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 3), (dict(S=0), 2), (dict(S=65), 2), (dict(V=0), 2), (dict(logits_stride_row=100), 2),
    (dict(B=-2), 2), (dict(gamma=float("nan")), 6), (dict(temperature=0.0), 6), (dict(temperature=-1.0), 6),
    (dict(temperature=float("inf")), 6), (dict(steps_left=0), 6), (dict(logits=None), 1), (dict(mask_in=None), 1),
    (dict(mask_out=None), 1), (dict(tokens=None), 1), (dict(logits=FAKE + 1), 4),
    (dict(dtype=TT_F32, logits=FAKE + 2), 4),
])
def test_unmask_validation(kw, code):
    rc = _lib.lib().tt_conf_unmask(ctypes.byref(unmask_ok(**kw)), None, 0, None)
    assert rc == code, (kw, _lib.STATUS.get(rc))


def test_unmask_needs_workspace_and_zero_batch_noop():
    L = _lib.lib()
    nb = L.tt_conf_unmask_workspace_bytes(ctypes.byref(unmask_ok()))
    assert nb > 0
    assert L.tt_conf_unmask(ctypes.byref(unmask_ok()), None, nb, None) == 5
    assert L.tt_conf_unmask(ctypes.byref(unmask_ok(B=0, logits=None)), None, 0, None) == 0
    assert L.tt_conf_unmask(None, None, 0, None) == 1


def test_unmask_gamma_extremes_are_valid_arguments():
    # any non-NaN gamma is allowed; the call then only lacks a workspace
    for g in (-1.0, 0.0, 1.0, 2.0, float("inf"), float("-inf")):
        assert _lib.lib().tt_conf_unmask(ctypes.byref(unmask_ok(gamma=g)), None, 0, None) == 5


@pytest.mark.parametrize("args,code", [
    ((0, FAKE, FAKE, 1, 1, 1, 64, FAKE, TT_F32, None), 2),
    ((2, FAKE, FAKE, 1, 0, 1, 64, FAKE, TT_F32, None), 2),
    ((2, FAKE, FAKE, 1, 1, 0, 64, FAKE, TT_F32, None), 2),
    ((2, FAKE, FAKE, 1, 1, 1, 6, FAKE, TT_F32, None), 2),
    ((2, FAKE, FAKE, 1, 1, 1, 64, FAKE, 7, None), 3),
    ((2, None, FAKE, 1, 1, 1, 64, FAKE, TT_F32, None), 1),
    ((2, FAKE, FAKE, 1, 1, 1, 64, None, TT_F32, None), 1),
    ((2, FAKE + 4, FAKE, 1, 1, 1, 64, FAKE, TT_F32, None), 4),
    ((2, FAKE, FAKE, 1, 1, 1, 12, FAKE, TT_BF16, None), 4),
    ((2, None, None, 0, 1, 1, 64, None, TT_F32, None), 0),
])
def test_merge_validation(args, code):
    rc = _lib.lib().tt_lse_merge(*args, None)
    assert rc == code


def append_ok(**kw):
    p = KvAppendParams()
    p.dtype, p.B, p.S, p.Hkv, p.head_dim = TT_BF16, 4, 16, 2, 128
    p.Kctx = p.Vctx = p.page_table = p.ctx_len = p.Knew = p.Vnew = p.status = FAKE
    p.page_size, p.num_pages, p.max_pages = 16, 64, 16
    p.new_stride_b, p.new_stride_s, p.new_stride_h = 16 * 2 * 128, 2 * 128, 128
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 3), (dict(B=-1), 2), (dict(S=0), 2), (dict(S=65), 2), (dict(Hkv=0), 2), (dict(head_dim=0), 2),
    (dict(page_size=0), 2), (dict(num_pages=0), 2), (dict(max_pages=0), 2), (dict(head_dim=4), 4),
    (dict(dtype=TT_F32, head_dim=2), 4), (dict(B=1 << 20, max_pages=1 << 10), 4),
    (dict(Kctx=None), 1), (dict(Vctx=None), 1), (dict(page_table=None), 1), (dict(ctx_len=None), 1),
    (dict(Knew=None), 1), (dict(Vnew=None), 1), (dict(status=None), 1), (dict(pool=FAKE), 1),
    (dict(pool_count=FAKE), 1), (dict(Knew=FAKE + 8), 4), (dict(Kctx=FAKE + 2), 4), (dict(new_stride_s=100), 4),
    (dict(new_stride_h=-8), 4),
])
def test_append_validation(kw, code):
    rc = _lib.lib().tt_kv_append(ctypes.byref(append_ok(**kw)), None)
    assert rc == code, (kw, _lib.STATUS.get(rc))


def test_append_zero_batch_is_a_noop():
    L = _lib.lib()
    assert L.tt_kv_append(ctypes.byref(append_ok(B=0, Kctx=None, Knew=None, status=None)), None) == 0
    assert L.tt_kv_append(None, None) == 1


def nll_ok(**kw):
    p = MaskedNllParams()
    p.dtype, p.B, p.S, p.V = TT_BF16, 4, 16, 131072
    p.logits = p.targets = p.mask = p.loss = FAKE
    p.logits_stride_row = 131072
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 3), (dict(B=-1), 2), (dict(S=0), 2), (dict(V=0), 2), (dict(logits_stride_row=100), 2),
    (dict(B=1 << 16, S=1 << 15), 2), (dict(logits=None), 1), (dict(targets=None), 1), (dict(mask=None), 1),
    (dict(loss=None), 1), (dict(logits=FAKE + 1), 4), (dict(dtype=TT_F32, logits=FAKE + 2), 4),
])
def test_nll_validation(kw, code):
    rc = _lib.lib().tt_masked_nll(ctypes.byref(nll_ok(**kw)), None, 0, None)
    assert rc == code, (kw, _lib.STATUS.get(rc))


def test_nll_needs_workspace_and_zero_batch_noop():
    L = _lib.lib()
    nb = L.tt_masked_nll_workspace_bytes(ctypes.byref(nll_ok()))
    assert nb > 0
    assert L.tt_masked_nll(ctypes.byref(nll_ok()), None, nb, None) == 5
    assert L.tt_masked_nll(ctypes.byref(nll_ok(B=0, logits=None)), None, 0, None) == 0
    assert L.tt_masked_nll(None, None, 0, None) == 1


def test_unmask_sampling_workspace_holds_the_draws():
    """With uniforms the workspace also holds one (token, confidence) pair of 8 bytes per position."""
    L = _lib.lib()
    g = L.tt_conf_unmask_workspace_bytes(ctypes.byref(unmask_ok()))
    s = L.tt_conf_unmask_workspace_bytes(ctypes.byref(unmask_ok(uniforms=FAKE)))
    assert s == g + 4 * 16 * 8


def test_unmask_sampling_vocabulary_bound():
    """With uniforms a vocabulary split may hold at most 2^21 logits, and a drawing step takes at
    most 64 splits (at least one per 16384 logits), so V = 2^27 + 512 is refused with TT_ERR_SHAPE
    by the host-side validation and V = 2^27 is not. The logits and workspace pointers are NULL:
    were the bound ever to pass, the call would stop at TT_ERR_NULL and still launch nothing."""
    L = _lib.lib()
    big = (1 << 27) + 512
    p = unmask_ok(B=256, S=16, V=big, logits_stride_row=big, uniforms=FAKE, logits=None)
    assert L.tt_conf_unmask_workspace_bytes(ctypes.byref(p)) == 0
    assert L.tt_conf_unmask(ctypes.byref(p), None, 0, None) == 2
    # the same vocabulary without uniforms, or a vocabulary within the bound, is not refused for its size
    assert L.tt_conf_unmask(ctypes.byref(unmask_ok(B=256, S=16, V=big, logits_stride_row=big, logits=None)),
                            None, 0, None) == 1
    ok = 1 << 27
    assert L.tt_conf_unmask(ctypes.byref(unmask_ok(B=256, S=16, V=ok, logits_stride_row=ok, uniforms=FAKE,
                                                   logits=None)), None, 0, None) == 1


# --------------------------------------------------------------------------- the Python binding

def _cpu_attn_tensors(B=2, S=16, Hq=32, Hkv=2, D=128, P=16, pages=8, max_pages=4):
    import torch
    bf = torch.bfloat16
    return dict(Q=torch.zeros(B, S, Hq, D, dtype=bf), Kc=torch.zeros(pages, Hkv, P, D, dtype=bf),
                Vc=torch.zeros(pages, Hkv, P, D, dtype=bf),
                page_table=torch.zeros(B, max_pages, dtype=torch.int32),
                ctx_len=torch.zeros(B, dtype=torch.int32), Kd=torch.zeros(B, S, Hkv, D, dtype=bf),
                Vd=torch.zeros(B, S, Hkv, D, dtype=bf))


@pytest.mark.parametrize("change", [
    "Kc_head_dim", "Vc_shape", "Kd_shape", "Vd_shape", "ctx_len_shape", "table_rows", "Kd_without_Vd",
    "cache_dtype", "out_shape", "lse_shape", "lse_dtype", "debug_dtype",
])
def test_attn_params_rejects_mismatched_tensors(change):
    """attn_params checks shapes and dtypes before anything reaches the library (CPU tensors: the
    checks come before any pointer is used)."""
    import torch
    from attention_eq_block_amd import api
    t = _cpu_attn_tensors()
    kw = {}
    if change == "Kc_head_dim":
        t["Kc"] = torch.zeros(8, 2, 16, 64, dtype=torch.bfloat16)
        t["Vc"] = t["Kc"].clone()
    elif change == "Vc_shape":
        t["Vc"] = torch.zeros(7, 2, 16, 128, dtype=torch.bfloat16)
    elif change == "Kd_shape":
        t["Kd"] = torch.zeros(2, 15, 2, 128, dtype=torch.bfloat16)
    elif change == "Vd_shape":
        t["Vd"] = torch.zeros(2, 16, 1, 128, dtype=torch.bfloat16)
    elif change == "ctx_len_shape":
        t["ctx_len"] = torch.zeros(3, dtype=torch.int32)
    elif change == "table_rows":
        t["page_table"] = torch.zeros(1, 4, dtype=torch.int32)
    elif change == "Kd_without_Vd":
        t["Vd"] = None
    elif change == "cache_dtype":
        t["Kc"] = t["Kc"].float()
        t["Vc"] = t["Vc"].float()
    elif change == "out_shape":
        kw["out"] = torch.zeros(2, 16, 32, 64, dtype=torch.bfloat16)
    elif change == "lse_shape":
        kw["lse"] = torch.zeros(2, 16, 32)
    elif change == "lse_dtype":
        kw["lse"] = torch.zeros(2, 32, 16, dtype=torch.float64)
    elif change == "debug_dtype":
        kw["debug_flags"] = torch.zeros(1, dtype=torch.int64)
    with pytest.raises((ValueError, TypeError)):
        api.attn_params(t["Q"], t["Kc"], t["Vc"], t["page_table"], t["ctx_len"], t["Kd"], t["Vd"], page_size=16,
                        max_ctx_len=64, **kw)


def test_attn_params_accepts_matching_tensors():
    from attention_eq_block_amd import api
    t = _cpu_attn_tensors()
    p = api.attn_params(t["Q"], t["Kc"], t["Vc"], t["page_table"], t["ctx_len"], t["Kd"], t["Vd"], page_size=16,
                        max_ctx_len=64)
    assert p.B == 2 and p.Hkv == 2 and p.debug_flags is None


@pytest.mark.parametrize("change", ["conf_dtype", "conf_shape", "num_masked_dtype", "num_masked_shape",
                                    "mask_out_dtype", "mask_out_shape"])
def test_unmask_params_rejects_mismatched_tensors(change):
    import torch
    from attention_eq_block_amd import api
    B, S, V = 2, 16, 1000
    x = torch.zeros(B, S, V, dtype=torch.bfloat16)
    mask = torch.ones(B, S, dtype=torch.uint8)
    tokens = torch.zeros(B, S, dtype=torch.int32)
    kw = {}
    if change == "conf_dtype":
        kw["conf"] = torch.zeros(B, S, dtype=torch.float64)
    elif change == "conf_shape":
        kw["conf"] = torch.zeros(B, S + 1)
    elif change == "num_masked_dtype":
        kw["num_masked"] = torch.zeros(B, dtype=torch.int64)
    elif change == "num_masked_shape":
        kw["num_masked"] = torch.zeros(B, S, dtype=torch.int32)
    elif change == "mask_out_dtype":
        kw["mask_out"] = torch.zeros(B, S, dtype=torch.int32)
    elif change == "mask_out_shape":
        kw["mask_out"] = torch.zeros(B, S - 1, dtype=torch.uint8)
    with pytest.raises(ValueError):
        api.unmask_params(x, mask, tokens, gamma=0.8, temperature=0.1, steps_left=16, **kw)


def test_noalloc_validates_and_refuses_oversized_calls_before_any_launch():
    """tt_block_attn_noalloc validates like tt_block_attn, and refuses a call whose workspace would
    exceed the library's fixed scratch (TT_NOALLOC_SCRATCH_BYTES = 64 MiB) with TT_ERR_WORKSPACE,
    before touching the device (the pointers here are fake)."""
    L = _lib.lib()
    f = L.tt_block_attn_noalloc
    assert f(None, None) == 1
    assert f(ctypes.byref(attn_ok(S=0)), None) == 2
    assert f(ctypes.byref(attn_ok(B=0, Q=None, O=None)), None) == 0
    big = attn_ok(B=1000, max_pages=1, max_ctx_len=16)
    assert L.tt_block_attn_workspace_bytes(ctypes.byref(big)) > 64 << 20
    assert f(ctypes.byref(big), None) == 5
