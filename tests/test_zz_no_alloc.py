"""tt_block_attn_noalloc against tt_block_attn through the C ABI.

The allocation-free entry point runs the same kernels with the library's fixed
scratch array in place of a caller workspace; its outputs must equal those of
tt_block_attn bit for bit, and both must match the float64 oracle (Eq. (1) of
Nemotron-TwoTower, section 2.1) to the bf16 bar. Two calls in a row, the second
with a smaller input, so that the second runs on scratch the first has filled.
"""
import ctypes

import pytest
import torch

from attention_eq_block_amd import api, synth

from parity import check_attn, oracle_attn, to_dev

pytestmark = pytest.mark.gpu


def _params(d, inp, case, out=None, lse=None):
    return api.attn_params(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"],
                           page_size=inp["page_size"], max_ctx_len=case.max_ctx_len, scale=inp["scale"],
                           out=out, lse=lse)


@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call(o_dtype):
    lib = api.lib()
    stream = torch.cuda.current_stream().cuda_stream
    cases = [synth.attn_case("loop"),                                                   # 64 pairs, all cut
             synth.AttnCase(5, 16, 32, 2, 128, [4000, 17, 0, 900, 2500], shuffle_pages=True)]  # smaller, ragged
    for i, case in enumerate(cases):
        inp = synth.make_attn_inputs(case, seed=20 + i)
        d = to_dev(inp)
        B, S, Hq, D = inp["Q"].shape
        p = _params(d, inp, case, out=torch.empty(B, S, Hq, D, dtype=o_dtype, device="cuda"))
        nb = api.block_attn_workspace_bytes(p)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        assert lib.tt_block_attn(ctypes.byref(p), ws.data_ptr(), nb, stream) == 0
        O_ws, L_ws = p._keep
        q = _params(d, inp, case, out=torch.full((B, S, Hq, D), 7.0, dtype=o_dtype, device="cuda"),
                    lse=torch.full((B, Hq, S), 7.0, device="cuda"))
        print(f"call {i}: B={B}, prefix up to {case.max_ctx_len}, scratch {nb} bytes")
        assert lib.tt_block_attn_noalloc(ctypes.byref(q), stream) == 0
        torch.cuda.synchronize()
        O_na, L_na = q._keep
        assert torch.equal(O_na, O_ws) and torch.equal(L_na, L_ws), f"call {i}: outputs differ from tt_block_attn"
        Or, Lr = oracle_attn(inp)
        print(check_attn(O_na, L_na, Or, Lr, torch.bfloat16, f"noalloc call {i}"))


def test_noalloc_refuses_more_than_its_scratch():
    """A call whose workspace would exceed TT_NOALLOC_SCRATCH_BYTES is refused before any launch."""
    lib = api.lib()
    case = synth.AttnCase(1000, 16, 32, 2, 128, [16] * 1000)
    inp = synth.make_attn_inputs(case, seed=1)
    d = to_dev(inp)
    p = _params(d, inp, case)
    assert api.block_attn_workspace_bytes(p) > 64 << 20
    assert lib.tt_block_attn_noalloc(ctypes.byref(p), torch.cuda.current_stream().cuda_stream) == 5
