"""Denoising steps captured as HIP graphs and replayed, against the same calls launched eagerly.

One step of Algorithm 2 (Nemotron-TwoTower, arXiv 2606.26493, section 2.2): the Eq. (1)
block attention of several layers and one ConfidenceSample, captured once with
torch.cuda.graph and replayed several times, with eager work (state resets, eager calls of
the same step) between the replays. Every replay must equal the eager result bit for bit:
the library's calls allocate nothing and clear nothing, so a captured call is the same
kernels on the same arguments.
"""
import pytest
import torch

from attention_eq_block_amd import api, synth

pytestmark = pytest.mark.gpu


def test_step_graph_replays_equal_eager():
    case = synth.AttnCase(4, 16, 32, 2, 128, [1000, 8, 4096, 333], shuffle_pages=True)
    layers = []
    for i in range(3):
        inp = synth.make_attn_inputs(case, seed=5, layer=i, device="cuda")
        p = api.attn_params(inp["Q"], inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp["Kd"],
                            inp["Vd"], page_size=16, max_ctx_len=case.max_ctx_len, scale=inp["scale"])
        nb = api.block_attn_workspace_bytes(p)
        p._inputs = inp  # the struct holds raw pointers: keep the input tensors alive with it
        layers.append((p, torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda"), nb))
    B, S, V = case.B, case.S, 4096
    logits = torch.randn((B, S, V), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).cuda()
    tokens = torch.empty((B, S), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, S), dtype=torch.uint8, device="cuda")
    nmask = torch.empty((B,), dtype=torch.int32, device="cuda")
    up = api.unmask_params(logits, mask, tokens, gamma=0.5, temperature=0.1, steps_left=4, num_masked=nmask)
    uws = torch.empty(max(16, api.conf_unmask_workspace_bytes(up)), dtype=torch.uint8, device="cuda")
    lib = api.lib()

    def reset():
        tokens.fill_(-1)
        mask.fill_(1)
        for p, _, _ in layers:
            p._keep[0].fill_(float("nan"))
            p._keep[1].fill_(float("nan"))

    def step(handle):
        for p, ws, nb in layers:
            assert lib.tt_block_attn(p, ws.data_ptr(), nb, handle) == 0
        assert lib.tt_conf_unmask(up, uws.data_ptr(), uws.numel(), handle) == 0

    def state():
        return [t.clone() for p, _, _ in layers for t in p._keep] + [tokens.clone(), mask.clone(), nmask.clone()]

    reset()
    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = state()
    assert all(torch.isfinite(t.float()).all() for t in ref[:2 * len(layers)])
    assert int(mask.sum()) < B * S, "the step committed nothing: the test would not see the unmask"

    cs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        step(cs.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, state())):
            assert torch.equal(a, b), f"replay {rep}, output {i} differs from the eager step"
        # eager work between replays, on the default stream: the same step launched from the host
        reset()
        step(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, state())):
            assert torch.equal(a, b), f"eager step after replay {rep}, output {i} differs"
