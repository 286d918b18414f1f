"""Consecutive blocks of block-diffusion decoding (Nemotron-TwoTower, section 2.1 "Bidirectional
attention" and Eq. (1); section 2.2, Algorithms 1 and 2) on the GPU against the oracle.

Each block starts fully masked and is denoised step by step: in every step each layer runs Eq. (1)
over its own paged context cache, then one confidence-unmasking step commits positions. Once the
block is committed, its K/V rows are appended to every layer's cache (the context update of
Algorithm 1), so the next block attends over a longer prefix that ends mid-page and whose new pages
come from the pool. The GPU and the oracle keep separate caches. After every append the caches,
tables, lengths and pool counts are compared exactly. Every attention output and every unmasking
step is compared at the bars of the single-call tests, with the GPU's own state carried forward.
The layers between attention and the logits need trained weights and are not part of this path, so
queries, block keys and values, logits and the committed rows' K/V are seeded synthetic inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_eq_block_amd import api, synth

from parity import check_attn, check_unmask, gpu_attn, oracle_attn

pytestmark = pytest.mark.gpu

LAYERS = 2
BLOCKS = 3
STEPS = 4       # T: the last step commits whatever is still masked
S = 16
HQ, HKV = 8, 2
V = 1000
SUB_Q, SUB_KD, SUB_VD, SUB_KN, SUB_VN = 40, 41, 42, 43, 44


def _states(ctx0, D, page_size, seed):
    """Per layer: the GPU's cache state (device tensors) and the oracle's (CPU), from one draw."""
    B = len(ctx0)
    max_pages = (max(ctx0) + BLOCKS * S + page_size - 1) // page_size + 1
    spare = B * ((BLOCKS * S + page_size - 1) // page_size + 1) + 3
    out = []
    for layer in range(LAYERS):
        inp = synth.make_append_inputs(B, S, HKV, D, page_size, max_pages=max_pages, ctx_lens=ctx0,
                                       spare_pages=spare, seed=seed + layer)
        ora = dict(Kc=inp["Kc"].clone(), Vc=inp["Vc"].clone(), page_table=inp["page_table"].clone(),
                   ctx_len=inp["ctx_len"].clone(), pool=inp["pool"].clone(), pool_count=inp["pool_count"])
        gpu = dict(Kc=inp["Kc"].cuda(), Vc=inp["Vc"].cuda(), page_table=inp["page_table"].cuda(),
                   ctx_len=inp["ctx_len"].cuda(), pool=inp["pool"].cuda(),
                   pool_count=torch.tensor([inp["pool_count"]], dtype=torch.int32, device="cuda"))
        out.append((gpu, ora))
    return out


def _attend(gpu, ora, Q, Kd, Vd, D, page_size, what):
    """Eq. (1) over each side's own cache; unassigned table entries (-1, past every length) are
    clamped to page 0 on both sides."""
    a = dict(Q=Q, Kc=gpu["Kc"], Vc=gpu["Vc"], page_table=gpu["page_table"].clamp(min=0), ctx_len=gpu["ctx_len"],
             Kd=Kd, Vd=Vd, page_size=page_size, scale=D ** -0.5)
    O, L = gpu_attn(a)
    r = dict(Q=Q, Kc=ora["Kc"], Vc=ora["Vc"], page_table=ora["page_table"].clamp(min=0), ctx_len=ora["ctx_len"],
             Kd=Kd, Vd=Vd, page_size=page_size, scale=D ** -0.5)
    Or, Lr = oracle_attn(r)
    check_attn(O, L, Or, Lr, torch.bfloat16, what)


def _commit(gpu, ora, Kn, Vn, what):
    st = api.kv_append(gpu["Kc"], gpu["Vc"], gpu["page_table"], gpu["ctx_len"], Kn.cuda(), Vn.cuda(),
                       pool=gpu["pool"], pool_count=gpu["pool_count"])
    torch.cuda.synchronize()
    ref = oracle.kv_append(ora["Kc"], ora["Vc"], ora["page_table"], ora["ctx_len"], Kn, Vn,
                           pool=ora["pool"].tolist(), pool_count=ora["pool_count"])
    assert int(st.item()) == 0 and ref["status"] == 0, (what, int(st.item()), ref["status"])
    ora.update(Kc=ref["Kc"], Vc=ref["Vc"], page_table=torch.from_numpy(ref["page_table"]),
               ctx_len=torch.from_numpy(ref["ctx_len"]), pool_count=ref["pool_count"])
    for k in ("Kc", "Vc"):
        assert torch.equal(gpu[k].cpu().view(torch.uint8), ora[k].view(torch.uint8)), f"{what}: {k} differs"
    assert torch.equal(gpu["page_table"].cpu(), ora["page_table"]), f"{what}: page table differs"
    assert torch.equal(gpu["ctx_len"].cpu(), ora["ctx_len"]), f"{what}: ctx_len differs"
    assert int(gpu["pool_count"].item()) == ora["pool_count"], f"{what}: pool count differs"


@pytest.mark.parametrize("ctx0,D,page_size,draw", [
    ([0, 37, 160], 128, 16, False),       # an empty prefix, one mid-page, one page-aligned
    ([5, 100, 0, 61], 64, 48, False),     # pages of 48 rows: each block ends at a new offset within a page
    ([23, 0, 64], 128, 32, True),         # tokens drawn at the temperature from caller uniforms
])
def test_blocks_with_commit_append(ctx0, D, page_size, draw):
    B = len(ctx0)
    seed = 50 + D + page_size
    layers = _states(ctx0, D, page_size, seed)
    ucase = synth.UnmaskCase(B, S, V, gamma=0.8, temperature=0.1)
    for j in range(BLOCKS):
        targets = synth.spike_targets(B, S, V, seed=seed + j)
        tokens, mask = synth.make_mask_state(B, S)
        for r in range(1, STEPS + 1):
            step = 100 * j + r
            for layer, (gpu, ora) in enumerate(layers):
                Q = synth.randn((B, S, HQ, D), seed, SUB_Q, layer, step, dtype=torch.bfloat16)
                Kd = synth.randn((B, S, HKV, D), seed, SUB_KD, layer, step, dtype=torch.bfloat16)
                Vd = synth.randn((B, S, HKV, D), seed, SUB_VD, layer, step, dtype=torch.bfloat16)
                _attend(gpu, ora, Q, Kd, Vd, D, page_size, f"block {j} step {r} layer {layer}")
            x = synth.make_logits(ucase, seed=seed + j, step=r, spike=1.0 * r, targets=targets)
            # B is 3 or 4: one sequence with a decision closer than the confidences' float32
            # resolution is left out of the exact comparison, as in the single-step tests
            u = synth.make_uniforms(B, S, seed=seed + j, step=r) if draw else None
            got, _, _ = check_unmask(x, mask, tokens, gamma=0.8, temperature=0.1, steps_left=STEPS - r + 1,
                                     what=f"block {j} step {r}", max_fragile_frac=0.34, uniforms=u)
            tokens = torch.from_numpy(got["tokens"])
            mask = torch.from_numpy(got["mask"])
            if int(mask.sum()) == 0:
                break
        assert int(mask.sum()) == 0, f"block {j} must complete within {STEPS} steps"
        for layer, (gpu, ora) in enumerate(layers):
            Kn = synth.randn((B, S, HKV, D), seed, SUB_KN, layer, j, dtype=torch.bfloat16)
            Vn = synth.randn((B, S, HKV, D), seed, SUB_VN, layer, j, dtype=torch.bfloat16)
            _commit(gpu, ora, Kn, Vn, f"commit of block {j}, layer {layer}")
    for gpu, _ in layers:
        assert np.array_equal(gpu["ctx_len"].cpu().numpy(), np.array(ctx0) + BLOCKS * S)
