"""tt_block_attn on seeded random shapes against the float64 oracle.

Eq. (1) of Nemotron-TwoTower (arXiv 2606.26493, section 2.1, "Bidirectional
attention"). Each seed draws one call: batch, block size S, query and KV heads,
head_dim, page size, prefix lengths (zero, short, ragged and page-unaligned ones
among them), page order, whether the block keys are present, input and output
dtype and value scale. Every output row and LSE is compared with the oracle at
the tolerances of parity.py. The shapes stay small enough for the oracle to
finish in about a second each, but span several tiles, row blocks and pieces.
"""
import numpy as np
import pytest
import torch

from attention_eq_block_amd import synth

from parity import check_attn, gpu_attn, oracle_attn

pytestmark = pytest.mark.gpu

HEADS = [(1, 1), (4, 1), (8, 2), (6, 3), (16, 2), (32, 2), (32, 8), (12, 4)]


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    S = int(rng.choice([1, 2, 5, 16, 31, 64]))
    Hq, Hkv = HEADS[int(rng.integers(len(HEADS)))]
    D = int(rng.choice([64, 128]))
    page_size = int(rng.choice([16, 32, 48, 64]))
    kind = int(rng.integers(4))
    if kind == 0:  # short and zero prefixes
        ctx = rng.integers(0, 80, size=B)
    elif kind == 1:  # ragged up to a few thousand
        ctx = rng.integers(1, 3000, size=B)
    elif kind == 2:  # one long, others short
        ctx = rng.integers(0, 200, size=B)
        ctx[int(rng.integers(B))] = int(rng.integers(2000, 6000))
    else:  # equal lengths, page-unaligned
        ctx = np.full(B, int(rng.integers(100, 2500)) | 1)
    dtype = torch.float32 if rng.random() < 0.2 else torch.bfloat16
    with_den = bool(rng.random() < 0.85)
    if not with_den and int(ctx.max()) == 0:
        ctx[0] = 17
    case = synth.AttnCase(B, S, Hq, Hkv, D, [int(x) for x in ctx], dtype=dtype, page_size=page_size,
                          shuffle_pages=bool(rng.random() < 0.7), with_den=with_den,
                          value_scale=float(rng.choice([1.0, 1.0 / np.sqrt(D)])),
                          spare_pages=int(rng.integers(0, 4)), poison_tail=bool(rng.random() < 0.3))
    o_dtype = torch.float32 if (dtype == torch.bfloat16 and rng.random() < 0.25) else None
    return case, o_dtype


@pytest.mark.parametrize("seed", range(300))
def test_random_shapes(seed):
    case, o_dtype = draw_case(seed)
    inp = synth.make_attn_inputs(case, seed=seed)
    O, L = gpu_attn(inp, o_dtype=o_dtype)
    Or, Lr = oracle_attn(inp)
    what = (f"seed {seed}: B={case.B} S={case.S} heads {case.Hq}/{case.Hkv} d={case.D} page {case.page_size} "
            f"ctx {list(case.ctx_lens)} den {case.with_den} {case.dtype} out {o_dtype}")
    print(what, check_attn(O, L, Or, Lr, case.dtype, what))
