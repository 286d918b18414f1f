"""tt_kv_append on seeded random appends against the oracle (the cache side of Algorithm 1's
context update after a block is committed, Nemotron-TwoTower section 2.1).

Each seed draws one append: batch, block size S, KV heads, head_dim, dtype, page size
(including sizes that are not a power of two), lengths (zero, mid-page, page-aligned, near
capacity), table capacity and spare pages. A pool one page short of what the append
needs, or an exactly full sequence, sometimes turns the call into an error that must
change nothing. Caches (byte for byte), page table, lengths, pool count and status must
equal the oracle's.
"""
import numpy as np
import pytest
import torch

from attention_eq_block_amd import synth

from test_gpu_append import _gpu, _oracle, _same

pytestmark = pytest.mark.gpu


def draw_append(seed):
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 12))
    S = int(rng.choice([1, 3, 8, 16, 33, 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([64, 128]))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    page_size = int(rng.choice([1, 3, 16, 24, 64]))
    max_pages = int(rng.integers(1, 40))
    cap = max_pages * page_size
    ctx = []
    for _ in range(B):
        r = rng.random()
        if r < 0.15:
            ctx.append(0)
        elif r < 0.3:
            ctx.append(max(0, cap - S))  # fills the sequence exactly
        elif r < 0.4:
            ctx.append(int(rng.integers(0, max(1, cap // page_size)) * page_size))  # page-aligned
        else:
            ctx.append(int(rng.integers(0, max(1, cap - S + 1))))
    # pages the append needs beyond those already assigned
    need = sum(max(0, -(-(c + S) // page_size) - (-(-c // page_size))) for c in ctx)
    short = rng.random() < 0.15 and need > 0
    spare = need - 1 if short else need + int(rng.integers(0, 5))
    inp = synth.make_append_inputs(B, S, Hkv, D, page_size, max_pages=max_pages, ctx_lens=ctx,
                                   spare_pages=max(spare, 0), dtype=dtype, seed=seed)
    return inp, dict(B=B, S=S, Hkv=Hkv, D=D, dtype=dtype, page_size=page_size, max_pages=max_pages, ctx=ctx,
                     short=short)


@pytest.mark.parametrize("seed", range(200))
def test_random_appends(seed):
    inp, info = draw_append(seed)
    ref = _oracle(inp)
    got = _gpu(inp)
    _same(got, ref, f"seed {seed}: {info}")
    if info["short"]:  # a pool one page short fails the call (unless capacity already does)
        assert ref["status"] in (1, 2), info
    print(seed, info, "status", ref["status"])
