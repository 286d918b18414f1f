"""tt_masked_nll on the GPU against the float64 oracle (L_MD, Nemotron-TwoTower section 2.2, Eq. (4)).

Tolerance: the kernel sums the exponentials of a row in float32 (up to 131072 terms, tree order)
and takes a float32 log, so ln Z carries a relative error of a few 1e-6; with nll values of order
ln V <= 12 the bar is |nll - nll_ref| <= 1e-4 + 1e-5 |nll_ref|, the same for the loss (a float64
mean of the float32 values)."""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_eq_block_amd import api, synth

pytestmark = pytest.mark.gpu


def _check(x, t, m, what, with_nll=True):
    xc, tc, mc = x.cuda(), t.cuda(), m.cuda()
    B, S, _ = x.shape
    nll = torch.full((B, S), 123.0, device="cuda") if with_nll else None
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    loss = api.masked_nll(xc, tc, mc, nll=nll, count=cnt)
    torch.cuda.synchronize()
    ref = oracle.masked_nll(x, t, m)
    assert int(cnt.item()) == ref["count"], what
    got_loss = float(loss.item())
    if math.isnan(ref["loss"]):
        assert math.isnan(got_loss), what
    else:
        assert abs(got_loss - ref["loss"]) <= 1e-4 + 1e-5 * abs(ref["loss"]), (what, got_loss, ref["loss"])
    if with_nll:
        g = nll.cpu().double().numpy()
        mk = m.numpy().astype(bool)
        r = ref["nll"]
        fin = mk & np.isfinite(r)
        assert np.all(np.abs(g[fin] - r[fin]) <= 1e-4 + 1e-5 * np.abs(r[fin])), (what, np.abs(g[fin] - r[fin]).max())
        assert np.all(np.isnan(g[mk & ~np.isfinite(r)])), what
        assert np.all(g[~mk] == 123.0), f"{what}: nll written at unmasked rows"
    return got_loss, ref


def test_loop_logits_all_masked():
    """The denoise loop's logits (32 x 16 x 131072 bf16, noise plus a spike at the target)."""
    c = synth.unmask_case("loop")
    targets = synth.spike_targets(c.B, c.S, c.V, seed=0)
    x = synth.make_logits(c, seed=0, step=3, spike=1.5, targets=targets)
    _check(x, targets.to(torch.int32), torch.ones(c.B, c.S, dtype=torch.uint8), "loop")


@pytest.mark.parametrize("V,dtype", [(1000, torch.float32), (999, torch.float32), (7, torch.bfloat16),
                                     (131071, torch.bfloat16), (4097, torch.float32)])
def test_ragged_mask_and_vocab_sizes(V, dtype):
    """Random masks, vocabularies whose rows are not 16-byte aligned, targets anywhere."""
    g = torch.Generator().manual_seed(V)
    x = (torch.randn(3, 11, V, generator=g) * 2).to(dtype)
    t = torch.randint(0, V, (3, 11), generator=g, dtype=torch.int32)
    m = (torch.rand(3, 11, generator=g) < 0.5).to(torch.uint8)
    m[0, 0] = 1
    _check(x, t, m, f"V={V} {dtype}")


def test_edge_cases():
    """No masked position (loss 0, count 0), a target outside the vocabulary (NaN), no nll output,
    -inf logits, a single finite logit (nll 0)."""
    x = torch.randn(2, 5, 300)
    t = torch.randint(0, 300, (2, 5), dtype=torch.int32)
    loss, ref = _check(x, t, torch.zeros(2, 5, dtype=torch.uint8), "none masked")
    assert loss == 0.0 and ref["count"] == 0
    t2 = t.clone()
    t2[1, 3] = 300
    m = torch.ones(2, 5, dtype=torch.uint8)
    _check(x, t2, m, "bad target")
    _check(x, t, m, "no nll output", with_nll=False)
    y = torch.full((1, 2, 64), float("-inf"))
    y[0, 0, 5] = 3.0
    y[0, 1, :] = torch.linspace(-4, 4, 64)
    loss, ref = _check(y, torch.tensor([[5, 63]], dtype=torch.int32), torch.ones(1, 2, dtype=torch.uint8), "-inf")
    assert ref["nll"][0, 0] == 0.0
