"""tt_conf_unmask on seeded random steps against the float64 oracle.

ConfidenceSample of Algorithm 2 (Nemotron-TwoTower, arXiv 2606.26493, section 2.2
"Sampling"). Each seed draws one step: batch, block size S, vocabulary V (tiny,
unaligned and large), logits dtype, logit scale and spikes (so that some rows pass gamma and
some do not), ties (logits rounded to a coarse grid), mask density, gamma,
temperature and steps left, and in about a third of the seeds caller uniforms
(the stochastic draw). Tokens, masks and counts are compared bit for bit and the
confidences to 1e-6 + 1e-5 * conf, with the exclusions stated in parity.py.
"""
import numpy as np
import pytest
import torch

from attention_eq_block_amd import synth

from parity import check_unmask

pytestmark = pytest.mark.gpu


def draw_step(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 9))
    S = int(rng.choice([1, 3, 8, 16, 17, 32, 64]))
    V = int(rng.choice([1, 7, 64, 1000, 4099, 32768, 50001]))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(B, S, V, generator=g) * float(rng.choice([0.5, 1.0, 3.0]))
    if rng.random() < 0.5:  # spikes: some rows confident enough to pass gamma
        tgt = torch.randint(0, V, (B, S), generator=g)
        h = torch.rand(B, S, generator=g) * float(rng.choice([4.0, 10.0]))
        base.scatter_add_(2, tgt.unsqueeze(-1), h.unsqueeze(-1))
    if rng.random() < 0.3:  # ties: a coarse grid makes equal maxima common
        base = torch.round(base * 2) / 2
    x = base.to(dtype)
    tokens, mask = synth.random_mask_state(B, S, float(rng.choice([0.3, 0.8, 1.0])), seed=seed)
    gamma = float(rng.choice([-0.5, 0.3, 0.8, 0.95, 1.0]))
    temperature = float(rng.choice([0.1, 0.5, 1.0]))
    steps_left = int(rng.integers(1, 17))
    uniforms = None
    if rng.random() < 0.35:
        uniforms = torch.rand(B, S, generator=g)
    return x, tokens, mask, gamma, temperature, steps_left, uniforms


@pytest.mark.parametrize("seed", range(300))
def test_random_steps(seed):
    x, tokens, mask, gamma, temperature, steps_left, uniforms = draw_step(seed)
    what = (f"seed {seed}: {tuple(x.shape)} {x.dtype} gamma {gamma} T {temperature} "
            f"R {steps_left} uniforms {uniforms is not None}")
    # tiny or coarse vocabularies can tie most confidences at the top-k cut, so any share of
    # sequences may be excluded; the others are compared bit for bit, every confidence to tolerance
    got, ref, skip = check_unmask(x, mask, tokens, gamma=gamma, temperature=temperature, steps_left=steps_left,
                                  what=what, max_fragile_frac=1.0, uniforms=uniforms)
    print(what, f"excluded {int(skip.sum())} of {len(skip)}")
