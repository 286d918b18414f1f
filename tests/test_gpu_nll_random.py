"""tt_masked_nll on seeded random batches against the float64 oracle (L_MD, Nemotron-TwoTower
section 2.2, Eq. (4)).

Each seed draws batch, block size, vocabulary (tiny to 131072, unaligned rows), dtype, logit
scale, mask density (empty masks included), -inf logits away from the target and, now and
then, targets outside the vocabulary (NaN for that row and the loss). The tolerances are
those of test_gpu_nll.py.
"""
import numpy as np
import pytest
import torch

from test_gpu_nll import _check

pytestmark = pytest.mark.gpu


def draw_batch(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 6))
    S = int(rng.choice([1, 4, 16, 33]))
    V = int(rng.choice([1, 2, 17, 1000, 4099, 65537, 131072]))
    dtype = torch.float32 if rng.random() < 0.4 else torch.bfloat16
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, S, V, generator=g) * float(rng.choice([0.3, 1.0, 4.0]))
    t = torch.randint(0, V, (B, S), generator=g, dtype=torch.int32)
    m = (torch.rand(B, S, generator=g) < float(rng.choice([0.0, 0.3, 1.0]))).to(torch.uint8)
    if V > 2 and rng.random() < 0.3:  # -inf logits, never at the target
        ninf = torch.rand(B, S, V, generator=g) < 0.2
        ninf.scatter_(2, t.long().unsqueeze(-1), False)
        x[ninf] = float("-inf")
    if rng.random() < 0.1:
        t[0, 0] = V + 5  # outside the vocabulary
    return x.to(dtype), t, m


@pytest.mark.parametrize("seed", range(120))
def test_random_batches(seed):
    x, t, m = draw_batch(seed)
    loss, ref = _check(x, t, m, f"seed {seed}: {tuple(x.shape)} {x.dtype} masked {int(m.sum())}")
    print(seed, tuple(x.shape), x.dtype, int(m.sum()), loss, ref["loss"])
