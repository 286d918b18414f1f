"""tt_conf_unmask on the GPU against the float64 oracle (Algorithm 2's ConfidenceSample,
Nemotron-TwoTower section 2.2). Tokens, masks and counts are compared bit for bit;
see parity.py for the exclusion of decisions within 1e-6 of a threshold."""
import numpy as np
import pytest
import torch

import oracle
from attention_eq_block_amd import api, synth

from parity import check_unmask, gpu_unmask

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("temperature", [1.0, 0.1])
def test_tiny_fp32(temperature):
    """Logits 16 x 1024 float32, N(0,1) + 4 at a seeded token, all masked, gamma 0.8."""
    c = synth.unmask_case("tiny", temperature=temperature)
    x = synth.make_logits(c, seed=0)
    tokens, mask = synth.make_mask_state(c.B, c.S)
    got, ref, _ = check_unmask(x, mask, tokens, gamma=0.8, temperature=temperature, steps_left=16, what="tiny")
    if temperature == 1.0:
        # nothing passes 0.8 at temperature 1: exactly one (the most confident) position commits
        assert int(got["num_masked"][0]) == 15


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
@pytest.mark.parametrize("temperature", [0.1, 1.0])
def test_ragged_full_size(gamma, temperature):
    """64 x 16 x 131072 bf16 logits, N(0,1) + U(0,8) spike per row, all masked, R = 16."""
    c = synth.unmask_case("ragged", temperature=temperature, gamma=gamma)
    x = _cached_ragged_logits()
    tokens, mask = synth.make_mask_state(c.B, c.S)
    got, ref, skip = check_unmask(x, mask, tokens, gamma=gamma, temperature=temperature, steps_left=16,
                                  what=f"ragged g={gamma} T={temperature}")
    print(f"excluded {skip.sum()} of {len(skip)}; committed {int((1 - got['mask']).sum())}")


_RAGGED = {}


def _cached_ragged_logits():
    if "x" not in _RAGGED:
        _RAGGED["x"] = synth.make_logits(synth.unmask_case("ragged"), seed=0)
    return _RAGGED["x"]


def test_ragged_argmax_ties_are_exercised():
    """bf16 logits tie at the max in a few percent of rows: the lowest index must win."""
    x = _cached_ragged_logits()
    xv = x.float()
    mx = xv.max(-1, keepdim=True).values
    n_ties = int(((xv == mx).sum(-1) > 1).sum())
    tokens, mask = synth.make_mask_state(64, 16)
    got = gpu_unmask(x, mask, tokens, gamma=-1.0, temperature=1.0, steps_left=16)  # gamma < 0: commit all
    assert got["mask"].sum() == 0
    first = xv.argmax(-1).numpy()  # torch returns the first maximal index on CPU
    ref_first = np.argmax(x.float().numpy(), axis=-1)
    assert np.array_equal(ref_first, first)
    assert np.array_equal(got["tokens"], ref_first.astype(np.int32)), "argmax must take the lowest tied index"
    print("rows with ties:", n_ties)


@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.95])
def test_denoise_loop_teacher_forced(gamma):
    """Algorithm 2 on the loop workload (32 x 16 x 131072, spike 0.5*t at step t, T = 16):
    each step's GPU output is compared with the oracle run from the GPU's own input state."""
    c = synth.unmask_case("loop", gamma=gamma)
    targets = synth.spike_targets(c.B, c.S, c.V, seed=0)
    tokens, mask = synth.make_mask_state(c.B, c.S)
    T = synth.LOOP_STEPS
    for r in range(1, T + 1):
        x = synth.make_logits(c, seed=0, step=r, spike=0.5 * r, targets=targets)
        got, ref, skip = check_unmask(x, mask, tokens, gamma=gamma, temperature=0.1, steps_left=T - r + 1,
                                      what=f"loop step {r}")
        tokens = torch.from_numpy(got["tokens"])
        mask = torch.from_numpy(got["mask"])
        if int(mask.sum()) == 0:
            break
    assert int(mask.sum()) == 0, "block must complete within T steps"


@pytest.mark.parametrize("T", [16, 8, 4])
def test_predict_and_noise_linear_schedule(T):
    """The predict-and-noise sampler with low-confidence remasking (section 2.2; the schedule
    alpha_t = 1 - t of Eq. (3)): every masked position is predicted and all but the ceil(M/R) most
    confident are masked again, which is the step with gamma = +inf. With S divisible by T the block
    then holds exactly S*(T - r)/T masked positions after step r, as the linear schedule says."""
    c = synth.unmask_case("loop")
    targets = synth.spike_targets(c.B, c.S, c.V, seed=0)
    tokens, mask = synth.make_mask_state(c.B, c.S)
    for r in range(1, T + 1):
        x = synth.make_logits(c, seed=1, step=r, spike=0.5 * r, targets=targets)
        # temperature 1: confidences stay well below 1 (no float32 saturation); every step is a top-k
        # choice, so near-ties within 1e-6 are more frequent than at gamma < 1 and up to 15% of the
        # sequences may be excluded from the exact comparison (the count check below covers all)
        got, ref, skip = check_unmask(x, mask, tokens, gamma=float("inf"), temperature=1.0, steps_left=T - r + 1,
                                      what=f"T={T} step {r}", max_fragile_frac=0.15)
        assert np.all(got["num_masked"] == c.S * (T - r) // T), (r, got["num_masked"][:4])
        tokens = torch.from_numpy(got["tokens"])
        mask = torch.from_numpy(got["mask"])
    assert int(mask.sum()) == 0


@pytest.mark.parametrize("V", [1, 5, 8, 1000, 4099])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_vocab_sizes(V, dtype):
    """Vocabularies that are tiny, not a multiple of 8, or leave a ragged last chunk."""
    g = torch.Generator().manual_seed(V)
    x = (torch.randn(3, 9, V, generator=g) * 2).to(dtype)
    tokens, mask = synth.random_mask_state(3, 9, 0.8, seed=V)
    for R in (1, 3, 9):
        check_unmask(x, mask, tokens, gamma=0.3, temperature=0.7, steps_left=R, what=f"V={V} R={R}",
                     max_fragile_frac=0.34)


def test_strided_rows_and_separate_mask_out():
    base = torch.randn(2, 5, 1043, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    x = base[:, :, 3:1003]  # rows 1043 apart, starting off a 16-byte boundary
    tokens, mask = synth.random_mask_state(2, 5, 0.6, seed=4)
    lg = base.cuda()[:, :, 3:1003]
    assert lg.stride(1) == 1043
    mk = mask.cuda()
    tk = tokens.cuda()
    mo = torch.full_like(mk, 9)
    api.conf_unmask(lg, mk, tk, gamma=0.2, temperature=0.5, steps_left=2, mask_out=mo)
    ref = oracle.conf_unmask(x, mask, tokens, gamma=oracle.f32(0.2), temperature=oracle.f32(0.5), steps_left=2)
    assert np.array_equal(tk.cpu().numpy(), ref["tokens"])
    assert np.array_equal(mo.cpu().numpy(), ref["mask"])
    assert torch.equal(mk.cpu(), mask), "mask_in must be left alone when mask_out is separate"


@pytest.mark.parametrize("S", [1, 2, 33, 64])
@pytest.mark.parametrize("gamma", [-0.5, 0.6, 1.0])
def test_block_sizes_and_gamma_extremes(S, gamma):
    g = torch.Generator().manual_seed(S)
    x = (torch.randn(4, S, 777, generator=g) * 3).to(torch.bfloat16)
    tokens, mask = synth.random_mask_state(4, S, 0.75, seed=S)
    for R in (1, 2, 5):
        got, ref, _ = check_unmask(x, mask, tokens, gamma=gamma, temperature=1.0, steps_left=R,
                                   what=f"S={S} gamma={gamma} R={R}", max_fragile_frac=0.5)
        M = mask.sum(1).numpy()
        k = -(-M // R)
        committed = M - got["num_masked"]
        if gamma < 0:
            assert np.all(got["num_masked"] == 0)
        if gamma >= 1.0:
            assert np.array_equal(committed, k)


def test_optional_outputs_and_empty_mask():
    x = torch.randn(2, 4, 64).to(torch.bfloat16).cuda()
    mk = torch.zeros(2, 4, dtype=torch.uint8, device="cuda")
    tk = torch.arange(8, dtype=torch.int32, device="cuda").reshape(2, 4)
    api.conf_unmask(x, mk, tk, gamma=0.5, temperature=1.0, steps_left=1)
    torch.cuda.synchronize()
    assert torch.equal(tk.cpu(), torch.arange(8, dtype=torch.int32).reshape(2, 4))
    assert int(mk.sum()) == 0
