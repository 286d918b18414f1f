"""Shared pieces of the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare them to the stated bar.

Tolerances (attention, Nemotron-TwoTower Eq. 1):
  float32 path:  O max-abs <= 1e-5, LSE max-abs <= 1e-5
  bf16 path:     O max-abs <= 2e-2 and rel-L2 ||O - O_ref|| / ||O_ref|| <= 4e-3 over the
                 tensor; LSE max-abs <= 4e-3. The kernel rounds the softmax weights P
                 to bf16 before the P.V product and sums them in fp32 before that
                 rounding, so O carries the bf16 rounding of P (about 2^-9 relative per
                 weight) and LSE the fp32 summation error of up to a few thousand
                 weights below 2^8 each (the running max may trail the true max by up
                 to 2^8); 4e-3 covers both with margin.
Confidence unmask (Algorithm 2): tokens, masks and counts bit-exact, except that a
sequence is excluded when one of its decisions sits within 1e-6 of a threshold in the
oracle's float64 values (a confidence within 1e-6 of gamma, or, on the fallback path,
the k-th and (k+1)-th confidences within 1e-6 of each other). conf within
1e-6 + 1e-5*conf.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from attention_eq_block_amd import api, synth

F32_TOL = 1e-5
BF16_MAXABS = 2e-2
BF16_RELL2 = 4e-3
BF16_LSE = 4e-3


def to_dev(inp, device="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def gpu_attn(inp, *, max_ctx_len=None, o_dtype=None, out=None, lse=None):
    d = to_dev(inp)
    if max_ctx_len is None:
        max_ctx_len = int(inp["ctx_len"].max()) if inp["ctx_len"].numel() else 0
    O, L = api.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d.get("Kd"), d.get("Vd"),
                          page_size=inp["page_size"], max_ctx_len=max_ctx_len, scale=inp["scale"],
                          o_dtype=o_dtype, out=out, lse=lse)
    torch.cuda.synchronize()
    return O, L


def oracle_attn(inp, rows=None):
    return oracle.block_attn(inp["Q"], inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp.get("Kd"),
                             inp.get("Vd"), page_size=inp["page_size"], scale=inp["scale"], rows=rows)


def check_attn(O_gpu, L_gpu, O_ref, L_ref, dtype, what=""):
    """Compare full outputs: O [B][S][Hq][D], LSE [B][Hq][S]."""
    O = O_gpu.detach().float().cpu().double().numpy()
    L = L_gpu.detach().float().cpu().double().numpy()
    assert O.shape == O_ref.shape, (O.shape, O_ref.shape)
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    err = np.abs(O - O_ref)
    lerr = np.where(np.isneginf(L_ref) & np.isneginf(L), 0.0, np.abs(L - L_ref))
    assert np.all(np.isfinite(lerr)), f"{what}: LSE mismatch in infinities"
    nrm = np.linalg.norm(O_ref)
    rel = np.linalg.norm(O - O_ref) / nrm if nrm > 0 else np.linalg.norm(O)
    stats = dict(maxabs=float(err.max()) if err.size else 0.0, rel_l2=float(rel),
                 lse_maxabs=float(lerr.max()) if lerr.size else 0.0)
    if dtype == torch.float32:
        assert stats["maxabs"] <= F32_TOL, f"{what}: {stats}"
        assert stats["lse_maxabs"] <= F32_TOL, f"{what}: {stats}"
    else:
        assert stats["maxabs"] <= BF16_MAXABS, f"{what}: {stats}"
        assert stats["rel_l2"] <= BF16_RELL2, f"{what}: {stats}"
        assert stats["lse_maxabs"] <= BF16_LSE, f"{what}: {stats}"
    return stats


def sample_rows(B, Hq, S, n, seed=0):
    """n distinct (b, h, s) triples, always including each sequence's first and last row."""
    rng = np.random.default_rng(seed)
    total = B * Hq * S
    idx = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    for b in range(B):
        idx.add(b * Hq * S)
        idx.add(b * Hq * S + Hq * S - 1)
    idx = np.array(sorted(idx))
    return np.stack([idx // (Hq * S), (idx // S) % Hq, idx % S], axis=1).astype(np.int32)


def check_attn_rows(O_gpu, L_gpu, inp, rows, dtype, what=""):
    """Compare sampled rows against the oracle computed for those rows only."""
    Or, Lr = oracle_attn(inp, rows)
    b, h, s = rows[:, 0], rows[:, 1], rows[:, 2]
    O = O_gpu.detach().float().cpu().double().numpy()[b, s, h]
    L = L_gpu.detach().float().cpu().double().numpy()[b, h, s]
    return check_attn(torch.from_numpy(O), torch.from_numpy(L), Or, Lr, dtype, what)


# ---------------------------------------------------------------------------
# confidence unmask
# ---------------------------------------------------------------------------

def gpu_unmask(logits, mask, tokens, *, gamma, temperature, steps_left, separate_out=False, want_conf=True):
    lg = logits.cuda()
    mk = mask.cuda().clone()
    tk = tokens.cuda().clone()
    B, S = mask.shape
    conf = torch.full((B, S), float("nan"), device="cuda") if want_conf else None
    nm = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    mo = torch.full_like(mk, 77) if separate_out else None
    api.conf_unmask(lg, mk, tk, gamma=gamma, temperature=temperature, steps_left=steps_left, mask_out=mo,
                    conf=conf, num_masked=nm)
    torch.cuda.synchronize()
    out_mask = mo if separate_out else mk
    return dict(tokens=tk.cpu().numpy(), mask=out_mask.cpu().numpy(), num_masked=nm.cpu().numpy(),
                conf=None if conf is None else conf.cpu().double().numpy())


def fragile(ref_conf, mask, gamma, steps_left, eps=1e-6):
    """Per sequence: True when a decision sits within eps of its threshold in the oracle's values."""
    B, S = mask.shape
    out = np.zeros(B, dtype=bool)
    for b in range(B):
        m = mask[b].astype(bool)
        c = ref_conf[b][m]
        if c.size == 0:
            continue
        if np.any(np.abs(c - gamma) < eps):
            out[b] = True
            continue
        M = c.size
        k = -(-M // steps_left)
        if int(np.sum(c > gamma)) < k and k < M:
            cs = np.sort(c)[::-1]
            if cs[k - 1] - cs[k] < eps:
                out[b] = True
    return out


def check_unmask(logits, mask, tokens, *, gamma, temperature, steps_left, separate_out=False, what="",
                 max_fragile_frac=0.05):
    """Run both sides from the same state and compare to the bar; returns the GPU result."""
    g32 = oracle.f32(gamma)
    t32 = oracle.f32(temperature)
    ref = oracle.conf_unmask(logits, mask, tokens, gamma=g32, temperature=t32, steps_left=steps_left)
    got = gpu_unmask(logits, mask, tokens, gamma=gamma, temperature=temperature, steps_left=steps_left,
                     separate_out=separate_out)
    mk = mask.cpu().numpy()
    skip = fragile(ref["conf"], mk, g32, steps_left)
    assert skip.mean() <= max_fragile_frac, f"{what}: {skip.sum()} of {len(skip)} sequences fragile"
    keep = ~skip
    assert np.array_equal(got["tokens"][keep], ref["tokens"][keep]), f"{what}: tokens differ"
    assert np.array_equal(got["mask"][keep], ref["mask"][keep]), f"{what}: masks differ"
    assert np.array_equal(got["num_masked"][keep], ref["num_masked"][keep]), f"{what}: num_masked differ"
    m = mk.astype(bool)
    dc = np.abs(got["conf"][m] - ref["conf"][m])
    assert np.all(dc <= 1e-6 + 1e-5 * ref["conf"][m]), f"{what}: conf max err {dc.max():.3e}"
    # rows that were not masked: conf untouched (NaN sentinel), tokens untouched
    assert np.all(np.isnan(got["conf"][~m])), f"{what}: conf written at unmasked rows"
    tk = tokens.cpu().numpy()
    assert np.array_equal(got["tokens"][~m], tk[~m]), f"{what}: unmasked tokens changed"
    return got, ref, skip
