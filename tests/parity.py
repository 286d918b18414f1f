"""Shared pieces of the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare them to the stated bar.

Tolerances (attention, Nemotron-TwoTower Eq. 1):
  float32 path:  O max-abs <= 1e-5, LSE max-abs <= 1e-5
  bf16 path:     O max-abs <= 2e-2 and rel-L2 ||O - O_ref|| / ||O_ref|| <= 4e-3 over the
                 tensor; LSE max-abs <= 1e-4. The kernel rounds the softmax weights P
                 to bf16 before the P.V product, so O carries the bf16 rounding of P
                 (about 2^-9 relative per weight; measured rel-L2 0.0025-0.0029 on the
                 five workloads). LSE is built from the fp32 scores and the fp32 sum of
                 the unrounded weights: its error is fp32 rounding of a value near
                 ln(keys) (measured at most 1.4e-6 on every workload), well inside 1e-4.
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
BF16_LSE = 1e-4


def to_dev(inp, device="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def gpu_attn(inp, *, max_ctx_len=None, o_dtype=None, out=None, lse=None, debug_flags=None):
    d = to_dev(inp)
    if max_ctx_len is None:
        max_ctx_len = int(inp["ctx_len"].max()) if inp["ctx_len"].numel() else 0
    O, L = api.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d.get("Kd"), d.get("Vd"),
                          page_size=inp["page_size"], max_ctx_len=max_ctx_len, scale=inp["scale"],
                          o_dtype=o_dtype, out=out, lse=lse, debug_flags=debug_flags)
    torch.cuda.synchronize()
    return O, L


def oracle_attn(inp, rows=None, max_ctx_len=None):
    return oracle.block_attn(inp["Q"], inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp.get("Kd"),
                             inp.get("Vd"), page_size=inp["page_size"], scale=inp["scale"], rows=rows,
                             max_ctx_len=max_ctx_len)


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

def gpu_unmask(logits, mask, tokens, *, gamma, temperature, steps_left, separate_out=False, want_conf=True,
               uniforms=None):
    lg = logits.cuda()
    mk = mask.cuda().clone()
    tk = tokens.cuda().clone()
    B, S = mask.shape
    conf = torch.full((B, S), float("nan"), device="cuda") if want_conf else None
    nm = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    mo = torch.full_like(mk, 77) if separate_out else None
    un = None if uniforms is None else uniforms.cuda()
    api.conf_unmask(lg, mk, tk, gamma=gamma, temperature=temperature, steps_left=steps_left, mask_out=mo,
                    conf=conf, num_masked=nm, uniforms=un)
    torch.cuda.synchronize()
    out_mask = mo if separate_out else mk
    return dict(tokens=tk.cpu().numpy(), mask=out_mask.cpu().numpy(), num_masked=nm.cpu().numpy(),
                conf=None if conf is None else conf.cpu().double().numpy())


def conf_tol(c):
    """Tolerance of a float32 confidence against the oracle's float64 one."""
    return 1e-6 + 1e-5 * np.abs(c)


def fragile(ref_conf, mask, gamma, steps_left):
    """Per sequence: True when a commit decision's margin in the oracle's values is within what the
    float32 confidences may be off by (reading R25): the larger of 1e-6 and 1e-5 of the values
    compared. That is a confidence within max(1e-6, 1e-5 c) of gamma, or the k-th and (k+1)-th
    largest confidences at the top-k cut closer than max(1e-6, 1e-5 (c_k + c_k+1)). Z is a float32
    sum: near a confidence of 1 (temperature 0.1) its tail terms, far below one float32 ulp of the
    leading 1, are partly lost and a confidence may be off by about 1e-6; small confidences are off
    by a small relative amount. A step with steps_left = 1 commits every masked position, and with
    gamma >= 1 no confidence (at most 1) is above gamma: neither decides anything against gamma."""
    B, S = mask.shape
    out = np.zeros(B, dtype=bool)
    if steps_left == 1:
        return out
    for b in range(B):
        m = mask[b].astype(bool)
        c = ref_conf[b][m]
        if c.size == 0:
            continue
        if gamma < 1.0 and np.any(np.abs(c - gamma) < np.maximum(1e-6, 1e-5 * np.abs(c))):
            out[b] = True
            continue
        M = c.size
        k = -(-M // steps_left)
        if int(np.sum(c > gamma)) < k and k < M:
            cs = np.sort(c)[::-1]
            if cs[k - 1] - cs[k] < max(1e-6, 1e-5 * (abs(cs[k - 1]) + abs(cs[k]))):
                out[b] = True
    return out


# The kernel's cumulative probabilities are float32 sums of up to 131072 terms (runs of a few hundred
# terms added in order, then a scan and the split masses): their error is of order 1e-6 of the total
# and below 256 * 2^-24 = 1.5e-5 in the worst case. A drawn token is valid when it is the exact
# inverse-transform draw for some uniform within DRAW_TOL of the given one. At temperature 1 over
# 131072 tokens each probability is about 7.6e-6, so the float32 and float64 draws often differ by
# a neighbour; that is the float32 rounding, not a different method.
DRAW_TOL = 3e-5


def settle_uniforms(logits, mask, uniforms, temperature, drawn):
    """Check every GPU draw against the exact float64 cumulative distribution and return uniforms
    that make the oracle draw the GPU's tokens: u itself where the GPU's token is the exact draw
    for u with room to spare, else the middle of the GPU token's bracket (after checking that u is
    within DRAW_TOL of that bracket). Also returns the number of moved uniforms and, per sequence,
    whether no float32 uniform could reproduce a draw (then the sequence is excluded)."""
    x = logits.float().numpy() if isinstance(logits, torch.Tensor) else np.asarray(logits, np.float32)
    B, S = mask.shape
    t = float(oracle.f32(temperature))
    u = uniforms.cpu().numpy().astype(np.float32).copy()
    moved, bad = 0, np.zeros(B, dtype=bool)
    for b, l in zip(*np.nonzero(mask)):
        z = x[b, l].astype(np.float64) / t
        e = np.exp(z - z.max())
        C = np.cumsum(e)
        a = int(drawn[b, l])
        assert 0 <= a < C.size and e[a] > 0, f"row ({b},{l}): drew token {a} of probability 0"
        lo = C[a - 1] / C[-1] if a > 0 else 0.0
        hi = C[a] / C[-1]
        uu = float(u[b, l])
        uu = 0.0 if not uu > 0 else min(uu, 1.0)
        assert lo - DRAW_TOL <= uu <= hi + DRAW_TOL, \
            f"row ({b},{l}): token {a} has bracket [{lo:.9f}, {hi:.9f}) but u = {uu:.9f}"
        if lo + 1e-9 < uu < hi - 1e-9:
            continue
        mid = np.float32((lo + hi) / 2)
        if lo + 1e-9 < float(mid) < hi - 1e-9:
            u[b, l] = mid
            moved += 1
        else:
            bad[b] = True
    return torch.from_numpy(u), moved, bad


def check_unmask(logits, mask, tokens, *, gamma, temperature, steps_left, separate_out=False, what="",
                 max_fragile_frac=0.05, uniforms=None):
    """Run both sides from the same state and compare to the bar; returns the GPU result."""
    g32 = oracle.f32(gamma)
    t32 = oracle.f32(temperature)
    mk = mask.cpu().numpy()
    bad = np.zeros(mk.shape[0], dtype=bool)
    u_ref = uniforms
    if uniforms is not None:
        # every draw, made visible by committing all positions (the draws do not depend on gamma)
        every = gpu_unmask(logits, mask, tokens, gamma=-1.0, temperature=temperature, steps_left=1,
                           want_conf=False, uniforms=uniforms)
        u_ref, moved, bad = settle_uniforms(logits, mk, uniforms, temperature, every["tokens"])
        print(f"{what}: {moved} of {int(mk.sum())} draws settled on a float32 neighbour within {DRAW_TOL}")
    ref = oracle.conf_unmask(logits, mask, tokens, gamma=g32, temperature=t32, steps_left=steps_left,
                             uniforms=u_ref)
    got = gpu_unmask(logits, mask, tokens, gamma=gamma, temperature=temperature, steps_left=steps_left,
                     separate_out=separate_out, uniforms=uniforms)
    skip = fragile(ref["conf"], mk, g32, steps_left) | bad
    assert skip.mean() <= max_fragile_frac, f"{what}: {skip.sum()} of {len(skip)} sequences fragile"
    keep = ~skip
    assert np.array_equal(got["tokens"][keep], ref["tokens"][keep]), f"{what}: tokens differ"
    assert np.array_equal(got["mask"][keep], ref["mask"][keep]), f"{what}: masks differ"
    assert np.array_equal(got["num_masked"][keep], ref["num_masked"][keep]), f"{what}: num_masked differ"
    m = mk.astype(bool)
    dc = np.abs(got["conf"][m] - ref["conf"][m])
    assert np.all(dc <= conf_tol(ref["conf"][m])), f"{what}: conf max err {dc.max() if dc.size else 0:.3e}"
    # rows that were not masked: conf untouched (NaN sentinel), tokens untouched
    um = ~mk.astype(bool)
    assert np.all(np.isnan(got["conf"][um])), f"{what}: conf written at unmasked rows"
    tk = tokens.cpu().numpy()
    assert np.array_equal(got["tokens"][um], tk[um]), f"{what}: unmasked tokens changed"
    return got, ref, skip
