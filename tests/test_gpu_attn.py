"""tt_block_attn and tt_lse_merge on the GPU against the float64 oracle.

Eq. (1) of Nemotron-TwoTower (arXiv 2606.26493, section 2.1). Every shape, the
full-size workloads included (in the launch configuration the benchmark times), is
compared element by element over all of O and LSE, rel-L2 over the whole tensor.
Tolerances are stated in parity.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_eq_block_amd import api, synth

from parity import check_attn, gpu_attn, oracle_attn, to_dev

pytestmark = pytest.mark.gpu


def case(B, S, Hq, Hkv, D, ctx, dtype=torch.bfloat16, **kw):
    return synth.AttnCase(B, S, Hq, Hkv, D, list(ctx), dtype=dtype, **kw)


def run_full(c, seed=0, what=""):
    inp = synth.make_attn_inputs(c, seed=seed)
    O, L = gpu_attn(inp)
    Or, Lr = oracle_attn(inp)
    return check_attn(O, L, Or, Lr, c.dtype, what or str(c))


# --------------------------------------------------------------------------- workloads

def test_tiny_fp32():
    """4 q-heads on 1 kv-head, d=64, prefix 48, S=16, float32 (the tiny workload)."""
    print(run_full(synth.attn_case("tiny")))


@pytest.mark.parametrize("variant", ["", "unscaled"])
def test_single_bf16(variant):
    """B=1, 32/2 heads, d=128, prefix 4096, S=16 (identity pages)."""
    print(run_full(synth.attn_case("single", variant)))


def pieces_per_pair(c, n_cu, piece_cost=3, tile=64, rows=256):
    """Segments that cut each (sequence, kv head, row block) pair of a bf16 call: the
    work split the library plans (one equal-cost segment per workgroup, a pair costing
    its tiles plus piece_cost), redone on the host to choose shapes for the test below."""
    G = c.Hq // c.Hkv
    n_rb = -(-c.S * G // rows)
    mult = c.Hkv * n_rb
    has_den = 1 if c.with_den else 0
    units = [-(-int(L) // tile) + has_den for L in c.ctx_lens]
    w_max = c.B * mult * max(units)
    cu8 = -(-n_cu // 8) * 8
    nseg = min(max(-(-((w_max + 1) // 2) // 8) * 8, 8), cu8)
    weighted = [mult * (u + piece_cost) if u > 0 else 0 for u in units]
    seg_len = -(-sum(weighted) // nseg)
    out, before = [], 0
    for u, w in zip(units, weighted):
        for pl in range(mult):
            if u > 0:
                U = before + pl * (u + piece_cost) + piece_cost
                out.append((U + u - 1) // seg_len - U // seg_len + 1)
        before += w
    return out


def test_merge_group_boundaries():
    """Pairs cut into 2, 8, 9, 16, 17 and 24-25 pieces: the merge reads partials eight
    at a time with the next group in flight, so these are its group edges (one group,
    a full group, a second group, two full groups, a third). With 32 or more pieces per
    pair the merge splits a pair's partials over eight thread groups: 40 pieces (five
    each), 64 (eight each, one batch) and 65 (a second batch in the first group)."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    found = {}
    for L in range(64, 16384, 16):
        c = case(1, 16, 32, 2, 128, [L])
        for k in pieces_per_pair(c, n_cu):
            for want in (2, 8, 9, 16, 17, 24, 25, 40, 64, 65):
                if k == want and want not in found:
                    found[want] = L
    assert {8, 9, 16, 17, 40, 64, 65}.issubset(found), found
    for want, L in sorted(found.items()):
        c = case(1, 16, 32, 2, 128, [L])
        print(want, L, run_full(c, what=f"{want} pieces, prefix {L}"))
    # float32 output (fp32 partials) where the merge splits each pair over eight thread groups
    c = synth.attn_case("single")
    inp = synth.make_attn_inputs(c, seed=2)
    O, Ls = gpu_attn(inp, o_dtype=torch.float32)
    Or, Lr = oracle_attn(inp)
    print("single, fp32 output", check_attn(O, Ls, Or, Lr, c.dtype, "single fp32 out"))


@pytest.mark.parametrize("kind", ["uniform_80", "one_short_80", "below_max", "uniform_odd"])
def test_equal_and_unequal_lengths(kind):
    """Batches whose sequences all have max_ctx_len keys and batches that miss it by little:
    80 equal sequences (the segment scan reads ctx_len in two chunks of 64), the same with one
    shorter sequence in the second chunk, equal sequences just below max_ctx_len (within the
    page table's capacity), and an equal odd length with pairs cut into many pieces."""
    if kind == "uniform_80":
        c, mx = case(80, 2, 8, 2, 64, [200] * 80, page_size=16, shuffle_pages=True), None
    elif kind == "one_short_80":
        ctx = [200] * 80
        ctx[70] = 150
        c, mx = case(80, 2, 8, 2, 64, ctx, page_size=16, shuffle_pages=True), None
    elif kind == "below_max":
        c, mx = case(3, 16, 32, 2, 128, [300] * 3, page_size=16, shuffle_pages=True), 304
    else:
        c, mx = case(2, 16, 32, 2, 128, [1999] * 2, page_size=32, shuffle_pages=True), None
    inp = synth.make_attn_inputs(c, seed=5)
    O, L = gpu_attn(inp, max_ctx_len=mx)
    Or, Lr = oracle_attn(inp)
    print(kind, check_attn(O, L, Or, Lr, c.dtype, kind))


def test_ragged_bf16_full_size():
    """B=64, prefix 16*U{32..512}, shuffled 16-token pages: every row at full size."""
    c = synth.attn_case("ragged")
    inp = synth.make_attn_inputs(c, seed=0)
    O, L = gpu_attn(inp, max_ctx_len=c.max_ctx_len)
    Or, Lr = oracle_attn(inp)
    print(check_attn(O, L, Or, Lr, c.dtype, "ragged"))


def test_ragged_unscaled_small_full_compare():
    c = case(8, 16, 32, 2, 128, synth.ragged_ctx_lens(8, 16, 1024, 16, seed=3), shuffle_pages=True)
    print(run_full(c))


def test_long_bf16_full_size():
    """B=4, prefix 131072, S=32 (two row blocks per kv head): every row."""
    c = synth.attn_case("long")
    inp = synth.make_attn_inputs(c, seed=0)
    O, L = gpu_attn(inp, max_ctx_len=131072)
    Or, Lr = oracle_attn(inp)
    print(check_attn(O, L, Or, Lr, c.dtype, "long"))


def test_loop_layer_full_size():
    """B=32, prefix 8192, S=16: one of the six layer caches of the denoise loop, every row."""
    c = synth.attn_case("loop")
    inp = synth.make_attn_inputs(c, seed=0, layer=3)
    O, L = gpu_attn(inp, max_ctx_len=8192)
    Or, Lr = oracle_attn(inp)
    print(check_attn(O, L, Or, Lr, c.dtype, "loop"))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_out_of_range_lengths_and_page_ids(dtype):
    """ctx_len below 0 and above max_ctx_len, and page ids below 0 and past the pool, read as their
    clamp into range (the library's stated behaviour, which the oracle implements); debug mode
    reports both kinds in the flags word, and a clean call leaves it 0."""
    c = case(5, 16, 32, 2, 128, [300, 64, 500, 129, 200], dtype=dtype, shuffle_pages=True, spare_pages=2)
    inp = synth.make_attn_inputs(c, seed=11)
    max_ctx = 400
    num_pages = inp["Kc"].shape[0]
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    O, L = gpu_attn(inp, max_ctx_len=c.max_ctx_len, debug_flags=flags)
    assert int(flags.item()) == 0, "clean data raised debug flags"
    flags.zero_()
    gpu_attn(inp, max_ctx_len=max_ctx, debug_flags=flags)  # sequence 2's 500 keys exceed max_ctx_len
    assert int(flags.item()) == 1, f"debug flags {int(flags.item())}, want TT_DEBUG_CTX_LEN"
    cl = torch.tensor([-7, 64, 500, 129, 1 << 30], dtype=torch.int32)
    pt = inp["page_table"].clone()
    pt[1, 0] = -5                   # a page sequence 1 reads
    pt[3, 8] = num_pages + 3        # the page of sequence 3's last key (128)
    bad = dict(inp, ctx_len=cl, page_table=pt)
    flags.zero_()
    O, L = gpu_attn(bad, max_ctx_len=max_ctx, debug_flags=flags)
    assert int(flags.item()) == 3, f"debug flags {int(flags.item())}, want TT_DEBUG_CTX_LEN | TT_DEBUG_PAGE_ID"
    Or, Lr = oracle_attn(bad, max_ctx_len=max_ctx)
    print(check_attn(O, L, Or, Lr, dtype, "clamped data"))
    # without debug mode the outputs are the same and nothing is reported
    O2, L2 = gpu_attn(bad, max_ctx_len=max_ctx)
    assert torch.equal(O2, O) and torch.equal(L2, L)


@pytest.mark.parametrize("kind", ["tiny", "single", "ragged", "long", "edges", "d64", "pages48", "empty", "f32"])
def test_debug_mode_lds_poison(kind):
    """Debug mode first fills every LDS buffer of the call with all-ones bytes (NaN in bf16 and
    fp32, page id -1). Outputs bit-identical to the call without debug mode and a zero flags
    word show that no LDS byte is read before a load or store of the call filled it: a poisoned
    read would put a NaN into O or LSE, or raise TT_DEBUG_PAGE_ID."""
    cases = {
        "tiny": lambda: synth.attn_case("tiny"),
        "single": lambda: synth.attn_case("single"),
        "ragged": lambda: synth.attn_case("ragged"),
        "long": lambda: synth.attn_case("long"),
        "edges": lambda: case(5, 16, 32, 2, 128, (15, 17, 63, 64, 65), shuffle_pages=True, spare_pages=3,
                              poison_tail=True),
        "d64": lambda: case(3, 16, 8, 2, 64, [100, 33, 512], shuffle_pages=True),
        "pages48": lambda: case(3, 16, 32, 2, 128, [100, 700, 257], page_size=48, shuffle_pages=True),
        "empty": lambda: case(3, 16, 32, 2, 128, [0, 300, 0], with_den=False),
        "f32": lambda: case(2, 5, 6, 3, 128, [37, 130], dtype=torch.float32, shuffle_pages=True),
    }
    c = cases[kind]()
    inp = synth.make_attn_inputs(c, seed=3)
    O, L = gpu_attn(inp)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    Od, Ld = gpu_attn(inp, debug_flags=flags)
    assert int(flags.item()) == 0, f"{kind}: debug flags {int(flags.item())}"
    assert torch.equal(Od, O), f"{kind}: O differs under the LDS fill"
    assert torch.equal(Ld.isnan(), L.isnan()) and torch.equal(torch.nan_to_num(Ld), torch.nan_to_num(L)), \
        f"{kind}: LSE differs under the LDS fill"


# --------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("ctx", [(0,), (0, 0, 5), (1,), (15, 17, 63, 64, 65), (129, 0, 200)])
def test_ragged_edges_with_poisoned_tails(ctx):
    """Prefix lengths off the tile and page grid; the unused slots of the last page and every
    unused page hold NaN, which must never reach the output."""
    c = case(len(ctx), 16, 32, 2, 128, ctx, shuffle_pages=True, spare_pages=3, poison_tail=True)
    print(run_full(c))


def test_empty_key_set():
    """ctx_len = 0 and no block keys: O = 0, LSE = -inf."""
    c = case(3, 16, 8, 2, 128, [0, 0, 0], with_den=False)
    inp = synth.make_attn_inputs(c)
    O, L = gpu_attn(inp)
    assert torch.all(O.float() == 0) and torch.all(torch.isneginf(L))


def test_empty_sequences_among_others():
    """Sequences with no keys at all next to ones with a prefix (no block keys): the empty ones get
    O = 0, LSE = -inf, the others their attention; pairs of the long ones span many segments."""
    c = case(5, 16, 32, 2, 128, [0, 300, 0, 4000, 0], with_den=False, shuffle_pages=True)
    print(run_full(c, what="empty sequences among prefix-only ones"))


def test_workspace_reused_across_calls_and_garbage():
    """One workspace, filled with random bytes, serves consecutive calls whose segment cuts differ:
    the per-pair arrival counts need no clearing between calls."""
    cases = [case(4, 16, 32, 2, 128, [4096, 900, 3000, 17]), case(4, 16, 32, 2, 128, [64, 5000, 128, 2500]),
             case(4, 16, 32, 2, 128, [4096, 900, 3000, 17])]
    inps = [synth.make_attn_inputs(c, seed=i) for i, c in enumerate(cases)]
    nb = 0
    for inp in inps:
        p = api.attn_params(*[to_dev(inp)[k] for k in ("Q", "Kc", "Vc", "page_table", "ctx_len", "Kd", "Vd")],
                            page_size=inp["page_size"], max_ctx_len=int(inp["ctx_len"].max()), scale=inp["scale"])
        nb = max(nb, api.block_attn_workspace_bytes(p))
    g = torch.Generator(device="cuda").manual_seed(7)
    ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda", generator=g)
    for i, (c, inp) in enumerate(zip(cases, inps)):
        d = to_dev(inp)
        O, L = api.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"],
                              page_size=inp["page_size"], max_ctx_len=int(inp["ctx_len"].max()), scale=inp["scale"],
                              workspace=ws)
        torch.cuda.synchronize()
        Or, Lr = oracle_attn(inp)
        print(check_attn(O, L, Or, Lr, c.dtype, f"call {i} on a shared workspace"))


def test_prefix_only_and_block_only():
    c = case(3, 16, 32, 2, 128, [300, 64, 1000], with_den=False, shuffle_pages=True)
    print(run_full(c, what="prefix only"))
    c = case(3, 16, 32, 2, 128, [0, 0, 0])
    print(run_full(c, what="block only (empty context: bidirectional attention over the block)"))


@pytest.mark.parametrize("S,Hq,Hkv", [(1, 32, 2), (3, 4, 4), (7, 6, 2), (64, 32, 2), (33, 8, 8), (16, 16, 1)])
def test_shapes(S, Hq, Hkv):
    """S from 1 to 64, GQA ratios 1..16, row counts S*G that do not fill a 256-row block
    and ones that need up to four row blocks."""
    c = case(2, S, Hq, Hkv, 128, [77, 190], shuffle_pages=True)
    print(run_full(c))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_head_dim_64(dtype):
    c = case(3, 16, 8, 2, 64, [100, 33, 512], dtype=dtype, shuffle_pages=True)
    print(run_full(c))


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
@pytest.mark.parametrize("prefix", [2000, 4096])
def test_head_dim_64_many_pieces(prefix, o_dtype):
    """One sequence at head_dim 64 whose pairs are cut into many pieces: a 2000-token prefix
    gives about 20 per pair (the merge splits each pair's partials over four thread groups), a
    4096-token prefix about 33 (eight groups of four rows); bf16 and fp32 partials."""
    c = case(1, 16, 32, 2, 64, [prefix])
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    k = pieces_per_pair(c, n_cu)
    print("pieces per pair", k)
    inp = synth.make_attn_inputs(c, seed=4)
    O, L = gpu_attn(inp, o_dtype=o_dtype)
    Or, Lr = oracle_attn(inp)
    print(check_attn(O, L, Or, Lr, c.dtype, f"d=64, prefix {prefix}, out {o_dtype}"))


@pytest.mark.parametrize("page_size", [32, 48, 64, 256])
def test_page_sizes(page_size):
    c = case(3, 16, 32, 2, 128, [100, 700, 257], page_size=page_size, shuffle_pages=True)
    print(run_full(c))


def test_fp32_shapes():
    c = case(2, 5, 6, 3, 128, [37, 130], dtype=torch.float32, shuffle_pages=True)
    print(run_full(c))


def test_contiguous_cache_as_one_page_per_sequence():
    """A dense [B][Hkv][L][d] cache is the paged layout with page_size = L and an identity table."""
    c = case(2, 16, 32, 2, 128, [1024, 1024], page_size=1024)
    print(run_full(c))


def test_strided_views_and_f32_output():
    """Q, K_den/V_den and O as strided views of larger buffers; bf16 inputs with a float32 O."""
    c = case(2, 16, 32, 2, 128, [333, 64], shuffle_pages=True)
    inp = synth.make_attn_inputs(c, seed=4)
    d = to_dev(inp)
    Qbig = torch.zeros(2, 16, 40, 128, dtype=torch.bfloat16, device="cuda")
    Qbig[:, :, 3:35] = d["Q"]
    Q = Qbig[:, :, 3:35]
    KVbig = torch.zeros(2, 16, 6, 128, dtype=torch.bfloat16, device="cuda")
    KVbig[:, :, 1:3] = d["Kd"]
    Kd = KVbig[:, :, 1:3]
    KVbig2 = torch.zeros(2, 16, 6, 128, dtype=torch.bfloat16, device="cuda")
    KVbig2[:, :, 1:3] = d["Vd"]
    Vd = KVbig2[:, :, 1:3]
    Obig = torch.full((2, 16, 36, 128), 5.0, dtype=torch.float32, device="cuda")
    O = Obig[:, :, 2:34]
    _, L = api.block_attn(Q, d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], Kd, Vd, page_size=16,
                          max_ctx_len=333, scale=inp["scale"], out=O)
    torch.cuda.synchronize()
    Or, Lr = oracle_attn(inp)
    check_attn(O, L, Or, Lr, torch.bfloat16, "strided")  # tolerances of the bf16 inputs
    assert torch.all(Obig[:, :, :2] == 5.0) and torch.all(Obig[:, :, 34:] == 5.0), "wrote outside the view"
    # float32 output of bf16 inputs is accurate beyond bf16 rounding
    err = (O.double().cpu().numpy() - Or)
    assert np.abs(err).max() < 2e-2


def test_lse_optional_and_batch_zero():
    c = case(2, 16, 32, 2, 128, [100, 50])
    inp = synth.make_attn_inputs(c)
    d = to_dev(inp)
    p = api.attn_params(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Kd"], d["Vd"], page_size=16,
                        max_ctx_len=100, scale=inp["scale"])
    p.LSE = None
    ws = torch.empty(api.block_attn_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    rc = api.lib().tt_block_attn(p, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    Or, _ = oracle_attn(inp)
    O = p._keep[0]
    assert np.abs(O.float().cpu().numpy() - Or).max() < 2e-2
    # B = 0: nothing to do
    e = torch.empty(0, 16, 32, 128, dtype=torch.bfloat16, device="cuda")
    api.block_attn(e, d["Kc"], d["Vc"], d["page_table"][:0], d["ctx_len"][:0], None, None, page_size=16,
                   max_ctx_len=0)


# --------------------------------------------------------------------------- properties on the GPU

def test_merge_of_prefix_and_block_partials():
    """Eq. (1) over the concatenation = tt_lse_merge(prefix-only partial, block-only partial)."""
    c = case(4, 16, 32, 2, 128, [1000, 64, 0, 4000], shuffle_pages=True)
    inp = synth.make_attn_inputs(c, seed=6)
    d = to_dev(inp)
    Of, Lf = gpu_attn(inp)
    O1, L1 = api.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], None, None, page_size=16,
                            max_ctx_len=4000, scale=inp["scale"], o_dtype=torch.float32)
    zero = torch.zeros_like(d["ctx_len"])
    O2, L2 = api.block_attn(d["Q"], d["Kc"], d["Vc"], d["page_table"], zero, d["Kd"], d["Vd"], page_size=16,
                            max_ctx_len=0, scale=inp["scale"], o_dtype=torch.float32)
    Om, Lm = api.lse_merge(torch.stack([O1, O2]).contiguous(), torch.stack([L1, L2]).contiguous(),
                           o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Or, Lr = oracle_attn(inp)
    print(check_attn(Om, Lm, Or, Lr, torch.bfloat16, "merged"))
    assert (Om.float() - Of.float()).abs().max().item() <= 2 ** -7, "merged vs direct"


def test_lse_merge_against_oracle_merge():
    rng = np.random.default_rng(5)
    P, B, S, Hq, d = 5, 3, 7, 6, 128
    O = rng.normal(size=(P, B, S, Hq, d)).astype(np.float32)
    lse = rng.normal(scale=4.0, size=(P, B, Hq, S)).astype(np.float32)
    lse[1, 0] = -np.inf        # an empty part
    lse[:, 2, 3] = -np.inf     # rows with every part empty
    Og, Lg = api.lse_merge(torch.from_numpy(O).cuda(), torch.from_numpy(lse).cuda())
    torch.cuda.synchronize()
    n = B * S * Hq
    Op = O.transpose(0, 1, 2, 3, 4).reshape(P, n, d).astype(np.float64)
    lp = lse.transpose(0, 1, 3, 2).reshape(P, n).astype(np.float64)
    Or, Lr = oracle.lse_merge(Op, lp)
    assert np.abs(Og.cpu().numpy().reshape(n, d) - Or).max() < 1e-5
    Lg = Lg.cpu().numpy().transpose(0, 2, 1).reshape(n).astype(np.float64)
    both = np.isneginf(Lg) & np.isneginf(Lr)
    assert np.all(np.where(both, 0, np.abs(Lg - Lr)) < 1e-5)
    # bf16 output
    Ob, _ = api.lse_merge(torch.from_numpy(O).cuda(), torch.from_numpy(lse).cuda(), o_dtype=torch.bfloat16)
    assert np.abs(Ob.float().cpu().numpy().reshape(n, d) - Or).max() < 2e-2


def test_weights_sum_to_one():
    """V = 1 everywhere: O is exactly 1 after rounding; V = c: O = c."""
    c = case(3, 16, 32, 2, 128, [900, 17, 4096], shuffle_pages=True, value_scale=3.0)
    inp = synth.make_attn_inputs(c, seed=2)
    for val in (1.0, -2.5):
        inp2 = dict(inp, Vc=torch.full_like(inp["Vc"], val), Vd=torch.full_like(inp["Vd"], val))
        O, _ = gpu_attn(inp2)
        assert torch.all(O.float() == val), f"V={val}: {O.float().unique()[:5]}"


def test_block_permutation_equivariance():
    c = case(2, 16, 32, 2, 128, [500, 77], shuffle_pages=True, value_scale=2.0)
    inp = synth.make_attn_inputs(c, seed=8)
    O, L = gpu_attn(inp)
    pi = torch.randperm(16, generator=torch.Generator().manual_seed(1))
    inp2 = dict(inp, Q=inp["Q"][:, pi].contiguous(), Kd=inp["Kd"][:, pi].contiguous(), Vd=inp["Vd"][:, pi].contiguous())
    O2, L2 = gpu_attn(inp2)
    assert (O2.float() - O[:, pi].float()).abs().max().item() <= 2 ** -7
    assert (L2 - L[:, :, pi]).abs().max().item() <= 1e-3


def test_deterministic():
    c = synth.attn_case("ragged")
    c.B = 16
    c.ctx_lens = c.ctx_lens[:16]
    inp = synth.make_attn_inputs(c, seed=1)
    O1, L1 = gpu_attn(inp)
    O2, L2 = gpu_attn(inp)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
