"""tt_kv_append on the GPU against the oracle (the cache side of Algorithm 1's context update after
a block is committed, Nemotron-TwoTower section 2.1). Byte and integer work: caches, page table,
ctx_len, pool count and status are compared exactly. Page assignment is deterministic (top of the
pool, sequence then position order), so the tables must match entry for entry."""
import numpy as np
import pytest
import torch

import oracle
from attention_eq_block_amd import api, synth

from parity import check_attn, gpu_attn, oracle_attn

pytestmark = pytest.mark.gpu


def _gpu(inp, pool_count=None, knew=None, vnew=None):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pc = torch.tensor([inp["pool_count"] if pool_count is None else pool_count], dtype=torch.int32, device="cuda")
    pool = d["pool"] if d["pool"].numel() else torch.zeros(1, dtype=torch.int32, device="cuda")
    st = api.kv_append(d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Knew"] if knew is None else knew,
                       d["Vnew"] if vnew is None else vnew, pool=pool, pool_count=pc)
    torch.cuda.synchronize()
    return dict(Kc=d["Kc"].cpu(), Vc=d["Vc"].cpu(), page_table=d["page_table"].cpu().numpy(),
                ctx_len=d["ctx_len"].cpu().numpy(), pool_count=int(pc.item()), status=int(st.item()))


def _oracle(inp, pool_count=None):
    return oracle.kv_append(inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp["Knew"], inp["Vnew"],
                            pool=inp["pool"].tolist(), pool_count=inp["pool_count"] if pool_count is None
                            else pool_count)


def _same(got, ref, what):
    assert got["status"] == ref["status"], (what, got["status"], ref["status"])
    for k in ("Kc", "Vc"):
        assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), f"{what}: {k} differs"
    assert np.array_equal(got["page_table"], ref["page_table"]), f"{what}: page table differs"
    assert np.array_equal(got["ctx_len"], ref["ctx_len"]), f"{what}: ctx_len differs"
    assert got["pool_count"] == ref["pool_count"], f"{what}: pool count differs"


@pytest.mark.parametrize("dtype,D,page_size,S", [
    (torch.bfloat16, 128, 16, 16), (torch.bfloat16, 64, 16, 32), (torch.float32, 64, 3, 5),
    (torch.float32, 128, 1, 1), (torch.bfloat16, 128, 64, 64),
])
def test_append_matches_oracle(dtype, D, page_size, S):
    """Ragged lengths (0, negative, mid-page, page-aligned), shuffled pages, partly unassigned table."""
    ctx = [0, -3, 5, 16, 47, 64, 1, 100, 31, 32]
    inp = synth.make_append_inputs(len(ctx), S, 2, D, page_size, max_pages=(200 + page_size - 1) // page_size,
                                   ctx_lens=ctx, spare_pages=400 // page_size + 20, dtype=dtype, seed=1)
    _same(_gpu(inp), _oracle(inp), f"{dtype} D={D} P={page_size} S={S}")


def test_loop_shape_and_many_sequences():
    """The denoise loop's shape (B=32, S=16, 2 KV heads, d=128, 16-token pages at prefix 8192) and
    B=100 (more sequences than one wave of the planning kernel)."""
    inp = synth.make_append_inputs(32, 16, 2, 128, 16, max_pages=520, ctx_lens=[8192] * 32, spare_pages=40,
                                   seed=2)
    _same(_gpu(inp), _oracle(inp), "loop shape")
    ctx = list(range(0, 300, 3))
    inp = synth.make_append_inputs(100, 7, 1, 64, 16, max_pages=20, ctx_lens=ctx, spare_pages=200, seed=3)
    _same(_gpu(inp), _oracle(inp), "B=100")


def test_errors_change_nothing():
    """Capacity (1), pool exhausted (2), page id out of range (3): status set, every output unchanged."""
    base = synth.make_append_inputs(6, 8, 2, 64, 16, max_pages=4, ctx_lens=[0, 10, 20, 33, 40, 8],
                                    spare_pages=12, seed=4)
    cases = []
    c = dict(base); c["ctx_len"] = base["ctx_len"].clone(); c["ctx_len"][3] = 4 * 16 - 7
    cases.append(("capacity", c, None, 1))
    cases.append(("pool short", base, 1, 2))
    c = dict(base); c["page_table"] = base["page_table"].clone(); c["page_table"][1, 0] = base["Kc"].shape[0] + 3
    cases.append(("bad table entry", c, None, 3))
    c = dict(base); c["pool"] = base["pool"].clone(); c["pool"][-1] = -1
    cases.append(("bad pool entry", c, None, 3))
    for what, c, pc, code in cases:
        got, ref = _gpu(c, pc), _oracle(c, pc)
        assert ref["status"] == code, what
        _same(got, ref, what)
        assert torch.equal(got["Kc"], c["Kc"]) and np.array_equal(got["ctx_len"], c["ctx_len"].numpy()), what
    # exactly to capacity succeeds
    c = dict(base); c["ctx_len"] = base["ctx_len"].clone(); c["ctx_len"][3] = 4 * 16 - 8
    _same(_gpu(c), _oracle(c), "exactly full")


def test_no_pool_needed_and_empty_batch():
    """Every needed page already assigned: no pool is passed and status is 0. B = 0 is a no-op."""
    inp = synth.make_append_inputs(4, 16, 2, 128, 16, max_pages=8, ctx_lens=[0, 17, 40, 96], spare_pages=0,
                                   assign_all=True, seed=5)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    st = api.kv_append(d["Kc"], d["Vc"], d["page_table"], d["ctx_len"], d["Knew"], d["Vnew"])
    torch.cuda.synchronize()
    ref = oracle.kv_append(inp["Kc"], inp["Vc"], inp["page_table"], inp["ctx_len"], inp["Knew"], inp["Vnew"])
    got = dict(Kc=d["Kc"].cpu(), Vc=d["Vc"].cpu(), page_table=d["page_table"].cpu().numpy(),
               ctx_len=d["ctx_len"].cpu().numpy(), pool_count=0, status=int(st.item()))
    ref["pool_count"] = 0
    _same(got, ref, "no pool")
    e = torch.empty((0, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    st = api.kv_append(d["Kc"], d["Vc"], d["page_table"][:0], d["ctx_len"][:0], e, e)
    torch.cuda.synchronize()


def test_strided_new_rows_and_two_appends():
    """New rows read through strides (a head slice of a wider tensor); a second append on the first's
    results matches the oracle applied twice."""
    inp = synth.make_append_inputs(5, 6, 2, 64, 16, max_pages=6, ctx_lens=[0, 9, 16, 30, 50], spare_pages=16,
                                   seed=6)
    wide_k = torch.randn(5, 6, 3, 64).to(torch.bfloat16)
    wide_v = torch.randn(5, 6, 3, 64).to(torch.bfloat16)
    inp["Knew"], inp["Vnew"] = wide_k[:, :, 1:], wide_v[:, :, 1:]
    gk, gv = wide_k.cuda()[:, :, 1:], wide_v.cuda()[:, :, 1:]
    assert gk.stride(1) == 3 * 64
    got = _gpu(inp, knew=gk, vnew=gv)
    ref = _oracle(inp)
    _same(got, ref, "strided")
    nxt = dict(Kc=ref["Kc"], Vc=ref["Vc"], page_table=torch.from_numpy(ref["page_table"]),
               ctx_len=torch.from_numpy(ref["ctx_len"]), Knew=inp["Knew"].flip(1).contiguous(),
               Vnew=inp["Vnew"].flip(1).contiguous(), pool=inp["pool"], pool_count=ref["pool_count"])
    _same(_gpu(nxt), _oracle(nxt), "second append")


def test_attention_over_the_appended_cache():
    """Eq. (1) over the cache the GPU appended equals the oracle's Eq. (1) over the cache the oracle
    appended (bf16 bar of the attention tests)."""
    B, S, Hq, Hkv, D, P = 4, 16, 8, 2, 128, 16
    inp = synth.make_append_inputs(B, S, Hkv, D, P, max_pages=12, ctx_lens=[0, 40, 64, 100], spare_pages=16,
                                   seed=7)
    got = _gpu(inp)
    ref = _oracle(inp)
    _same(got, ref, "append before attention")
    Q = synth.randn((B, S, Hq, D), 7, 30, dtype=torch.bfloat16)
    Kd = synth.randn((B, S, Hkv, D), 7, 31, dtype=torch.bfloat16)
    Vd = synth.randn((B, S, Hkv, D), 7, 32, dtype=torch.bfloat16)
    a = dict(Q=Q, Kc=got["Kc"], Vc=got["Vc"], page_table=torch.from_numpy(got["page_table"]).clamp(min=0),
             ctx_len=torch.from_numpy(got["ctx_len"]), Kd=Kd, Vd=Vd, page_size=P, scale=D ** -0.5)
    O, L = gpu_attn(a)
    r = dict(a); r["Kc"], r["Vc"] = ref["Kc"], ref["Vc"]
    r["page_table"] = torch.from_numpy(ref["page_table"]).clamp(min=0)
    Oref, Lref = oracle_attn(r)
    check_attn(O, L, Oref, Lref, torch.bfloat16, "attention after append")
