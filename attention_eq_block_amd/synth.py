"""Seeded synthetic inputs for the block-attention step and the confidence unmask.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the HIP path and the CPU oracle are fed from it.

Every tensor is drawn from its own ``torch.Generator`` whose seed is
``seed + sub-seed + 100*layer + 10000*step`` (sub-seeds: Q=1, Kctx=2, Vctx=3,
Kden=4, Vden=5, ctx_len=6, page permutation=7, logit noise=8, spike index=9,
spike height=10). Draws are N(0,1) or uniform in float32, scaled where a
workload says so, then rounded to the working dtype (bf16 round-to-nearest-even
through ``Tensor.to``). On ``device="cpu"`` the values are identical on every
machine; on a GPU device the generator is the device's own (used by the
benchmark to fill multi-GB workloads quickly).

The workloads mirror the operating point of Nemotron-TwoTower (arXiv
2606.26493): block size S=16, T=16 denoising steps, six attention layers per
tower (section 2.1), gamma=0.8 and temperature 0.1 (the generation example of
the release notes). Head counts, head_dim and vocabulary size are not on the
pages; 32 query heads sharing 2 KV heads, head_dim 128 and V=131072 are used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

SUB_Q, SUB_KCTX, SUB_VCTX, SUB_KDEN, SUB_VDEN = 1, 2, 3, 4, 5
SUB_CTXLEN, SUB_PAGEPERM, SUB_NOISE, SUB_SPIKE_IDX, SUB_SPIKE_H = 6, 7, 8, 9, 10

MASK_TOKEN_ID = 3  # the [MASK] id used in the release's generation example


def _gen(seed: int, sub: int, layer: int = 0, step: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + sub + 100 * layer + 10000 * step)
    return g


def randn(shape, seed, sub, layer=0, step=0, device="cpu", scale=1.0, dtype=torch.float32):
    g = _gen(seed, sub, layer, step, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


# ----------------------------------------------------------------------------
# attention step
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class AttnCase:
    """Shapes and value recipe of one block-attention call.

    ``ctx_lens`` lists the prefix length of every sequence (tokens of the
    prompt plus committed blocks). Pages of ``page_size`` tokens come from one
    pool; ``shuffle_pages`` draws their order with a seeded permutation,
    otherwise sequence b owns a contiguous run of pages (identity table).
    """
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    ctx_lens: Sequence[int]
    dtype: torch.dtype = torch.bfloat16
    page_size: int = 16
    shuffle_pages: bool = False
    value_scale: float = 1.0      # multiply N(0,1) draws by this before rounding
    with_den: bool = True         # False: context-only partial (Kden=Vden=NULL)
    spare_pages: int = 0          # unused pages appended to the pool
    poison_tail: bool = False     # fill slots past ctx_len with NaN (never read)
    name: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_ctx_len(self) -> int:
        return max(self.ctx_lens) if len(self.ctx_lens) else 0

    def pages_of(self, L: int) -> int:
        return (L + self.page_size - 1) // self.page_size

    @property
    def max_pages(self) -> int:
        return max(1, max((self.pages_of(L) for L in self.ctx_lens), default=0))

    def kv_bytes(self) -> int:
        eb = torch.tensor([], dtype=self.dtype).element_size()
        return sum(self.ctx_lens) * self.Hkv * self.D * 2 * eb

    def algorithmic_bytes(self) -> int:
        """Bytes the step must move: prefix K/V, Q, in-block K/V, O and LSE."""
        eb = torch.tensor([], dtype=self.dtype).element_size()
        n = self.B * self.S
        den = 2 * self.Hkv * self.D * eb if self.with_den else 0
        return self.kv_bytes() + n * (2 * self.Hq * self.D * eb + den + 4 * self.Hq)

    def flops(self) -> int:
        keys = sum(L + (self.S if self.with_den else 0) for L in self.ctx_lens)
        return 4 * self.Hq * self.D * self.S * keys


def make_attn_inputs(case: AttnCase, seed: int = 0, layer: int = 0, device="cpu"):
    """Draw Q, the paged prefix cache, the in-block K/V and the page table."""
    B, S, Hq, Hkv, D, P = case.B, case.S, case.Hq, case.Hkv, case.D, case.page_size
    dt = case.dtype
    sc = case.value_scale
    ctx_len = torch.tensor(list(case.ctx_lens), dtype=torch.int32)
    n_pages = [case.pages_of(int(L)) for L in case.ctx_lens]
    num_pages = max(1, sum(n_pages) + case.spare_pages)
    if case.shuffle_pages:
        perm = torch.randperm(num_pages, generator=_gen(seed, SUB_PAGEPERM, layer)).to(torch.int32)
    else:
        perm = torch.arange(num_pages, dtype=torch.int32)
    page_table = torch.full((B, case.max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        page_table[b, : n_pages[b]] = perm[off: off + n_pages[b]]
        off += n_pages[b]

    Q = randn((B, S, Hq, D), seed, SUB_Q, layer, device=device, scale=sc, dtype=dt)
    Kc = randn((num_pages, Hkv, P, D), seed, SUB_KCTX, layer, device=device, scale=sc, dtype=dt)
    Vc = randn((num_pages, Hkv, P, D), seed, SUB_VCTX, layer, device=device, scale=sc, dtype=dt)
    if case.poison_tail:
        for b in range(B):
            L = int(case.ctx_lens[b])
            if L % P:
                pg = int(page_table[b, L // P])
                Kc[pg, :, L % P:, :] = float("nan")
                Vc[pg, :, L % P:, :] = float("nan")
        used = set(int(x) for x in page_table.flatten().tolist() if x >= 0)
        for pg in range(num_pages):
            if pg not in used:
                Kc[pg] = float("nan")
                Vc[pg] = float("nan")
    if case.with_den:
        Kd = randn((B, S, Hkv, D), seed, SUB_KDEN, layer, device=device, scale=sc, dtype=dt)
        Vd = randn((B, S, Hkv, D), seed, SUB_VDEN, layer, device=device, scale=sc, dtype=dt)
    else:
        Kd = Vd = None
    return dict(Q=Q, Kc=Kc, Vc=Vc, page_table=page_table.to(device), ctx_len=ctx_len.to(device),
                Kd=Kd, Vd=Vd, page_size=P, scale=1.0 / math.sqrt(D))


def ragged_ctx_lens(B: int, lo: int, hi: int, multiple: int, seed: int = 0) -> List[int]:
    """Prefix lengths drawn uniformly from {lo, lo+multiple, ..., hi}."""
    g = _gen(seed, SUB_CTXLEN)
    k = torch.randint(lo // multiple, hi // multiple + 1, (B,), generator=g)
    return [int(x) * multiple for x in k]


# ----------------------------------------------------------------------------
# confidence unmask
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class UnmaskCase:
    """Logits of one SampleStep: N(0,1) noise plus one spike per row.

    The spike sits at a seeded target token of each (b, position); its height
    is either a constant or drawn per row from U(0, spike_hi).
    """
    B: int
    S: int
    V: int
    dtype: torch.dtype = torch.bfloat16
    spike: float = 4.0               # constant height (used when spike_hi is None)
    spike_hi: Optional[float] = None  # draw height from U(0, spike_hi) per row
    gamma: float = 0.8
    temperature: float = 0.1
    steps_left: int = 16
    name: str = ""

    def algorithmic_bytes(self, n_masked_rows: int) -> int:
        eb = torch.tensor([], dtype=self.dtype).element_size()
        return n_masked_rows * self.V * eb


def spike_targets(B: int, S: int, V: int, seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(seed, SUB_SPIKE_IDX)
    return torch.randint(0, V, (B, S), generator=g, dtype=torch.int64).to(device)


def make_logits(case: UnmaskCase, seed: int = 0, step: int = 0, spike: Optional[float] = None,
                targets: Optional[torch.Tensor] = None, device="cpu") -> torch.Tensor:
    B, S, V = case.B, case.S, case.V
    x = randn((B, S, V), seed, SUB_NOISE, 0, step, device=device)
    if targets is None:
        targets = spike_targets(B, S, V, seed, device=device)
    if case.spike_hi is not None:
        g = _gen(seed, SUB_SPIKE_H, 0, step, device)
        h = torch.rand((B, S), generator=g, device=device) * case.spike_hi
    else:
        h = torch.full((B, S), case.spike if spike is None else spike, device=device)
    x.scatter_add_(2, targets.to(device).unsqueeze(-1), h.unsqueeze(-1))
    return x.to(case.dtype)


def make_mask_state(B: int, S: int, device="cpu"):
    """A fresh block: every position is [MASK]."""
    tokens = torch.full((B, S), MASK_TOKEN_ID, dtype=torch.int32, device=device)
    mask = torch.ones((B, S), dtype=torch.uint8, device=device)
    return tokens, mask


def random_mask_state(B: int, S: int, p_masked: float, seed: int = 0, device="cpu"):
    g = _gen(seed, 11)
    mask = (torch.rand((B, S), generator=g) < p_masked).to(torch.uint8)
    tokens = torch.randint(0, 1000, (B, S), generator=g, dtype=torch.int32)
    tokens[mask.bool()] = MASK_TOKEN_ID
    return tokens.to(device), mask.to(device)


SUB_UNIFORM = 17


def make_uniforms(B: int, S: int, seed: int = 0, step: int = 0, device="cpu") -> torch.Tensor:
    """One float32 uniform in [0, 1) per block position, for the stochastic draw."""
    return torch.rand((B, S), generator=_gen(seed, SUB_UNIFORM, 0, step)).to(device)


# ----------------------------------------------------------------------------
# commit-time cache append
# ----------------------------------------------------------------------------

SUB_APPEND = 12


def make_append_inputs(B: int, S: int, Hkv: int, D: int, page_size: int, max_pages: int, ctx_lens,
                       spare_pages: int, dtype=torch.bfloat16, seed: int = 0, assign_all: bool = False):
    """Paged caches and one committed block of new K/V rows per sequence.

    The cache holds the pages each sequence uses for its ctx_lens (every page of
    max_pages when ``assign_all``) plus ``spare_pages`` free ones, all in one seeded
    random order; table entries past the used pages are -1 and the free pages form
    the pool. Cache contents and new rows are N(0,1). CPU tensors; the pool is int32.
    """
    ctx = [int(c) for c in ctx_lens]
    used = [max_pages if assign_all else (max(c, 0) + page_size - 1) // page_size for c in ctx]
    num_pages = sum(used) + spare_pages
    perm = torch.randperm(num_pages, generator=_gen(seed, SUB_APPEND)).to(torch.int32)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    k = 0
    for b in range(B):
        table[b, :used[b]] = perm[k:k + used[b]]
        k += used[b]
    pool = perm[k:].clone()
    Kc = randn((num_pages, Hkv, page_size, D), seed, SUB_APPEND + 1, dtype=dtype)
    Vc = randn((num_pages, Hkv, page_size, D), seed, SUB_APPEND + 2, dtype=dtype)
    Kn = randn((B, S, Hkv, D), seed, SUB_APPEND + 3, dtype=dtype)
    Vn = randn((B, S, Hkv, D), seed, SUB_APPEND + 4, dtype=dtype)
    return dict(Kc=Kc, Vc=Vc, page_table=table, ctx_len=torch.tensor(ctx, dtype=torch.int32), Knew=Kn, Vnew=Vn,
                pool=pool, pool_count=int(pool.numel()))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def attn_case(name: str, variant: str = "") -> AttnCase:
    """Attention shapes of the named workload.

    tiny      fp32, B=1, 4 q-heads on 1 kv-head, d=64, prefix 48, S=16
    single    bf16, B=1, 32/2 heads, d=128, prefix 4096, S=16, values N(0,1)/sqrt(128)
    ragged    bf16, B=64, prefix 16*U{32..512}, shuffled 16-token pages
    long      bf16, B=4, prefix 131072, S=32, values N(0,1)
    loop      bf16, B=32, prefix 8192, S=16 (one of six layer caches)
    ``variant="unscaled"`` draws N(0,1) values where the workload scales them.
    """
    s128 = 1.0 / math.sqrt(128.0)
    vs = 1.0 if variant == "unscaled" else s128
    if name == "tiny":
        return AttnCase(1, 16, 4, 1, 64, [48], dtype=torch.float32, name=name)
    if name == "single":
        return AttnCase(1, 16, 32, 2, 128, [4096], value_scale=vs, name=name)
    if name == "ragged":
        return AttnCase(64, 16, 32, 2, 128, ragged_ctx_lens(64, 512, 8192, 16), shuffle_pages=True,
                        value_scale=vs, name=name)
    if name == "long":
        return AttnCase(4, 32, 32, 2, 128, [131072] * 4, name=name)
    if name == "loop":
        return AttnCase(32, 16, 32, 2, 128, [8192] * 32, value_scale=vs, name=name)
    raise KeyError(name)


def unmask_case(name: str, temperature: float = 0.1, gamma: float = 0.8) -> UnmaskCase:
    if name == "tiny":
        return UnmaskCase(1, 16, 1024, dtype=torch.float32, spike=4.0, gamma=gamma,
                          temperature=temperature, name=name)
    if name == "ragged":
        return UnmaskCase(64, 16, 131072, spike_hi=8.0, gamma=gamma, temperature=temperature, name=name)
    if name == "loop":
        return UnmaskCase(32, 16, 131072, spike=0.5, gamma=gamma, temperature=temperature, name=name)
    raise KeyError(name)


LOOP_LAYERS = 6
LOOP_STEPS = 16
