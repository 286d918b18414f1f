"""libtwotower_attn for MI355X: the TwoTower block-attention step (Eq. 1) and
confidence-unmask SampleStep (Algorithm 2) of Nemotron-TwoTower (arXiv
2606.26493), as hand-written gfx950 HIP kernels behind a C ABI.

``attention_eq_block_amd.api`` holds the Python calls; ``synth`` the seeded
synthetic workloads. Importing the package does not load the library; the
first call does, and raises if it was not built.
"""
from .api import (abi_version, block_attn, conf_unmask, lse_merge,  # noqa: F401
                  status_string)
