"""Oracle for the deterministic MoE layer step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU implementation of what one GPU's share of a Mixture-of-
Kittens MoE layer step computes (router top-k gating, stable expert
permutation, SwiGLU expert FFN, weighted combine, and the backward pass with
router-weight gradients). It shares no code with the GPU library and imports
nothing from it. Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import it.

Sources (the pages describing Mixture-of-Kittens):
  * "Cursor Mixture-of-Kittens cuts MoE training latency by 5.8x"
    (dothoosh.com), section "Technical details of the MoK mechanism":
    one schedule table for dispatch, combine, reverse-combine and
    reverse-dispatch; BF16 and MXFP8; router-weight gradients fused into the
    SwiGLU backward (SonicMoE-style); a fixed ring buffer so no token is
    dropped.
  * kwkr.cn MoK explainer, section 4.1: top-k gating; section 2: determinism
    (same inputs give the same outputs).
  * aikraft.ru MoK article, section 04: pull dispatch, push combine.

MXFP8 quantisation and the MXFP8 step are in ``oracle.mx``.

Every function is pinned by tests in tests/test_oracle_*.py against closed
forms, brute force, torch.autograd on a dense formulation, and finite
differences (see the docstrings of those tests).
"""
from .moe import *  # noqa: F401,F403
from . import mx  # noqa: F401
