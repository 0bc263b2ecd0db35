"""CPU oracle for the Dynamic Cache Updating (DCU) step and the Frechet-profile commit rule.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, numpy fp64 statement of what the GPU path
computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import it.
The product path (the HIP library and its Python binding) never imports, links or calls anything
here, and this package imports nothing from the product path.

Sources (web pages about the method; each function cites the part it follows):

* "Dynamic-dLLM: Dynamic Cache-Budget and Adaptive Parallel Decoding for Training-Free Acceleration
  of Diffusion LLM" (papernotes.org reading notes, ICLR 2026), section "Key designs":
  design 1 (DCU: token distance, layer dynamics, proportional budget, top-B recompute),
  design 2 (forced update window), design 3 (APD thresholds).
* "Fast-dLLM++: Frechet Profile Decoding for Faster Diffusion LLM Inference" (papernotes.org
  reading notes, ICML 2026 workshop), section "Key designs": design 1 (Theorem 4.1 certificate),
  design 2 (selection rule n* = max{n : G_n > delta}, else 1), design 3 (Proposition 4.3 /
  Corollary 4.4 decomposition G_n = F_n + B_n).

Modules: distance, budget, select, layer (with optional rotary position embedding), confidence,
frechet, apd (adaptive parallel decoding), step (the per-step driver, open or closed loop).

Parity status: every function is pinned by the tests under tests/test_oracle_*.py (closed forms,
exact rational or high-precision brute force, library routines, the pages' worked example). The
internal structure of the transformer layer (pre-norm RMSNorm, scale 1/sqrt(head_dim), rotary
embedding of q and k in the rotate-half pairing when a base is given) is a reading the pages do
not fix: the layer function is pinned as an implementation of that reading, but the reading itself
is "parity unpinned" by the pages.
"""
from . import apd, budget, confidence, distance, frechet, layer, select, step  # noqa: F401
