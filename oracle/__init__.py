"""CPU oracle for EntmaxKV support-aware paged sparse alpha-entmax decode.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code written from the
EntmaxKV pages ("EntmaxKV: Support-Aware Decoding for Entmax Attention",
arXiv 2605.21649: the gist.science technical summary, sections 2.A-2.C and 3,
and the authors' abstract).  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it; the product path (the HIP
library and its Python binding) never does, and shares no code with it.

Modules:
  entmax    exact sort-based alpha-entmax threshold (and a bisection variant)
  metadata  brute-force per-page k_min / k_max / mean / variance
  scoring   bounding-box upper bound and Gaussian page score model
  select    fixed-budget top-k and the Gaussian-aware threshold selector
  decode    exact entmax attention over a token set, dropped mass, error bound
  softmax   softmax attention over a token set and its dropped mass (comparison)

Where the pages are silent (the bound's formula, the Gaussian expectation,
the estimated maximum, GQA sharing, tie rules) each function states the
reading it implements.  Parity status: every function is pinned by tests in
tests/test_oracle_*.py except the ones whose docstring says
"parity unpinned".
"""
from . import entmax, metadata, scoring, select, decode, softmax  # noqa: F401
