"""CPU oracle for mixed FP8 / TQ3 paged decode attention (Minima-KV).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library under
``mixed_format_paged_amd/`` and its Python binding) imports, calls or links
anything here.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use this package.

What it is: a plain, slow, numpy implementation of what the hot path computes,
written from the Minima-KV pages (arXiv 2608.23834, abstract on page 1; the
"Technical Deep Dive" of the setupai.cc summary on page 2 only as a hint):

* ``fp8``       -- OCP E4M3FN encode (round-to-nearest-even, saturating) and decode
* ``tq3``       -- the TQ3 3-bit symmetric group quantiser (scale rule, codes)
* ``layout``    -- byte layout of FP8 and TQ3 pages, 8-codes-in-3-bytes packing
* ``pool``      -- a byte-level page pool: append, FP8->TQ3 demotion, page-table gather
* ``attention`` -- dense fp64 softmax decode attention and the log-sum-exp merge
* ``dense``     -- bf16 rounding and the dense materialisation of pages
* ``rotation``  -- the rotated TQ3 variant: sign flip and Walsh-Hadamard rotation

Every floating-point step of attention is carried out in fp64 on the
dequantised values; quantisation steps are done exactly (integer / exact
fp32 threshold arithmetic) so the byte outputs are the unique results of the
stated rules.  Where the pages are silent the reading taken is stated in the
function that implements it.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(exhaustive codec tables, brute-force quantiser, closed forms, a library
SDPA cross-check and merge invariance).  The pages' own headline figures
(18.3 KiB/token, 3.625x, 0.9821x, RULER/LongBench deltas) are context only:
parity unpinned, because the model, control and tier mix behind them are not
given on the pages.
"""
from . import fp8, tq3, layout, pool, attention, build, dense  # noqa: F401
