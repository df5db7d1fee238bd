"""fp64 CPU oracle for block-diagonal (per-document causal) packed attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links
or runs anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path (no
kernels, headers, helpers or table generators); the only code both sides use
is the seeded input generator in ``synthetic``, which holds no attention
arithmetic.

What it computes follows the Automodel page "feat(distributed): block-diagonal
varlen CP for packed sequences":
  * Summary / Motivation: attention inside a packed row is block-causal per
    document -- a query attends a key only in its own document and only at or
    before its own position -- and a dense masked-SDPA computation is the
    plain definition the varlen kernel must reproduce;
  * Design overview (kernels.py): the dense ``[B,1,L,S]`` mask of the L local
    query rows against all S keys of the row;
  * Design overview (batch.py, packed.py) and key property 1: a rank holds a
    contiguous query chunk starting at ``row_offset`` and the K/V of the whole
    row; ``row_offset = 0`` with the full length is the single-rank case;
  * key property 2: a document that starts left of the chunk gives its first
    segment more keys than queries, aligned bottom-right.

Modules:
  segment   -- reference segment table (varlen metadata) and per-row /
               per-key mask bounds, from the document lengths.
  attention -- dense and windowed fp64 forward (O, LSE) and a hand-derived
               backward (dQ, dK, dV) from the softmax Jacobian.
  brute     -- pure-Python scalar loops for tiny inputs.
  kvplan    -- reference needed-only K/V exchange plan (halo / all-to-all-v
               ranges) from the dense mask.
  dropout   -- attention-dropout keep masks from Philox4x32-10 (the
               counter-based generator of Salmon et al., SC'11) under a
               stated counter layout; attention.forward / backward take an
               optional Dropout.
  parallel  -- process-pool runner (slicing and reassembly only).

Parity status: every function here is pinned by CPU tests against values
independent of its own code (torch SDPA as a library special case, closed
forms, finite differences, brute force, hand-worked fixtures); see the test
module docstrings.  The bf16 output rounding convention and the padding-row
convention (O = 0, LSE = -inf) are conventions, not pinned values.
"""
from . import attention, brute, dropout, kvplan, segment  # noqa: F401
