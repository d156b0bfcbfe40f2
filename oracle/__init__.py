"""Plain CPU oracle for the shared-round verify step (test infrastructure).

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(the HIP library and its Python binding) never calls into it, and it imports
nothing from the product path: no kernels, headers, helpers or tables are
shared.

Everything here is written from the pages' description of the method, as
slow, direct NumPy float64 code:

* ``bf16``   -- bfloat16 bit patterns to float64 and back (single RNE rounding).
* ``table``  -- the segment table of a shared round (row offsets, row map,
  visible-key counts, 16-row tiles, the split plan and partial offsets).
  PR #1377 "LFM2: shared-round decode", the shared-round commit of its
  commit log (a table of per-stream cache addresses, row offsets and key
  counts; the partials of each stream kept apart).
* ``conv``   -- a host replay, row by row, of the gated short conv against each
  stream's own conv state (same commit: the stream conv is checked against a
  host replay of the conv steps).
* ``attn``   -- float64 softmax attention per row and head, the split-K
  partials, and their merge (same commit: the stream attention is checked
  against float64 attention; the attention merge kernel of the inline-bodies
  commit).
* ``argmax`` -- a scalar first-maximum scan with nonfinite flags (PR #1377,
  the GPU-pick commit and the kernel contract entry for the argmax: the host
  draw's pick, ties to the lower id, nonfinite rows flagged).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library routines, brute force and hand-written golden cases.
"""

from . import argmax, attn, bf16, conv, table  # noqa: F401

__all__ = ["argmax", "attn", "bf16", "conv", "table"]
