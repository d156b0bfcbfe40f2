"""Greedy per-row pick with nonfinite flags (oracle; test infrastructure only).

PR #1377 "LFM2: shared-round decode", the GPU-pick commit and the "Kernel
contract and exactness" section: each head row's pick is the first largest
of its 128,000 bf16 logits (ties go to the lower id, as in the host draw),
and a row holding a nonfinite logit is flagged so that its draw stays on the
host. The pick of a flagged row is never used there, so its value is left
open by the pages; the reading taken (listed in the design notes) is:

* NaN is skipped; +Inf and -Inf are ordered as usual;
* -0 and +0 compare equal, so they tie and the lower id wins;
* a row with no non-NaN value picks 0;
* flag = the row holds a NaN or an infinity.

``scan_row`` is the definition, a scalar loop; ``row_argmax`` is the same
rule over whole rows with NumPy, pinned against ``scan_row`` in the tests.
"""

import math

import numpy as np

from . import bf16


def scan_row(bits):
    """Scalar scan of one row of bf16 bit patterns -> (pick, flag)."""
    vals = bf16.to_f64(bits)
    best_i = None
    best_v = None
    flag = False
    for i, v in enumerate(vals.tolist()):
        if not math.isfinite(v):
            flag = True
        if math.isnan(v):
            continue
        if best_v is None or v > best_v:
            best_v, best_i = v, i
    return (0 if best_i is None else best_i), flag


def row_argmax(logits):
    """logits: uint16 [R][V] bf16 bit patterns -> (pick int32 [R], flag uint8 [R])."""
    L = np.asarray(logits, dtype=np.uint16)
    if L.ndim == 1:
        L = L[None, :]
    R = L.shape[0]
    pick = np.zeros(R, dtype=np.int32)
    flag = np.zeros(R, dtype=np.uint8)
    for r in range(R):
        v = bf16.to_f64(L[r])
        nan = np.isnan(v)
        flag[r] = np.uint8(bool((~np.isfinite(v)).any()))
        if nan.all():
            pick[r] = 0
            continue
        vmax = v[~nan].max()
        # first index holding the maximum among non-NaN values; -0 == +0
        pick[r] = int(np.flatnonzero((~nan) & (v == vmax))[0])
    return pick, flag
