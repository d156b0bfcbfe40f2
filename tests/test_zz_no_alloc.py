"""asv_row_argmax_noalloc against asv_row_argmax, through the C ABI.

The allocation-free entry point takes its workspace from the library's own
device array; its picks and flags must equal those of asv_row_argmax (the
same kernels over a caller workspace) bit for bit. Two calls in a row, the
second smaller (fewer rows, a ragged vocabulary and a padded row stride), so
the second runs over what the first left in the shared array.
"""

import numpy as np
import pytest
import torch

import attention_stream_verify_amd as asv
import workloads
from oracle import argmax as oargmax

pytestmark = pytest.mark.gpu


def _both(logits, rows, vocab, stride):
    pick_ws = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    flag_ws = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(16, asv.row_argmax_workspace(rows, vocab)), dtype=torch.uint8, device="cuda")
    asv.row_argmax(logits, rows, vocab, stride, pick_ws, flag_ws, ws)
    pick_na = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    flag_na = torch.full((rows,), 9, dtype=torch.uint8, device="cuda")
    asv.row_argmax_noalloc(logits, rows, vocab, stride, pick_na, flag_na)
    torch.cuda.synchronize()
    return (pick_ws.cpu().numpy(), flag_ws.cpu().numpy(), pick_na.cpu().numpy(),
            flag_na.cpu().numpy())


def test_noalloc_argmax_equals_workspace_argmax_twice():
    # first call: the 2,048-row scratch round's logits (ties, nonfinite rows)
    print("\n[no-alloc] call 1: 2,048 rows x 128,000", flush=True)
    rnd = workloads.Round(4, device="cuda", n_conv=0, n_attn=0)
    R, V = rnd.logits.shape
    p_ws, f_ws, p_na, f_na = _both(rnd.logits, R, V, V)
    assert np.array_equal(p_na, p_ws) and np.array_equal(f_na, f_ws)
    assert f_na.sum() == 8
    # second call: fewer rows, a ragged vocabulary, a padded stride
    print("[no-alloc] call 2: 37 rows x 20,001 (stride 20,008)", flush=True)
    rows, vocab, stride = 37, 20001, 20008
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((rows, stride)) * 3).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    bits[0, [5, 19999]] = 0x4300           # a tie, the lower id first
    bits[1, 8192] = 0x7FC0                  # a NaN on a chunk boundary
    bits[2, :] = 0x7FC0                     # an all-NaN row
    bits[3, vocab:] = 0x7F80                # +Inf past the vocabulary: never read
    L = torch.from_numpy(bits.view(np.int16)).cuda()
    p_ws, f_ws, p_na, f_na = _both(L, rows, vocab, stride)
    assert np.array_equal(p_na, p_ws) and np.array_equal(f_na, f_ws)
    ep, ef = oargmax.row_argmax(bits[:, :vocab])
    assert np.array_equal(p_na, ep) and np.array_equal(f_na, ef)
    assert p_na[0] == 5 and f_na[1] == 1 and p_na[2] == 0 and f_na[3] == 0


def test_noalloc_argmax_refusals():
    """Sizes past the library's array are refused before any launch."""
    L = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    pick = torch.zeros(4, dtype=torch.int32, device="cuda")
    flag = torch.zeros(4, dtype=torch.uint8, device="cuda")
    # 262,145 one-chunk rows need one record more than the 4 MiB array holds
    with pytest.raises(asv.AsvError) as e:
        asv.row_argmax_noalloc(L, 262145, 64, 64, pick, flag)
    assert e.value.code == -4
    with pytest.raises(asv.AsvError) as e:
        asv.row_argmax_noalloc(L, 2, 64, 60, pick, flag)
    assert e.value.code == -2
    asv.row_argmax_noalloc(L, 0, 64, 64, pick, flag)   # zero rows: nothing to do
