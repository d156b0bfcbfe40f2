"""Pins of the oracle's bf16 helpers and argmax (CPU only).

The bf16 rounding is pinned to torch's float32 -> bfloat16 cast (a library
routine, round to nearest even) where the input is a float32, to the IEEE
definition at hand-picked midpoints, and to a double-rounding trap that a
float32 detour would fail. The argmax is pinned to hand-derived golden cases
(tests/golden/argmax_cases.json), to numpy.argmax on NaN-free rows (it returns
the first maximum), and the vectorised form to the scalar definition.
"""

import json
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import argmax, bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ bf16

def test_bf16_roundtrip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = bf16.round_f64(bf16.to_f64(bits))
    nan = bf16.is_nan_bits(bits)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_matches_torch_cast_on_float32_inputs():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 3,
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),      # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),       # near overflow
        rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]
    ours = bf16.round_f64(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_to_even_by_hand():
    # bf16 step on [1, 2) is 2^-7
    assert bf16.round_f64(1 + 2**-8) == 0x3F80            # midpoint 1 | 1+2^-7 -> even (1)
    assert bf16.round_f64(1 + 3 * 2**-8) == 0x3F82        # midpoint 1+2^-7 | 1+2^-6 -> even
    assert bf16.round_f64(-(1 + 2**-8)) == 0xBF80
    assert bf16.round_f64(1 + 2**-8 + 2**-20) == 0x3F81   # above the midpoint


def test_bf16_single_rounding_not_via_float32():
    # 1 + 2^-8 + 2^-30 lies just above a midpoint; a float32 detour drops 2^-30
    # and the tie then goes to even (1.0). The correct single rounding is up.
    x = 1.0 + 2.0**-8 + 2.0**-30
    assert bf16.round_f64(x) == 0x3F81
    assert torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() == 0x3F80


def test_bf16_overflow_and_specials():
    big = (2 - 2**-7) * 2.0**127                    # largest finite bf16
    assert bf16.round_f64(big) == 0x7F7F
    assert bf16.round_f64(2.0**128 - 2.0**119) == 0x7F80     # midpoint above max -> inf (even)
    assert bf16.round_f64(2.0**128 - 2.0**119 - 2.0**100) == 0x7F7F
    assert bf16.round_f64(-np.inf) == 0xFF80
    assert bf16.round_f64(np.nan) == 0x7FC0
    assert bf16.round_f64(-0.0) == 0x8000
    assert bf16.round_f64(-1e-300) == 0x8000
    assert bf16.round_f64(2.0**-133) == 0x0001       # smallest subnormal
    assert bf16.round_f64(2.0**-134) == 0x0000       # half of it, ties to even (0)
    assert bf16.round_f64(3 * 2.0**-134) == 0x0002   # 1.5 quanta -> 2 (even)


# ---------------------------------------------------------------- argmax

def _golden_argmax():
    with open(os.path.join(GOLDEN, "argmax_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_argmax(), ids=lambda c: c["name"])
def test_argmax_golden(case):
    row = np.array([int(h, 16) for h in case["row"]], dtype=np.uint16)
    assert argmax.scan_row(row) == (case["pick"], bool(case["flag"]))
    pick, flag = argmax.row_argmax(row[None, :])
    assert (int(pick[0]), int(flag[0])) == (case["pick"], case["flag"])


def test_argmax_matches_numpy_first_max_on_finite_rows():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20, 4000)) * 3).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # plant ties: copy each row's max to a random lower position
    vals = bf16.to_f64(bits)
    for r in range(20):
        a = int(np.argmax(vals[r]))
        if a > 0:
            bits[r, rng.integers(0, a)] = bits[r, a]
    pick, flag = argmax.row_argmax(bits)
    assert np.array_equal(pick, np.argmax(bf16.to_f64(bits), axis=1))
    assert not flag.any()


def test_argmax_full_width_row_with_planted_anomalies():
    rng = np.random.default_rng(11)
    V = 128000
    x = (rng.standard_normal((3, V)) * 3).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = bf16.to_f64(bits)
    a = int(np.argmax(vals[0]))
    bits[0, V - 1] = bits[0, a]            # tie above: pick stays a
    bits[1, 5] = 0x7FC0                    # NaN row
    bits[2, 99999] = 0x7F80                # +Inf row
    pick, flag = argmax.row_argmax(bits)
    assert pick[0] == a and flag[0] == 0
    assert flag[1] == 1 and pick[1] == argmax.scan_row(bits[1])[0]
    assert pick[2] == 99999 and flag[2] == 1


_special = st.sampled_from([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x3F80, 0xBF80])


@settings(max_examples=300, deadline=None)
@given(st.lists(st.one_of(st.integers(0, 65535), _special), min_size=1, max_size=40))
def test_argmax_vectorised_equals_scalar_definition(row):
    bits = np.array(row, dtype=np.uint16)
    p, f = argmax.row_argmax(bits[None, :])
    assert (int(p[0]), bool(f[0])) == argmax.scan_row(bits)
