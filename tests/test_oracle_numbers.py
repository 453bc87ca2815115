"""Pins for the oracle's number decoding (no GPU)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_matches_hand_worked_values():
    cases = json.load(open(os.path.join(GOLDEN, "bf16_values.json")))["cases"]
    bits = np.array([int(c["bits"], 16) for c in cases], dtype=np.uint16)
    got = O.decode_bf16(bits)
    for c, g in zip(cases, got):
        want = float(c["value"])
        assert (g == want) and (math.copysign(1.0, g) == math.copysign(1.0, want)), (c, g)


def test_bf16_decode_matches_torch_on_every_finite_pattern():
    # every one of the 65,536 patterns except NaNs; torch's widening is a library routine
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.decode_bf16(bits)
    finite = ~np.isnan(t)
    assert np.array_equal(mine[finite], t[finite])
    assert np.isnan(mine[~finite]).all()


def test_f32_inputs_widen_exactly():
    x = np.array([1.0, -3.5, 1e-30, 7.0e30, np.float32(0.1)], dtype=np.float32)
    assert np.array_equal(O.to_f64(x, "f32"), x.astype(np.float64))
    with pytest.raises(ValueError):
        O.to_f64(x, "f16")
