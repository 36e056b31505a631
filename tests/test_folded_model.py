"""CPU checks of the test suite's model of the bf16 merge arithmetic (tests/helpers.py,
folded_gate_model) against the oracle: the model may differ from the exact method
only by rounding the folded coefficient times B to bf16."""
import numpy as np
import torch

from helpers import folded_bound, folded_gate_model, to64
from oracle import adafuse as O
from weight_merge_amd import synth


def test_unit_coefficient_is_the_exact_merge():
    # s * g = 1: c B is B itself, already bf16, so the model is the exact fp64 merge
    W, Aw, Bw = synth.adapter_bank(3, 4, 8, 24, 40, "bf16")
    x, _ = folded_gate_model(W, Aw, Bw, [(2, 0.5, 2.0)])
    ref = O.merge(to64(W), to64(Aw), to64(Bw), np.array([2]), np.array([0.5]), 2.0)
    assert np.allclose(x, ref, rtol=1e-13, atol=1e-15)


def test_folding_error_is_within_its_bound_and_present():
    W, Aw, Bw = synth.adapter_bank(5, 6, 16, 32, 48, "bf16")
    idx, gate = np.array([4, 1, 3]), np.array([0.45, 0.33, 0.22])
    slots = [(int(e), float(np.float32(g)), 2.0) for e, g in zip(idx, gate)]
    g32 = np.array([s[1] for s in slots])
    x, mag = folded_gate_model(W, Aw, Bw, slots)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx, g32, 2.0)
    err = np.abs(x - ref)
    assert np.all(err <= folded_bound(Aw, Bw, idx, g32, 2.0))
    assert err.max() > 0.0  # c B was rounded: the model is not the exact method
    assert np.all(mag >= np.abs(to64(W)))


def test_negated_coefficients_undo_the_merge_in_the_model():
    W, Aw, Bw = synth.adapter_bank(9, 4, 8, 16, 24, "bf16")
    slots = [(1, 0.6, 2.0), (3, 0.4, 2.0)]
    x, _ = folded_gate_model(W, Aw, Bw, slots + [(e, g, -s) for e, g, s in slots])
    assert np.allclose(x, to64(W), rtol=0, atol=1e-12)
    assert isinstance(W, torch.Tensor)
