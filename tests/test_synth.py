"""The seeded input generators: bf16 workloads draw fp32 values and round
them to the nearest bf16 number, ties to even (checked against torch's cast,
a library routine), and every draw is reproducible from its seed alone."""

import numpy as np
import pytest

import synth


def test_bf16_activations_are_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    w = synth.get_workload("decode")
    rng = synth.workloads._rng(w, synth.workloads._S_ACT, 3)
    raw = rng.standard_normal((8, w.hidden), dtype=np.float32)
    got = synth.draw_activations(w, 3, 8)["x_qkv"]
    want = torch.from_numpy(raw).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # every value is a bf16 number, so the bit extraction accepts it
    assert synth.bf16_bits(got).dtype == np.uint16


def test_bf16_rounding_ties_go_to_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20],
                    np.float32)
    got = synth.workloads._to_dtype_values(vals, "bf16")
    assert got.tolist() == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]
    assert synth.workloads._to_dtype_values(vals, "f32") is vals


def test_draws_are_reproducible():
    w = synth.get_workload("tiny")
    a = synth.draw_activations(w, 0, 12)
    b = synth.draw_activations(w, 0, 12)
    for k in a:
        assert np.array_equal(a[k], b[k])
