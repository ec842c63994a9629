"""The HIP layer, through the C ABI, against the fixtures under tests/golden/:
the closed-form worked example and the stored oracle output of the tiny layer.
Routing is compared bit for bit, h within one FP16 rounding of the stored
value, y to the parity tolerance."""
import types

import numpy as np
import pytest

from golden_util import load, oracle_fixture_arrays, worked_example_expected, worked_example_inputs
from layer_util import gpu_layer
from parity_util import assert_close_rows, f16_to_f64
from w4a16_routed_expert_amd import synth

pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _one_ulp(got_bits, want_bits):
    g, w = f16_to_f64(got_bits), f16_to_f64(want_bits)
    ulp = np.spacing(np.abs(w).astype(np.float16)).astype(np.float64)
    return np.all(np.abs(g - w) <= ulp)


def test_worked_example_on_gpu():
    d = load("worked_example.json")
    x, wr, rows = worked_example_inputs(d)
    logits, ids, w, h, y = worked_example_expected(d)
    cfg = types.SimpleNamespace(H=d["H"], I=d["I"], E=d["E"], k=d["k"])
    got = gpu_layer(cfg, rows, wr, x)
    assert np.array_equal(got["logits"].astype(np.float64), logits)
    assert np.array_equal(got["ids"], ids)
    assert np.allclose(got["w"], w, rtol=1e-6, atol=0)
    # grouped position pos holds pair sorted_pairs[pos]
    h_grouped = np.repeat(h[got["sorted_pairs"]][:, None], d["I"], axis=1)
    assert _one_ulp(got["h"].view(np.uint16), h_grouped)
    assert_close_rows(got["y"].view(np.uint16), y, "worked example y")


def test_stored_tiny_layer_on_gpu():
    d = load("oracle_tiny_T5.json")
    cfg = synth.CONFIGS[d["config"]]
    want = oracle_fixture_arrays(d)
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, d["T"])
    got = gpu_layer(cfg, rows, wr, x)
    assert np.array_equal(got["logits"].view(np.uint32), want["logits"].view(np.uint32))
    for key in ("ids", "offsets", "sorted_pairs"):
        assert np.array_equal(got[key], want[key]), key
    assert np.array_equal(got["active"][:len(want["active"])], want["active"])
    assert np.allclose(got["w"], want["w"], rtol=1e-5, atol=1e-7)
    assert_close_rows(got["h"].view(np.uint16), want["h"][want["sorted_pairs"]], "stored tiny h")
    assert_close_rows(got["y"].view(np.uint16), want["y"], "stored tiny y")
