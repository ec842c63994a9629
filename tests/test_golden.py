"""The oracle against the fixtures under tests/golden/.

worked_example.json is derived in closed form (derive_worked_example.py uses
only the definitions, no oracle call), so it pins the whole layer
composition: routing order, which weight goes with which expert, the SwiGLU
rounding point, the down matrix's row-to-column mapping and the combine.
oracle_tiny_T5.json is the oracle's own output on a seeded tiny layer, kept
so that any later change to the oracle's arithmetic shows up as a diff.
"""
import numpy as np

import oracle
from golden_util import load, oracle_fixture_arrays, worked_example_expected, worked_example_inputs
from w4a16_routed_expert_amd import synth


def test_worked_example_closed_form():
    d = load("worked_example.json")
    x, wr, rows = worked_example_inputs(d)
    logits, ids, w, h, y = worked_example_expected(d)
    ref = oracle.layer(x, wr, rows, d["H"], d["I"], d["E"], d["k"], want_h=True)
    assert np.array_equal(ref["logits"].astype(np.float64), logits)
    assert np.array_equal(ref["ids"], ids)
    assert np.allclose(ref["w"], w, rtol=4e-16, atol=0)
    # h is one value per pair across all I rows
    assert np.array_equal(ref["h"], np.repeat(h[:, None], d["I"], axis=1))
    assert np.array_equal(ref["y"], y)


def test_worked_example_is_not_degenerate():
    # Distinct experts per token, both signs in y, and a zero column class
    # (down code 8) so that a swapped or shifted column mapping is visible.
    d = load("worked_example.json")
    _, ids, w, _, y = worked_example_expected(d)
    assert len({tuple(r) for r in ids}) == 2 and np.all(w[:, 0] > w[:, 1])
    yv = y.view(np.float16).astype(np.float64)
    assert (yv > 0).any() and (yv < 0).any()
    assert np.all(yv[:, 8::16] == 0) and np.all(yv[:, 9::16] != 0)


def test_oracle_reproduces_stored_tiny_layer():
    d = load("oracle_tiny_T5.json")
    cfg = synth.CONFIGS[d["config"]]
    T = d["T"]
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    want = oracle_fixture_arrays(d)
    assert np.array_equal(ref["logits"].view(np.uint32), want["logits"].view(np.uint32))
    for key in ("ids", "offsets", "sorted_pairs", "active", "h", "y"):
        assert np.array_equal(ref[key], want[key]), key
    assert np.array_equal(ref["w"], want["w"])
