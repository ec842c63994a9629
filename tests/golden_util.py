"""Loads the fixtures under tests/golden/ and builds the worked example's
inputs (qpacked expert rows, router, activations) from its description."""
import json
import os

import numpy as np

from w4a16_routed_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def worked_example_inputs(d):
    """(x [T,H] FP16, W_r [H,E] FP16, rows uint8 [E,row_bytes]) of worked_example.json."""
    H, I, E = d["H"], d["I"], d["E"]
    x = np.array([[v] * H for v in d["x_per_token"]], np.float16)
    wr = np.tile(np.array(d["router_column"], np.float16), (H, 1))
    rows = []
    for ex in d["experts"]:
        gate = (np.full((I, H), ex["gate_code"], np.uint8), np.full((I, synth.n_blocks(H)), ex["gate_scale"], np.float16))
        up = (np.full((I, H), ex["up_code"], np.uint8), np.full((I, synth.n_blocks(H)), ex["up_scale"], np.float16))
        down_codes = np.repeat((np.arange(H) % 16).astype(np.uint8)[:, None], I, axis=1)
        down = (down_codes, np.full((H, synth.n_blocks(I)), ex["down_scale"], np.float16))
        rows.append(synth.pack_expert_row(H, I, gate, up, down))
    return x, wr, np.stack(rows)


def worked_example_expected(d):
    """Expected logits [T,E] float64, ids [T,k], weights [T,k], h bits [T*k]
    (one value per pair, pair p = t*k + j), y bits [T,H]."""
    H = d["H"]
    toks = d["tokens"]
    logits = np.array([t["logits"] for t in toks])
    ids = np.array([t["ids"] for t in toks], np.int32)
    w = np.array([t["weights"] for t in toks])
    h = np.array([p["h_bits"] for t in toks for p in t["pairs"]], np.uint16)
    y = np.array([[t["y_bits_by_col_mod16"][c % 16] for c in range(H)] for t in toks], np.uint16)
    return logits, ids, w, h, y


def oracle_fixture_arrays(d):
    """Arrays of oracle_tiny_T5.json in the oracle's own dtypes."""
    return dict(
        logits=np.array(d["logits_f32_bits"], np.uint32).view(np.float32),
        ids=np.array(d["ids"], np.int32),
        w=np.array(d["weights"]),
        offsets=np.array(d["offsets"], np.int32),
        sorted_pairs=np.array(d["sorted_pairs"], np.int32),
        active=np.array(d["active"], np.int32),
        h=np.stack([np.frombuffer(bytes.fromhex(r), np.uint16) for r in d["h_f16_hex"]]),
        y=np.stack([np.frombuffer(bytes.fromhex(r), np.uint16) for r in d["y_f16_hex"]]),
    )
