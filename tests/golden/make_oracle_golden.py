"""Writes oracle_tiny_T5.json: the oracle's routing, grouping and layer output
for five tokens of the seeded tiny layer (8 experts, top-2, H = 256, I = 512).

The values come from `oracle/` alone, on inputs from the seeded generators of
`w4a16_routed_expert_amd.synth`.  The CPU tests re-run the oracle and require
the same bits (a change to the oracle's arithmetic shows up here and has to be
justified from the pages); the GPU tests hold the HIP path to them.

Run from the repository root:  python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from w4a16_routed_expert_amd import synth  # noqa: E402

T = 5


def main():
    cfg = synth.CONFIGS["tiny"]
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    fixture = dict(
        description="oracle.layer on the tiny layer (synth config 'tiny', layer 0, step 0), T = 5",
        config="tiny", T=T,
        logits_f32_bits=ref["logits"].view("u4").tolist(),
        ids=ref["ids"].tolist(),
        weights=ref["w"].tolist(),
        offsets=ref["offsets"].tolist(),
        sorted_pairs=ref["sorted_pairs"].tolist(),
        active=ref["active"].tolist(),
        h_f16_hex=[r.tobytes().hex() for r in ref["h"]],
        y_f16_hex=[r.tobytes().hex() for r in ref["y"]],
    )
    out = os.path.join(HERE, "oracle_tiny_T5.json")
    with open(out, "w") as f:
        json.dump(fixture, f, indent=0)
        f.write("\n")
    print(out)


if __name__ == "__main__":
    main()
