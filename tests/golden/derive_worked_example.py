"""Writes worked_example.json: a routed-expert layer small enough to follow by
hand, with every expected value derived in closed form from the definitions
(no call into the oracle or the HIP library).

Definitions followed ("Horizon RunMap - architecture", "Representation and
computation"; "horizonrunmap.com/en", "08 / Precision & quality", "06 / Follow
a token"):
  weight       = (code - 8) * FP16 block scale           (INT4, 256-value blocks)
  logit[e]     = sum_h x[h] * W_r[h, e]                   (exact, then FP32)
  ids          = the k largest logits, ties to the lower expert index
  p_j          = softmax over the k chosen logits
  g, u         = W_gate x, W_up x;   h = RN16(silu(g) * u),  silu(g) = g / (1 + e^-g)
  o            = W_down h
  y            = RN16(sum_j p_j o_j)

The inputs are built so that every sum collapses to a product:
  * each token's x is one constant v_t across all H columns;
  * W_r column e is the constant r_e, so logit[e] = H * v_t * r_e;
  * an expert's gate and up matrices are constant (one code, one scale), so
    g = H * v * a and u = H * v * b for every intermediate row, and h is one
    FP16 value per (token, expert);
  * the down matrix row c holds code (c mod 16) in every column with one scale
    s_d, so o[c] = I * (c mod 16 - 8) * s_d * h -- the output pins that row c
    of the down matrix lands in output column c.
Every product and sum above is exact in binary64 (small integers times powers
of two), so the only roundings are the ones the definitions name.  Sums start
from +0, so a sum of zero terms (down code 8) is +0, never -0.

Run from the repository root:  python tests/golden/derive_worked_example.py
"""
import json
import math
import os
import struct

H, I, E, K = 256, 128, 4, 2
X = [1.0, -0.5]                                 # token t: x[t, :] = X[t]
ROUTER = [1 * 2.0 ** -8, 3 * 2.0 ** -8, 2 * 2.0 ** -8, 0.0]   # W_r[:, e] = ROUTER[e]
# expert e: (gate code, gate scale, up code, up scale, down scale); down codes = row mod 16
EXPERTS = [
    (10, 2.0 ** -9, 4, 2.0 ** -8, 2.0 ** -10),
    (5, 2.0 ** -8, 11, 2.0 ** -9, 3 * 2.0 ** -11),
    (15, 2.0 ** -8, 7, 2.0 ** -7, 2.0 ** -9),
    (0, 2.0 ** -10, 14, 2.0 ** -10, 5 * 2.0 ** -12),
]


def f16_bits(v: float) -> int:
    """Round-to-nearest-even binary16 bit pattern of a binary64 value."""
    return struct.unpack("<H", struct.pack("<e", v))[0]


def f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def main():
    tokens = []
    for t, v in enumerate(X):
        logits = [f32(H * v * r) + 0.0 for r in ROUTER]      # + 0.0: an exact zero sum is +0
        order = sorted(range(E), key=lambda e: (-logits[e], e))
        ids = order[:K]
        top = logits[ids[0]]
        den = sum(math.exp(logits[e] - top) for e in ids)
        p = [math.exp(logits[e] - top) / den for e in ids]
        pairs, o_cols = [], []
        for e in ids:
            gc, gs, uc, us, ds = EXPERTS[e]
            g = H * v * (gc - 8) * gs
            u = H * v * (uc - 8) * us
            h_bits = f16_bits(g / (1.0 + math.exp(-g)) * u)
            h = f16_value(h_bits)
            # output column c uses o[c % 16]; sums start from +0, so a zero sum is +0
            o = [0.0 + I * (m - 8) * ds * h for m in range(16)]
            pairs.append(dict(expert=e, g=g, u=u, h_bits=h_bits, h=h, o_by_col_mod16=o))
            o_cols.append(o)
        y_bits = [f16_bits(0.0 + p[0] * o_cols[0][m] + p[1] * o_cols[1][m]) for m in range(16)]
        tokens.append(dict(x=v, logits=logits, ids=ids, weights=p, pairs=pairs, y_bits_by_col_mod16=y_bits))
    fixture = dict(
        description="Hand-derivable routed-expert layer; see derive_worked_example.py for the derivation.",
        H=H, I=I, E=E, k=K, x_per_token=X, router_column=ROUTER,
        experts=[dict(gate_code=a, gate_scale=b, up_code=c, up_scale=d, down_scale=s, down_code="row mod 16")
                 for a, b, c, d, s in EXPERTS],
        tokens=tokens)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example.json")
    with open(out, "w") as f:
        json.dump(fixture, f, indent=1)
        f.write("\n")
    print(out)


if __name__ == "__main__":
    main()
