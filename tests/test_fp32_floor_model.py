"""Why the end-to-end tolerance on y needs a floor, and how large it must be.

The oracle evaluates the layer in fp64 and rounds h = silu(g) * u to FP16 at
the point the pages' FP16 activations fix ("horizonrunmap.com/en", section
"08 / Precision & quality", paragraph "Compute").  A GPU that sums in FP32
(the accumulation the pages name) in another order gets g and u a few FP32
ulps away from the fp64 values, so wherever h sits next to an FP16 rounding
midpoint the two round to neighbouring FP16 values (about one element in
300).  Each such one-ulp flip of h moves every output of that expert by
|w_down| * ulp(h), an absolute change; outputs that are small through
cancellation then see a large relative change, which no floor-free relative
bound can absorb.

This test evaluates each workload shape with plain FP32 arithmetic (numpy
float32 matrix products on the oracle's own dequantized weights: one valid
FP32 evaluation order among many) and computes the smallest floor f, as a
fraction of each token's largest |y|, for which
    |y32 - y| <= 2e-3 * max(|y|, f * max_c |y[t, c]|)
holds everywhere, over several input batches, and asserts that it stays
below parity_util.FLOOR, the floor the GPU parity tests use.  Measured here:
up to 2^-3.6 on the tiny layer (H 256, I 512: short sums, so a single flip
weighs more), 2^-4.8 .. 2^-5.2 on the OLMoE shape, 2^-6.1 on the Qwen shape
with its shared expert.  The GPU parity tests add a stage-wise check that has
no such flips (the oracle's down projection on the GPU's own h) at the
survey's 2^-8 floor, and hold h itself to one FP16 ulp.
"""
import numpy as np
import pytest

import oracle
from layer_util import oracle_tokens
from parity_util import FLOOR, REL, f16_to_f64
from w4a16_routed_expert_amd import synth


def fp32_layer(cfg, rows, x, ref, shared=None):
    """The layer in FP32 on the oracle's routing: h rounded to FP16, y to FP16."""
    k = cfg.k
    T = x.shape[0]
    y32 = np.zeros((T, cfg.H), np.float32)
    xf = f16_to_f64(x.view(np.uint16)).astype(np.float32)
    ids = ref["ids"].reshape(-1)
    w = ref["w"].reshape(-1).astype(np.float32)
    for e in np.unique(ids):
        Wg, Wu, Wd = (m.astype(np.float32) for m in oracle.dequant_expert(rows[e], cfg.H, cfg.I))
        ps = np.nonzero(ids == e)[0]
        X = xf[ps // k]
        G = X @ Wg.T
        U = X @ Wu.T
        Hh = (G / (np.float32(1) + np.exp(-G)) * U).astype(np.float16).astype(np.float32)
        O = Hh @ Wd.T
        for i, p in enumerate(ps):
            y32[p // k] += w[p] * O[i]
    if shared is not None:
        Wsg, Wsu, Wsd, wg = (f16_to_f64(np.asarray(m).view(np.uint16)).astype(np.float32) for m in shared)
        G = xf @ Wsg.T
        U = xf @ Wsu.T
        Hs = (G / (np.float32(1) + np.exp(-G)) * U).astype(np.float16).astype(np.float32)
        sig = np.float32(1) / (np.float32(1) + np.exp(-(xf @ wg)))
        y32 += sig[:, None] * (Hs @ Wsd.T)
    return y32.astype(np.float16).astype(np.float64)


def floor_needed(y_model, y_ref_bits):
    yr = f16_to_f64(y_ref_bits)
    m = np.abs(yr).max(axis=1, keepdims=True)
    d = np.abs(y_model - yr)
    need = np.maximum(d / REL - np.abs(yr), 0.0) / np.where(m > 0, m, 1.0)
    return float(need.max())


CASES = [
    # name, config, T, bias, shared, input batches
    ("tiny T=300", "tiny", 300, None, False, range(4, 12)),
    ("tiny T=300, every token on experts 5 and 2", "tiny", 300, "skew", False, range(4, 12)),
    ("OLMoE decode T=32", "olmoe", 32, None, False, range(4, 6)),
    ("OLMoE stack layer 3 (Zipf bias) T=32", "olmoe_stack", 32, "zipf", False, range(4, 5)),
    ("Qwen decode + shared expert T=64", "qwen", 64, None, True, range(4, 5)),
]


@pytest.mark.parametrize("name,cname,T,bias_kind,with_shared,steps", CASES, ids=[c[0] for c in CASES])
def test_fp32_evaluation_needs_less_than_the_floor(name, cname, T, bias_kind, with_shared, steps):
    cfg = synth.CONFIGS[cname]
    layer = 3 if bias_kind == "zipf" else 0
    rows = synth.make_expert_rows(cfg if cname != "olmoe_stack" else synth.CONFIGS["olmoe"])
    wr = synth.make_router(cfg, layer=layer)
    bias = None
    if bias_kind == "skew":
        bias = np.zeros(cfg.E, np.float32)
        bias[5], bias[2] = 50.0, 40.0
    elif bias_kind == "zipf":
        bias = synth.make_zipf_bias(cfg, layer=layer)
    shared = synth.make_shared(cfg) if with_shared else None
    worst = 0.0
    for step in steps:
        x = synth.make_x(cfg, T, step=step, layer=layer)
        ref = oracle_tokens(x, wr, rows, cfg, bias=bias, shared=shared)
        f = floor_needed(fp32_layer(cfg, rows, x, ref, shared), ref["y"])
        print(f"{name}, batch {step}: an FP32 evaluation needs a floor of {f:.3g} "
              f"(2^{np.log2(f) if f > 0 else -99:.2f})")
        worst = max(worst, f)
    assert worst <= FLOOR, f"{name}: FP32 evaluation needs floor {worst:.3g} > FLOOR = {FLOOR}"
