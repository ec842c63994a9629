"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with a closed form, a hand-worked value,
an exact-rational brute force, or a library routine (numpy / scipy), chosen so
that a dropped term, a wrong sign, a swapped nibble or a transposed operand in
the oracle fails at least one of them.  CPU only.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.special

import oracle
from w4a16_routed_expert_amd import synth


# ------------------------------------------------------------------ helpers
def f16(vals):
    return np.asarray(vals, dtype=np.float16)


def frac_of_f16(h) -> Fraction:
    return Fraction(float(np.float16(h)))          # fp16 -> float64 is exact


def rn32_fraction(F: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational, ties to even (independent of the oracle)."""
    if F == 0:
        return np.float32(0.0)
    c = np.float32(float(F))                         # within one fp32 ulp of F
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for v in cands:
        d = abs(Fraction(float(v)) - F)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(v).view(np.uint32)) & 1) == 0):
            best = (d, v)
    return np.float32(best[1])


def dense_from_codes(codes, scales):
    """Dequantized weights straight from the quantizer's codes/scales (no qpacked bytes)."""
    R, K = codes.shape
    s = scales.astype(np.float64)
    cols = np.arange(K) // 256
    return (codes.astype(np.float64) - 8.0) * s[:, cols]


def np_silu(g):
    return g / (1.0 + np.exp(-g))


def f16_ulps_apart(a_bits, b_bits):
    """Distance in FP16 units-in-last-place between finite FP16 bit patterns."""
    def key(b):
        b = np.asarray(b, dtype=np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


# -------------------------------------------------------------- FP16 codec
def test_half_to_double_matches_numpy_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.half_to_double(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isinf(got[np.isinf(ref)]))


def test_double_to_half_matches_numpy_round_to_nearest_even():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.integers(-9, 6, 20000),
        # exact midpoints between neighbouring FP16 values (ties go to even)
        (np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -3,
        [0.0, -0.0, 65504.0, 65519.99, 6.1e-5, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26],
    ])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = oracle.double_to_half(v)
    assert np.array_equal(got, ref)
    assert oracle.double_to_half(np.array([65520.0]))[0] == 0x7C00      # rounds to +inf
    assert oracle.double_to_half(np.array([2.0 ** -25]))[0] == 0x0000   # tie -> even (zero)
    assert oracle.double_to_half(np.array([3 * 2.0 ** -25]))[0] == 0x0002


# ------------------------------------------------------- qpacked v1 layout
def _one_matrix(R, K, codes, scales):
    return synth.pack_nibbles(codes), synth.pack_scales(scales)


def test_all_eight_codes_are_zero_weights():
    R, K = 32, 512
    codes = np.full((R, K), 8, np.uint8)
    scales = np.full((R, 2), 1.5, np.float16)
    nib, sc = _one_matrix(R, K, codes, scales)
    assert not np.any(oracle.dequant_matrix(nib, sc, R, K))


def test_ramp_codes_give_minus8_to_7():
    R, K = 16, 256
    codes = (np.arange(K)[None, :] % 16).repeat(R, 0).astype(np.uint8)
    scales = np.ones((R, 1), np.float16)
    nib, sc = _one_matrix(R, K, codes, scales)
    W = oracle.dequant_matrix(nib, sc, R, K)
    assert np.array_equal(W, np.tile((np.arange(K) % 16) - 8.0, (R, 1)))


def test_hand_placed_nibble_is_read_at_the_documented_position():
    # Worked by hand from the qpacked v1 description: a 32 x 256 matrix has
    # K/128 = 2 tiles per row group.  Row 17, column 200 -> row group 1, r 1,
    # tile column 1, chunk group g = (200-128)//32 = 2, offset 8 inside the
    # chunk -> tile 1*2+1 = 3, chunk 16*2+1 = 33, byte 3*1024 + 33*16 + 4 = 3604,
    # low nibble (even column).  Column 201 is the high nibble of that byte.
    R, K = 32, 256
    nib = np.full(R * K // 2, 0x88, np.uint8)
    sc = np.ones(R * 1, np.float16)
    nib[3604] = 0x8F
    W = oracle.dequant_matrix(nib, sc, R, K)
    assert W[17, 200] == 7.0 and np.count_nonzero(W) == 1
    nib[3604] = 0x08
    W = oracle.dequant_matrix(nib, sc, R, K)
    assert W[17, 201] == -8.0 and W[17, 200] == 0.0 and np.count_nonzero(W) == 1
    # scale of row 17, block 0: element (rg*nb + b)*16 + r = (1*1+0)*16 + 1 = 17
    sc2 = np.ones(R, np.float16)
    sc2[17] = np.float16(0.25)
    W = oracle.dequant_matrix(nib, sc2, R, K)
    assert W[17, 201] == -2.0


@pytest.mark.parametrize("s,expect", [(2.0 ** -24, 7 * 2.0 ** -24), (2.0 ** -14, 7 * 2.0 ** -14),
                                      (65504.0, 458528.0)])
def test_extreme_scales_are_exact(s, expect):
    R, K = 16, 256
    codes = np.full((R, K), 15, np.uint8)
    scales = np.full((R, 1), s, np.float16)
    nib, sc = _one_matrix(R, K, codes, scales)
    W = oracle.dequant_matrix(nib, sc, R, K)
    assert np.all(W == expect)          # 7 * 65504 overflows FP16; the oracle keeps it exact


def test_short_last_block_has_its_own_scale():
    R, K = 16, 1408                     # 5 full 256-blocks + one 128-wide block
    codes = np.full((R, K), 9, np.uint8)
    scales = np.ones((R, 6), np.float16)
    scales[:, 5] = np.float16(3.0)
    nib, sc = _one_matrix(R, K, codes, scales)
    W = oracle.dequant_matrix(nib, sc, R, K)
    assert np.all(W[:, :1280] == 1.0) and np.all(W[:, 1280:] == 3.0)


def test_packer_and_oracle_agree_on_random_codes():
    # The packer (numpy reshapes) and the oracle reader (scalar address
    # arithmetic) are two independent implementations of the same layout.
    g = np.random.default_rng(3)
    R, K = 48, 384
    codes = g.integers(0, 16, (R, K)).astype(np.uint8)
    scales = (g.random((R, 2)) + 0.5).astype(np.float16)
    nib, sc = _one_matrix(R, K, codes, scales)
    assert np.array_equal(oracle.dequant_matrix(nib, sc, R, K), dense_from_codes(codes, scales))


def test_quantizer_error_bound_and_fixed_point():
    g = np.random.default_rng(11)
    R, K = 32, 1408
    w = (g.standard_normal((R, K)) * 0.02).astype(np.float32)
    codes, scales = synth.quantize_q4(w)
    nib, sc = _one_matrix(R, K, codes, scales)
    W = oracle.dequant_matrix(nib, sc, R, K)
    s = scales.astype(np.float64)[:, np.arange(K) // 256]
    assert np.all(codes >= 1) and np.all(codes <= 15)
    # |w - w_hat| <= s/2, plus the slack from rounding the scale to FP16
    assert np.all(np.abs(w - W) <= s * (0.5 + 7 * 2.0 ** -11) + 1e-12)
    # requantizing the dequantized weights reproduces the same codes and scales
    c2, s2 = synth.quantize_q4(W.astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2.view(np.uint16), scales.view(np.uint16))


def test_expert_row_offsets_agree_with_packer():
    for H, I in ((256, 512), (2048, 1024), (2048, 1408)):
        assert oracle.row_offsets(H, I) == synth.expert_row_layout(H, I)
    assert synth.expert_row_layout(2048, 1024)["row_bytes"] == 3_194_880
    assert synth.expert_row_layout(2048, 1408)["row_bytes"] == 4_395_008


# ------------------------------------------------------------ router logits
def _exact_logit(x_row, w_col) -> Fraction:
    return sum((frac_of_f16(a) * frac_of_f16(b) for a, b in zip(x_row, w_col)), Fraction(0))


def test_router_logits_equal_exact_rational_brute_force():
    g = np.random.default_rng(5)
    T, H, E = 3, 48, 5
    x = (g.standard_normal((T, H)) * 10.0 ** g.integers(-6, 3, (T, H))).astype(np.float16)
    wr = (g.standard_normal((H, E)) * 10.0 ** g.integers(-7, 4, (H, E))).astype(np.float16)
    x[0, :4] = f16([2.0 ** -24, -2.0 ** -24, 65504.0, -6.0e-8])       # subnormals and the max value
    got = oracle.router_logits(x, wr)
    for t in range(T):
        for e in range(E):
            assert got[t, e] == rn32_fraction(_exact_logit(x[t], wr[:, e]))


def test_router_logits_closed_forms():
    # exact cancellation: 65504 + 2^-24 - 65504 = 2^-24 (a sequential FP32 sum gives 0)
    x = f16([[1.0, 1.0, 1.0]])
    wr = f16([[65504.0], [2.0 ** -24], [-65504.0]])
    assert oracle.router_logits(x, wr)[0, 0] == np.float32(2.0 ** -24)
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2 -> even (2^24); 2^24 + 3 -> 2^24 + 4
    x = f16([[4096.0, 1.0], [4096.0, 3.0]])
    wr = f16([[4096.0], [1.0]])
    out = oracle.router_logits(x, wr)
    assert out[0, 0] == np.float32(2.0 ** 24) and out[1, 0] == np.float32(2.0 ** 24 + 4)
    # zero router -> zero logits; one-hot token -> that router row, exactly
    g = np.random.default_rng(1)
    wr = (g.standard_normal((64, 6)) * 0.02).astype(np.float16)
    assert not np.any(oracle.router_logits(g.standard_normal((2, 64)).astype(np.float16), np.zeros_like(wr)))
    xo = np.zeros((1, 64), np.float16); xo[0, 17] = 1.0
    assert np.array_equal(oracle.router_logits(xo, wr)[0], wr[17].astype(np.float32))
    # bias is one FP32 add after rounding
    b = np.float32([0.5, -1.0, 0, 0, 0, 3.25])
    assert np.array_equal(oracle.router_logits(xo, wr, b)[0], wr[17].astype(np.float32) + b)


# ------------------------------------------------------- top-k and softmax
def test_topk_matches_a_full_sort_with_ties_to_lower_index():
    g = np.random.default_rng(9)
    T, E, k = 200, 64, 8
    l = (g.integers(-20, 20, (T, E)) / 8.0).astype(np.float32)       # many exact ties
    ids, w = oracle.topk_softmax(l, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))
        assert list(ids[t]) == order[:k]
        assert float(l[t, order[k - 1]]) >= max(float(l[t, e]) for e in order[k:])
        assert np.allclose(w[t], scipy.special.softmax(l[t, ids[t]].astype(np.float64)), rtol=1e-14, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-15


def test_zero_logits_pick_first_k_with_equal_weights():
    for E, k in ((8, 2), (60, 4), (64, 8)):
        ids, w = oracle.topk_softmax(np.zeros((3, E), np.float32), k)
        assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))
        assert np.all(w == 1.0 / k)


# ---------------------------------------------------------------- grouping
def test_grouping_equals_stable_sort_brute_force():
    g = np.random.default_rng(2)
    for T, E, k in ((1, 64, 8), (7, 8, 2), (33, 60, 4), (64, 64, 8)):
        ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        if T > 3:
            ids[: T // 2] = ids[0]                 # skew: many tokens on the same experts
        gr = oracle.group(ids, E)
        pairs = sorted(range(T * k), key=lambda p: (int(ids.flat[p]), p))
        assert list(gr["sorted_pairs"]) == pairs
        cnt = np.bincount(ids.reshape(-1), minlength=E)
        assert np.array_equal(gr["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
        assert np.array_equal(gr["pair_pos"][gr["sorted_pairs"]], np.arange(T * k))
        assert list(gr["active"]) == [e for e in range(E) if cnt[e] > 0]


# -------------------------------------------------------------- expert FFN
def _tiny_expert(H, I, seed):
    g = np.random.default_rng(seed)
    mats = []
    for R, K in ((I, H), (I, H), (H, I)):
        mats.append(synth.quantize_q4((g.standard_normal((R, K)) * 0.05).astype(np.float32)))
    return mats


def test_single_expert_layer_is_a_textbook_swiglu():
    # E = 1, k = 1: routing is trivial (w = 1) and the layer reduces to
    # y = fp16(Wd fp16(silu(Wg x) * (Wu x))) with weights (code-8)*scale.
    H, I, T = 256, 384, 5
    (gc, gs), (uc, us), (dc, ds) = _tiny_expert(H, I, 21)
    row = synth.pack_expert_row(H, I, (gc, gs), (uc, us), (dc, ds))[None, :]
    x = np.random.default_rng(4).standard_normal((T, H)).astype(np.float16)
    wr = np.ones((H, 1), np.float16)
    out = oracle.layer(x, wr, row, H, I, E=1, k=1, want_h=True)
    Wg, Wu, Wd = dense_from_codes(gc, gs), dense_from_codes(uc, us), dense_from_codes(dc, ds)
    xd = x.astype(np.float64)
    h_ref = (np_silu(xd @ Wg.T) * (xd @ Wu.T)).astype(np.float16)
    y_ref = (h_ref.astype(np.float64) @ Wd.T).astype(np.float16)
    assert np.all(out["w"] == 1.0) and np.all(out["ids"] == 0)
    # identical up to the summation order of fp64 (BLAS vs sequential): at most 1 FP16 ulp
    assert f16_ulps_apart(out["h"], h_ref.view(np.uint16)).max() <= 1
    assert f16_ulps_apart(out["y"], y_ref.view(np.uint16)).max() <= 1
    assert np.mean(out["y"] == y_ref.view(np.uint16)) > 0.99


def test_closed_form_constant_expert():
    # Every gate weight a, up weight b, down weight c, and x = 1:
    # g = H a, u = H b, h = fp16(silu(H a) H b), o = I c h, y = fp16(o) (k = 1).
    H, I = 256, 128
    a, b, c = 2.0 ** -6, -3 * 2.0 ** -7, 5 * 2.0 ** -9          # codes 9, 5, 13 with scales below
    def mat(R, K, code, s):
        return np.full((R, K), code, np.uint8), np.full((R, (K + 255) // 256), s, np.float16)
    row = synth.pack_expert_row(H, I, mat(I, H, 9, a), mat(I, H, 5, -b / 3), mat(H, I, 13, c / 5))[None]
    x = np.ones((1, H), np.float16)
    out = oracle.layer(x, np.ones((H, 1), np.float16), row, H, I, E=1, k=1, want_h=True)
    g, u = H * a, H * b
    h = float(np.float16(g / (1 + math.exp(-g)) * u))
    assert np.all(out["h"] == np.float16(h).view(np.uint16))
    assert np.all(out["o"] == I * c * h)
    assert np.all(out["y"] == np.float16(I * c * h).view(np.uint16))


def _tiny_layer(E, k, H, I, T, seed, identical=False):
    g = np.random.default_rng(seed)
    rows = []
    for e in range(E):
        mats = _tiny_expert(H, I, seed * 100 + (0 if identical else e))
        rows.append((synth.pack_expert_row(H, I, *mats), mats))
    x = g.standard_normal((T, H)).astype(np.float16)
    wr = (g.standard_normal((H, E)) * 0.05).astype(np.float16)
    return x, wr, rows


def test_layer_equals_dense_masked_brute_force():
    # All experts on all tokens with numpy fp64 matmuls, then the routing mask.
    E, k, H, I, T = 8, 2, 256, 256, 6
    x, wr, rows = _tiny_layer(E, k, H, I, T, seed=8)
    packed = np.stack([r for r, _ in rows])
    out = oracle.layer(x, wr, packed, H, I, E, k)
    xd = x.astype(np.float64)
    o_all = []
    for _, ((gc, gs), (uc, us), (dc, ds)) in rows:
        Wg, Wu, Wd = dense_from_codes(gc, gs), dense_from_codes(uc, us), dense_from_codes(dc, ds)
        h = (np_silu(xd @ Wg.T) * (xd @ Wu.T)).astype(np.float16).astype(np.float64)
        o_all.append(h @ Wd.T)
    o_all = np.stack(o_all)                                   # [E, T, H]
    logits = np.array([[float(rn32_fraction(_exact_logit(x[t], wr[:, e]))) for e in range(E)] for t in range(T)])
    y_ref = np.zeros((T, H))
    for t in range(T):
        sel = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        p = scipy.special.softmax(logits[t, sel])
        y_ref[t] = sum(p[j] * o_all[sel[j], t] for j in range(k))
        assert list(out["ids"][t]) == sel
    y_ref16 = y_ref.astype(np.float16).view(np.uint16)
    assert f16_ulps_apart(out["y"], y_ref16).max() <= 1
    assert np.mean(out["y"] == y_ref16) > 0.98


def test_identical_experts_make_routing_irrelevant():
    E, k, H, I, T = 8, 2, 256, 128, 4
    x, wr, rows = _tiny_layer(E, k, H, I, T, seed=3, identical=True)
    packed = np.stack([r for r, _ in rows])
    y_routed = oracle.layer(x, wr, packed, H, I, E, k)["y"]
    y_single = oracle.layer(x, np.ones((H, 1), np.float16), packed[:1], H, I, 1, 1)["y"]
    assert f16_ulps_apart(y_routed, y_single).max() <= 1          # sum of weights is 1
    assert np.mean(y_routed == y_single) > 0.99


def test_doubling_down_scales_doubles_the_output_exactly():
    E, k, H, I, T = 4, 2, 256, 256, 3
    x, wr, rows = _tiny_layer(E, k, H, I, T, seed=12)
    packed = np.stack([r for r, _ in rows])
    lay = synth.expert_row_layout(H, I)
    doubled = packed.copy()
    s = doubled[:, lay["down_s"]:lay["down_s"] + H * (I // 256) * 2].copy().view(np.float16)
    doubled[:, lay["down_s"]:lay["down_s"] + s.size * 2] = (s.astype(np.float32) * 2).astype(np.float16).view(np.uint8)
    a = oracle.layer(x, wr, packed, H, I, E, k)
    b = oracle.layer(x, wr, doubled, H, I, E, k)
    assert np.array_equal(b["o"], 2 * a["o"])
    ya = a["y"].view(np.float16).astype(np.float64)
    assert np.array_equal(b["y"].view(np.float16).astype(np.float64), 2 * ya)


def test_batch_invariance():
    E, k, H, I, T = 8, 2, 256, 128, 5
    x, wr, rows = _tiny_layer(E, k, H, I, T, seed=6)
    packed = np.stack([r for r, _ in rows])
    y = oracle.layer(x, wr, packed, H, I, E, k)["y"]
    for t in range(T):
        assert np.array_equal(oracle.layer(x[t:t + 1], wr, packed, H, I, E, k)["y"][0], y[t])


# ------------------------------------------------------------ shared expert
def test_tile8_packer_places_values_at_the_documented_positions():
    # The shared expert's kernels read its matrices in the tile8 layout; the
    # oracle reads them row-major, so the packer is the only link between the
    # two.  A hand-computed position: R = 16, K = 256 (two 128-column tiles
    # per row group), W[9][161]: 8-row tile r8 = 1, row r = 1; column 161 =
    # 128 + 32*1 + 8*0 + 1, so kt = 1, piece s = 1, g = 0, c = 1; flat index
    # ((r8 * 2 + kt) * 4 + s) * 256 + (8 g + r) * 8 + c = 13 * 256 + 9.
    w = np.zeros((16, 256), np.float16)
    w[9, 161] = 1.0
    p = synth.pack_fp16_tile8(w)
    assert np.flatnonzero(p).tolist() == [13 * 256 + 9]
    # every position, by the documented index formula written as loops
    R, K = 24, 384
    w = (np.arange(R * K) % 2039).astype(np.float16).reshape(R, K)          # integers, exact in FP16
    p = synth.pack_fp16_tile8(w)
    NT = K // 128
    for r8 in range(R // 8):
        for kt in range(NT):
            for s_ in range(4):
                for g in range(4):
                    for r in range(8):
                        for c in range(8):
                            idx = ((r8 * NT + kt) * 4 + s_) * 256 + (8 * g + r) * 8 + c
                            assert p[idx] == w[8 * r8 + r, 128 * kt + 32 * s_ + 8 * g + c]
    # a permutation: nothing lost or duplicated
    assert np.array_equal(np.sort(p), np.sort(w.reshape(-1)))


def test_shared_expert_matches_numpy():
    g = np.random.default_rng(31)
    T, H, Is = 3, 128, 96
    x = g.standard_normal((T, H)).astype(np.float16)
    Wsg, Wsu = [(g.standard_normal((Is, H)) * 0.05).astype(np.float16) for _ in range(2)]
    Wsd = (g.standard_normal((H, Is)) * 0.05).astype(np.float16)
    wgate = (g.standard_normal(H) * 0.05).astype(np.float16)
    os_, sig = oracle.shared_ffn(x, Wsg, Wsu, Wsd, wgate)
    xd = x.astype(np.float64)
    h = (np_silu(xd @ Wsg.astype(np.float64).T) * (xd @ Wsu.astype(np.float64).T)).astype(np.float16)
    ref = h.astype(np.float64) @ Wsd.astype(np.float64).T
    assert np.allclose(os_, ref, rtol=2e-3, atol=1e-3 * np.abs(ref).max())
    assert np.allclose(sig, scipy.special.expit(xd @ wgate.astype(np.float64)), rtol=1e-14)


# ------------------------------------------------------------------ combine
def test_combine_closed_form():
    o = np.array([[1.0, -2.0, 4.0], [3.0, 2.0, 0.5]])          # pairs (0,0), (0,1)
    w = np.array([[0.25, 0.75]])
    y = oracle.combine(o, w)
    assert np.array_equal(y.view(np.float16).astype(np.float64), [[2.5, 1.0, 1.375]])
    os_ = np.array([[8.0, 8.0, 8.0]]); sig = np.array([0.5])
    y = oracle.combine(o, w, os_, sig)
    assert np.array_equal(y.view(np.float16).astype(np.float64), [[6.5, 5.0, 5.375]])


# ----------------------------------------------- offload-qpacked profile (FP16 execution slots)
def test_fp16_slot_weights_are_the_nearest_fp16_values():
    # Every weight of the FP16-slot profile is (code - 8) * scale rounded to the
    # nearest FP16 value, ties to even (numpy's float16 conversion, an
    # independent implementation of that rounding); scales that leave values
    # between FP16 neighbours, and large and subnormal results, included.
    H, I = 256, 256
    g = np.random.default_rng(21)
    mats = []
    for R, K in ((I, H), (I, H), (H, I)):
        codes = g.integers(0, 16, size=(R, K)).astype(np.uint8)
        scales = (g.random((R, (K + 255) // 256)) * 0.05).astype(np.float16)
        scales[0, 0] = np.float16(65504.0)           # 7 * 65504 overflows FP16 -> inf
        scales[1, 0] = np.float16(2.0 ** -24)        # results deep in the subnormal range
        scales[2, 0] = np.float16(0.0123)
        mats.append((codes, scales))
    row = synth.pack_expert_row(H, I, *mats)
    exact = oracle.dequant_expert(row, H, I)
    slots = oracle.dequant_expert(row, H, I, fp16=True)
    for e, s in zip(exact, slots):
        with np.errstate(over="ignore"):
            want = e.astype(np.float16).astype(np.float64)
        assert np.array_equal(np.isinf(want), np.isinf(s))
        fin = np.isfinite(want)
        assert np.array_equal(s[fin], want[fin])
    # the rounding changes something, so the profile is not silently the exact one
    assert any(not np.array_equal(e, s) for e, s in zip(exact, slots))


def test_fp16_slot_layer_equals_the_exact_layer_when_weights_are_fp16_values():
    # With power-of-two scales every (code - 8) * scale is an FP16 value, so
    # the offload-qpacked layer and the exact layer agree bit for bit; with
    # ordinary scales they differ.
    E, k, H, I, T = 4, 2, 256, 256, 5
    g = np.random.default_rng(22)
    rows = []
    for e in range(E):
        mats = []
        for R, K in ((I, H), (I, H), (H, I)):
            codes = g.integers(1, 16, size=(R, K)).astype(np.uint8)
            scales = np.exp2(g.integers(-9, -4, size=(R, (K + 255) // 256))).astype(np.float16)
            mats.append((codes, scales))
        rows.append(synth.pack_expert_row(H, I, *mats))
    rows = np.stack(rows)
    x = g.standard_normal((T, H)).astype(np.float16)
    wr = (g.standard_normal((H, E)) * 0.05).astype(np.float16)
    a = oracle.layer(x, wr, rows, H, I, E, k, want_h=True)
    b = oracle.layer(x, wr, rows, H, I, E, k, want_h=True, fp16_slots=True)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["h"], b["h"]) and np.array_equal(a["o"], b["o"])
    x2, wr2, rows2 = _tiny_layer(E, k, H, I, T, seed=23)
    packed = np.stack([r for r, _ in rows2])
    c = oracle.layer(x2, wr2, packed, H, I, E, k)
    d = oracle.layer(x2, wr2, packed, H, I, E, k, fp16_slots=True)
    assert np.array_equal(c["ids"], d["ids"])                  # routing does not use expert weights
    assert not np.array_equal(c["o"], d["o"])
