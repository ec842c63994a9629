"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Routing (logits, ids) and grouping are compared bit for bit; routing weights,
the SwiGLU activations h, the per-pair expert outputs and the layer output y
within the tolerance of parity_util (2e-3 relative after FP16 rounding, with
a per-row floor).  Shapes: the tiny layer, the OLMoE-shaped and Qwen-shaped
decode layers at their batch sizes, ragged and skewed batches, and sampled
tokens of the 4096-token prefill batch.
"""
import numpy as np
import pytest

import oracle
from layer_util import check_full, gpu_layer, rows_of
from parity_util import assert_close_rows
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- tiny layer
@pytest.mark.parametrize("T", [4, 1, 3, 17, 33, 100])
def test_tiny_layer(T):
    cfg = synth.CONFIGS["tiny"]
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x), ref, f"tiny T={T}", rows=rows)


def test_skewed_routing_many_tokens_per_expert():
    # A large bias on experts 5 and 2 sends every token to them: 40 tokens per
    # expert = three 16-token tiles with a ragged tail.
    cfg = synth.CONFIGS["tiny"]
    T = 40
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=3)
    bias = np.zeros(cfg.E, np.float32)
    bias[5], bias[2] = 50.0, 40.0
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias, want_h=True)
    assert ref["n_active"] == 2
    check_full(cfg, gpu_layer(cfg, rows, wr, x, bias=bias), ref, "tiny skewed", rows=rows)


def test_zero_router_ties_go_to_lower_index():
    cfg = synth.CONFIGS["tiny"]
    T = 5
    rows, x = rows_of("tiny"), synth.make_x(cfg, T)
    wr = np.zeros((cfg.H, cfg.E), np.float16)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    got = gpu_layer(cfg, rows, wr, x)
    assert np.array_equal(got["ids"], np.tile(np.arange(cfg.k), (T, 1)))
    assert np.all(got["w"] == np.float32(1.0 / cfg.k))
    check_full(cfg, got, ref, "tiny zero router", rows=rows)


def test_empty_batch():
    cfg = synth.CONFIGS["tiny"]
    x = np.zeros((0, cfg.H), np.float16)
    got = gpu_layer(cfg, rows_of("tiny"), synth.make_router(cfg), x)
    assert got["y"].shape == (0, cfg.H)


def test_identical_experts_ignore_routing():
    cfg = synth.CONFIGS["tiny"]
    T = 6
    rows = np.repeat(rows_of("tiny")[3:4], cfg.E, axis=0)
    wr, x = synth.make_router(cfg), synth.make_x(cfg, T, step=1)
    single = oracle.layer(x, np.ones((cfg.H, 1), np.float16), rows[:1], cfg.H, cfg.I, 1, 1)
    got = gpu_layer(cfg, rows, wr, x)
    assert_close_rows(got["y"].view(np.uint16), single["y"], "identical experts")


def test_absent_expert_sets_status_and_zero_output():
    cfg = synth.CONFIGS["tiny"]
    T = 4
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    missing = int(ref["active"][0])
    slot_map = np.arange(cfg.E, dtype=np.int32)
    slot_map[missing] = -1
    got = gpu_layer(cfg, rows, wr, x, slot_map=slot_map)
    assert got["status"] == 7
    lo, hi = ref["offsets"][missing], ref["offsets"][missing + 1]
    assert np.all(got["pair_out"][lo:hi] == 0) and np.all(got["h"][lo:hi] == 0)


# H, I: reduction axes with an odd tile count (a short last scale block), one
# tile (I = 128: the down projection reads a single 128-column tile), and
# output row counts that are not a multiple of the 8 row groups of an item.
@pytest.mark.parametrize("H,I", [(384, 384), (128, 128), (640, 128), (256, 640)])
def test_streaming_odd_shapes(H, I):
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.LayerConfig(f"odd{H}x{I}", 9, E=4, k=2, H=H, I=I, batches=(40,), resident=4)
    T = 40
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    B.moe_set_ffn_path(B.MOE_FFN_PATH_STREAM)
    try:
        got = gpu_layer(cfg, rows, wr, x)
    finally:
        B.moe_set_ffn_path(B.MOE_FFN_PATH_AUTO)
    check_full(cfg, got, ref, f"streaming H={H} I={I}", rows=rows)


# Expert counts at the edges: one expert with k = 1 (every routing weight 1),
# and 37 experts (not a multiple of 16) with k = 5; both FFN kernel families.
@pytest.mark.parametrize("E,k,H,I,T", [(1, 1, 256, 128, 3), (37, 5, 384, 256, 50)])
@pytest.mark.parametrize("path", ["stream", "gemm"])
def test_expert_count_edges(E, k, H, I, T, path):
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.LayerConfig(f"edge{E}x{k}", 10, E=E, k=k, H=H, I=I, batches=(T,), resident=E)
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    B.moe_set_ffn_path(B.MOE_FFN_PATH_STREAM if path == "stream" else B.MOE_FFN_PATH_GEMM)
    try:
        got = gpu_layer(cfg, rows, wr, x)
    finally:
        B.moe_set_ffn_path(B.MOE_FFN_PATH_AUTO)
    check_full(cfg, got, ref, f"{path} E={E} k={k}", rows=rows)


def test_run_to_run_bit_identical():
    cfg = synth.CONFIGS["tiny"]
    T = 33
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T)
    a = gpu_layer(cfg, rows, wr, x)
    lay = a["layer"]
    xd = torch.from_numpy(x).cuda()
    for _ in range(3):
        y = lay.forward(xd)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), a["y"].view(np.uint16))


# ------------------------------------------------------- full-size decode layers
@pytest.mark.parametrize("T", [1, 8, 32])
def test_olmoe_decode_layer(T):
    cfg = synth.CONFIGS["olmoe"]
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x), ref, f"olmoe T={T}", rows=rows)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_qwen_routed_decode_layer(T):
    cfg = synth.CONFIGS["qwen"]
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x), ref, f"qwen T={T}", rows=rows)


def test_olmoe_zipf_biased_layer():
    cfg = synth.CONFIGS["olmoe_stack"]
    T = 32
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg, layer=3), synth.make_x(cfg, T, layer=3)
    bias = synth.make_zipf_bias(cfg, layer=3)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x, bias=bias), ref, "olmoe zipf T=32", rows=rows)


def test_prefill_batch_sampled_tokens():
    # 4096 tokens: every token's routing depends on that token only, so the
    # oracle of a sampled subset gives those tokens' ids, weights and outputs.
    cfg = synth.CONFIGS["prefill"]
    T = 4096
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T)
    got = gpu_layer(cfg, rows, wr, x)
    k, E = cfg.k, cfg.E
    ids = got["ids"]
    # grouping properties on the full batch
    sp = got["sorted_pairs"]
    assert np.array_equal(np.sort(sp), np.arange(T * k))
    assert np.array_equal(got["pair_pos"][sp], np.arange(T * k))
    flat = ids.reshape(-1)
    assert np.array_equal(got["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    key = flat[sp].astype(np.int64) * (T * k) + sp
    assert np.all(np.diff(key) > 0), "grouping is not sorted by (expert, pair)"
    assert np.all(np.sort(ids, axis=1)[:, 1:] != np.sort(ids, axis=1)[:, :-1])
    sample = np.random.default_rng(0).choice(T, 24, replace=False)
    ref = oracle.layer(x[sample], wr, rows, cfg.H, cfg.I, E, k)
    assert np.array_equal(ids[sample], ref["ids"])
    assert np.array_equal(got["logits"][sample].view(np.uint32), ref["logits"].view(np.uint32))
    assert np.allclose(got["w"][sample], ref["w"], rtol=1e-5, atol=1e-7)
    assert_close_rows(got["y"][sample].view(np.uint16), ref["y"], "prefill sampled y")
