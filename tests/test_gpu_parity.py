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
    got = gpu_layer(cfg, rows, wr, x, mode=B.MOE_FFN_PATH_STREAM)
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
    got = gpu_layer(cfg, rows, wr, x, mode=B.MOE_FFN_PATH_STREAM if path == "stream" else B.MOE_FFN_PATH_GEMM)
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


def test_prefill_batch_full_routing_and_item_edges():
    # 4096 tokens, the grouped-GEMM path.  The oracle routes and groups the
    # whole batch (logits bit for bit, top-k, softmax, the stable grouping);
    # expert outputs are checked on the tokens of the first and the last pair
    # of every expert's first and last 128-pair item (every token's output
    # depends on that token only).
    from layer_util import oracle_tokens
    from parity_util import assert_h_close
    cfg = synth.CONFIGS["prefill"]
    T = 4096
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T)
    got = gpu_layer(cfg, rows, wr, x)
    k, E = cfg.k, cfg.E
    logits = oracle.router_logits(x, wr)
    assert np.array_equal(got["logits"].view(np.uint32), logits.view(np.uint32)), "prefill logits not bit-exact"
    ids, w = oracle.topk_softmax(logits, k)
    assert np.array_equal(got["ids"], ids), "prefill expert ids differ"
    assert np.allclose(got["w"], w, rtol=1e-5, atol=1e-7), "prefill routing weights differ"
    grp = oracle.group(ids, E)
    for key in ("offsets", "sorted_pairs", "pair_pos"):
        assert np.array_equal(got[key], grp[key]), f"prefill grouping: {key} differs"
    assert got["n_active"] == grp["n_active"]
    assert np.array_equal(got["active"][:grp["n_active"]], grp["active"])
    off, sp = grp["offsets"], grp["sorted_pairs"]
    pos = set()
    for e in range(E):
        n = off[e + 1] - off[e]
        if n == 0:
            continue
        last_item = 128 * ((n - 1) // 128)
        for q in (0, min(127, n - 1), last_item, n - 1):
            pos.add(int(off[e] + q))
    toks = np.array(sorted({int(sp[p]) // k for p in pos}))
    ref = oracle_tokens(x[toks], wr, rows, cfg, want_h=True)
    assert np.array_equal(got["ids"][toks], ref["ids"])
    assert_close_rows(got["y"][toks].view(np.uint16), ref["y"], "prefill item-edge tokens: y")
    pairs = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    gpu_h = got["h"][got["pair_pos"][pairs]].view(np.uint16)
    eq = assert_h_close(gpu_h, ref["h"], "prefill item-edge tokens: h")
    o_gpu = got["pair_out"][got["pair_pos"][pairs]].astype(np.float64)
    assert_close_rows(o_gpu, ref["o"], "prefill item-edge tokens: expert outputs", floor=1.0)
    print(f"prefill: {len(toks)} item-edge tokens, h bit-identical {eq:.5f}")
