"""GPU parity of the grouped-GEMM expert FFN (the kernels moe_w4a16_* use for
large batches) against the CPU oracle, through the C ABI.

The GEMM path is forced with the calls' mode argument so that small, oracle-sized
layers exercise it: several 128-pair items per expert with a ragged last one,
reduction lengths with an odd number of 128-column tiles (a padded tile),
output row counts that leave a partial row block, one tile per row, absent
experts, and the OLMoE and Qwen shapes.  The full 4096-token prefill batch,
where the automatic choice takes this path, is checked on sampled tokens in
test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle
from layer_util import check_full, gpu_layer, rows_of
from parity_util import assert_close_rows
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


GEMM = 2          # MOE_FFN_PATH_GEMM
STREAM = 1        # MOE_FFN_PATH_STREAM


@pytest.mark.parametrize("T", [1, 4, 33, 100, 300])
def test_tiny_layer(T):
    cfg = synth.CONFIGS["tiny"]
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=5)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x, mode=GEMM), ref, f"gemm tiny T={T}", rows=rows)


def test_skewed_routing_ragged_items():
    # Every token goes to experts 5 and 2: 300 pairs each = items of 128, 128
    # and 44 pairs.
    cfg = synth.CONFIGS["tiny"]
    T = 300
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=6)
    bias = np.zeros(cfg.E, np.float32)
    bias[5], bias[2] = 50.0, 40.0
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias, want_h=True)
    assert ref["n_active"] == 2
    check_full(cfg, gpu_layer(cfg, rows, wr, x, bias=bias, mode=GEMM), ref, "gemm tiny skewed", rows=rows)


# H, I: odd tile counts of the reduction axis (padded tile), partial row blocks
# (gate/up items cover 128 rows of I, down items 256 rows of H), one tile.
@pytest.mark.parametrize("H,I", [(384, 384), (384, 256), (128, 128), (640, 128), (256, 640)])
def test_odd_shapes(H, I):
    cfg = synth.LayerConfig(f"odd{H}x{I}", 9, E=4, k=2, H=H, I=I, batches=(150,), resident=4)
    T = 150
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x, mode=GEMM), ref, f"gemm H={H} I={I}", rows=rows)


def test_olmoe_layer():
    cfg = synth.CONFIGS["olmoe"]
    T = 32
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x, mode=GEMM), ref, "gemm olmoe T=32", rows=rows)


def test_qwen_layer():
    # I = 1408: 11 reduction tiles in the down projection, 11 row blocks in gate/up
    cfg = synth.CONFIGS["qwen"]
    T = 64
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=2)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, gpu_layer(cfg, rows, wr, x, mode=GEMM), ref, "gemm qwen T=64", rows=rows)


def test_absent_expert():
    cfg = synth.CONFIGS["tiny"]
    T = 200
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    missing = int(ref["active"][1])
    slot_map = np.arange(cfg.E, dtype=np.int32)
    slot_map[missing] = -1
    got = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, mode=GEMM)
    assert got["status"] == 7
    lo, hi = ref["offsets"][missing], ref["offsets"][missing + 1]
    assert hi - lo > 0
    assert np.all(got["pair_out"][lo:hi] == 0) and np.all(got["h"][lo:hi] == 0)
    keep = np.ones(T * cfg.k, bool)
    keep[lo:hi] = False
    o_ref = ref["o"][ref["sorted_pairs"]]
    assert_close_rows(got["pair_out"][keep].astype(np.float64), o_ref[keep], "gemm present experts", floor=1.0)


def test_run_to_run_bit_identical():
    cfg = synth.CONFIGS["tiny"]
    T = 300
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T)
    a = gpu_layer(cfg, rows, wr, x, mode=GEMM)
    lay = a["layer"]
    xd = torch.from_numpy(x).cuda()
    for _ in range(3):
        y = lay.forward(xd, mode=GEMM)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), a["y"].view(np.uint16))


def test_auto_path_and_stream_path_agree():
    # T*k = 600 >= 64*E: the automatic choice is the GEMM, bit-identical to
    # forcing it; the streaming kernels give the same layer within tolerance.
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["tiny"]
    T = 300
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=7)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    auto = gpu_layer(cfg, rows, wr, x)
    gemm = gpu_layer(cfg, rows, wr, x, mode=B.MOE_FFN_PATH_GEMM)
    stream = gpu_layer(cfg, rows, wr, x, mode=B.MOE_FFN_PATH_STREAM)
    assert np.array_equal(auto["y"].view(np.uint16), gemm["y"].view(np.uint16))
    assert_close_rows(gemm["y"].view(np.uint16), ref["y"], "gemm y")
    assert_close_rows(stream["y"].view(np.uint16), ref["y"], "stream y")


def test_olmoe_512_tokens_sampled():
    # Automatic choice at 4096 pairs (64 per expert on average): the GEMM.
    cfg = synth.CONFIGS["olmoe"]
    T = 512
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T, step=9)
    got = gpu_layer(cfg, rows, wr, x)
    sample = np.random.default_rng(1).choice(T, 16, replace=False)
    ref = oracle.layer(x[sample], wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    assert np.array_equal(got["ids"][sample], ref["ids"])
    assert_close_rows(got["y"][sample].view(np.uint16), ref["y"], "gemm olmoe T=512 sampled y")

