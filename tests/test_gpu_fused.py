"""GPU parity of the one-call layer (moe_layer_forward) against the CPU oracle,
through the C ABI.

For decode batches the call runs four launches: routing in one (the last
block to finish its logits runs the top-k and the grouping), gate/up, down
and the combine.  Every stage is compared with the oracle as in
test_gpu_parity.py (routing and grouping bit for bit, h within one FP16 ulp,
expert outputs and y within tolerance, plus the stage-wise check), and y must
equal the separate calls' y bit for bit.  Shapes: the OLMoE-shaped layer at
T = 1/8/32, the Qwen-shaped layer with its shared expert (on a second stream,
joined by an event before the combine) at T = 1/16/64, the tiny layer, odd
shapes, an absent expert, batches that take the separate kernels, repeated
calls and graph replay.
"""
import numpy as np
import pytest

import oracle
from layer_util import check_full, gpu_layer, rows_of
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def both(cfg, rows, wr, x, **kw):
    fused = gpu_layer(cfg, rows, wr, x, fused=True, **kw)
    sep = gpu_layer(cfg, rows, wr, x, **kw)
    assert np.array_equal(fused["y"].view(np.uint16), sep["y"].view(np.uint16)), \
        "one-call layer and separate calls differ"
    return fused


def workspace_is_zero(lay, T):
    """The one-call layer leaves its counter zero (the routing launch's done counter, the first
    256 bytes of the workspace)."""
    ws = lay.layer_ws.cpu().numpy()
    return not ws[:256].any()


@pytest.mark.parametrize("T", [1, 8, 32])
def test_olmoe_decode_layer_one_call(T):
    cfg = synth.CONFIGS["olmoe"]
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T, step=11)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    got = both(cfg, rows, wr, x)
    check_full(cfg, got, ref, f"one-call olmoe T={T}", rows=rows)
    assert workspace_is_zero(got["layer"], T)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_qwen_decode_layer_one_call_with_shared_expert(T):
    cfg = synth.CONFIGS["qwen"]
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=12)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = both(cfg, rows, wr, x, shared=shared)
    check_full(cfg, got, ref, f"one-call qwen + shared T={T}", rows=rows)


@pytest.mark.parametrize("T", [1, 4, 33, 256])
def test_tiny_layer_one_call(T):
    cfg = synth.CONFIGS["tiny"]
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=13)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, both(cfg, rows, wr, x), ref, f"one-call tiny T={T}", rows=rows)


@pytest.mark.parametrize("H,I", [(384, 384), (640, 128), (256, 640)])
def test_odd_shapes_one_call(H, I):
    # odd tile counts of the down projection's reduction axis (one output row
    # group per unit) and partial row chunks
    cfg = synth.LayerConfig(f"odd{H}x{I}", 9, E=4, k=2, H=H, I=I, batches=(40,), resident=4)
    T = 40
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    check_full(cfg, both(cfg, rows, wr, x, mode=1), ref, f"one-call H={H} I={I}", rows=rows)


def test_batches_that_take_the_separate_kernels():
    # T > 256 and the grouped GEMM: the call runs the separate kernels
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["tiny"]
    rows, wr = rows_of("tiny"), synth.make_router(cfg)
    for T, mode in ((300, B.MOE_FFN_PATH_AUTO), (300, B.MOE_FFN_PATH_STREAM), (40, B.MOE_FFN_PATH_GEMM)):
        x = synth.make_x(cfg, T, step=14)
        ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
        check_full(cfg, both(cfg, rows, wr, x, mode=mode), ref, f"one-call tiny T={T} mode {mode}", rows=rows)


def test_absent_expert_one_call():
    cfg = synth.CONFIGS["tiny"]
    T = 8
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=15)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    missing = int(ref["active"][0])
    slot_map = np.arange(cfg.E, dtype=np.int32)
    slot_map[missing] = -1
    got = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, fused=True)
    sep = gpu_layer(cfg, rows, wr, x, slot_map=slot_map)
    assert got["status"] == 7
    lo, hi = ref["offsets"][missing], ref["offsets"][missing + 1]
    assert np.all(got["pair_out"][lo:hi] == 0)
    assert np.array_equal(got["y"].view(np.uint16), sep["y"].view(np.uint16))
    assert workspace_is_zero(got["layer"], T)


def test_repeated_calls_and_graph_replay():
    # calls of different sizes in a row reuse the workspace (its counters are
    # left zero); a captured call replays to the same bits between eager calls
    cfg = synth.CONFIGS["olmoe"]
    dev = torch.device("cuda:0")
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    rows, wr = rows_of("olmoe"), synth.make_router(cfg)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev), torch.from_numpy(wr).to(dev),
                            max_T=32, device=dev)
    xs = {T: torch.from_numpy(synth.make_x(cfg, T, step=16 + T)).to(dev) for T in (32, 1, 8)}
    want = {T: lay.forward(x).clone() for T, x in xs.items()}
    torch.cuda.synchronize()
    for _ in range(2):
        for T, x in xs.items():
            y = lay.forward_fused(x)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want[T].view(torch.int16)), f"T={T}"
            assert workspace_is_zero(lay, 32)
    y32 = torch.empty((32, cfg.H), dtype=torch.float16, device=dev)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        lay.forward_fused(xs[32], y32)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y32.view(torch.int16), want[32].view(torch.int16)), "graph replay differs"
        y1 = lay.forward_fused(xs[1])
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), want[1].view(torch.int16)), "eager call between replays differs"
