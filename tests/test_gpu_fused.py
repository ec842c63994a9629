"""GPU parity of the one-call layer (moe_layer_forward) against the CPU oracle,
through the C ABI.

For decode batches the call routes in one launch (the last block to finish
its logits runs the top-k and the grouping).  With the streaming kernels it
then runs gate/up, down and the combine, and y must equal the separate calls'
y bit for bit; with the K-split expert FFN (MOE_FFN_PATH_KSPLIT, opt-in)
gate/up and down run in one launch that writes partial outputs per slice of
the intermediate axis, and the combine adds them.  Every stage is compared with the oracle as in
test_gpu_parity.py (routing and grouping bit for bit, h within one FP16 ulp,
expert outputs and y within tolerance, plus the stage-wise check).  Shapes:
the OLMoE-shaped layer, the Qwen-shaped layer with its shared expert (on a
second stream, joined by an event before the combine), the tiny layer, odd
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


STREAM, KSPLIT, ONE = 1, 3, 4    # MOE_FFN_PATH_STREAM, MOE_FFN_PATH_KSPLIT, MOE_FFN_PATH_ONE_LAUNCH


def both(cfg, rows, wr, x, mode=STREAM, **kw):
    """The one-call layer and the separate calls with the same kernel family: y bit-identical."""
    fused = gpu_layer(cfg, rows, wr, x, fused=True, mode=mode, **kw)
    sep = gpu_layer(cfg, rows, wr, x, mode=mode, **kw)
    assert np.array_equal(fused["y"].view(np.uint16), sep["y"].view(np.uint16)), \
        "one-call layer and separate calls differ"
    return fused


def workspace_is_zero(lay, T):
    """The one-call layer leaves its control words zero (the routing launch's done counter and
    the one-launch layer's counters: the first 1024 bytes of the workspace)."""
    ws = lay.layer_ws.cpu().numpy()
    return not ws[:1024].any()


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


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 2), ("olmoe", 3), ("olmoe", 8), ("olmoe", 16),
                                    ("qwen", 1), ("qwen", 5), ("qwen", 16), ("tiny", 1), ("tiny", 16)])
def test_ksplit_expert_ffn_one_call(name, T):
    # gate/up and down of a slice of the intermediate axis in one block,
    # partial outputs per slice added by the combine: slice widths 32 (T = 1
    # to 3 on the OLMoE shape, 44 planes on the Qwen shape), 64 and 128, and
    # the tiny layer's H = 256 (two tiles, one wave per row group)
    cfg = synth.CONFIGS[name]
    rows, wr, x = rows_of(name), synth.make_router(cfg), synth.make_x(cfg, T, step=30 + T)
    shared = synth.make_shared(cfg) if cfg.shared_I else None
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = gpu_layer(cfg, rows, wr, x, fused=True, mode=KSPLIT, shared=shared)
    assert got["status"] == 0
    check_full(cfg, got, ref, f"k-split {name} T={T}", rows=rows)
    assert workspace_is_zero(got["layer"], T)


@pytest.mark.parametrize("T,path", [(1, STREAM), (8, STREAM), (32, STREAM)])
def test_auto_keeps_the_streaming_ffn_in_one_call(T, path):
    # AUTO runs the same kernels as the forced mode, so the bits agree (the
    # K-split launch is opt-in: measured slower)
    cfg = synth.CONFIGS["olmoe"]
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T, step=40)
    auto = gpu_layer(cfg, rows, wr, x, fused=True)
    forced = gpu_layer(cfg, rows, wr, x, fused=True, mode=path)
    assert np.array_equal(auto["y"].view(np.uint16), forced["y"].view(np.uint16))


def test_ksplit_absent_expert():
    # an expert without a device row: status word set, its pairs' outputs
    # zero, the other pairs as with the streaming kernels (within tolerance:
    # the down projection's FP32 summation order differs)
    cfg = synth.CONFIGS["tiny"]
    T = 6
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=41)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    missing = int(ref["active"][0])
    slot_map = np.arange(cfg.E, dtype=np.int32)
    slot_map[missing] = -1
    got = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, fused=True, mode=KSPLIT)
    st = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, fused=True, mode=STREAM)
    assert got["status"] == 7 and st["status"] == 7
    lo, hi = ref["offsets"][missing], ref["offsets"][missing + 1]
    assert np.all(got["pair_out"][lo:hi] == 0) and np.all(got["h"][lo:hi] == 0)
    np.testing.assert_allclose(got["pair_out"], st["pair_out"], rtol=2e-3, atol=2e-3 * np.abs(st["pair_out"]).max())


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
    got = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, fused=True, mode=STREAM)
    sep = gpu_layer(cfg, rows, wr, x, slot_map=slot_map, mode=STREAM)
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
    # references: T = 32 the separate calls (same kernels), the small batches
    # a first one-call run (the K-split expert FFN, which the separate calls
    # do not have)
    want = {T: (lay.forward(x) if T == 32 else lay.forward_fused(x)).clone() for T, x in xs.items()}
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


# ---------------------------------------------------------------- the one-launch layer
# MOE_FFN_PATH_ONE_LAUNCH: routing, gate/up, down and the combine in one
# persistent launch whose blocks hand results to each other through
# device-scope counters.  Same kernels' arithmetic and splits as the separate
# calls, so y (and h, pair_out, the routing results) must be bit-identical to
# them, and every stage is checked against the oracle.

def one_vs_separate(cfg, rows, wr, x, **kw):
    one = gpu_layer(cfg, rows, wr, x, fused=True, mode=ONE, **kw)
    sep = gpu_layer(cfg, rows, wr, x, mode=STREAM, **kw)
    for key in ("ids", "w", "offsets", "sorted_pairs", "pair_pos", "active", "h", "pair_out"):
        assert np.array_equal(one[key], sep[key]), f"one-launch layer: {key} differs from the separate calls"
    assert np.array_equal(one["y"].view(np.uint16), sep["y"].view(np.uint16)), \
        "one-launch layer and separate calls differ"
    assert workspace_is_zero(one["layer"], x.shape[0])
    return one


@pytest.mark.parametrize("T", [1, 2, 4, 8, 32])
def test_one_launch_olmoe_decode(T):
    # T = 1, 2-4 and 8-32 take the reduction-axis splits 4, 2 and 1
    cfg = synth.CONFIGS["olmoe"]
    rows, wr, x = rows_of("olmoe"), synth.make_router(cfg), synth.make_x(cfg, T, step=50 + T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    got = one_vs_separate(cfg, rows, wr, x)
    assert got["status"] == 0
    check_full(cfg, got, ref, f"one-launch olmoe T={T}", rows=rows)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_one_launch_qwen_decode_with_shared_expert(T):
    cfg = synth.CONFIGS["qwen"]
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=60 + T)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = one_vs_separate(cfg, rows, wr, x, shared=shared)
    assert got["status"] == 0
    check_full(cfg, got, ref, f"one-launch qwen + shared T={T}", rows=rows)


@pytest.mark.parametrize("T", [1, 5, 16, 64])
def test_one_launch_tiny(T):
    cfg = synth.CONFIGS["tiny"]
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=70 + T)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True)
    got = one_vs_separate(cfg, rows, wr, x)
    check_full(cfg, got, ref, f"one-launch tiny T={T}", rows=rows)


def test_one_launch_absent_expert():
    # an expert without a device row: status word set, its outputs zero, the
    # rest as the separate calls compute them
    cfg = synth.CONFIGS["tiny"]
    T = 8
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=15)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k)
    missing = int(ref["active"][0])
    slot_map = np.arange(cfg.E, dtype=np.int32)
    slot_map[missing] = -1
    got = one_vs_separate(cfg, rows, wr, x, slot_map=slot_map)
    assert got["status"] == 7
    lo, hi = ref["offsets"][missing], ref["offsets"][missing + 1]
    assert np.all(got["pair_out"][lo:hi] == 0)


def test_one_launch_rejects_what_it_is_not_built_for():
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["olmoe"]
    rows, wr = rows_of("olmoe"), synth.make_router(cfg)
    x = synth.make_x(cfg, 65, step=1)              # T above the one-launch maximum of 64
    with pytest.raises(B.MoeError) as ei:
        gpu_layer(cfg, rows, wr, x, fused=True, mode=ONE)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED


def test_one_launch_repeated_calls_and_graph_replay():
    # calls of different sizes in a row reuse the workspace (the last block of
    # each call zeroes the counters); a captured call replays to the same bits
    # between eager calls
    cfg = synth.CONFIGS["olmoe"]
    dev = torch.device("cuda:0")
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    rows, wr = rows_of("olmoe"), synth.make_router(cfg)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev), torch.from_numpy(wr).to(dev),
                            max_T=32, device=dev)
    xs = {T: torch.from_numpy(synth.make_x(cfg, T, step=80 + T)).to(dev) for T in (32, 1, 8)}
    want = {T: lay.forward(x, mode=STREAM).clone() for T, x in xs.items()}
    torch.cuda.synchronize()
    for _ in range(3):
        for T, x in xs.items():
            y = lay.forward_fused(x, mode=ONE)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want[T].view(torch.int16)), f"T={T}"
            assert workspace_is_zero(lay, 32)
            assert int(lay.status.cpu()[0]) == 0
    y32 = torch.empty((32, cfg.H), dtype=torch.float16, device=dev)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for _ in range(3):
            lay.forward_fused(xs[32], y32, mode=ONE)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y32.view(torch.int16), want[32].view(torch.int16)), "graph replay differs"
        y1 = lay.forward_fused(xs[1], mode=ONE)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), want[1].view(torch.int16)), "eager call between replays differs"
    assert workspace_is_zero(lay, 32)


def test_one_launch_wait_gives_up_on_a_workspace_that_was_not_zeroed():
    # The routing counter of the one-launch layer starts at a value the
    # election never reaches, so no block publishes the routing and every
    # wait for it runs into its poll limit (the kernel still ends: the waits
    # are bounded): MOE_ERR_TIMEOUT in the status word.  The last block to
    # leave zeroes the counters, so the next call is correct again.
    from w4a16_routed_expert_amd import binding as B
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    cfg = synth.CONFIGS["tiny"]
    dev = torch.device("cuda:0")
    T = 4
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=90)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev), torch.from_numpy(wr).to(dev),
                            max_T=T, device=dev)
    xd = torch.from_numpy(x).to(dev)
    want = lay.forward(xd, mode=STREAM).clone()
    torch.cuda.synchronize()
    lay.layer_ws[:4].view(torch.int32).fill_(1 << 20)         # logits counter far past any task count
    lay.forward_fused(xd, mode=ONE)
    torch.cuda.synchronize()
    assert int(lay.status.cpu()[0]) == B.MOE_ERR_TIMEOUT
    assert workspace_is_zero(lay, T)
    lay.status.zero_()
    y = lay.forward_fused(xd, mode=ONE)
    torch.cuda.synchronize()
    assert int(lay.status.cpu()[0]) == 0
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))


# ---------------------------------------------------------------- the layer with its shared expert on one stream
# moe_layer_forward_shared: for decode batches the routing launch also runs
# the FP16 shared expert's gate/up pass (extra blocks of the same grid), then
# the expert FFN, the rest of the shared expert and the combine follow on the
# same stream.  Every block computes what the separate launches compute, so
# y, the routing results, h, pair_out and the shared expert's outputs must be
# bit-identical to the shared expert on a second stream beside the one-call
# layer; other batches and modes take the separate calls in stream order.

SHARED_KEYS = ("ids", "w", "offsets", "sorted_pairs", "pair_pos", "active", "h", "pair_out", "shared_os",
               "shared_sigma", "shared_hs")


def shared_one_stream(cfg, rows, wr, x, shared, mode=None):
    one = gpu_layer(cfg, rows, wr, x, shared=shared, one_stream=True, mode=mode)
    two = gpu_layer(cfg, rows, wr, x, shared=shared, fused=True, mode=mode)
    for key in SHARED_KEYS:
        assert np.array_equal(one[key], two[key]), f"one-stream shared layer: {key} differs"
    assert np.array_equal(one["y"].view(np.uint16), two["y"].view(np.uint16)), \
        "one-stream shared layer and the two-stream call differ"
    assert workspace_is_zero(one["layer"], x.shape[0])
    return one


@pytest.mark.parametrize("T", [1, 5, 16, 24, 64, 100])
def test_qwen_layer_with_shared_expert_on_one_stream(T):
    # T = 1, 5 and 16 take the routing + shared gate/up launch (8-row units
    # over the whole axis); T = 24, 64 and 100 (16-row units with 2 or 4 token
    # tiles) the separate calls in stream order
    cfg = synth.CONFIGS["qwen"]
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=120 + T)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = shared_one_stream(cfg, rows, wr, x, shared)
    assert got["status"] == 0
    check_full(cfg, got, ref, f"one-stream qwen + shared T={T}", rows=rows)


@pytest.mark.parametrize("T", [1, 7, 16])
def test_tiny_layer_with_shared_expert_on_one_stream(T):
    # a small grid: 8 experts, H = 256, a 512-wide shared expert
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], shared_I=512)
    rows, wr, x = rows_of("tiny"), synth.make_router(cfg), synth.make_x(cfg, T, step=130 + T)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = shared_one_stream(cfg, rows, wr, x, shared)
    check_full(cfg, got, ref, f"one-stream tiny + shared T={T}", rows=rows)


@pytest.mark.parametrize("E,k,T", [(37, 5, 3), (8, 2, 9)])
def test_shared_on_one_stream_shapes_off_the_fused_path(E, k, T):
    # an odd expert count (37) takes the separate calls; H = 384 (three
    # 128-column tiles) and a 640-wide shared expert exercise other plans
    cfg = synth.LayerConfig(f"edge{E}x{k}s", 11, E=E, k=k, H=384, I=256, batches=(T,), resident=E, shared_I=640)
    rows, wr, x = synth.make_expert_rows(cfg), synth.make_router(cfg), synth.make_x(cfg, T)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = shared_one_stream(cfg, rows, wr, x, shared)
    check_full(cfg, got, ref, f"one-stream E={E} k={k} T={T} + shared", rows=rows)


@pytest.mark.parametrize("mode", [2, 3, 4])   # GEMM, K-split, one launch: the separate calls
def test_shared_on_one_stream_other_modes(mode):
    cfg = synth.CONFIGS["qwen"]
    T = 4
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=140 + mode)
    shared = synth.make_shared(cfg)
    shared_one_stream(cfg, rows, wr, x, shared, mode=mode)


def test_shared_on_one_stream_repeated_calls_and_graph_replay():
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer, SharedExpert
    cfg = synth.CONFIGS["qwen"]
    dev = torch.device("cuda:0")
    rows, wr = rows_of("qwen"), synth.make_router(cfg)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev), torch.from_numpy(wr).to(dev),
                            max_T=16, device=dev)
    sh = SharedExpert(*(torch.from_numpy(np.ascontiguousarray(m)).to(dev) for m in synth.make_shared(cfg)),
                      max_T=16, device=dev)
    xs = {T: torch.from_numpy(synth.make_x(cfg, T, step=150 + T)).to(dev) for T in (16, 1, 9)}
    want = {T: lay.forward_fused(x, shared=sh).clone() for T, x in xs.items()}
    torch.cuda.synchronize()
    for _ in range(2):
        for T, x in xs.items():
            y = lay.forward_shared(x, sh)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want[T].view(torch.int16)), f"T={T}"
            assert workspace_is_zero(lay, 16)
    y16 = torch.empty((16, cfg.H), dtype=torch.float16, device=dev)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        lay.forward_shared(xs[16], sh, y16)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int16), want[16].view(torch.int16)), "graph replay differs"
        y1 = lay.forward_shared(xs[1], sh)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), want[1].view(torch.int16)), "eager call between replays differs"
    assert workspace_is_zero(lay, 16)
