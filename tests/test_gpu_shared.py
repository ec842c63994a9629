"""GPU parity of the FP16 shared expert (moe_shared_ffn) and of the layer with it.

The shared expert is checked stage by stage: its FP16 activation hs within one
FP16 ulp of the oracle's (parity_util.assert_h_close), its output against the
FP16 down weights applied to the GPU's own hs (elementwise, the stage floor)
and against the oracle per token row (normwise: single outputs move with
one-ulp flips of hs); the sigmoid gate to 1e-6 absolute; the layer output y
with the elementwise rule of parity_util.
"""
import numpy as np
import pytest

import oracle
from parity_util import assert_close_rows
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def small_shared(H, Is, seed):
    g = np.random.default_rng(seed)
    mk = lambda *shape: (g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    return mk(Is, H), mk(Is, H), mk(H, Is), mk(H)


def run_shared(x, shared):
    from w4a16_routed_expert_amd import binding as B
    dev = torch.device("cuda:0")
    from w4a16_routed_expert_amd import synth
    # the kernels read the tile8 layout; packed here by the numpy packer (the
    # library's own packer is checked against it below)
    Wsg, Wsu, Wsd = (torch.from_numpy(synth.pack_fp16_tile8(m)).to(dev) for m in shared[:3])
    wg = torch.from_numpy(np.ascontiguousarray(shared[3])).to(dev)
    T, H = x.shape
    Is = shared[0].shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out = torch.full((max(T, 1), H), float("nan"), dtype=torch.float32, device=dev)
    sig = torch.full((max(T, 1),), float("nan"), dtype=torch.float32, device=dev)
    nb = B.moe_shared_ffn_workspace_size(T, H, Is)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    B.moe_shared_ffn(xd, Wsg, Wsu, Wsd, wg, T, H, Is, out, sig, ws, nb)
    torch.cuda.synchronize()
    hs = ws[:T * Is * 2].cpu().numpy().view(np.uint16).reshape(T, Is).copy()    # hs leads the workspace
    return out.cpu().numpy()[:T], sig.cpu().numpy()[:T], hs


def check_shared(x, shared, what):
    from layer_util import check_shared_stages
    os_ref, sig_ref = oracle.shared_ffn(x, *shared)
    os_gpu, sig_gpu, hs = run_shared(x, shared)
    assert np.all(np.isfinite(os_gpu)) and np.all(np.isfinite(sig_gpu)), f"{what}: unwritten outputs"
    check_shared_stages(dict(x=x, shared_hs=hs, shared_os=os_gpu.astype(np.float64),
                             shared_sigma=sig_gpu.astype(np.float64)),
                        dict(shared_os=os_ref, shared_sigma=sig_ref), shared, what)


@pytest.mark.parametrize("R,K", [(8, 128), (16, 256), (40, 384), (2048, 5632)])
def test_tile8_packer_matches_numpy(R, K):
    from w4a16_routed_expert_amd import binding as B, synth
    dev = torch.device("cuda:0")
    w = (np.random.default_rng(R + K).standard_normal((R, K)) * 4).astype(np.float16)
    got = B.pack_tile8(torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    want = synth.pack_fp16_tile8(w)
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16)), f"tile8 {R}x{K}"


@pytest.mark.parametrize("T", [1, 5, 16, 20, 33, 70])
def test_small_shared_expert(T):
    # H = 256: a unit has 2 tiles, so 6 of the 8 wavefronts of a block load
    # nothing; T = 20 and 33 take 16-row units, T = 70 two token passes of 64
    x = (np.random.default_rng(T).standard_normal((T, 256))).astype(np.float16)
    check_shared(x, small_shared(256, 512, 7), f"small shared T={T}")


@pytest.mark.parametrize("H,Is,T", [(640, 1408, 20), (384, 2048, 3), (1024, 2816, 40), (8192, 1024, 2),
                                    (1024, 8192, 1)])
def test_odd_shared_shapes(H, Is, T):
    # reduction axes of 3 to 64 tiles: 8-row units with one or two tiles per
    # wavefront, 16-row units with chunk counts above one (uneven chunks,
    # one or two token tiles, two tiles per wavefront)
    x = (np.random.default_rng(H + T).standard_normal((T, H))).astype(np.float16)
    check_shared(x, small_shared(H, Is, 11), f"shared H={H} Is={Is} T={T}")


@pytest.mark.parametrize("T", [1, 16, 64, 100])
def test_qwen_shared_expert(T):
    cfg = synth.CONFIGS["qwen"]
    check_shared(synth.make_x(cfg, T, step=2), synth.make_shared(cfg), f"qwen shared T={T}")


def test_shared_run_to_run_bit_identical():
    # chunk partial sums meet in a fixed order
    cfg = synth.CONFIGS["qwen"]
    x, shared = synth.make_x(cfg, 16, step=6), synth.make_shared(cfg)
    a_out, a_sig, _ = run_shared(x, shared)
    b_out, b_sig, _ = run_shared(x, shared)
    assert np.array_equal(a_out.view(np.uint32), b_out.view(np.uint32))
    assert np.array_equal(a_sig.view(np.uint32), b_sig.view(np.uint32))


@pytest.mark.parametrize("T", [1, 16, 64])
def test_qwen_layer_with_shared_expert(T):
    # The whole Qwen-shaped layer: routed experts, the FP16 shared expert on a
    # second stream, the gated combine; every stage against the oracle.
    from layer_util import check_full, gpu_layer, rows_of
    cfg = synth.CONFIGS["qwen"]
    rows, wr, x = rows_of("qwen"), synth.make_router(cfg), synth.make_x(cfg, T, step=4)
    shared = synth.make_shared(cfg)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, shared=shared, want_h=True)
    got = gpu_layer(cfg, rows, wr, x, shared=shared)
    check_full(cfg, got, ref, f"qwen layer + shared T={T}", rows=rows)


def test_concurrent_shared_expert_equals_sequential():
    # The layer can run the shared expert on a second stream beside the routing
    # and the routed experts; the output must equal the one-stream order bit for
    # bit, also when the forked step is captured in a graph and replayed between
    # other (eager) layer calls.
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer, SharedExpert
    cfg = synth.CONFIGS["qwen"]
    T = 16
    dev = torch.device("cuda:0")
    rows, wr = synth.make_expert_rows(cfg), synth.make_router(cfg)
    xa = torch.from_numpy(synth.make_x(cfg, T, step=7)).to(dev)
    xb = torch.from_numpy(synth.make_x(cfg, T, step=8)).to(dev)
    Wsg, Wsu, Wsd, wg = (torch.from_numpy(np.ascontiguousarray(m)).to(dev) for m in synth.make_shared(cfg))
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev), torch.from_numpy(wr).to(dev),
                            max_T=T, device=dev)
    # one stream: shared expert first, then the routed layer
    seq = SharedExpert(Wsg, Wsu, Wsd, wg, max_T=T, device=dev)
    want = {}
    for name, x in (("a", xa), ("b", xb)):
        seq.run(x)
        want[name] = lay.forward(x, shared_out=seq.out, shared_gate=seq.gate).clone()
    torch.cuda.synchronize()
    conc = SharedExpert(Wsg, Wsu, Wsd, wg, max_T=T, device=dev)
    y = torch.empty((T, cfg.H), dtype=torch.float16, device=dev)
    lay.forward(xa, y, shared=conc)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), want["a"].view(torch.int16))
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        lay.forward(xa, y, shared=conc)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want["a"].view(torch.int16)), "graph replay differs"
        yb = lay.forward(xb, shared=conc)            # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(yb.view(torch.int16), want["b"].view(torch.int16)), "eager call differs"
