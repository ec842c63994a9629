"""GPU routing: the fast path (fp64 sums certified against an error bound)
must give the same bits as the exact integer path and as the oracle, also on
inputs built so that exact logits sit on FP32 rounding midpoints or cancel."""
import numpy as np
import pytest

import oracle
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_route(x, wr, k, bias=None, exact=False):
    from w4a16_routed_expert_amd import binding as B
    dev = torch.device("cuda:0")
    T, H = x.shape
    E = wr.shape[1]
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    wd = torch.from_numpy(np.ascontiguousarray(wr)).to(dev)
    bd = None if bias is None else torch.from_numpy(bias).to(dev)
    out = dict(logits=torch.empty((T, E), dtype=torch.float32, device=dev),
               ids=torch.empty((T, k), dtype=torch.int32, device=dev),
               w=torch.empty((T, k), dtype=torch.float32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_pairs=torch.empty(T * k, dtype=torch.int32, device=dev),
               pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
               active=torch.empty(E, dtype=torch.int32, device=dev),
               n_active=torch.empty(1, dtype=torch.int32, device=dev))
    args = (out["logits"], out["ids"], out["w"], out["offsets"], out["sorted_pairs"], out["pair_pos"],
            out["active"], out["n_active"])
    nb = B.moe_route_workspace_size(T, H, E)
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    if exact:
        B.moe_route_exact(xd, wd, bd, T, H, E, k, *args, ws, nb)
    else:
        B.moe_route(xd, wd, bd, T, H, E, k, *args, ws, nb)
    # and once more without the logits output
    ids2 = torch.empty_like(out["ids"])
    args2 = (None, ids2) + args[2:]
    B.moe_route(xd, wd, bd, T, H, E, k, *args2, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(ids2, out["ids"])
    return {n: t.cpu().numpy() for n, t in out.items()}


def assert_same(a, b, what):
    for n in a:
        if a[n].dtype == np.float32:
            assert np.array_equal(a[n].view(np.uint32), b[n].view(np.uint32)), f"{what}: {n} differs"
        else:
            assert np.array_equal(a[n], b[n]), f"{what}: {n} differs"


@pytest.mark.parametrize("name,T", [("tiny", 9), ("olmoe", 32), ("qwen", 16)])
def test_fast_route_equals_exact_route(name, T):
    cfg = synth.CONFIGS[name]
    x, wr = synth.make_x(cfg, T, step=5), synth.make_router(cfg)
    fast = run_route(x, wr, cfg.k)
    exact = run_route(x, wr, cfg.k, exact=True)
    assert_same(fast, exact, f"{name} T={T}")
    assert np.array_equal(fast["logits"].view(np.uint32), oracle.router_logits(x, wr).view(np.uint32))


def crafted_router_inputs():
    """Rows whose exact logits are FP32 ties (2^24 + 1 -> 2^24, 2^24 + 3 -> 2^24 + 4),
    near-ties, and cancellations that lose everything in FP32 and little in fp64."""
    H, E = 256, 8
    g = np.random.default_rng(17)
    wr = (g.standard_normal((H, E)) * 1e-3).astype(np.float16)
    x = (g.standard_normal((6, H)) * 1e-3).astype(np.float16)
    # crafted tokens 0..3 use only rows 0..3 of the router (x is zero elsewhere),
    # so their logits are exactly the crafted sums; tokens 4, 5 stay random
    wr[:4] = 0
    x[:4] = 0
    x[4:, :4] = 0
    x[0, 0], x[0, 1] = 4096, 1
    wr[0, 0], wr[1, 0] = 4096, 1                       # token 0, expert 0: 2^24 + 1 -> tie to even 2^24
    wr[0, 1], wr[1, 1] = 4096, 3                       # expert 1: 2^24 + 3 -> 2^24 + 4
    wr[0, 2], wr[1, 2] = 4096, 2                       # expert 2: 2^24 + 2 (representable)
    x[1, 0], x[1, 1], x[1, 2] = 1, 1, 1
    wr[0, 3], wr[1, 3], wr[2, 3] = 65504, 2.0 ** -24, -65504   # cancellation: exact 2^-24
    x[2, :4] = [2048, 2048, 1, 0]
    wr[0, 4], wr[1, 4], wr[2, 4] = 2048, 2048, 1       # token 2, expert 4: 2^23 + 2^22 ... + 1 (exact in FP32)
    x[3, 0], x[3, 1] = 8192, 2.0 ** -10
    wr[0, 5], wr[1, 5] = 8192, 2.0 ** -14              # 2^26 + 2^-24: far below FP32 resolution, rounds down
    return x, wr


def test_midpoint_and_cancellation_logits_are_exact():
    x, wr = crafted_router_inputs()
    ref = oracle.router_logits(x, wr)
    assert ref[0, 0] == np.float32(2.0 ** 24) and ref[0, 1] == np.float32(2.0 ** 24 + 4)
    assert ref[1, 3] == np.float32(2.0 ** -24)
    fast = run_route(x, wr, 2)
    exact = run_route(x, wr, 2, exact=True)
    assert np.array_equal(fast["logits"].view(np.uint32), ref.view(np.uint32))
    assert_same(fast, exact, "crafted")
    ids, w = oracle.topk_softmax(ref, 2)
    assert np.array_equal(fast["ids"], ids)
    assert np.allclose(fast["w"], w, rtol=1e-6, atol=0)


def check_grouping(got, ids, E, what):
    """Offsets, sorted pairs, pair positions and the active list against the
    oracle's stable counting sort of the routed ids."""
    ref = oracle.group(ids, E)
    assert np.array_equal(got["offsets"], ref["offsets"]), f"{what}: offsets"
    assert np.array_equal(got["sorted_pairs"], ref["sorted_pairs"]), f"{what}: sorted pairs"
    assert np.array_equal(got["pair_pos"], ref["pair_pos"]), f"{what}: pair positions"
    na = ref["n_active"]
    assert int(got["n_active"][0]) == na and np.array_equal(got["active"][:na], ref["active"]), f"{what}: active list"
    assert np.all(got["active"][na:] == -1), f"{what}: active list padding"


# Batches above the 256-token switch take the multi-block path (4 tokens per
# logits block, per-segment counts of 256 pairs, segment-wise scatter): a
# partial last token block and a partial last segment (T*k not a multiple of
# 256), several segments per expert, and experts absent from the batch.
@pytest.mark.parametrize("name,T", [("tiny", 1001), ("olmoe", 300), ("qwen", 257)])
def test_large_batch_route_and_grouping(name, T):
    cfg = synth.CONFIGS[name]
    x, wr = synth.make_x(cfg, T, step=11), synth.make_router(cfg)
    fast = run_route(x, wr, cfg.k)
    exact = run_route(x, wr, cfg.k, exact=True)
    assert_same(fast, exact, f"{name} T={T}")
    ref = oracle.router_logits(x, wr)
    assert np.array_equal(fast["logits"].view(np.uint32), ref.view(np.uint32))
    ids, w = oracle.topk_softmax(ref, cfg.k)
    assert np.array_equal(fast["ids"], ids)
    assert np.allclose(fast["w"], w, rtol=1e-5, atol=1e-7)
    check_grouping(fast, ids, cfg.E, f"{name} T={T}")


def test_large_batch_skewed_grouping():
    # every token prefers experts 5 and 2 (bias): 600 pairs each spread over
    # five segments, the other experts absent
    cfg = synth.CONFIGS["tiny"]
    T = 600
    x, wr = synth.make_x(cfg, T, step=12), synth.make_router(cfg)
    bias = np.zeros(cfg.E, np.float32)
    bias[5], bias[2] = 50.0, 40.0
    got = run_route(x, wr, cfg.k, bias=bias)
    ref = oracle.router_logits(x, wr, bias)
    ids, _ = oracle.topk_softmax(ref, cfg.k)
    assert np.array_equal(got["ids"], ids)
    assert set(np.unique(ids)) == {2, 5}
    check_grouping(got, ids, cfg.E, "skewed T=600")


# Edges of the supported envelope: one expert (k = 1, every weight 1), k = E,
# an expert count that is not a multiple of 16, the largest hidden size the
# exact accumulators allow (H = 4096) on both paths, and the largest batch of
# the split-logits path (T = 256) next to the smallest of the other (257).
@pytest.mark.parametrize("H,E,k,T", [(256, 1, 1, 7), (256, 3, 3, 20), (512, 37, 5, 300), (4096, 64, 8, 5),
                                     (4096, 64, 8, 300), (2048, 64, 8, 256), (2048, 64, 8, 257)])
def test_route_envelope_edges(H, E, k, T):
    g = np.random.default_rng(H * 131 + E * 7 + T)
    x = g.standard_normal((T, H)).astype(np.float16)
    wr = (g.standard_normal((H, E)) * 0.02).astype(np.float16)
    got = run_route(x, wr, k)
    ref = oracle.router_logits(x, wr)
    assert np.array_equal(got["logits"].view(np.uint32), ref.view(np.uint32)), "logits"
    ids, w = oracle.topk_softmax(ref, k)
    assert np.array_equal(got["ids"], ids), "ids"
    assert np.allclose(got["w"], w, rtol=1e-5, atol=1e-7), "weights"
    if E == 1:
        assert np.all(got["w"] == 1.0)
    check_grouping(got, ids, E, f"H={H} E={E} k={k} T={T}")
