"""moe_route_static (routing without a caller workspace: its scratch is a fixed
device array inside the library) against moe_route with a caller workspace,
through the C ABI: every output bit for bit, on two calls in a row (a
large-batch call, then a smaller decode call that reuses the same array), and
the rejection of a batch whose workspace would exceed the array."""
import numpy as np
import pytest

from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def outputs(T, E, k, dev):
    """Fresh output buffers, filled with a sentinel so unwritten entries show."""
    n = max(T * k, 1)
    return dict(logits=torch.full((T, E), float("nan"), dtype=torch.float32, device=dev),
                ids=torch.full((T, k), -7, dtype=torch.int32, device=dev),
                w=torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
                offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                sorted_pairs=torch.full((n,), -7, dtype=torch.int32, device=dev),
                pair_pos=torch.full((n,), -7, dtype=torch.int32, device=dev),
                active=torch.full((E,), -7, dtype=torch.int32, device=dev),
                n_active=torch.full((1,), -7, dtype=torch.int32, device=dev))


def host(o):
    return {key: v.cpu().numpy() for key, v in o.items()}


def route_pair(cfg, T, step, bias_np=None):
    from w4a16_routed_expert_amd import binding as B
    dev = torch.device("cuda:0")
    E, k, H = cfg.E, cfg.k, cfg.H
    x = torch.from_numpy(synth.make_x(cfg, T, step=step)).to(dev)
    wr = torch.from_numpy(synth.make_router(cfg)).to(dev)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    ref = outputs(T, E, k, dev)
    nb = B.moe_route_workspace_size(T, H, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    B.moe_route(x, wr, bias, T, H, E, k, ref["logits"], ref["ids"], ref["w"], ref["offsets"], ref["sorted_pairs"],
                ref["pair_pos"], ref["active"], ref["n_active"], ws, nb)
    got = outputs(T, E, k, dev)
    B.moe_route_static(x, wr, bias, T, H, E, k, got["logits"], got["ids"], got["w"], got["offsets"],
                       got["sorted_pairs"], got["pair_pos"], got["active"], got["n_active"])
    torch.cuda.synchronize()
    return host(ref), host(got)


def test_static_route_equals_workspace_route_on_two_calls():
    from w4a16_routed_expert_amd import binding as B
    assert B.moe_route_static_max_bytes() == 1 << 20
    # first call: 1000 tokens of the prefill shape (the large-batch kernels,
    # per-segment counts in the scratch); second call, smaller: 32 tokens of the
    # Zipf-biased decode layer (logits handed between kernels in the scratch)
    cases = [(synth.CONFIGS["prefill"], 1000, 3, None),
             (synth.CONFIGS["olmoe_stack"], 32, 5, synth.make_zipf_bias(synth.CONFIGS["olmoe_stack"], layer=0))]
    for cfg, T, step, bias in cases:
        assert B.moe_route_workspace_size(T, cfg.H, cfg.E) <= B.moe_route_static_max_bytes()
        ref, got = route_pair(cfg, T, step, bias)
        for key in ref:
            a, b = ref[key], got[key]
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), \
                f"{cfg.name} T={T}: {key} differs from moe_route"
        assert int(got["n_active"][0]) > 0 and np.all(got["ids"] >= 0)


def test_static_route_rejects_a_batch_beyond_its_array():
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["prefill"]
    T = 5000                                     # 5000 x 64 FP32 logits > 1 MiB
    assert B.moe_route_workspace_size(T, cfg.H, cfg.E) > B.moe_route_static_max_bytes()
    dev = torch.device("cuda:0")
    o = outputs(T, cfg.E, cfg.k, dev)
    x = torch.zeros((T, cfg.H), dtype=torch.float16, device=dev)
    wr = torch.zeros((cfg.H, cfg.E), dtype=torch.float16, device=dev)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route_static(x, wr, None, T, cfg.H, cfg.E, cfg.k, o["logits"], o["ids"], o["w"], o["offsets"],
                           o["sorted_pairs"], o["pair_pos"], o["active"], o["n_active"])
    assert ei.value.code == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.all(o["ids"].cpu().numpy() == -7), "a rejected call must enqueue nothing"
