"""GPU parity of the offload-qpacked profile (FP16 execution slots) through the C ABI.

The low-bit source is dequantized on the GPU into FP16 slots
(moe_dequant_expert_rows) and the expert FFN reads the slots
(moe_fp16_expert_ffn).  The slots are compared bit for bit with the oracle's
FP16 weights, read out of the documented tile layout; the layer with the
oracle's FP16-slot profile (oracle.layer(..., fp16_slots=True)) stage by
stage as in test_gpu_parity.py; and a resident expert table holding FP16
slots (misses copied qpacked, dequantized on the GPU) against the same layer
with every slot present.
"""
import numpy as np
import pytest

import oracle
from layer_util import check_full, gpu_layer, rows_of
from parity_util import assert_close_rows, f16_to_f64
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def unpack_slot_matrix(buf, R, K):
    """An FP16 slot matrix (tile layout of the header) -> dense [R][K] FP16 bits."""
    t = buf.view(np.uint16).reshape(R // 16, K // 128, 4, 4, 16, 8)    # rg, kt, q, g, r, e
    return t.transpose(0, 4, 1, 3, 2, 5).reshape(R, K)                  # rg r | kt g q e


@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen"])
def test_dequantized_slots_equal_the_oracle_fp16_weights(name):
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS[name]
    rows = rows_of(name)[:3]
    dev = torch.device("cuda:0")
    q = torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
    fb = B.moe_expert_row_bytes_fp16(cfg.H, cfg.I)
    assert fb == 3 * cfg.I * cfg.H * 2
    fstride = (fb + 255) // 256 * 256
    slots = torch.empty((3, fstride), dtype=torch.uint8, device=dev)
    B.moe_dequant_expert_rows(q, q.stride(0), slots, fstride, 3, cfg.H, cfg.I)
    torch.cuda.synchronize()
    got = slots.cpu().numpy()
    m = cfg.I * cfg.H * 2
    for e in range(3):
        want = oracle.dequant_expert(rows[e], cfg.H, cfg.I, fp16=True)
        for i, (R, K) in enumerate(((cfg.I, cfg.H), (cfg.I, cfg.H), (cfg.H, cfg.I))):
            dense = unpack_slot_matrix(got[e, i * m:(i + 1) * m].copy(), R, K)
            w = oracle.double_to_half(want[i])
            assert np.array_equal(dense, w), f"{name} expert {e} matrix {i}: slot values differ"


@pytest.mark.parametrize("name,T", [("tiny", 33), ("olmoe", 1), ("olmoe", 8), ("olmoe", 32), ("qwen", 1),
                                    ("qwen", 64)])
def test_fp16_slot_layer_matches_the_oracle_profile(name, T):
    cfg = synth.CONFIGS[name]
    rows, wr, x = rows_of(name), synth.make_router(cfg), synth.make_x(cfg, T, step=40)
    ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, want_h=True, fp16_slots=True)
    got = gpu_layer(cfg, rows, wr, x, fp16_slots=True)
    check_full(cfg, got, ref, f"fp16 slots {name} T={T}", rows=None)
    # stage-wise: the profile's own down projection on the GPU's h
    T_, k = got["ids"].shape
    sp, off = got["sorted_pairs"], got["offsets"]
    o = np.zeros((T_ * k, cfg.H))
    for e in np.unique(got["ids"]):
        _, _, Wd = oracle.dequant_expert(rows[e], cfg.H, cfg.I, fp16=True)
        lo, hi = off[e], off[e + 1]
        o[sp[lo:hi]] = f16_to_f64(got["h"][lo:hi].view(np.uint16)) @ Wd.T
    assert_close_rows(got["pair_out"].astype(np.float64), o[sp], f"fp16 slots {name} T={T}: o from the GPU's h",
                      floor=2.0 ** -8)


def test_fp16_slot_table_partial_residency():
    # The table holds FP16 slots: each miss is copied as qpacked bytes and
    # dequantized on the GPU into its slot; the output equals the layer with
    # every slot present, bit for bit, and the profile's oracle.
    from w4a16_routed_expert_amd.layer import ResidentExpertTable, RoutedExpertLayer
    cfg = synth.CONFIGS["olmoe_stack"]
    T = 8
    dev = torch.device("cuda:0")
    rows = synth.make_expert_rows(cfg, layer=2)
    wr, bias = synth.make_router(cfg, layer=2), synth.make_zipf_bias(cfg, layer=2)
    tab = ResidentExpertTable(rows, cfg.H, cfg.I, cfg.resident, min(cfg.E - cfg.resident, T * cfg.k), 2,
                              top_k=cfg.k, max_tokens=T, fp16_slots=True)
    _, stride, _ = tab.device()
    assert stride >= 3 * cfg.I * cfg.H * 2
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.empty((1, stride), dtype=torch.uint8, device=dev),
                            torch.from_numpy(wr).to(dev), torch.from_numpy(bias).to(dev), max_T=T, device=dev)
    for s in range(3):
        x = synth.make_x(cfg, T, step=50 + s, layer=2)
        y = lay.forward(torch.from_numpy(x).to(dev), table=tab)
        torch.cuda.synchronize()
        lay.check_status()
        full = gpu_layer(cfg, rows, wr, x, bias=bias, fp16_slots=True)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), full["y"].view(np.uint16)), f"step {s}"
        ref = oracle.layer(x, wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias, fp16_slots=True)
        assert_close_rows(y.cpu().numpy().view(np.uint16), ref["y"], f"fp16 slot table step {s} vs oracle")
    st = tab.stats()
    assert st["misses"] > 0 and st["h2d_bytes"] == st["misses"] * synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
    tab.close()
