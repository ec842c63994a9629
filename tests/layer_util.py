"""Helpers of the GPU layer tests: cached expert rows, one layer call through
the C ABI with every intermediate read back, and the full comparison with the
oracle (routing bit for bit, h / expert outputs / y within tolerance)."""
import numpy as np

import oracle
from parity_util import STAGE_FLOOR, assert_close_rows, error_report, f16_to_f64
from w4a16_routed_expert_amd import synth

_ROWS = {}


def rows_of(name):
    if name not in _ROWS:
        _ROWS[name] = synth.make_expert_rows(synth.CONFIGS[name])
    return _ROWS[name]


def gpu_layer(cfg, rows_np, wr, x, bias=None, slot_map=None, rows_dev=None):
    import torch
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    dev = torch.device("cuda:0")
    T = x.shape[0]
    if rows_dev is None:
        rows_dev = torch.from_numpy(rows_np).to(dev)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, rows_dev, torch.from_numpy(wr).to(dev),
                            None if bias is None else torch.from_numpy(bias).to(dev),
                            None if slot_map is None else torch.from_numpy(slot_map).to(dev),
                            max_T=max(T, 1), device=dev)
    y = lay.forward(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    n = T * cfg.k
    na = int(lay.n_active.cpu()[0]) if T else 0
    return dict(y=y.cpu().numpy(), logits=lay.logits.cpu().numpy()[:T], ids=lay.topk_ids.cpu().numpy()[:T],
                w=lay.topk_w.cpu().numpy()[:T], offsets=lay.expert_offsets.cpu().numpy(),
                sorted_pairs=lay.sorted_pairs.cpu().numpy()[:n], pair_pos=lay.pair_pos.cpu().numpy()[:n],
                active=lay.active_list.cpu().numpy(), n_active=na, h=lay.h.cpu().numpy()[:n],
                pair_out=lay.pair_out.cpu().numpy()[:n], status=int(lay.status.cpu()[0]), layer=lay)


def stagewise(cfg, got, rows):
    """The oracle's down projection and combine applied to the GPU's own h and
    routing weights: expert outputs o (pair order t*k+j, fp64) and FP16 y.
    Removes the effect of h values that an FP32 and an fp64 evaluation round
    to neighbouring FP16 values, so what remains is the error of the down
    projection and the combine alone."""
    T, k = got["ids"].shape
    sp, off = got["sorted_pairs"], got["offsets"]
    o = np.zeros((T * k, cfg.H))
    for e in np.unique(got["ids"]):
        _, _, Wd = oracle.dequant_expert(rows[e], cfg.H, cfg.I)
        lo, hi = off[e], off[e + 1]
        o[sp[lo:hi]] = f16_to_f64(got["h"][lo:hi].view(np.uint16)) @ Wd.T
    return o, oracle.combine(o, got["w"].astype(np.float64))


def check_full(cfg, got, ref, what, rows=None):
    T, k = got["ids"].shape
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32)), f"{what}: logits not bit-exact"
    assert np.array_equal(got["ids"], ref["ids"]), f"{what}: expert ids differ"
    assert np.allclose(got["w"], ref["w"], rtol=1e-5, atol=1e-7), f"{what}: routing weights differ"
    assert np.allclose(got["w"].sum(axis=1), 1.0, atol=k * 2.0 ** -23)
    assert np.array_equal(got["offsets"], ref["offsets"]), f"{what}: expert offsets differ"
    assert np.array_equal(got["sorted_pairs"], ref["sorted_pairs"]), f"{what}: sorted pairs differ"
    assert np.array_equal(got["pair_pos"], ref["pair_pos"]), f"{what}: pair positions differ"
    assert got["n_active"] == ref["n_active"]
    assert np.array_equal(got["active"][:ref["n_active"]], ref["active"])
    assert np.all(got["active"][ref["n_active"]:] == -1)
    if ref.get("h") is not None:
        # grouped position pos holds pair sorted_pairs[pos]
        assert_close_rows(got["h"].view(np.uint16), ref["h"][ref["sorted_pairs"]], f"{what}: h")
    # Per-pair expert outputs are compared normwise (2e-3 of each pair's largest
    # output): a 1-ulp flip of a large FP16 h (ulp 2^-8 for h in [4, 8)) times a
    # large down weight moves single outputs by ~1e-4, which an elementwise test
    # of these unrounded intermediates would flag.  The layer output y below is
    # held to the elementwise criterion.
    o_ref = ref["o"][ref["sorted_pairs"]]
    assert_close_rows(got["pair_out"].astype(np.float64), o_ref, f"{what}: expert outputs", floor=1.0)
    assert_close_rows(got["y"].view(np.uint16), ref["y"], f"{what}: y")
    if rows is not None:
        o_st, y_st = stagewise(cfg, got, rows)
        assert_close_rows(got["pair_out"].astype(np.float64), o_st[got["sorted_pairs"]],
                          f"{what}: expert outputs from the GPU's h", floor=STAGE_FLOOR)
        assert_close_rows(got["y"].view(np.uint16), y_st, f"{what}: y from the GPU's h", floor=STAGE_FLOOR)
    rel, norm = error_report(got["y"].view(np.uint16), ref["y"])
    print(f"{what}: max rel err (no floor) {rel:.3g}, max normwise {norm:.3g}")


