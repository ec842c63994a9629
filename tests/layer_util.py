"""Helpers of the GPU layer tests: cached expert rows, one layer call through
the C ABI with every intermediate read back, and the full comparison with the
oracle (routing bit for bit, h / expert outputs / y within tolerance)."""
import numpy as np

import oracle
from parity_util import STAGE_FLOOR, assert_close_rows, assert_h_close, error_report, f16_to_f64
from w4a16_routed_expert_amd import synth

_ROWS = {}


def rows_of(name):
    if name not in _ROWS:
        _ROWS[name] = synth.make_expert_rows(synth.CONFIGS[name])
    return _ROWS[name]


def gpu_layer(cfg, rows_np, wr, x, bias=None, slot_map=None, rows_dev=None, mode=None, shared=None, fused=False,
              fp16_slots=False, one_stream=False):
    """One layer call through the C ABI; mode: None (automatic) or a B.MOE_FFN_PATH_* value;
    shared: None or the FP16 shared expert (Wsg, Wsu, Wsd, wgate) as numpy arrays, run on a
    second stream beside the routed experts; fused: the one-call layer (moe_layer_forward)
    instead of the separate calls; one_stream: the layer with its shared expert in one call on
    one stream (moe_layer_forward_shared)."""
    import torch
    from w4a16_routed_expert_amd import binding as B
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer, SharedExpert
    dev = torch.device("cuda:0")
    T = x.shape[0]
    sh = None
    if shared is not None:
        sh = SharedExpert(*(torch.from_numpy(np.ascontiguousarray(m)).to(dev) for m in shared), max_T=max(T, 1),
                          device=dev)
    if rows_dev is None:
        rows_dev = torch.from_numpy(rows_np).to(dev)
    if fp16_slots:
        # every expert's row dequantized on the GPU into an FP16 execution slot
        fstride = (B.moe_expert_row_bytes_fp16(cfg.H, cfg.I) + 255) // 256 * 256
        slots = torch.empty((rows_dev.shape[0], fstride), dtype=torch.uint8, device=dev)
        B.moe_dequant_expert_rows(rows_dev, rows_dev.stride(0), slots, fstride, rows_dev.shape[0], cfg.H, cfg.I)
        rows_dev = slots
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, rows_dev, torch.from_numpy(wr).to(dev),
                            None if bias is None else torch.from_numpy(bias).to(dev),
                            None if slot_map is None else torch.from_numpy(slot_map).to(dev),
                            max_T=max(T, 1), device=dev)
    xd = torch.from_numpy(x).to(dev)
    if fp16_slots:
        y = lay.forward(xd, shared=sh, fp16_slots=True)
    elif one_stream:
        y = lay.forward_shared(xd, sh, mode=B.MOE_FFN_PATH_AUTO if mode is None else mode)
    else:
        fwd = lay.forward_fused if fused else lay.forward
        y = fwd(xd, mode=B.MOE_FFN_PATH_AUTO if mode is None else mode, shared=sh)
    torch.cuda.synchronize()
    n = T * cfg.k
    na = int(lay.n_active.cpu()[0]) if T else 0
    extra = {}
    if sh is not None:
        Is = shared[0].shape[0]
        extra = dict(shared_os=sh.out.cpu().numpy()[:T].astype(np.float64),
                     shared_sigma=sh.gate.cpu().numpy()[:T].astype(np.float64),
                     shared_hs=sh.ws[:T * Is * 2].cpu().numpy().view(np.uint16).reshape(T, Is).copy(),
                     shared=shared)
    return dict(**extra, y=y.cpu().numpy(), logits=lay.logits.cpu().numpy()[:T], ids=lay.topk_ids.cpu().numpy()[:T],
                w=lay.topk_w.cpu().numpy()[:T], offsets=lay.expert_offsets.cpu().numpy(),
                sorted_pairs=lay.sorted_pairs.cpu().numpy()[:n], pair_pos=lay.pair_pos.cpu().numpy()[:n],
                active=lay.active_list.cpu().numpy(), n_active=na, h=lay.h.cpu().numpy()[:n],
                pair_out=lay.pair_out.cpu().numpy()[:n], status=int(lay.status.cpu()[0]), layer=lay, x=x)


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
    return o, oracle.combine(o, got["w"].astype(np.float64), got.get("shared_os"), got.get("shared_sigma"))


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
        eq = assert_h_close(got["h"].view(np.uint16), ref["h"][ref["sorted_pairs"]], f"{what}: h")
        print(f"{what}: h bit-identical fraction {eq:.5f}")
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
    if ref.get("shared_os") is not None and got.get("shared_os") is not None:
        check_shared_stages(got, ref, got["shared"], f"{what}: shared expert")
    rel, norm = error_report(got["y"].view(np.uint16), ref["y"])
    print(f"{what}: max rel err (no floor) {rel:.3g}, max normwise {norm:.3g}")


def oracle_shared_h(x, shared, workers=None):
    """The oracle's FP16 shared-expert activations hs [T][Is] (oracle.swiglu_dense on the
    FP16 weights read exactly as doubles, one token per call, on host threads)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    Wsg, Wsu, Wsd, _ = (f16_to_f64(np.asarray(m).view(np.uint16)) for m in shared)
    T = x.shape[0]
    if workers is None:
        workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        hs = list(ex.map(lambda t: oracle.swiglu_dense(Wsg, Wsu, Wsd, x[t])[0], range(T)))
    return np.stack(hs) if T else np.zeros((0, Wsg.shape[0]), np.uint16)


def check_shared_stages(got, ref, shared, what):
    """Shared expert stage by stage: hs within one FP16 ulp of the oracle's; shared_out
    against the FP16 down weights applied to the GPU's own hs (elementwise, stage floor);
    the gate within 1e-6; shared_out against the oracle normwise."""
    x = got["x"]
    hs_ref = oracle_shared_h(x, shared)
    eq = assert_h_close(got["shared_hs"], hs_ref, f"{what}: hs")
    Wsd = f16_to_f64(np.asarray(shared[2]).view(np.uint16))
    os_st = f16_to_f64(got["shared_hs"]) @ Wsd.T
    assert_close_rows(got["shared_os"], os_st, f"{what}: shared_out from the GPU's hs", floor=STAGE_FLOOR)
    assert_close_rows(got["shared_os"], ref["shared_os"], f"{what}: shared_out", floor=1.0)
    assert np.allclose(got["shared_sigma"], ref["shared_sigma"], rtol=0, atol=1e-6), f"{what}: gate"
    print(f"{what}: hs bit-identical fraction {eq:.5f}")




def oracle_tokens(x, wr, rows, cfg, bias=None, shared=None, want_h=False, chunk=8, workers=None):
    """oracle.layer on a set of tokens, split into chunks run on host threads.

    Every token's route, expert outputs and y depend on that token only, so the
    per-token results equal one oracle call on all of them (the grouping
    fields, which depend on the whole batch, are dropped).  The oracle is plain
    C called through ctypes, which releases the GIL."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    T = x.shape[0]
    if workers is None:
        workers = max(1, min(16, os.cpu_count() or 1))
    parts = [(i, min(T, i + chunk)) for i in range(0, T, chunk)]

    def run(p):
        a, b = p
        sh = None if shared is None else shared
        return oracle.layer(x[a:b], wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias, shared=sh, want_h=want_h)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(run, parts))
    out = {}
    for key in ("y", "logits", "ids", "w", "o"):
        out[key] = np.concatenate([r[key] for r in res], axis=0)
    if want_h:
        out["h"] = np.concatenate([r["h"] for r in res], axis=0)
    if shared is not None:
        out["shared_os"] = np.concatenate([r["shared_os"] for r in res], axis=0)
        out["shared_sigma"] = np.concatenate([r["shared_sigma"] for r in res], axis=0)
    return out
