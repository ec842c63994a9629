"""GPU tests of the resident expert table (moe_table_*): misses travel host ->
pinned staging -> spare device rows, are published after the copies, least
recently used experts lose their copy above capacity, and the layer's output
with partial residency is bit-identical to the output with every expert
resident (same kernels, same bytes).
"""
import ctypes

import numpy as np
import pytest

import oracle
from parity_util import assert_close_rows
from w4a16_routed_expert_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def read_device(addr: int, nbytes: int) -> np.ndarray:
    """Copy device memory at a raw address to the host (HIP runtime, device-to-host)."""
    hip = ctypes.CDLL("libamdhip64.so")
    out = np.empty(nbytes, dtype=np.uint8)
    rc = hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(addr), ctypes.c_size_t(nbytes),
                       ctypes.c_int(2))
    assert rc == 0
    return out


class LruModel:
    """The table's policy restated in plain Python: spare rows lowest index first; above
    capacity, the least recently used experts outside the current step lose their copy
    (ties: lower expert id)."""

    def __init__(self, E, capacity, spare, initial):
        self.E, self.c = E, capacity
        self.slot_of = {e: i for i, e in enumerate(initial)}
        self.expert_in = list(initial) + [-1] * spare
        self.last = [0] * E
        self.step = 0
        self.active = set()
        self.n_misses = 0

    def misses(self, active):
        self.step += 1
        self.active = set()
        out = []
        for e in active:
            if e in self.active:
                continue
            self.active.add(e)
            self.last[e] = self.step
            if e not in self.slot_of:
                out.append(e)
        self.n_misses += len(out)
        return out

    def evict_one(self):
        cand = [e for e in self.slot_of if e not in self.active]
        if not cand:
            return False
        v = min(cand, key=lambda e: (self.last[e], e))
        self.expert_in[self.slot_of.pop(v)] = -1
        return True

    def upload(self, misses):
        while sum(e < 0 for e in self.expert_in) < len(misses):
            assert self.evict_one()
        spare = [s for s, e in enumerate(self.expert_in) if e < 0]
        for e, s in zip(misses, spare):
            self.slot_of[e] = s
            self.expert_in[s] = e
        while len(self.slot_of) > self.c and self.evict_one():
            pass

    def published(self):
        m = np.full(self.E, -1, np.int32)
        for e, s in self.slot_of.items():
            m[e] = s
        return m


def make_table(cfg, rows, capacity, spare, initial=None, staging=2):
    from w4a16_routed_expert_amd.layer import ResidentExpertTable
    return ResidentExpertTable(rows, cfg.H, cfg.I, capacity, spare, staging, initial)


def test_uploads_publish_lru_and_bytes():
    cfg = synth.CONFIGS["tiny"]
    rows = synth.make_expert_rows(cfg)
    digest = rows.sum(dtype=np.uint64), rows.tobytes()[:4096]
    tab = make_table(cfg, rows, capacity=3, spare=2)
    model = LruModel(cfg.E, 3, 2, [0, 1, 2])       # 5 rows: a 5-expert step evicts before uploading
    assert np.array_equal(tab.published(), model.published())
    for active in ([0, 5], [1, 2, 6], [6, 7], [3, 3, 4], [3, 0, 1], [2, 4, 5, 6, 7], [0, 1, 3]):
        want = model.misses(active)
        got = tab.prepare(np.array(active, np.int32))
        model.upload(want)
        assert list(got) == want, f"misses for {active}"
        assert np.array_equal(tab.published(), model.published()), f"published map after {active}"
        torch.cuda.synchronize()
        rows_dev, stride, smap = tab.device()
        dev_map = read_device(smap, 4 * cfg.E).view(np.int32)
        assert np.array_equal(dev_map, model.published()), "device map differs from the host mirror"
        row_bytes = synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
        for e, s in model.slot_of.items():
            assert np.array_equal(read_device(rows_dev + s * stride, row_bytes), rows[e, :row_bytes]), \
                f"device row of expert {e} (slot {s}) differs from the host source"
    st = tab.stats()
    row_bytes = synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
    assert st["misses"] == model.n_misses and st["h2d_bytes"] == st["misses"] * row_bytes
    assert st["expert_d2h_bytes"] == 0 and st["host_writes"] == 0
    assert st["hits"] + st["misses"] == 2 + 3 + 2 + 2 + 3 + 5 + 3
    assert (rows.sum(dtype=np.uint64), rows.tobytes()[:4096]) == digest, "the host source was written"
    tab.close()


def test_more_misses_than_spare_rows_is_a_capacity_error():
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["tiny"]
    tab = make_table(cfg, synth.make_expert_rows(cfg), capacity=3, spare=1)
    # 5 active experts need 5 rows; the table has 4 (0, 1, 2 are active, so none can be evicted)
    misses = B.moe_table_misses(tab.handle, np.array([0, 1, 2, 4, 5], np.int32))
    assert list(misses) == [4, 5]
    with pytest.raises(B.MoeError) as ei:
        B.moe_upload_expert_rows(tab.handle, misses)
    assert ei.value.code == B.MOE_ERR_CAPACITY
    with pytest.raises(B.MoeError) as ei:          # an expert already published is not a miss
        B.moe_upload_expert_rows(tab.handle, np.array([0], np.int32))
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    tab.close()


def run_layer(cfg, rows, wr, xs, bias=None, table=None):
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    dev = torch.device("cuda:0")
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev),
                            torch.from_numpy(wr).to(dev), None if bias is None else torch.from_numpy(bias).to(dev),
                            max_T=max(x.shape[0] for x in xs), device=dev)
    ys = []
    for x in xs:
        y = lay.forward(torch.from_numpy(x).to(dev), table=table)
        torch.cuda.synchronize()
        assert int(lay.status.cpu()[0]) == 0, "an active expert had no published row"
        ys.append(y.cpu().numpy().view(np.uint16).copy())
    return ys


# spare rows = min(E - capacity, T*k): enough for any step; the Qwen-shaped layer keeps 39 of
# its 60 experts resident
@pytest.mark.parametrize("name,capacity,spare,T", [("tiny", 3, 5, 4), ("olmoe_stack", 40, 24, 8),
                                                   ("qwen", 39, 21, 16), ("qwen", 39, 4, 1)])
def test_partial_residency_output_equals_full_residency(name, capacity, spare, T):
    cfg = synth.CONFIGS[name]
    rows = synth.make_expert_rows(cfg)
    wr = synth.make_router(cfg, layer=1)
    bias = synth.make_zipf_bias(cfg, layer=1)
    xs = [synth.make_x(cfg, T, step=s, layer=1) for s in range(4)]
    full = run_layer(cfg, rows, wr, xs, bias)
    tab = make_table(cfg, rows, capacity, spare)
    part = run_layer(cfg, rows, wr, xs, bias, table=tab)
    for s, (a, b) in enumerate(zip(full, part)):
        assert np.array_equal(a, b), f"{name} step {s}: output with partial residency differs"
    st = tab.stats()
    assert st["misses"] > 0 and st["expert_d2h_bytes"] == 0
    ref = oracle.layer(xs[0], wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias)
    assert_close_rows(part[0], ref["y"], f"{name} partial residency vs oracle")
    tab.close()
