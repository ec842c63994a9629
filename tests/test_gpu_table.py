"""GPU tests of the resident expert table (moe_table_*): misses travel host ->
pinned staging -> spare device rows on the table's copy stream, each
transaction publishes a new generation after its copies, least recently used
experts lose their copy above capacity, an open lease keeps the rows its
generation names, and the layer's output with partial residency is
bit-identical to the output with every expert resident (same kernels, same
bytes) and matches the oracle, over consecutive layers of the Zipf-biased
OLMoE-shaped stack and on the Qwen-shaped layer with its shared expert.
The state machine itself is also tested without a GPU (test_table_cpu.py).
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
    """The table's policy restated in plain Python: misses take the lowest rows that the
    current generation does not name (no leases are held here); above capacity, the least
    recently used experts outside the current step lose their copy (ties: lower expert id)."""

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
        spare = [s for s, e in enumerate(self.expert_in) if e < 0]
        assert len(spare) >= len(misses)
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


def make_table(cfg, rows, capacity, spare, max_tokens, initial=None, staging=2, digests=None):
    from w4a16_routed_expert_amd.layer import ResidentExpertTable
    return ResidentExpertTable(rows, cfg.H, cfg.I, capacity, spare, staging, initial, top_k=cfg.k,
                               max_tokens=max_tokens, row_digests=digests)


def test_uploads_publish_lru_and_bytes():
    cfg = synth.CONFIGS["tiny"]
    rows = synth.make_expert_rows(cfg)
    digest = rows.sum(dtype=np.uint64), rows.tobytes()[:4096]
    # steps of up to 3 tokens x top-2: 5 spare rows (every expert fits)
    from w4a16_routed_expert_amd import binding as B
    tab = make_table(cfg, rows, capacity=3, spare=5, max_tokens=3,
                     digests=[B.moe_row_digest(rows[e]) for e in range(cfg.E)])
    model = LruModel(cfg.E, 3, 5, [0, 1, 2])
    assert np.array_equal(tab.published(), model.published())
    n_transactions = 0
    for active in ([0, 5], [1, 2, 6], [6, 7], [3, 3, 4], [3, 0, 1], [2, 4, 5, 6, 7], [0, 1, 3]):
        want = model.misses(active)
        n_transactions += len(want) > 0
        got = tab.prepare(np.array(active, np.int32))
        model.upload(want)
        assert list(got) == want, f"misses for {active}"
        assert np.array_equal(tab.published(), model.published()), f"published map after {active}"
        lease = tab.acquire()
        torch.cuda.synchronize()
        rows_dev, stride, smap = lease.rows_dev, lease.row_stride, lease.slot_map_dev
        assert (rows_dev, stride, smap) == tab.device()
        dev_map = read_device(smap, 4 * cfg.E).view(np.int32)
        assert np.array_equal(dev_map, model.published()), "device map differs from the host mirror"
        row_bytes = synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
        for e, s in model.slot_of.items():
            assert np.array_equal(read_device(rows_dev + int(s) * stride, row_bytes), rows[e, :row_bytes]), \
                f"device row of expert {e} (slot {s}) differs from the host source"
        tab.release(lease)
    st = tab.stats()
    row_bytes = synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
    assert st["misses"] == model.n_misses and st["h2d_bytes"] == st["misses"] * row_bytes
    assert st["expert_d2h_bytes"] == 0 and st["host_writes"] == 0 and st["open_leases"] == 0
    assert st["hits"] + st["misses"] == 2 + 3 + 2 + 2 + 3 + 5 + 3
    assert st["generation"] == 1 + n_transactions
    tab.verify_source()
    assert (rows.sum(dtype=np.uint64), rows.tobytes()[:4096]) == digest, "the host source was written"
    tab.close()


def test_open_lease_holds_rows_then_release_frees_them():
    # 5 rows (capacity 3 + 2 spares, steps of one token x top-2).  A lease on
    # generation 1 keeps rows 0-2 (experts 0, 1, 2); the first step puts 4, 5
    # into the spares and drops 0, 1 above capacity; the second step finds no
    # row its transaction may write until the lease is released.
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["tiny"]
    rows = synth.make_expert_rows(cfg)
    tab = make_table(cfg, rows, capacity=3, spare=2, max_tokens=1)
    held = tab.acquire()
    assert held.generation == 1
    tab.prepare(np.array([4, 5], np.int32))
    misses = tab.misses(np.array([6, 7], np.int32))
    assert list(misses) == [6, 7]
    with pytest.raises(B.MoeError) as ei:
        tab.upload(misses)
    assert ei.value.code == B.MOE_ERR_CAPACITY
    st = tab.stats()
    assert st["generation"] == 2 and st["open_leases"] == 1
    tab.release(held)
    tab.upload(misses)
    lease = tab.acquire()
    torch.cuda.synchronize()
    m = read_device(lease.slot_map_dev, 4 * cfg.E).view(np.int32)
    row_bytes = synth.expert_row_layout(cfg.H, cfg.I)["row_bytes"]
    for e in (6, 7):
        assert m[e] >= 0
        assert np.array_equal(read_device(lease.rows_dev + int(m[e]) * lease.row_stride, row_bytes),
                              rows[e, :row_bytes])
    tab.release(lease)
    with pytest.raises(B.MoeError) as ei:          # an expert already published is not a miss
        B.moe_upload_expert_rows(tab.handle, np.array([6], np.int32))
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    tab.close()


def test_source_identity_is_checked():
    from w4a16_routed_expert_amd import binding as B
    cfg = synth.CONFIGS["tiny"]
    rows = synth.make_expert_rows(cfg)
    dig = [B.moe_row_digest(rows[e]) for e in range(cfg.E)]
    tab = make_table(cfg, rows, capacity=3, spare=5, max_tokens=4, digests=dig)
    tab.verify_source()
    rows[2, 17] ^= 1                                   # the caller breaks its promise
    with pytest.raises(B.MoeError) as ei:
        tab.verify_source()
    assert ei.value.code == B.MOE_ERR_SOURCE and tab.stats()["host_writes"] == 1
    tab.close()


def run_layer(cfg, rows, wr, xs, bias=None, table=None, shared=None):
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    dev = torch.device("cuda:0")
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev),
                            torch.from_numpy(wr).to(dev), None if bias is None else torch.from_numpy(bias).to(dev),
                            max_T=max(x.shape[0] for x in xs), device=dev)
    sh = None
    if shared is not None:
        from w4a16_routed_expert_amd.layer import SharedExpert
        sh = SharedExpert(*(torch.from_numpy(np.ascontiguousarray(m)).to(dev) for m in shared),
                          max_T=max(x.shape[0] for x in xs), device=dev)
    ys = []
    for x in xs:
        y = lay.forward(torch.from_numpy(x).to(dev), table=table, shared=sh)
        torch.cuda.synchronize()
        lay.check_status()
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
    tab = make_table(cfg, rows, capacity, spare, max_tokens=T)
    part = run_layer(cfg, rows, wr, xs, bias, table=tab)
    for s, (a, b) in enumerate(zip(full, part)):
        assert np.array_equal(a, b), f"{name} step {s}: output with partial residency differs"
    st = tab.stats()
    assert st["misses"] > 0 and st["expert_d2h_bytes"] == 0
    ref = oracle.layer(xs[0], wr, rows, cfg.H, cfg.I, cfg.E, cfg.k, bias=bias)
    assert_close_rows(part[0], ref["y"], f"{name} partial residency vs oracle")
    tab.close()


def test_page_locked_source_is_copied_directly():
    # A pinned host source: misses go straight from it to the device (no
    # staging); the output equals full residency and every miss is a direct copy.
    cfg = synth.CONFIGS["olmoe_stack"]
    T = 8
    rows = synth.make_expert_rows(cfg, layer=4)
    wr = synth.make_router(cfg, layer=4)
    bias = synth.make_zipf_bias(cfg, layer=4)
    xs = [synth.make_x(cfg, T, step=s, layer=4) for s in range(3)]
    full = run_layer(cfg, rows, wr, xs, bias)
    from w4a16_routed_expert_amd.layer import ResidentExpertTable
    tab = ResidentExpertTable(rows, cfg.H, cfg.I, cfg.resident, min(cfg.E - cfg.resident, T * cfg.k),
                              top_k=cfg.k, max_tokens=T, pinned_source=True)
    part = run_layer(cfg, rows, wr, xs, bias, table=tab)
    for s, (a, b) in enumerate(zip(full, part)):
        assert np.array_equal(a, b), f"step {s}: pinned-source table differs from full residency"
    st = tab.stats()
    assert st["misses"] > 0 and st["direct_copies"] == st["misses"] and st["staging_waits"] == 0
    tab.close()


def test_table_forward_on_a_stream_that_is_not_current():
    # forward(table=..., stream=s) with s not torch's current stream: the
    # active-expert list is read back after the routing on s (not on the
    # current stream), the misses are uploaded before the FFN on s reads
    # them, and the output equals full residency; the status word stays clear.
    from w4a16_routed_expert_amd.layer import RoutedExpertLayer
    cfg = synth.CONFIGS["olmoe_stack"]
    T = 8
    rows = synth.make_expert_rows(cfg, layer=3)
    wr = synth.make_router(cfg, layer=3)
    bias = synth.make_zipf_bias(cfg, layer=3)
    xs = [synth.make_x(cfg, T, step=s, layer=3) for s in range(3)]
    full = run_layer(cfg, rows, wr, xs, bias)
    dev = torch.device("cuda:0")
    tab = make_table(cfg, rows, cfg.resident, min(cfg.E - cfg.resident, T * cfg.k), max_tokens=T)
    lay = RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.from_numpy(rows).to(dev),
                            torch.from_numpy(wr).to(dev), torch.from_numpy(bias).to(dev), max_T=T, device=dev)
    side = torch.cuda.Stream(device=dev)
    for s, x in enumerate(xs):
        xd = torch.from_numpy(x).to(dev)
        side.wait_stream(torch.cuda.current_stream())   # x was copied on the current stream
        y = lay.forward(xd, stream=side, table=tab)
        side.synchronize()
        lay.check_status(side)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), full[s]), f"step {s}"
    st = tab.stats()
    assert st["misses"] > 0 and st["open_leases"] == 0
    tab.close()


@pytest.mark.parametrize("T", [1, 32])
def test_olmoe_stack_two_layers_partial_residency_vs_oracle(T):
    # Two consecutive layers of the OLMoE-shaped stack (own weights, router and
    # Zipf(1.1) bias each), 40 of 64 experts resident, spare rows by the
    # create-time rule; three steps per layer; every layer's y against the
    # oracle and bit-identical to full residency.
    from layer_util import oracle_tokens
    cfg = synth.CONFIGS["olmoe_stack"]
    spare = min(cfg.E - cfg.resident, T * cfg.k)
    for layer in (5, 6):
        rows = synth.make_expert_rows(cfg, layer=layer)
        wr = synth.make_router(cfg, layer=layer)
        bias = synth.make_zipf_bias(cfg, layer=layer)
        xs = [synth.make_x(cfg, T, step=s, layer=layer) for s in range(3)]
        tab = make_table(cfg, rows, cfg.resident, spare, max_tokens=T)
        part = run_layer(cfg, rows, wr, xs, bias, table=tab)
        st = tab.stats()
        full = run_layer(cfg, rows, wr, xs, bias)
        for s, (a, b) in enumerate(zip(full, part)):
            assert np.array_equal(a, b), f"layer {layer} step {s}: partial residency differs from full"
        for s, x in enumerate(xs):
            ref = oracle_tokens(x, wr, rows, cfg, bias=bias)
            assert_close_rows(part[s], ref["y"], f"olmoe stack layer {layer} T={T} step {s} vs oracle")
        assert st["misses"] > 0 and st["expert_d2h_bytes"] == 0 and st["open_leases"] == 0
        tab.close()


def test_qwen_partial_residency_with_shared_expert_T64():
    # 39 of 60 experts resident, 64 tokens, the FP16 shared expert beside.
    from layer_util import oracle_tokens
    cfg = synth.CONFIGS["qwen"]
    T = 64
    rows = synth.make_expert_rows(cfg)
    wr = synth.make_router(cfg)
    shared = synth.make_shared(cfg)
    xs = [synth.make_x(cfg, T, step=s, layer=2) for s in range(2)]
    tab = make_table(cfg, rows, cfg.resident, min(cfg.E - cfg.resident, T * cfg.k), max_tokens=T)
    part = run_layer(cfg, rows, wr, xs, table=tab, shared=shared)
    full = run_layer(cfg, rows, wr, xs, shared=shared)
    for s, x in enumerate(xs):
        assert np.array_equal(full[s], part[s]), f"step {s}: partial residency differs from full"
        ref = oracle_tokens(x, wr, rows, cfg, shared=shared)
        assert_close_rows(part[s], ref["y"], f"qwen partial T=64 step {s} vs oracle")
    assert tab.stats()["misses"] > 0
    tab.close()


def test_residual_add_is_the_correctly_rounded_sum():
    # out = RN16(a + b): random values over the FP16 range, plus pairs whose sum
    # needs more bits than FP32 holds (a large value and a tiny one) and sums on
    # FP16 rounding midpoints
    from w4a16_routed_expert_amd import binding as B
    g = np.random.default_rng(3)
    a = (g.standard_normal(50_000) * np.exp2(g.integers(-14, 14, 50_000))).astype(np.float16)
    b = (g.standard_normal(50_000) * np.exp2(g.integers(-24, 14, 50_000))).astype(np.float16)
    a[:4] = np.array([2048.0, 1.0, 65504.0, -0.5], np.float16)
    b[:4] = np.array([1.0, 2.0 ** -11, 8.0, 2.0 ** -24], np.float16)      # ties and far-apart magnitudes
    want = oracle.double_to_half(oracle.half_to_double(a.view(np.uint16)) + oracle.half_to_double(b.view(np.uint16)))
    dev = torch.device("cuda:0")
    ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    out = torch.empty_like(ta)
    B.moe_residual_add(ta, tb, out, a.size)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), f"{int((got != want).sum())} sums differ"


def make_stack(cfg, L, T, prefetch, layer0=0):
    from w4a16_routed_expert_amd.layer import DecodeStack, RoutedExpertLayer
    dev = torch.device("cuda:0")
    layers, tables, host = [], [], []
    for l in range(layer0, layer0 + L):
        rows = synth.make_expert_rows(cfg, layer=l)
        host.append((rows, synth.make_router(cfg, layer=l), synth.make_zipf_bias(cfg, layer=l)))
        tab = make_table(cfg, rows, cfg.resident, min(cfg.E - cfg.resident, T * cfg.k), max_tokens=T)
        _, stride, _ = tab.device()
        layers.append(RoutedExpertLayer(cfg.H, cfg.I, cfg.E, cfg.k, torch.empty((1, stride), dtype=torch.uint8,
                                                                               device=dev),
                                        torch.from_numpy(host[-1][1]).to(dev), torch.from_numpy(host[-1][2]).to(dev),
                                        max_T=T, device=dev))
        tables.append(tab)
    return DecodeStack(layers, tables, prefetch=prefetch), host


@pytest.mark.parametrize("T", [1, 8])
def test_stack_prefetch_is_transparent_and_layers_match_the_oracle(T):
    # Four chained layers of the OLMoE-shaped stack (Zipf-biased routers, 40 of
    # 64 experts resident), three steps, with and without next-layer prefetch:
    # every layer's y and the stack's output are bit-identical either way;
    # prefetch turns demand misses into prefetch hits; each layer's y matches
    # the oracle on that layer's input, and the residual chain matches its
    # definition.
    from layer_util import oracle_tokens
    cfg = synth.CONFIGS["olmoe_stack"]
    L = 4
    dev = torch.device("cuda:0")
    runs = {}
    for prefetch in (False, True):
        stack, host = make_stack(cfg, L, T, prefetch)
        outs = []
        for s in range(3):
            x0 = torch.from_numpy(synth.make_x(cfg, T, step=30 + s)).to(dev)
            ys = []
            xL = stack.step(x0, ys=ys)
            torch.cuda.synchronize()
            for lay in stack.layers:
                lay.check_status()
            outs.append(([y.cpu().numpy().view(np.uint16).copy() for y in ys], xL.cpu().numpy().view(np.uint16)))
        st = [t.stats() for t in stack.tables]
        for t in stack.tables:
            t.close()
        runs[prefetch] = (outs, st, host)
    for s in range(3):
        for l in range(L):
            assert np.array_equal(runs[False][0][s][0][l], runs[True][0][s][0][l]), f"step {s} layer {l}: y differs"
        assert np.array_equal(runs[False][0][s][1], runs[True][0][s][1]), f"step {s}: stack output differs"
    plain, pre = runs[False][1], runs[True][1]
    assert sum(t["prefetched"] for t in plain) == 0
    assert sum(t["prefetch_hits"] for t in pre) > 0
    assert sum(t["misses"] for t in pre) < sum(t["misses"] for t in plain), "prefetch did not remove demand misses"
    # per-layer oracle on the first step, with the chain rebuilt from the GPU's own y
    ys, xL = runs[True][0][0]
    host = runs[True][2]
    x = synth.make_x(cfg, T, step=30)
    for l in range(L):
        rows, wr, bias = host[l]
        ref = oracle_tokens(x, wr, rows, cfg, bias=bias)
        assert_close_rows(ys[l], ref["y"], f"stack layer {l} T={T} vs oracle")
        x = oracle.double_to_half(oracle.half_to_double(x.view(np.uint16)) + oracle.half_to_double(ys[l]))
        x = x.view(np.float16)
    assert np.array_equal(x.view(np.uint16), xL), "residual chain differs from RN16(x + y)"
