"""Device-buffer plumbing around the C ABI: one routed-expert layer.

RoutedExpertLayer owns the torch device buffers the C calls write into and
runs route -> expert FFN -> combine on one stream (a SharedExpert, if given,
on a second stream beside them).  It does no arithmetic of
its own: torch provides memory and streams, the HIP library does the work.
"""
from __future__ import annotations

import torch

from . import binding as B


class RoutedExpertLayer:
    """W4A16 routed-expert layer over qpacked expert rows that already sit in HBM.

    rows: uint8 CUDA tensor [n_slots, row_stride] (256-byte aligned rows).
    router: float16 CUDA tensor [H, E].  bias: float32 CUDA tensor [E] or None.
    slot_map: int32 CUDA tensor [E] (slot of each expert, -1 = absent) or None
    (expert e in slot e).
    """

    def __init__(self, H: int, I: int, E: int, k: int, rows: torch.Tensor, router: torch.Tensor,
                 bias: torch.Tensor | None = None, slot_map: torch.Tensor | None = None, max_T: int = 64,
                 device: str | torch.device = "cuda:0"):
        self.H, self.I, self.E, self.k = H, I, E, k
        self.row_bytes, self.offsets6 = B.moe_expert_row_bytes(H, I)
        if rows.dtype != torch.uint8 or rows.dim() != 2 or rows.shape[1] < self.row_bytes:
            raise ValueError("rows must be uint8 [n_slots, >= row_bytes]")
        self.rows, self.router, self.bias, self.slot_map = rows, router, bias, slot_map
        self.row_stride = rows.stride(0)
        self.device = torch.device(device)
        self.max_T = 0
        self._alloc(max_T)

    def _alloc(self, T: int):
        d, E, k, H, I = self.device, self.E, self.k, self.H, self.I
        n = max(T * k, 1)
        self.max_T = T
        self.logits = torch.empty((max(T, 1), E), dtype=torch.float32, device=d)
        self.topk_ids = torch.empty((max(T, 1), k), dtype=torch.int32, device=d)
        self.topk_w = torch.empty((max(T, 1), k), dtype=torch.float32, device=d)
        self.expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
        self.sorted_pairs = torch.empty(n, dtype=torch.int32, device=d)
        self.pair_pos = torch.empty(n, dtype=torch.int32, device=d)
        self.active_list = torch.empty(E, dtype=torch.int32, device=d)
        self.n_active = torch.empty(1, dtype=torch.int32, device=d)
        self.ws_bytes = B.moe_route_workspace_size(T, H, E)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=d)
        self.h = torch.empty((n, I), dtype=torch.float16, device=d)
        self.pair_out = torch.empty((n, H), dtype=torch.float32, device=d)
        self.status = torch.zeros(1, dtype=torch.int32, device=d)
        # host copy of [n_active, active_list] (pinned, so the copies are asynchronous), and the
        # event the host waits on for it
        self._act_host = torch.empty(E + 1, dtype=torch.int32, pin_memory=True)
        self._act_evt = torch.cuda.Event()
        # workspace of the one-call layer: zero-filled once, left zero by every call
        self.layer_ws = torch.zeros(max(B.moe_layer_workspace_size(T, H, I, E, k), 256), dtype=torch.uint8, device=d)
        self._bufs = B.layer_buffers(self.logits, self.topk_ids, self.topk_w, self.expert_offsets, self.sorted_pairs,
                                     self.pair_pos, self.active_list, self.n_active, self.h, self.pair_out,
                                     self.status, self.layer_ws, self.layer_ws.numel())

    def _rows(self, rows):
        """Rows, stride and slot map: the layer's own, or an explicit rows tensor with its stride."""
        if rows is None:
            return self.rows, self.row_stride, self.slot_map
        return rows, rows.stride(0), self.slot_map

    def route(self, x: torch.Tensor, stream=None, exact: bool = False):
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        if exact:
            B.moe_route_exact(x, self.router, self.bias, T, self.H, self.E, self.k, self.logits, self.topk_ids,
                              self.topk_w, self.expert_offsets, self.sorted_pairs, self.pair_pos, self.active_list,
                              self.n_active, self.ws, self.ws_bytes, stream)
        else:
            B.moe_route(x, self.router, self.bias, T, self.H, self.E, self.k, self.logits, self.topk_ids,
                        self.topk_w, self.expert_offsets, self.sorted_pairs, self.pair_pos, self.active_list,
                        self.n_active, self.ws, self.ws_bytes, stream)

    def ffn(self, x: torch.Tensor, stream=None, rows=None, lease=None, mode: int = B.MOE_FFN_PATH_AUTO,
            fp16_slots: bool = False):
        """Expert FFN over the rows tensor (or `rows`), or over the rows and map of a table lease
        (ResidentExpertTable.acquire).  mode: kernel family (B.MOE_FFN_PATH_AUTO / _STREAM / _GEMM).
        fp16_slots: the rows are FP16 execution slots (moe_fp16_expert_ffn) instead of qpacked rows."""
        T = x.shape[0]
        if lease is not None:
            rows_dev, stride, smap = lease.rows_dev, lease.row_stride, lease.slot_map_dev
        else:
            rows_dev, stride, smap = self._rows(rows)
        if fp16_slots:
            B.moe_fp16_expert_ffn(x, T, self.H, self.I, self.E, self.k, rows_dev, stride, smap, self.expert_offsets,
                                  self.sorted_pairs, self.active_list, self.n_active, self.h, self.pair_out,
                                  status=self.status, stream=stream)
            return
        B.moe_w4a16_expert_ffn(x, T, self.H, self.I, self.E, self.k, rows_dev, stride, smap, self.expert_offsets,
                               self.sorted_pairs, self.active_list, self.n_active, self.h, self.pair_out,
                               status=self.status, mode=mode, stream=stream)

    def combine(self, T: int, y: torch.Tensor, shared_out=None, shared_gate=None, stream=None):
        B.moe_combine(self.pair_out, self.pair_pos, self.topk_w, shared_out, shared_gate, T, self.H, self.k, y,
                      stream)

    def forward(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None, rows=None,
                shared_out=None, shared_gate=None, table=None, shared: "SharedExpert | None" = None,
                mode: int = B.MOE_FFN_PATH_AUTO, fp16_slots: bool = False) -> torch.Tensor:
        """y = layer(x); x float16 [T, H] on the device.  With a ResidentExpertTable the
        routed experts' misses are uploaded (host round trip of the active list; the copies
        run on the table's copy stream) and the expert FFN reads the rows and map of a lease
        on the new generation, released after it.  With a SharedExpert its FFN runs on a
        second stream, concurrently with the routing and the routed experts (it needs x
        only), and the combine waits for both."""
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float16, device=self.device)
        main = _torch_stream(stream)
        if shared is not None:
            side = shared.side_stream()
            side.wait_stream(main)
            shared.run(x, side)
            shared_out, shared_gate = shared.out, shared.gate
        self.route(x, main)
        lease = None
        if table is not None:
            table.prepare(self.active_experts(main), main)
            lease = table.acquire(main)
        self.ffn(x, main, rows, lease, mode, fp16_slots=fp16_slots or (table is not None and table.fp16_slots))
        if lease is not None:
            table.release(lease, main)
        if shared is not None:
            main.wait_stream(side)
        self.combine(T, y, shared_out, shared_gate, main)
        return y

    def forward_fused(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None, rows=None, lease=None,
                      shared: "SharedExpert | None" = None, mode: int = B.MOE_FFN_PATH_AUTO) -> torch.Tensor:
        """y = layer(x) through the one-call layer (moe_layer_forward: three or four launches for
        decode batches, no host round trip; mode B.MOE_FFN_PATH_KSPLIT forces the one-launch expert
        FFN of small batches).  rows/lease as for ffn().  With a SharedExpert its FFN runs
        on a second stream beside the routed work and the combine waits for its event (for
        decode batches forward_shared, which runs both on one stream with the shared gate/up
        pass inside the routing launch, was measured faster: Qwen shape T = 1 40.6 against
        48.9 us, T = 16 72.5 against 80.4)."""
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float16, device=self.device)
        main = _torch_stream(stream)
        if lease is not None:
            rows_dev, stride, smap = lease.rows_dev, lease.row_stride, lease.slot_map_dev
        else:
            rows_dev, stride, smap = self._rows(rows)
        sh_out = sh_gate = ready = None
        if shared is not None:
            side = shared.side_stream()
            side.wait_stream(main)
            shared.run(x, side)
            ready = shared.ready_event()
            ready.record(side)
            sh_out, sh_gate = shared.out, shared.gate
        B.moe_layer_forward(x, self.router, self.bias, T, self.H, self.I, self.E, self.k, rows_dev, stride, smap,
                            sh_out, sh_gate, ready, y, self._bufs, mode, main)
        if shared is not None:
            main.wait_stream(shared.side_stream())   # the side stream's work is joined before reuse
        return y

    def forward_shared(self, x: torch.Tensor, shared: "SharedExpert", y: torch.Tensor | None = None, stream=None,
                       rows=None, lease=None, mode: int = B.MOE_FFN_PATH_AUTO) -> torch.Tensor:
        """y = layer(x) with the shared expert, all on one stream (moe_layer_forward_shared): for
        decode batches the routing launch also runs the shared expert's gate/up pass; the
        result equals forward_fused's with the same shared expert."""
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float16, device=self.device)
        shared.ensure(T)
        if lease is not None:
            rows_dev, stride, smap = lease.rows_dev, lease.row_stride, lease.slot_map_dev
        else:
            rows_dev, stride, smap = self._rows(rows)
        B.moe_layer_forward_shared(x, self.router, self.bias, T, self.H, self.I, self.E, self.k, rows_dev, stride,
                                   smap, shared.wg, shared.wu, shared.wd, shared.wgate, shared.Is, shared.out,
                                   shared.gate, shared.ws, shared.ws.numel(), y, self._bufs, mode,
                                   _torch_stream(stream))
        return y

    def active_experts(self, stream=None):
        """Active expert ids of the last route, on the host.  The copies are ordered after
        the work already enqueued on `stream` (the stream the route ran on; None = the
        current stream), and the call waits for them."""
        self.enqueue_active_copy(stream).synchronize()
        return self.host_active()

    def enqueue_active_copy(self, stream=None) -> torch.cuda.Event:
        """Enqueues the copy of n_active and the active list to pinned host memory on `stream`
        (None = the current stream) and returns the event recorded after it; read them with
        host_active() once that event has completed.  Lets several layers' lists come back with
        one wait."""
        s = _torch_stream(stream)
        with torch.cuda.stream(s):
            self._act_host[:1].copy_(self.n_active, non_blocking=True)
            self._act_host[1:].copy_(self.active_list, non_blocking=True)
        self._act_evt.record(s)
        return self._act_evt

    def host_active(self):
        """The active expert ids copied by the last enqueue_active_copy (after its stream's wait)."""
        n = int(self._act_host[0])
        return self._act_host[1:1 + n].numpy().copy()

    def check_status(self, stream=None):
        """Raises MoeError if an expert FFN call since this layer's buffers were made
        found a routed expert without a device row (the status word is sticky; waits
        for `stream`)."""
        with torch.cuda.stream(_torch_stream(stream)):
            st = int(self.status.cpu()[0])
        if st != B.MOE_OK:
            raise B.MoeError(st, "expert FFN status word: a routed expert had no published device row"
                             if st == B.MOE_ERR_ABSENT_EXPERT else "expert FFN status word set")


def _torch_stream(stream):
    """A torch stream object for None (the current stream), a torch stream or a raw handle."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


class SharedExpert:
    """FP16 shared expert (moe_shared_ffn) with its output buffers and workspace.

    wg, wu: row-major float16 CUDA tensors [Is, H]; wd: [H, Is]; wgate: [H] (16-byte aligned).
    The matrices are packed into the tile8 layout the kernels read (moe_pack_fp16_tile8) once,
    here; the row-major inputs are not kept.
    out (FP32 [T, H]) and gate (FP32 [T]) hold the last run's shared_out and shared_gate.
    """

    def __init__(self, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor, wgate: torch.Tensor,
                 max_T: int = 64, device: str | torch.device = "cuda:0"):
        self.Is, self.H = wg.shape
        self.wg, self.wu, self.wd = B.pack_tile8(wg), B.pack_tile8(wu), B.pack_tile8(wd)
        self.wgate = wgate
        self.device = torch.device(device)
        self._side = None
        self.max_T = 0
        self.ws = torch.empty(256, dtype=torch.uint8, device=self.device)
        self._alloc(max_T)

    def _alloc(self, T: int):
        self.max_T = T
        self.out = torch.empty((max(T, 1), self.H), dtype=torch.float32, device=self.device)
        self.gate = torch.empty((max(T, 1),), dtype=torch.float32, device=self.device)

    def ready_event(self) -> torch.cuda.Event:
        """Event recorded after this expert's kernels (the one-call layer waits for it)."""
        if getattr(self, "_ready", None) is None:
            self._ready = torch.cuda.Event()
        return self._ready

    def side_stream(self) -> torch.cuda.Stream:
        """The second stream the layer forks this expert onto (default priority)."""
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
        return self._side

    def ensure(self, T: int):
        """Output buffers and workspace for a batch of T tokens (grown, never shrunk)."""
        if T > self.max_T:
            self._alloc(T)
        need = B.moe_shared_ffn_workspace_size(T, self.H, self.Is)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)

    def run(self, x: torch.Tensor, stream=None):
        T = x.shape[0]
        self.ensure(T)
        B.moe_shared_ffn(x, self.wg, self.wu, self.wd, self.wgate, T, self.H, self.Is, self.out, self.gate,
                         self.ws, self.ws.numel(), stream)


class ResidentExpertTable:
    """A resident expert table (moe_table_*) over an immutable host source of qpacked rows.

    host_rows: uint8 numpy array [E, stride] holding every expert's row; kept referenced (and
    never written) for the table's lifetime.  capacity experts stay published between steps;
    spare_rows device rows receive misses (at least what steps of max_tokens tokens with top_k
    experts need; moe_table_create checks it).  pinned_source: keep the source in page-locked
    host memory (a pinned copy made here), which the table copies misses from directly instead
    of through its staging buffers.
    """

    def __init__(self, host_rows, H: int, I: int, capacity: int, spare_rows: int, staging_rows: int = 2,
                 initial_resident=None, top_k: int = 1, max_tokens: int = 1, row_digests=None,
                 fp16_slots: bool = False, pinned_source: bool = False):
        import numpy as np
        self._pinned = None
        if pinned_source:
            self._pinned = torch.empty(host_rows.shape, dtype=torch.uint8, pin_memory=True)
            self._pinned.numpy()[...] = host_rows
            host_rows = self._pinned.numpy()
        self.host_rows = np.ascontiguousarray(host_rows)
        self.E = self.host_rows.shape[0]
        self.fp16_slots = fp16_slots
        self.handle = B.moe_table_create(self.E, H, I, capacity, spare_rows, staging_rows, top_k, max_tokens,
                                         self.host_rows, self.host_rows.strides[0], initial_resident, row_digests,
                                         slot_format=B.MOE_SLOT_FP16 if fp16_slots else B.MOE_SLOT_QPACKED)

    def device(self):
        """(rows, stride, map) of the current generation, without a lease."""
        return B.moe_table_device(self.handle)

    def misses(self, active):
        return B.moe_table_misses(self.handle, active)

    def upload(self, misses, stream=None):
        """One miss transaction; `stream` is ordered after the new generation's publication."""
        if len(misses):
            B.moe_upload_expert_rows(self.handle, misses, stream)

    def prepare(self, active, stream=None):
        """Start a step with these active experts: upload and publish the misses. Returns the misses."""
        misses = self.misses(active)
        self.upload(misses, stream)
        return misses

    def prefetch(self, expert_ids):
        """Speculative load of experts a later step is expected to route (no stream waits for it)."""
        B.moe_table_prefetch(self.handle, expert_ids)

    def acquire(self, stream=None):
        """Lease on the current generation (stream ordered after its publication)."""
        return B.moe_table_acquire(self.handle, stream)

    def release(self, lease, stream=None):
        B.moe_table_release(self.handle, lease, stream)

    def verify_source(self):
        B.moe_table_verify_source(self.handle)

    def stats(self) -> dict:
        return B.moe_table_stats(self.handle)

    def published(self):
        return B.moe_table_published(self.handle, self.E)

    def close(self):
        if self.handle:
            B.moe_table_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DecodeStack:
    """Decode through a stack of routed-expert layers with partial residency, chained by the
    residual stream: x_{l+1} = RN16(x_l + y_l) (moe_residual_add).

    Each layer: route, bring the active experts to the host, one miss transaction on the layer's
    ResidentExpertTable (copies on its copy stream), a lease on the new generation, the expert FFN
    on the lease's rows, release, combine (and the FP16 shared expert where given).  With
    prefetch, layer l+1's router is also applied to x_l before the host round trip of layer l (one
    wait serves both), and the experts it selects are loaded into layer l+1's table right after
    layer l's kernels are enqueued, so those copies overlap layer l's compute; layer l+1 then
    routes its real input and loads only what the prediction missed.  Speculative next-layer
    loading is named among related systems' staging semantics ("Horizon RunMap - Architecture,
    Experimental Evidence and Scope", "Architecture comparison matrix", row "Publication/staging
    semantics"); predicting from the residual stream is this implementation's reading.
    Results do not depend on prefetching: the same kernels read the same bytes.
    """

    def __init__(self, layers, tables, shared=None, prefetch: bool = False):
        self.layers, self.tables = list(layers), list(tables)
        self.shared = shared
        self.prefetch = prefetch
        self.L = len(self.layers)
        lay = self.layers[0]
        # predictors: the next layer's router (and bias) on buffers of their own
        self.preds = [None] + [RoutedExpertLayer(l.H, l.I, l.E, l.k, l.rows, l.router, l.bias, max_T=l.max_T,
                                                 device=l.device) for l in self.layers[1:]] if prefetch else None
        self.device = lay.device

    def step(self, x0: torch.Tensor, ys=None, timer=None) -> torch.Tensor:
        """Runs every layer on x0 (float16 [T, H]); returns x_L.  ys: optional list receiving each
        layer's y (copies).  timer: optional callable(layer, phase) for event timing."""
        T, H = x0.shape
        x = x0
        main = torch.cuda.current_stream()
        for l in range(self.L):
            lay, tab = self.layers[l], self.tables[l]
            lay.route(x, main)
            nxt = self.preds[l + 1] if self.prefetch and l + 1 < self.L else None
            if nxt is not None:
                nxt.route(x, main)
            sh = self.shared[l] if self.shared is not None else None
            if sh is not None:
                sh.run(x, main)
            # one wait brings back this layer's active list and the predicted next-layer list
            ev = lay.enqueue_active_copy(main)
            if nxt is not None:
                ev = nxt.enqueue_active_copy(main)
            ev.synchronize()
            active = lay.host_active()
            predicted = nxt.host_active() if nxt is not None else None
            tab.prepare(active, main)
            lease = tab.acquire(main)
            if timer:
                timer(l, "ffn_begin")
            lay.ffn(x, main, lease=lease, fp16_slots=tab.fp16_slots)
            if timer:
                timer(l, "ffn_end")
            tab.release(lease, main)
            y = torch.empty((T, H), dtype=torch.float16, device=self.device)
            if sh is not None:
                lay.combine(T, y, sh.out, sh.gate, main)
            else:
                lay.combine(T, y, stream=main)
            if predicted is not None:
                self.tables[l + 1].prefetch(predicted)
            if ys is not None:
                ys.append(y)
            x_next = torch.empty_like(x)
            B.moe_residual_add(x, y, x_next, T * H, main)
            x = x_next
        return x
