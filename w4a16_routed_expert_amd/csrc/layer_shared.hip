// The routed-expert layer of a decode batch together with its FP16 shared
// expert (the Qwen-shaped layer: routed experts plus one non-routed expert
// with a sigmoid gate; non-routed weights stay FP16, "horizonrunmap.com/en",
// section "08 / Precision & quality", paragraph "Other components").
//
// The shared expert needs x only, so it could run beside the routing, which
// is bound by latency and leaves HBM idle.  Two streams do not get there on
// this GPU: every launch's grid takes every compute unit, so a kernel of the
// other stream waits for CUs (measured: the Qwen-shaped step took as long
// with the shared expert on a second stream as with everything on one).
// Here the routing launch itself carries the shared expert's gate/up pass as
// extra blocks: blocks below the routing task count run the fused routing
// (logits of one (token, expert group) task, the last one also the top-k and
// the grouping), the others the gate/up units of the shared expert and its
// sigmoid gate.  For the one-token-tile plans fused here the kernel needs
// 103-245 VGPRs, and routing blocks run beside the pass's blocks, so the
// shared weights stream while the logits and the top-k run.  Then the
// routed expert FFN, the rest of the shared expert and the combine follow on
// the same stream.  Every block computes exactly what the
// separate launches compute (the same units with the same block stride), so
// the outputs are bit-identical to moe_shared_ffn followed by
// moe_layer_forward.
#include "route_dev.h"
#include "shared_dev.h"

namespace {

template <int MT>
union RouteSharedLds {
    FusedRouteLds r;
    shx::StreamLds<true, MT> s;
};

// Blocks [0, ntask): fused routing task blockIdx.x.  Blocks from ntask on:
// block b - ntask of the shared expert's gate/up pass as planned (RU-row
// units, MT token tiles per pass, NTW tiles per wavefront, nkc chunks of the
// reduction axis: with more than one, FP32 partial sums to the workspace;
// n_main unit blocks, then the sigmoid-gate blocks).
template <int MT, int NTW, int RU>
__global__ __launch_bounds__(kSelThreads) void route_shared_kernel(RouteArgs ra, unsigned int *done, int ntask,
                                                                  shx::SArgs sa, int nkc, int n_main)
{
    __shared__ RouteSharedLds<MT> L;
    __shared__ int s_last;
    if ((int)blockIdx.x < ntask) {
        fused_route_task<2>(ra, L.r, s_last, done, blockIdx.x, ntask);
        return;
    }
    shx::fp16_stream_block<true, MT, NTW, RU>(sa, nkc, n_main, sa.part, (int)blockIdx.x - ntask,
                                              (int)gridDim.x - ntask, L.s);
}

template <int MT, int NTW, int RU>
int launch_route_shared(const RouteArgs &ra, unsigned int *done, const shx::SArgs &sa, int nkc, hipStream_t s)
{
    const int ntask = ra.T * ((ra.E + kGroupE - 1) / kGroupE);
    int n_main = 0, n_sig = 0;
    shx::gateup_blocks(sa, &n_main, &n_sig);
    const unsigned int grid = (unsigned int)(ntask + n_main + n_sig);
    hipLaunchKernelGGL((route_shared_kernel<MT, NTW, RU>), dim3(grid), dim3(kSelThreads), 0, s, ra, done, ntask, sa,
                       nkc, n_main);
    return moe::check_launch("moe_layer_forward_shared (routing + shared gate/up)");
}

// The batches that take the fused launch: those whose gate/up pass is one
// token tile in 8-row units over the whole reduction axis (1-4 tiles per
// wavefront), where the routing occupies a few CUs and the pass streams on
// the rest.  Wider plans (16-row units, 2 or 4 token tiles, split axis) were
// measured no faster fused (Qwen shape T = 32 95.6 against 94.8 us per step,
// T = 64 111.9 against 111.8): the routing then has a block on most CUs, and
// the pass, planned for one block per CU, shares them.
bool plan_fused(const shx::GateupPlan &p) { return p.ru == 8 && p.mt == 1 && p.ntw >= 1 && p.ntw <= 4; }

int launch_planned(const shx::GateupPlan &p, const RouteArgs &ra, unsigned int *done, const shx::SArgs &sa,
                   hipStream_t s)
{
    switch (p.ntw) {
    case 1: return launch_route_shared<1, 1, 8>(ra, done, sa, p.nkc, s);
    case 2: return launch_route_shared<1, 2, 8>(ra, done, sa, p.nkc, s);
    case 3: return launch_route_shared<1, 3, 8>(ra, done, sa, p.nkc, s);
    default: return launch_route_shared<1, 4, 8>(ra, done, sa, p.nkc, s);
    }
}

}  // namespace

extern "C" {

int moe_layer_forward_shared(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I,
                             int E, int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                             const void *w_sgate_proj_dev, const void *w_sup_dev, const void *w_sdown_dev,
                             const void *w_sgate_dev, int Is, float *shared_out_dev, float *shared_gate_dev,
                             void *shared_ws_dev, size_t shared_ws_bytes, void *y_dev, const moe_layer_buffers *b,
                             int mode, void *stream)
{
    moe::clear_error();
    const char *who = "moe_layer_forward_shared";
    hipStream_t s = (hipStream_t)stream;
    shx::SArgs sa;
    int rc = shx::make_args(sa, x_dev, w_sgate_proj_dev, w_sup_dev, w_sdown_dev, w_sgate_dev, T, H, Is,
                            shared_out_dev, shared_gate_dev, shared_ws_dev, shared_ws_bytes, who);
    if (rc) return rc < 0 ? MOE_OK : rc;
    rc = moe::check_shape(T, H, I, E, k, true);
    if (rc) return rc;
    // the layer's own arguments first, so that a rejected call launches nothing
    if (mode != MOE_FFN_PATH_AUTO && mode != MOE_FFN_PATH_STREAM && mode != MOE_FFN_PATH_GEMM &&
        mode != MOE_FFN_PATH_KSPLIT && mode != MOE_FFN_PATH_ONE_LAUNCH)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: unknown mode %d", who, mode);
    if (!b || !w_router_dev || !rows_dev || !y_dev || !b->topk_ids || !b->topk_w || !b->expert_offsets ||
        !b->sorted_pairs || !b->pair_pos || !b->active_list || !b->n_active || !b->h || !b->pair_out)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: null pointer argument", who);
    if (!moe::aligned(b->pair_out, 16) || !moe::aligned(y_dev, 8))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: pair_out needs 16-byte and y 8-byte alignment", who);
    const size_t need = moe_layer_workspace_size(T, H, I, E, k);
    if (!b->ws || b->ws_bytes < need || !moe::aligned(b->ws, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "%s: the layer workspace needs %zu bytes, 256-byte aligned", who, need);
    const shx::GateupPlan plan = shx::gateup_plan(T, H, Is);
    const bool stream_kernels = mode == MOE_FFN_PATH_STREAM || (mode == MOE_FFN_PATH_AUTO && (long long)T * k < 64LL * E);
    const bool fused = plan_fused(plan) && stream_kernels && T <= moe::kFusedMaxT && H <= kMaxH && E % 2 == 0 &&
                       moe::aligned(w_router_dev, 4) && moe::aligned(x_dev, 8);
    if (!fused) {
        // any other batch or mode: the shared expert, then the one-call layer, in stream order (a
        // shape that mode rejects is reported by moe_layer_forward, after the shared expert ran)
        rc = moe_shared_ffn(x_dev, w_sgate_proj_dev, w_sup_dev, w_sdown_dev, w_sgate_dev, T, H, Is, shared_out_dev,
                            shared_gate_dev, shared_ws_dev, shared_ws_bytes, stream);
        if (rc) return rc;
        return moe_layer_forward(x_dev, w_router_dev, bias_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev,
                                 shared_out_dev, shared_gate_dev, nullptr, y_dev, b, mode, stream);
    }
    RouteArgs a;
    a.x = (const uint16_t *)x_dev;
    a.wr = (const uint16_t *)w_router_dev;
    a.bias = bias_dev;
    a.T = T; a.H = H; a.E = E; a.k = k;
    a.logits = b->logits;
    a.ids = b->topk_ids;
    a.w = b->topk_w;
    a.offsets = b->expert_offsets;
    a.sorted_pairs = b->sorted_pairs;
    a.pair_pos = b->pair_pos;
    a.active = b->active_list;
    a.n_active = b->n_active;
    a.force_exact = 0;
    // the layer workspace: control words (the routing counter first), then the logits
    a.lbuf = (float *)((uint8_t *)b->ws + moe::kLayerCtrlBytes);
    unsigned int *done = (unsigned int *)b->ws;
    rc = launch_planned(plan, a, done, sa, s);
    if (rc) return rc;
    rc = moe_w4a16_expert_ffn(x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, b->expert_offsets,
                              b->sorted_pairs, b->active_list, b->n_active, b->h, b->pair_out, b->status, mode, stream);
    if (rc) return rc;
    rc = shx::launch_rest(sa, s, who);
    if (rc) return rc;
    return moe_combine(b->pair_out, b->pair_pos, b->topk_w, shared_out_dev, shared_gate_dev, T, H, k, y_dev, stream);
}

}  // extern "C"
