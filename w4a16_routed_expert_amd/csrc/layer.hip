// The whole routed-expert layer in one call: route -> W4A16 gate/up + SiLU*up
// -> W4A16 down -> weighted combine (+ the gated shared-expert term).
//
// Decode batches (the streaming kernels, T <= 256) run with no host round
// trip and no wait of one block for another: routing in one launch (the last
// block to finish its logits runs the top-k and the grouping, 4 KB of logits
// handed over at device scope), then gate/up, down and the combine - four
// launches - or, on request (MOE_FFN_PATH_KSPLIT), the K-split expert FFN
// (gate/up and down of a slice of the intermediate axis in one block,
// partial outputs in planes) and the combine over the planes - three.  A combine
// folded into the down projection's epilogue (the
// last unit of a token combining it) was measured slower: the outputs of one
// launch would cross the XCDs' L2 caches either by write-back of whole
// caches per unit or by uncombined device-scope stores, costing more than the
// launch saved.  Larger batches (and the grouped GEMM) run the separate
// calls in order.  The pages' executors for the same layer (a scalar path,
// "Grouped T3", "top4-fused-v1": "Horizon RunMap - architecture", section
// "Regimes and executor boundaries") are prior art; their kernels are not
// published.
#include "moe_internal.h"

namespace {

constexpr size_t kCtrl = moe::kLayerCtrlBytes;      // control words: routing counter, one-launch layer counters
// AUTO never takes the K-split FFN: measured on the MI355X it loses to the
// streaming pair at every batch (OLMoE shape, one-call layer: T = 1 31.3 us
// against 28.1 us, the planes' combine costing more than the launch saved;
// T = 8 76.8 against 48.4 us); MOE_FFN_PATH_KSPLIT selects it.
constexpr int kKsplitAutoMaxT = 0;

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Bytes of the K-split planes of a batch of T tokens (0 if the path does not apply).
size_t planes_bytes_at(int T, int H, int I, int E, int k)
{
    const int w = moe::ffn_ksplit_width(T, H, I, E, k);
    return w ? (size_t)(I / w) * T * k * H * sizeof(float) : 0;
}

// The workspace serves every T' <= T: the planes part is the largest over
// those batches (the slice width, hence the plane count, depends on T').
size_t layer_ws_bytes(int T, int H, int I, int E, int k)
{
    size_t planes = 0;
    for (int t = 1; t <= T && t <= 16; ++t) {
        const size_t b = planes_bytes_at(t, H, I, E, k);
        if (b > planes) planes = b;
    }
    return kCtrl + moe::route_logits_bytes(T, E) + align256(planes);
}

}  // namespace

extern "C" {

size_t moe_layer_workspace_size(int T, int H, int I, int E, int k)
{
    if (T < 0 || T > 65536 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK || H <= 0 ||
        I <= 0)
        return 0;
    return layer_ws_bytes(T, H, I, E, k);
}

int moe_layer_forward(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I,
                      int E, int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                      const float *shared_out_dev, const float *shared_gate_dev, void *shared_ready_event,
                      void *y_dev, const moe_layer_buffers *b, int mode, void *stream)
{
    moe::clear_error();
    const char *who = "moe_layer_forward";
    int rc = moe::check_shape(T, H, I, E, k, true);
    if (rc) return rc;
    if (mode != MOE_FFN_PATH_AUTO && mode != MOE_FFN_PATH_STREAM && mode != MOE_FFN_PATH_GEMM &&
        mode != MOE_FFN_PATH_KSPLIT && mode != MOE_FFN_PATH_ONE_LAUNCH)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: unknown mode %d", who, mode);
    if (mode == MOE_FFN_PATH_ONE_LAUNCH && T > 0 && !moe::layer_persistent_supported(T, H, I, E, k))
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: the one-launch layer takes decode batches (1 <= T <= %d, "
                         "T*k < 64*E, E even) of the shapes it is built for, H/128 and I/128 in {(2, 4), (16, 8), "
                         "(16, 11)} (T=%d, H=%d, I=%d, E=%d, k=%d)", who, moe::kPersistentMaxT, T, H, I, E, k);
    const int width = T >= 1 ? moe::ffn_ksplit_width(T, H, I, E, k) : 0;
    if (mode == MOE_FFN_PATH_KSPLIT && T > 0 && width == 0)
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: the K-split expert FFN needs T <= 16, H <= 2048 with H/128 even "
                         "and I <= 2048 (T=%d, H=%d, I=%d)", who, T, H, I);
    if (T == 0) return MOE_OK;
    if (!b || !x_dev || !w_router_dev || !rows_dev || !y_dev || !b->topk_ids || !b->topk_w || !b->expert_offsets ||
        !b->sorted_pairs || !b->pair_pos || !b->active_list || !b->n_active || !b->h || !b->pair_out)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: null pointer argument", who);
    if ((shared_out_dev == nullptr) != (shared_gate_dev == nullptr))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: shared_out and shared_gate must both be given or both NULL", who);
    if (!moe::aligned(b->pair_out, 16) || !moe::aligned(y_dev, 8) || (shared_out_dev && !moe::aligned(shared_out_dev, 16)))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: pair_out/shared_out need 16-byte and y 8-byte alignment", who);
    const size_t need = layer_ws_bytes(T, H, I, E, k);
    if (!b->ws || b->ws_bytes < need || !moe::aligned(b->ws, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "%s: the workspace needs %zu bytes, 256-byte aligned", who, need);
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)b->ws;
    unsigned int *done = (unsigned int *)ws;
    void *route_ws = ws + kCtrl;
    const size_t route_ws_bytes = moe::route_logits_bytes(T, E);
    if (mode == MOE_FFN_PATH_ONE_LAUNCH) {
        if (shared_ready_event) {
            const hipError_t e = hipStreamWaitEvent(s, (hipEvent_t)shared_ready_event, 0);
            if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, "%s: waiting for the shared expert: %s", who,
                                                  hipGetErrorString(e));
        }
        return moe::layer_persistent(x_dev, w_router_dev, bias_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev,
                                     shared_out_dev, shared_gate_dev, y_dev, b, (float *)route_ws, (uint32_t *)ws, s);
    }
    const bool stream_kernels = mode == MOE_FFN_PATH_STREAM || mode == MOE_FFN_PATH_KSPLIT ||
                                (mode == MOE_FFN_PATH_AUTO && (long long)T * k < 64LL * E);
    const bool ksplit = mode == MOE_FFN_PATH_KSPLIT ||
                        (mode == MOE_FFN_PATH_AUTO && stream_kernels && width > 0 && T <= kKsplitAutoMaxT);
    if (stream_kernels && T <= moe::kFusedMaxT)
        rc = moe::route_fused(x_dev, w_router_dev, bias_dev, T, H, E, k, b->logits, b->topk_ids, b->topk_w,
                              b->expert_offsets, b->sorted_pairs, b->pair_pos, b->active_list, b->n_active,
                              (float *)route_ws, done, s);
    else
        rc = moe_route(x_dev, w_router_dev, bias_dev, T, H, E, k, b->logits, b->topk_ids, b->topk_w,
                       b->expert_offsets, b->sorted_pairs, b->pair_pos, b->active_list, b->n_active, route_ws,
                       route_ws_bytes, stream);
    if (rc) return rc;
    float *planes = (float *)(ws + kCtrl + route_ws_bytes);
    if (ksplit)
        rc = moe::ffn_ksplit(x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, b->expert_offsets,
                             b->sorted_pairs, b->active_list, b->n_active, b->h, b->status, planes, width, s);
    else
        rc = moe_w4a16_expert_ffn(x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, b->expert_offsets,
                                  b->sorted_pairs, b->active_list, b->n_active, b->h, b->pair_out, b->status,
                                  mode, stream);
    if (rc) return rc;
    if (shared_ready_event) {
        const hipError_t e = hipStreamWaitEvent(s, (hipEvent_t)shared_ready_event, 0);
        if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, "%s: waiting for the shared expert: %s", who,
                                              hipGetErrorString(e));
    }
    if (ksplit)
        return moe::combine_planes(planes, (size_t)T * k * H, I / width, b->pair_out, b->pair_pos, b->topk_w,
                                   shared_out_dev, shared_gate_dev, T, H, k, y_dev, s);
    return moe_combine(b->pair_out, b->pair_pos, b->topk_w, shared_out_dev, shared_gate_dev, T, H, k, y_dev, stream);
}

}  // extern "C"
