// Weighted top-k combine of the routed expert outputs (plus an optional gated
// shared-expert term), rounded once to the FP16 output activation
// ("horizonrunmap.com/en", section "08 / Precision & quality": FP16
// activations, FP32 accumulation stages and explicit rounding).
//
// One thread produces 4 consecutive output columns of one token; the k pair
// outputs are summed in FP32 in slot order j = 0..k-1, so the result is the
// same on every run.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 64;

__global__ __launch_bounds__(kThreads) void combine_kernel(const float *pair_out, const int32_t *pair_pos,
                                                           const float *topk_w, const float *shared_out,
                                                           const float *shared_gate, int T, int H, int k,
                                                           uint16_t *y)
{
    const int per_token = (H / 4 + kThreads - 1) / kThreads;
    const int t = blockIdx.x / per_token;
    const int c4 = (blockIdx.x % per_token) * kThreads + threadIdx.x;
    if (c4 * 4 >= H) return;
    // all k positions and weights first, then all k row loads, so the loads overlap
    int pos[MOE_MAX_TOPK];
    float w[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        pos[j] = -1;
        w[j] = 0.0f;
        if (j < k) {
            pos[j] = pair_pos[(size_t)t * k + j];
            w[j] = topk_w[(size_t)t * k + j];
        }
    }
    float4 v[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (pos[j] >= 0 && pos[j] < T * k)       // a corrupted grouping is skipped, never read out of bounds
            v[j] = *reinterpret_cast<const float4 *>(pair_out + (size_t)pos[j] * H + c4 * 4);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j < k) {
            acc.x += w[j] * v[j].x; acc.y += w[j] * v[j].y; acc.z += w[j] * v[j].z; acc.w += w[j] * v[j].w;
        }
    }
    if (shared_out) {
        const float g = shared_gate[t];
        const float4 sv = *reinterpret_cast<const float4 *>(shared_out + (size_t)t * H + c4 * 4);
        acc.x += g * sv.x; acc.y += g * sv.y; acc.z += g * sv.z; acc.w += g * sv.w;
    }
    const _Float16 hx = (_Float16)acc.x, hy = (_Float16)acc.y, hz = (_Float16)acc.z, hw = (_Float16)acc.w;
    uint2 packed;
    packed.x = (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
    packed.y = (uint32_t)__builtin_bit_cast(uint16_t, hz) | ((uint32_t)__builtin_bit_cast(uint16_t, hw) << 16);
    *reinterpret_cast<uint2 *>(y + (size_t)t * H + c4 * 4) = packed;
}

}  // namespace

extern "C" int moe_combine(const float *pair_out_dev, const int32_t *pair_pos_dev, const float *topk_w_dev,
                           const float *shared_out_dev, const float *shared_gate_dev,
                           int T, int H, int k, void *y_dev, void *stream)
{
    moe::clear_error();
    if (T < 0 || T > 65536 || H <= 0 || H % 128 || k < 1 || k > MOE_MAX_TOPK)
        return moe::fail(MOE_ERR_UNSUPPORTED, "moe_combine: bad shape T=%d H=%d k=%d", T, H, k);
    if (T == 0) return MOE_OK;
    if (!pair_out_dev || !pair_pos_dev || !topk_w_dev || !y_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer argument");
    if ((shared_out_dev == nullptr) != (shared_gate_dev == nullptr))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_combine: shared_out and shared_gate must both be given or both NULL");
    if (!moe::aligned(pair_out_dev, 16) || !moe::aligned(y_dev, 8) || (shared_out_dev && !moe::aligned(shared_out_dev, 16)))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_combine: pair_out/shared_out need 16-byte and y 8-byte alignment");
    const int per_token = (H / 4 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned int)(T * per_token)), dim3(kThreads), 0, (hipStream_t)stream,
                       pair_out_dev, pair_pos_dev, topk_w_dev, shared_out_dev, shared_gate_dev, T, H, k,
                       (uint16_t *)y_dev);
    return moe::check_launch("moe_combine");
}
