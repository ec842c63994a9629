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
    moe::combine_cols4(pair_out, pair_pos, topk_w, shared_out, shared_gate, T, H, k, t, c4, y);
}

// out = RN16(a + b) elementwise for FP16 a, b: the sum of two FP16 values is
// exact in fp64, so one rounding to FP16 gives the correctly rounded result.
__global__ __launch_bounds__(256) void residual_add_kernel(const uint16_t *a, const uint16_t *b, uint16_t *out,
                                                           long long n)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const double s = (double)(float)__builtin_bit_cast(_Float16, a[i]) +
                     (double)(float)__builtin_bit_cast(_Float16, b[i]);
    out[i] = __builtin_bit_cast(uint16_t, (_Float16)s);
}

}  // namespace

extern "C" int moe_residual_add(const void *a_dev, const void *b_dev, void *out_dev, long long n, void *stream)
{
    moe::clear_error();
    if (n < 0) return moe::fail(MOE_ERR_INVALID_ARG, "moe_residual_add: n=%lld", n);
    if (n == 0) return MOE_OK;
    if (!a_dev || !b_dev || !out_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_residual_add: null pointer argument");
    hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned int)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t *)a_dev, (const uint16_t *)b_dev, (uint16_t *)out_dev, n);
    return moe::check_launch("moe_residual_add");
}

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
