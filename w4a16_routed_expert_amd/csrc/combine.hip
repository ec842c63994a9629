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

// The combine over `planes` planes of partial pair outputs (the K-split
// expert FFN of the one-call layer).  Block = (token t, 64 columns); its 256
// threads are 16 plane groups x 16 column quads: thread (g, q) sums planes
// g, g + 16, ... (ascending) of the token's k pairs at columns 4q .. 4q+3 of
// the block; the 16 group sums of a pair meet in LDS in group order (the
// pair's output, also written to sum_out); then the threads of group 0 weight
// the k pairs in slot order, add the shared term and round, with the same
// arithmetic as the plain combine.  Every order is fixed: the result is the
// same on every run.
constexpr int kPG = 16, kPQ = 16, kPThreads = kPG * kPQ;

__global__ __launch_bounds__(kPThreads) void combine_planes_kernel(const float *planes_, size_t plane_stride,
                                                                   int planes, float *sum_out, const int32_t *pair_pos,
                                                                   const float *topk_w, const float *shared_out,
                                                                   const float *shared_gate, int T, int H, int k,
                                                                   uint16_t *y)
{
    __shared__ float4 red[kPG][MOE_MAX_TOPK][kPQ];
    __shared__ float4 tot[MOE_MAX_TOPK][kPQ];
    const int nb = H / 64;
    const int t = blockIdx.x / nb;
    const int col = (blockIdx.x % nb) * 64 + 4 * (threadIdx.x % kPQ);
    const int g = threadIdx.x / kPQ, q = threadIdx.x % kPQ;
    int pos[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        pos[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
        if (pos[j] >= T * k) pos[j] = -1;        // a corrupted grouping is skipped, never read out of bounds
    }
    float4 v[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = g; s < planes; s += kPG) {
        float4 u[MOE_MAX_TOPK];
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            if (pos[j] >= 0)
                u[j] = *reinterpret_cast<const float4 *>(planes_ + s * plane_stride + (size_t)pos[j] * H + col);
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            if (pos[j] >= 0) {
                v[j].x += u[j].x; v[j].y += u[j].y; v[j].z += u[j].z; v[j].w += u[j].w;
            }
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) red[g][j][q] = v[j];
    __syncthreads();
    if (g < k) {
        float4 o = red[0][g][q];
        for (int gg = 1; gg < kPG; ++gg) {
            const float4 r = red[gg][g][q];
            o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
        }
        tot[g][q] = o;
        if (sum_out && pos[g] >= 0) *reinterpret_cast<float4 *>(sum_out + (size_t)pos[g] * H + col) = o;
    }
    __syncthreads();
    if (g != 0) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j < k) {
            const float w = topk_w[(size_t)t * k + j];
            const float4 vj = tot[j][q];
            acc.x += w * vj.x; acc.y += w * vj.y; acc.z += w * vj.z; acc.w += w * vj.w;
        }
    }
    if (shared_out) {
        const float gs = shared_gate[t];
        const float4 sv = *reinterpret_cast<const float4 *>(shared_out + (size_t)t * H + col);
        acc.x += gs * sv.x; acc.y += gs * sv.y; acc.z += gs * sv.z; acc.w += gs * sv.w;
    }
    const _Float16 hx = (_Float16)acc.x, hy = (_Float16)acc.y, hz = (_Float16)acc.z, hw = (_Float16)acc.w;
    uint2 packed;
    packed.x = (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
    packed.y = (uint32_t)__builtin_bit_cast(uint16_t, hz) | ((uint32_t)__builtin_bit_cast(uint16_t, hw) << 16);
    *reinterpret_cast<uint2 *>(y + (size_t)t * H + col) = packed;
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

int moe::combine_planes(const float *planes, size_t plane_stride, int n_planes, float *sum_out,
                        const int32_t *pair_pos_dev, const float *topk_w_dev, const float *shared_out_dev,
                        const float *shared_gate_dev, int T, int H, int k, void *y_dev, hipStream_t s)
{
    if (T == 0) return MOE_OK;
    hipLaunchKernelGGL(combine_planes_kernel, dim3((unsigned int)(T * (H / 64))), dim3(kPThreads), 0, s, planes,
                       plane_stride, n_planes, sum_out, pair_pos_dev, topk_w_dev, shared_out_dev, shared_gate_dev, T,
                       H, k, (uint16_t *)y_dev);
    return moe::check_launch("moe_layer_forward (combine)");
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
