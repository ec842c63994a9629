// Dequantization of qpacked expert rows into FP16 execution slots (the
// offload-qpacked profile: "Horizon RunMap - architecture", section
// "Historical contracts remain distinct"; "Horizon technical notes —
// publication edition v1", section "Precision is profile-specific").
//
// Each weight becomes the FP16 value nearest (code - 8) * scale: the product
// of a 4-bit integer and an FP16 scale is exact in FP32, so one conversion to
// FP16 rounds it once.  Slot layout of a matrix with R rows and K columns:
// 4096-byte tiles, tile (rg, kt) = rows 16rg..16rg+15 x columns
// 128kt..128kt+127 at byte (rg*K/128 + kt)*4096; piece q (1024 bytes at
// q*1024) holds, at byte (16g + r)*16, row 16rg + r, columns
// 128kt + 32g + 8q .. +7 as 8 FP16 values in order.  One thread writes one
// 16-byte group (coalesced) from 4 bytes of codes and one scale.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(const uint8_t *q_rows, size_t q_stride,
                                                                uint8_t *f_rows, size_t f_stride, int H, int I,
                                                                int off_q0, int off_q1, int off_q2, int off_s0,
                                                                int off_s1, int off_s2)
{
    const int row = blockIdx.z, m = blockIdx.y;                 // expert row, matrix (gate, up, down)
    const int R = m < 2 ? I : H, K = m < 2 ? H : I;
    const long long c = (long long)blockIdx.x * kThreads + threadIdx.x;   // 16-byte group of the matrix
    if (c >= (long long)R * K / 8) return;
    const int tile = (int)(c >> 8), q = (int)((c >> 6) & 3), lane = (int)(c & 63);
    const int g = lane >> 4, r = lane & 15;
    const int KT = K / 128, NB = (K + 255) / 256;
    const int rg = tile / KT, kt = tile % KT;
    const int off_q = m == 0 ? off_q0 : (m == 1 ? off_q1 : off_q2);
    const int off_s = m == 0 ? off_s0 : (m == 1 ? off_s1 : off_s2);
    const uint8_t *src = q_rows + (size_t)row * q_stride;
    const uint32_t codes = *reinterpret_cast<const uint32_t *>(src + off_q + (size_t)tile * 1024 + (16 * g + r) * 16 +
                                                               4 * q);
    const float s = (float)*reinterpret_cast<const _Float16 *>(src + off_s +
                                                               ((size_t)(rg * NB + kt / 2) * 16 + r) * 2);
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = (codes >> (8 * i)) & 0xFFu;          // columns 2i (low nibble) and 2i + 1
        const _Float16 lo = (_Float16)((float)((int)(b & 15u) - 8) * s);
        const _Float16 hi = (_Float16)((float)((int)(b >> 4) - 8) * s);
        out[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    uint8_t *dst = f_rows + (size_t)row * f_stride + (size_t)m * ((size_t)I * H * 2) + (size_t)tile * 4096 +
                   (size_t)q * 1024 + (size_t)lane * 16;
    *reinterpret_cast<uint4 *>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace

int moe::dequant_rows(const void *q_rows, size_t q_stride, void *f_rows, size_t f_stride, int n, int H, int I,
                      hipStream_t s)
{
    size_t off[6];
    const size_t qb = moe::row_bytes(H, I, off);
    const size_t fb = moe::row_bytes_fp16(H, I, nullptr);
    if (qb == 0 || H > 2048 || I > 2048)
        return moe::fail(MOE_ERR_UNSUPPORTED, "moe_dequant_expert_rows: H=%d, I=%d (multiples of 128, at most 2048)",
                         H, I);
    if (n < 0 || n > 65535) return moe::fail(MOE_ERR_INVALID_ARG, "moe_dequant_expert_rows: n=%d", n);
    if (n == 0) return MOE_OK;
    if (!q_rows || !f_rows || q_stride < qb || f_stride < fb || !moe::aligned(q_rows, 256) ||
        !moe::aligned(f_rows, 256) || q_stride % 256 || f_stride % 256)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_dequant_expert_rows: rows must be 256-byte aligned with strides "
                         ">= %zu (qpacked) and %zu (FP16), multiples of 256", qb, fb);
    const long long groups = (long long)H * I / 8;              // per matrix (all three have H*I values)
    const dim3 grid((unsigned int)((groups + kThreads - 1) / kThreads), 3, (unsigned int)n);
    hipLaunchKernelGGL(dequant_rows_kernel, grid, dim3(kThreads), 0, s, (const uint8_t *)q_rows, q_stride,
                       (uint8_t *)f_rows, f_stride, H, I, (int)off[0], (int)off[1], (int)off[2], (int)off[3],
                       (int)off[4], (int)off[5]);
    return moe::check_launch("moe_dequant_expert_rows");
}

extern "C" int moe_dequant_expert_rows(const void *q_rows_dev, size_t q_stride, void *f_rows_dev, size_t f_stride,
                                       int n, int H, int I, void *stream)
{
    moe::clear_error();
    return moe::dequant_rows(q_rows_dev, q_stride, f_rows_dev, f_stride, n, H, I, (hipStream_t)stream);
}
