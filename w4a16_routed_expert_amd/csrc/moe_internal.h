// Internal helpers shared by the HIP sources of libmoe_w4a16 (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/moe_w4a16.h"

namespace moe {

// Inclusive prefix sum of an int over the 64 lanes of a wavefront (DPP row
// shifts, then two row broadcasts carry the row totals forward).
__device__ inline int wave_inclusive_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Cross-lane sums without the LDS crossbar.  add_row_ror<N>: each lane adds
// the value N lanes away inside its row of 16 (DPP rotation); add_partner:
// adds the value of lane l ^ 16 (SIXTEEN) or l ^ 32 (gfx950 permlane swaps).
template <int N>
__device__ inline uint32_t ror_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xf, 0xf, false);
}

template <int N>
__device__ inline double add_row_ror(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = (uint64_t)ror_u32<N>((uint32_t)b) | ((uint64_t)ror_u32<N>((uint32_t)(b >> 32)) << 32);
    return v + __builtin_bit_cast(double, r);
}

template <int N>
__device__ inline float add_row_ror(float v)
{
    return v + __builtin_bit_cast(float, ror_u32<N>(__builtin_bit_cast(uint32_t, v)));
}

// One of the two swap results is the lane's own value, so XOR-ing both with
// it leaves the partner's.
template <bool SIXTEEN>
__device__ inline uint32_t partner_u32(uint32_t v)
{
    const auto r = SIXTEEN ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] ^ r[1] ^ v;
}

template <bool SIXTEEN>
__device__ inline double add_partner(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = (uint64_t)partner_u32<SIXTEEN>((uint32_t)b) |
                       ((uint64_t)partner_u32<SIXTEEN>((uint32_t)(b >> 32)) << 32);
    return v + __builtin_bit_cast(double, r);
}

template <bool SIXTEEN>
__device__ inline float add_partner(float v)
{
    return v + __builtin_bit_cast(float, partner_u32<SIXTEEN>(__builtin_bit_cast(uint32_t, v)));
}

// Sum over the lanes of the wavefront that share lane % EQ (EQ a power of two <= 64).
template <int EQ, typename V>
__device__ inline V sum_phases(V v)
{
    if constexpr (EQ <= 1) v = add_row_ror<1>(v);
    if constexpr (EQ <= 2) v = add_row_ror<2>(v);
    if constexpr (EQ <= 4) v = add_row_ror<4>(v);
    if constexpr (EQ <= 8) v = add_row_ror<8>(v);
    if constexpr (EQ <= 16) v = add_partner<true>(v);
    if constexpr (EQ <= 32) v = add_partner<false>(v);
    return v;
}

// Resident blocks per compute unit of kernel `kern` at `threads` threads on
// the current device, asked of the runtime once per device and kept in
// `cache` (one array per kernel: the caller's function-local static).  The
// query is host work on every launch otherwise.
template <typename K>
inline int blocks_per_cu(K kern, int threads, int (&cache)[64])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int occ = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (occ > 0) return occ;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess || occ <= 0) occ = 1;
    __atomic_store_n(&cache[dev], occ, __ATOMIC_RELAXED);
    return occ;
}

// Data handed between blocks of one launch.  Stores and loads at device
// scope (relaxed atomics: the sc1 bit, coherent across the XCDs' L2 caches)
// reach every block without write-back or invalidation of whole L2 caches
// (a device-scope fence does both, which costs microseconds per wave); a
// wave orders its device-scope stores before a counter update by waiting
// for them to complete (s_waitcnt vmcnt(0)).  Worth it for small data only:
// scattered device-scope stores bypass the L2's write combining.
__device__ inline void store_dev(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float load_dev(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ inline void store_dev(int32_t *p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline int32_t load_dev(const int32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void store_dev(uint32_t *p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline uint32_t load_dev(const uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Store or load plainly, or at device scope when DEV.
template <bool DEV, typename V>
__device__ inline void put(V *p, V v)
{
    if constexpr (DEV) store_dev(p, v);
    else *p = v;
}
template <bool DEV, typename V>
__device__ inline V get(const V *p)
{
    if constexpr (DEV) return load_dev(p);
    else return *p;
}
// Cache-policy operand of the buffer intrinsics for device-scope accesses
// (sc1: coherent across the XCDs' L2 caches, like the relaxed atomics above).
constexpr int kDevScope = 16;

// y[t][c4*4 .. c4*4+3] = RN16( sum_{j<k} topk_w[t][j] * pair_out[pair_pos[t*k+j]][..]
// (+ shared_gate[t] * shared_out[t][..]) ), FP32 in slot order: the combine of
// one token's 4 columns.
__device__ inline void combine_cols4(const float *pair_out, const int32_t *pair_pos, const float *topk_w,
                                     const float *shared_out, const float *shared_gate, int T, int H, int k, int t,
                                     int c4, uint16_t *y)
{
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

// Thread-local message behind moe_last_error().
void set_error(const char *fmt, ...);
void vset_error(const char *fmt, va_list ap);
void clear_error();

// Returns `code` after recording the formatted message.
int fail(int code, const char *fmt, ...);

// Checks the launch that was just enqueued.
int check_launch(const char *what);

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape envelope shared by every entry point.
int check_shape(int T, int H, int I, int E, int k, bool need_I);

size_t row_bytes(int H, int I, size_t *off6);
// FP16 execution-slot row (gate, up, down in 4096-byte tiles; no scale planes).
size_t row_bytes_fp16(int H, int I, size_t *off6);
// Dequantizes n qpacked rows into FP16 slot rows (dequant.hip).
int dequant_rows(const void *q_rows, size_t q_stride, void *f_rows, size_t f_stride, int n, int H, int I,
                 hipStream_t s);

// Pieces of the fused layer (moe_layer_forward).
constexpr int kFusedMaxT = 256;        // largest batch routed in one launch
// The layer workspace starts with this many bytes of control words (the
// routing launch's counter first, then the one-launch layer's counters); the
// routing logits follow.
constexpr size_t kLayerCtrlBytes = 1024;

// route.hip: logits, top-k and grouping of 1 <= T <= kFusedMaxT tokens in one
// launch.  lbuf: FP32 [T][E] (route_logits_bytes); done: a counter that is 0
// before the call and 0 after it.
int route_fused(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int E, int k,
                float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev, int32_t *expert_offsets_dev,
                int32_t *sorted_pairs_dev, int32_t *pair_pos_dev, int32_t *active_list_dev, int32_t *n_active_dev,
                float *lbuf, unsigned int *done, hipStream_t s);
size_t route_logits_bytes(int T, int E);

// combine.hip: the combine over n_planes planes of partial pair outputs
// (plane stride in floats), writing each pair's plane sum to sum_out.
int combine_planes(const float *planes, size_t plane_stride, int n_planes, float *sum_out,
                   const int32_t *pair_pos_dev, const float *topk_w_dev, const float *shared_out_dev,
                   const float *shared_gate_dev, int T, int H, int k, void *y_dev, hipStream_t s);

// expert_ffn.hip: the K-split expert FFN of the one-call layer (batches of at
// most 16 tokens): its slice width for a shape (0 = not applicable), and the
// launch, which writes h and the I / width planes of partial pair outputs
// [I/width][T*k][H] (FP32).
int ffn_ksplit_width(int T, int H, int I, int E, int k);
int ffn_ksplit(const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev, size_t row_stride,
               const int32_t *slot_map_dev, const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
               const int32_t *active_list_dev, const int32_t *n_active_dev, void *h_dev, int32_t *status_dev,
               float *planes, int width, hipStream_t s);

// layer_persistent.hip: the routed layer of a decode batch in one launch.
// The control words (layer_persistent_ctl_bytes, at the start of the layer
// workspace) are zero before and after each call; lbuf: FP32 [T][E].
constexpr int kPersistentMaxT = 64;
size_t layer_persistent_ctl_bytes();
bool layer_persistent_supported(int T, int H, int I, int E, int k);
int layer_persistent(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I, int E,
                     int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                     const float *shared_out_dev, const float *shared_gate_dev, void *y_dev,
                     const moe_layer_buffers *b, float *lbuf, uint32_t *ctl, hipStream_t s);

}  // namespace moe
