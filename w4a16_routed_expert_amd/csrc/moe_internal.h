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

}  // namespace moe
