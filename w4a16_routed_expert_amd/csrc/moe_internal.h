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

// Thread-local message behind moe_last_error().
void set_error(const char *fmt, ...);
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
