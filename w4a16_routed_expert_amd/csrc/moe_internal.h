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
