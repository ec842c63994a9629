// Host-side glue of libmoe_w4a16: error reporting, shape checks, row layout.
#include "moe_internal.h"

#include <cstring>

namespace moe {

static thread_local char g_err[512];

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void vset_error(const char *fmt, va_list ap) { vsnprintf(g_err, sizeof(g_err), fmt, ap); }

void clear_error() { g_err[0] = '\0'; }

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

int check_shape(int T, int H, int I, int E, int k, bool need_I)
{
    if (T < 0 || T > 65536) return fail(MOE_ERR_UNSUPPORTED, "T=%d outside [0, 65536]", T);
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
    if (k < 1 || k > E || k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k=%d outside [1, min(E, %d)]", k, MOE_MAX_TOPK);
    if (H <= 0 || H % 128) return fail(MOE_ERR_UNSUPPORTED, "H=%d must be a positive multiple of 128", H);
    if (need_I && (I <= 0 || I % 128)) return fail(MOE_ERR_UNSUPPORTED, "I=%d must be a positive multiple of 128", I);
    if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "T*k too large");
    return MOE_OK;
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t row_bytes(int H, int I, size_t *off6)
{
    if (H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
    const size_t nbH = (size_t)(H + 255) / 256, nbI = (size_t)(I + 255) / 256;
    const size_t sz[6] = {(size_t)I * H / 2, (size_t)I * H / 2, (size_t)H * I / 2,
                          (size_t)I * nbH * 2, (size_t)I * nbH * 2, (size_t)H * nbI * 2};
    size_t o = 0;
    for (int i = 0; i < 6; ++i) {
        if (off6) off6[i] = o;
        o = align256(o + sz[i]);
    }
    return o;
}

size_t row_bytes_fp16(int H, int I, size_t *off6)
{
    if (H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
    const size_t m = (size_t)I * H * 2;        // one FP16 matrix, a multiple of 4096 bytes
    if (off6) {
        off6[0] = 0;
        off6[1] = m;
        off6[2] = 2 * m;
        off6[3] = off6[4] = off6[5] = 3 * m;   // no scale planes
    }
    return 3 * m;
}

}  // namespace moe

extern "C" {

size_t moe_expert_row_bytes_fp16(int H, int I) { return moe::row_bytes_fp16(H, I, nullptr); }

int moe_version(void) { return 100; }

const char *moe_last_error(void) { return moe::g_err; }

size_t moe_expert_row_bytes(int H, int I, size_t *off6) { return moe::row_bytes(H, I, off6); }

}  // extern "C"
