// Resident expert table on the GPU: the HIP transport of the table's state
// machine (table_core.h) and the moe_table_* C ABI.
//
// The contract follows "Horizon RunMap - architecture", section "Immutable
// authority and miss lifecycle", and "Horizon technical notes — publication
// edition v1", section "Immutable cache — the scope of ADR 0009"; the state
// machine that implements it is host code in table_core.h (also built and
// tested without a GPU).  This file supplies the device side: allocations,
// the copy stream, events, host-to-device copies and a one-block kernel that
// writes a generation's map.
#include "moe_internal.h"
#include "table_core.h"

namespace {

struct MapArgs {
    int32_t slot[MOE_MAX_EXPERTS];
};

// Writes one generation's map: one lane per expert.  Launched on the copy
// stream after the row copies, so kernels ordered after it read the new map
// and the rows it points to.
__global__ void publish_map_kernel(int32_t *map, MapArgs m, int E)
{
    const int e = threadIdx.x;
    if (e < E) map[e] = m.slot[e];
}

class HipTransport final : public tcore::Transport {
public:
    int alloc_device(void **p, size_t n) override { return note(hipMalloc(p, n)); }
    void free_device(void *p) override { (void)hipFree(p); }
    int alloc_pinned(void **p, size_t n) override { return note(hipHostMalloc(p, n, hipHostMallocDefault)); }
    void free_pinned(void *p) override { (void)hipHostFree(p); }
    int create_event(void **ev) override
    {
        hipEvent_t e = nullptr;
        const int rc = note(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        *ev = e;
        return rc;
    }
    void destroy_event(void *ev) override { (void)hipEventDestroy((hipEvent_t)ev); }
    int create_stream(void **s) override
    {
        hipStream_t st = nullptr;
        const int rc = note(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
        *s = st;
        return rc;
    }
    void destroy_stream(void *s) override { (void)hipStreamDestroy((hipStream_t)s); }
    int h2d_async(void *dst, const void *src, size_t n, void *s) override
    {
        return note(hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, (hipStream_t)s));
    }
    int record(void *ev, void *s) override { return note(hipEventRecord((hipEvent_t)ev, (hipStream_t)s)); }
    int event_sync(void *ev) override { return note(hipEventSynchronize((hipEvent_t)ev)); }
    int event_done(void *ev) override
    {
        const hipError_t e = hipEventQuery((hipEvent_t)ev);
        if (e == hipSuccess) return 1;
        if (e == hipErrorNotReady) return 0;
        note(e);
        return -1;
    }
    int stream_wait(void *s, void *ev) override
    {
        return note(hipStreamWaitEvent((hipStream_t)s, (hipEvent_t)ev, 0));
    }
    int stream_sync(void *s) override { return note(hipStreamSynchronize((hipStream_t)s)); }
    int publish(int32_t *map_dev, const int32_t *slots, int E, void *s) override
    {
        MapArgs m;
        for (int e = 0; e < MOE_MAX_EXPERTS; ++e) m.slot[e] = e < E ? slots[e] : -1;
        hipLaunchKernelGGL(publish_map_kernel, dim3(1), dim3(64), 0, (hipStream_t)s, map_dev, m, E);
        return note(hipGetLastError());
    }
    const char *message() override { return msg_; }
    // Page-locked host memory (hipHostMalloc, pinned torch tensors) reports
    // hipMemoryTypeHost; pageable memory is unregistered (or an error, which
    // is cleared so the next launch check does not see it).
    bool host_pinned(const void *p, size_t n) override
    {
        if (!p || n == 0) return false;
        auto pinned = [](const void *q) {
            hipPointerAttribute_t a{};
            if (hipPointerGetAttributes(&a, q) != hipSuccess) {
                (void)hipGetLastError();
                return false;
            }
            return a.type == hipMemoryTypeHost;
        };
        return pinned(p) && pinned(static_cast<const uint8_t *>(p) + n - 1);
    }
    // FP16 execution slots: the qpacked row goes to a device staging row, then
    // is dequantized into the slot (same stream, so the staging row is free
    // again for the next row)
    int row_upload(void *dst, const void *src, size_t n, void *s) override
    {
        if (!dev_stage_) return h2d_async(dst, src, n, s);
        if (h2d_async(dev_stage_, src, n, s)) return 1;
        if (moe::dequant_rows(dev_stage_, stage_stride_, dst, slot_stride_, 1, H_, I_, (hipStream_t)s) != MOE_OK) {
            msg_ = moe_last_error();
            return 1;
        }
        return 0;
    }
    int init_fp16_slots(int H, int I)
    {
        H_ = H;
        I_ = I;
        stage_stride_ = (moe::row_bytes(H, I, nullptr) + 255) / 256 * 256;
        slot_stride_ = (moe::row_bytes_fp16(H, I, nullptr) + 255) / 256 * 256;
        return alloc_device(&dev_stage_, stage_stride_);
    }
    ~HipTransport() override
    {
        if (dev_stage_) (void)hipFree(dev_stage_);
    }

private:
    int note(hipError_t e)
    {
        if (e == hipSuccess) return 0;
        msg_ = hipGetErrorString(e);
        return 1;
    }
    const char *msg_ = "";
    void *dev_stage_ = nullptr;
    int H_ = 0, I_ = 0;
    size_t stage_stride_ = 0, slot_stride_ = 0;
};

}  // namespace

int tcore::fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    moe::vset_error(fmt, ap);
    va_end(ap);
    return code;
}

struct moe_table {
    HipTransport tr;
    tcore::Table *core = nullptr;
};

extern "C" {

uint64_t moe_row_digest(const void *p, size_t n) { return p ? tcore::digest(p, n) : 0; }

int moe_table_create(moe_table **out, const moe_table_desc *d, void *stream)
{
    (void)stream;
    moe::clear_error();
    if (!out || !d) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_create: null pointer argument");
    *out = nullptr;
    moe_table *t = new (std::nothrow) moe_table;
    if (!t) return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: out of host memory");
    if (d->slot_format == MOE_SLOT_FP16 && moe::row_bytes(d->H, d->I, nullptr) != 0 &&
        t->tr.init_fp16_slots(d->H, d->I) != 0) {
        const int rc = moe::fail(MOE_ERR_CAPACITY, "moe_table_create: device staging row: %s", t->tr.message());
        delete t;
        return rc;
    }
    const int rc = tcore::Table::create(&t->tr, d, &t->core);
    if (rc) {
        delete t;
        return rc;
    }
    *out = t;
    return MOE_OK;
}

void moe_table_destroy(moe_table *t)
{
    if (!t) return;
    delete t->core;
    delete t;
}

int moe_table_device(const moe_table *t, const void **rows_dev, size_t *row_stride, const int32_t **slot_map_dev)
{
    moe::clear_error();
    if (!t || !rows_dev || !row_stride || !slot_map_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_device: null pointer argument");
    return t->core->device(rows_dev, row_stride, slot_map_dev);
}

int moe_table_misses(moe_table *t, const int32_t *active_host, int n, int32_t *miss_out, int *n_miss)
{
    moe::clear_error();
    if (!t || (n > 0 && (!active_host || !miss_out)) || !n_miss)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_misses: null pointer argument");
    return t->core->misses(active_host, n, miss_out, n_miss);
}

int moe_upload_expert_rows(moe_table *t, const int32_t *expert_ids, int n, void *stream)
{
    moe::clear_error();
    if (!t || (n > 0 && !expert_ids)) return moe::fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: null pointer");
    return t->core->upload(expert_ids, n, stream);
}

int moe_table_prefetch(moe_table *t, const int32_t *expert_ids, int n)
{
    moe::clear_error();
    if (!t || (n > 0 && !expert_ids)) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_prefetch: null pointer");
    return t->core->prefetch(expert_ids, n);
}

int moe_table_acquire(moe_table *t, void *stream, moe_table_lease *lease)
{
    moe::clear_error();
    if (!t || !lease) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_acquire: null pointer argument");
    return t->core->acquire(stream, lease);
}

int moe_table_release(moe_table *t, const moe_table_lease *lease, void *stream)
{
    moe::clear_error();
    if (!t || !lease) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_release: null pointer argument");
    return t->core->release(lease, stream);
}

int moe_table_verify_source(moe_table *t)
{
    moe::clear_error();
    if (!t) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_verify_source: null table");
    return t->core->verify_source();
}

int moe_table_stats(const moe_table *t, moe_table_counters *out)
{
    moe::clear_error();
    if (!t || !out) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_stats: null pointer argument");
    t->core->stats(out);
    return MOE_OK;
}

int moe_table_published(const moe_table *t, int32_t *slot_map_host)
{
    moe::clear_error();
    if (!t || !slot_map_host) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_published: null pointer argument");
    t->core->published(slot_map_host);
    return MOE_OK;
}

}  // extern "C"
