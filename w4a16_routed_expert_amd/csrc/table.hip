// Resident expert table: which experts have a published device row, and the
// miss path that brings a missing row to the GPU.
//
// The contract follows "Horizon RunMap - architecture", section "Immutable
// authority and miss lifecycle", and "Horizon technical notes — publication
// edition v1", section "Immutable cache — the scope of ADR 0009":
//   * the complete host source (every expert's qpacked row) belongs to the
//     caller, stays immutable and outlives the table; the table never writes
//     it and never copies an expert from the device back to the host;
//   * device rows are disposable copies; a miss moves the row through bounded
//     pinned staging into a row that readers do not see (a spare row), and
//     the new map is published only after the copies, in stream order;
//   * eviction discards a device copy (least recently used first); a row is
//     refilled only after the consumers recorded for earlier generations have
//     finished;
//   * capacity is fixed when the table is created.
// Host code plus one tiny kernel that writes the published map.
#include "moe_internal.h"

#include <condition_variable>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

namespace {

struct MapArgs {
    int32_t slot[MOE_MAX_EXPERTS];
};

// Publishes a map generation: one lane per expert.  Launched on the upload
// stream after the row copies, so kernels later in that stream read the new
// map and the rows it points to.
__global__ void publish_map_kernel(int32_t *map, MapArgs m, int E)
{
    const int e = threadIdx.x;
    if (e < E) map[e] = m.slot[e];
}

// Host copy of one row into pinned staging, split over a few persistent
// threads: one thread copying from pageable memory runs at about half the
// host-to-device link rate, so the link would wait for it.  copy() returns
// when every part is done; one caller at a time (calls on a table are
// serialized).
class CopyPool {
public:
    explicit CopyPool(int workers)
    {
        for (int i = 0; i < workers; ++i) th_.emplace_back([this, i] { run(i); });
    }
    ~CopyPool()
    {
        {
            std::lock_guard<std::mutex> lk(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto &t : th_) t.join();
    }
    void copy(uint8_t *dst, const uint8_t *src, size_t n)
    {
        const int parts = (int)th_.size() + 1;
        if (n < kMinSplit || th_.empty()) {
            std::memcpy(dst, src, n);
            return;
        }
        {
            std::lock_guard<std::mutex> lk(m_);
            dst_ = dst;
            src_ = src;
            n_ = n;
            pending_ = (int)th_.size();
            ++gen_;
        }
        cv_.notify_all();
        part(parts - 1, parts);           // the caller takes the last part
        std::unique_lock<std::mutex> lk(m_);
        done_.wait(lk, [this] { return pending_ == 0; });
    }

private:
    static constexpr size_t kMinSplit = 256 * 1024;

    void part(int i, int parts)
    {
        const size_t chunk = (n_ / parts + 63) / 64 * 64;
        const size_t b = (size_t)i * chunk, e = b + chunk < n_ ? b + chunk : n_;
        if (b < e) std::memcpy(dst_ + b, src_ + b, e - b);
    }
    void run(int i)
    {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(m_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            lk.unlock();
            part(i, (int)th_.size() + 1);
            lk.lock();
            if (--pending_ == 0) done_.notify_one();
        }
    }

    std::vector<std::thread> th_;
    std::mutex m_;
    std::condition_variable cv_, done_;
    uint8_t *dst_ = nullptr;
    const uint8_t *src_ = nullptr;
    size_t n_ = 0;
    int pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

constexpr int kCopyWorkers = 3;           // plus the calling thread

}  // namespace

struct moe_table {
    int E = 0, H = 0, I = 0;
    int capacity = 0, spare = 0, nslots = 0;
    size_t row_bytes = 0, row_stride = 0, host_stride = 0;
    const uint8_t *host = nullptr;          // caller's immutable source
    uint8_t *rows = nullptr;                // device [nslots][row_stride]
    int32_t *map_dev = nullptr;             // device [E]
    std::vector<int32_t> slot_of;           // published map (host mirror), -1 = absent
    std::vector<int32_t> expert_in;         // slot -> published expert, -1 = spare
    std::vector<uint64_t> last_use;         // expert -> step of last use
    std::vector<uint8_t> active_now;        // expert -> in the current step's active set
    uint64_t step = 0;
    std::vector<uint8_t *> staging;         // pinned host buffers of row_bytes
    std::vector<hipEvent_t> staging_done;   // copy out of staging i finished
    std::vector<bool> staging_used;
    size_t next_staging = 0;
    hipEvent_t consumers = nullptr;         // last recorded consumer event
    bool consumers_recorded = false;
    bool faulted = false;
    moe_table_counters ctr{};
    CopyPool *pool = nullptr;               // host-side staging copies
};

namespace {

int table_fail(moe_table *t, int code, const char *what, hipError_t e)
{
    if (t && code == MOE_ERR_FAULTED) t->faulted = true;
    return moe::fail(code, "%s: %s", what, hipGetErrorString(e));
}

void release(moe_table *t)
{
    if (!t) return;
    for (size_t i = 0; i < t->staging.size(); ++i) {
        if (t->staging_done[i]) (void)hipEventDestroy(t->staging_done[i]);
        if (t->staging[i]) (void)hipHostFree(t->staging[i]);
    }
    if (t->consumers) (void)hipEventDestroy(t->consumers);
    if (t->rows) (void)hipFree(t->rows);
    if (t->map_dev) (void)hipFree(t->map_dev);
    delete t->pool;
    delete t;
}

// Copies one expert's host row into device slot `slot` through a staging buffer.
int upload_row(moe_table *t, int e, int slot, hipStream_t s)
{
    const size_t i = t->next_staging;
    t->next_staging = (i + 1) % t->staging.size();
    if (t->staging_used[i]) {
        // the staging buffer is refilled only after its previous copy has left it
        if (hipEventQuery(t->staging_done[i]) == hipErrorNotReady) t->ctr.staging_waits++;
        hipError_t err = hipEventSynchronize(t->staging_done[i]);
        if (err != hipSuccess) return table_fail(t, MOE_ERR_FAULTED, "moe_upload_expert_rows (staging)", err);
    }
    t->pool->copy(t->staging[i], t->host + (size_t)e * t->host_stride, t->row_bytes);
    hipError_t err = hipMemcpyAsync(t->rows + (size_t)slot * t->row_stride, t->staging[i], t->row_bytes,
                                    hipMemcpyHostToDevice, s);
    if (err == hipSuccess) err = hipEventRecord(t->staging_done[i], s);
    if (err != hipSuccess) return table_fail(t, MOE_ERR_FAULTED, "moe_upload_expert_rows (copy)", err);
    t->staging_used[i] = true;
    t->ctr.h2d_bytes += t->row_bytes;
    return MOE_OK;
}

// Published expert outside the current step with the oldest use (ties: lower
// expert id), or -1.
int lru_outside_step(const moe_table *t)
{
    int victim = -1;
    for (int e = 0; e < t->E; ++e)
        if (t->slot_of[e] >= 0 && !t->active_now[e] && (victim < 0 || t->last_use[e] < t->last_use[victim]))
            victim = e;
    return victim;
}

int publish(moe_table *t, hipStream_t s)
{
    MapArgs m;
    for (int e = 0; e < MOE_MAX_EXPERTS; ++e) m.slot[e] = e < t->E ? t->slot_of[e] : -1;
    hipLaunchKernelGGL(publish_map_kernel, dim3(1), dim3(64), 0, s, t->map_dev, m, t->E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return table_fail(t, MOE_ERR_FAULTED, "moe_upload_expert_rows (publish)", err);
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_table_create(moe_table **out, const moe_table_desc *d, void *stream)
{
    moe::clear_error();
    if (!out || !d) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_create: null pointer argument");
    *out = nullptr;
    int rc = moe::check_shape(0, d->H, d->I, d->E, 1, true);
    if (rc) return rc;
    if (d->capacity < 1 || d->capacity > d->E || d->spare_rows < 0 || d->capacity + d->spare_rows > 4 * MOE_MAX_EXPERTS)
        return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: capacity %d / spare rows %d outside the envelope",
                         d->capacity, d->spare_rows);
    if (d->staging_rows < 1 || d->staging_rows > 16)
        return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: staging_rows %d outside [1, 16]", d->staging_rows);
    size_t off[6];
    const size_t rb = moe::row_bytes(d->H, d->I, off);
    if (!d->host_source || d->host_row_stride < rb)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_create: host source missing or stride < %zu", rb);
    std::vector<uint8_t> seen(d->E, 0);
    for (int i = 0; i < d->capacity; ++i) {
        const int e = d->initial_resident ? d->initial_resident[i] : i;
        if (e < 0 || e >= d->E || seen[e])
            return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_create: initial resident list invalid at %d", i);
        seen[e] = 1;
    }

    moe_table *t = new (std::nothrow) moe_table;
    if (!t) return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: out of host memory");
    t->E = d->E; t->H = d->H; t->I = d->I;
    t->capacity = d->capacity;
    t->spare = d->spare_rows;
    t->nslots = d->capacity + d->spare_rows;
    t->row_bytes = rb;
    t->row_stride = (rb + 255) / 256 * 256;
    t->host_stride = d->host_row_stride;
    t->host = (const uint8_t *)d->host_source;
    t->pool = new (std::nothrow) CopyPool(kCopyWorkers);
    if (!t->pool) {
        release(t);
        return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: out of host memory");
    }
    t->slot_of.assign(t->E, -1);
    t->expert_in.assign(t->nslots, -1);
    t->last_use.assign(t->E, 0);
    t->active_now.assign(t->E, 0);
    hipError_t err = hipMalloc(&t->rows, (size_t)t->nslots * t->row_stride);
    if (err == hipSuccess) err = hipMalloc(&t->map_dev, sizeof(int32_t) * t->E);
    for (int i = 0; err == hipSuccess && i < d->staging_rows; ++i) {
        uint8_t *p = nullptr;
        hipEvent_t ev = nullptr;
        err = hipHostMalloc(&p, rb, hipHostMallocDefault);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        t->staging.push_back(p);
        t->staging_done.push_back(ev);
        t->staging_used.push_back(false);
    }
    if (err == hipSuccess) err = hipEventCreateWithFlags(&t->consumers, hipEventDisableTiming);
    if (err != hipSuccess) {
        release(t);
        return moe::fail(MOE_ERR_CAPACITY, "moe_table_create: allocation failed: %s", hipGetErrorString(err));
    }
    // initial residents in slots 0..capacity-1, then the first map generation
    hipStream_t s = (hipStream_t)stream;
    for (int i = 0; i < t->capacity; ++i) {
        const int e = d->initial_resident ? d->initial_resident[i] : i;
        rc = upload_row(t, e, i, s);
        if (rc) {
            release(t);
            return rc;
        }
        t->slot_of[e] = i;
        t->expert_in[i] = e;
    }
    rc = publish(t, s);
    if (rc == MOE_OK && (err = hipStreamSynchronize(s)) != hipSuccess)
        rc = moe::fail(MOE_ERR_HIP, "moe_table_create: %s", hipGetErrorString(err));
    if (rc) {
        release(t);
        return rc;
    }
    t->ctr = moe_table_counters{};          // creation traffic is not a miss
    *out = t;
    return MOE_OK;
}

void moe_table_destroy(moe_table *t)
{
    if (!t) return;
    (void)hipDeviceSynchronize();           // no copy or kernel may still use the rows or staging
    release(t);
}

int moe_table_device(const moe_table *t, const void **rows_dev, size_t *row_stride, const int32_t **slot_map_dev)
{
    moe::clear_error();
    if (!t || !rows_dev || !row_stride || !slot_map_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_device: null pointer argument");
    *rows_dev = t->rows;
    *row_stride = t->row_stride;
    *slot_map_dev = t->map_dev;
    return MOE_OK;
}

int moe_table_misses(moe_table *t, const int32_t *active_host, int n, int32_t *miss_out, int *n_miss)
{
    moe::clear_error();
    if (!t || (n > 0 && (!active_host || !miss_out)) || !n_miss)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_misses: null pointer argument");
    if (t->faulted) return moe::fail(MOE_ERR_FAULTED, "moe_table_misses: the table faulted earlier");
    if (n < 0 || n > t->E) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_misses: n=%d outside [0, E]", n);
    for (int i = 0; i < n; ++i)
        if (active_host[i] < 0 || active_host[i] >= t->E)
            return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_misses: expert id %d outside [0, E)", active_host[i]);
    t->step++;
    std::fill(t->active_now.begin(), t->active_now.end(), 0);
    int m = 0;
    for (int i = 0; i < n; ++i) {
        const int e = active_host[i];
        if (t->active_now[e]) continue;         // listed twice
        t->active_now[e] = 1;
        t->last_use[e] = t->step;
        if (t->slot_of[e] >= 0) {
            t->ctr.hits++;
        } else {
            t->ctr.misses++;
            miss_out[m++] = e;
        }
    }
    t->ctr.steps++;
    *n_miss = m;
    return MOE_OK;
}

int moe_upload_expert_rows(moe_table *t, const int32_t *expert_ids, int n, void *stream)
{
    moe::clear_error();
    if (!t || (n > 0 && !expert_ids)) return moe::fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: null pointer");
    if (t->faulted) return moe::fail(MOE_ERR_FAULTED, "moe_upload_expert_rows: the table faulted earlier");
    if (n < 0 || n > t->E) return moe::fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: n=%d", n);
    std::vector<uint8_t> want(t->E, 0);
    for (int i = 0; i < n; ++i) {
        const int e = expert_ids[i];
        if (e < 0 || e >= t->E) return moe::fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: expert id %d", e);
        if (t->slot_of[e] >= 0 || want[e])
            return moe::fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: expert %d is resident or listed twice", e);
        want[e] = 1;
    }
    // rows readers of the coming step do not need: spare slots, and if there
    // are too few, the rows of least recently used experts outside this step
    int n_spare = 0;
    for (int sl = 0; sl < t->nslots; ++sl) n_spare += t->expert_in[sl] < 0;
    int n_free = n_spare;
    for (int e = 0; e < t->E; ++e) n_free += t->slot_of[e] >= 0 && !t->active_now[e];
    if (n_free < n)
        return moe::fail(MOE_ERR_CAPACITY, "moe_upload_expert_rows: %d misses but %d spare or evictable rows", n,
                         n_free);
    if (n == 0) return MOE_OK;
    while (n_spare < n) {
        const int victim = lru_outside_step(t);
        t->expert_in[t->slot_of[victim]] = -1;
        t->slot_of[victim] = -1;
        t->ctr.evictions++;
        ++n_spare;
    }
    std::vector<int> spare;
    for (int sl = 0; sl < t->nslots; ++sl)
        if (t->expert_in[sl] < 0) spare.push_back(sl);
    hipStream_t s = (hipStream_t)stream;
    if (t->consumers_recorded) {
        // spare rows may still be read by kernels of an earlier generation
        hipError_t err = hipStreamWaitEvent(s, t->consumers, 0);
        if (err != hipSuccess) return table_fail(t, MOE_ERR_HIP, "moe_upload_expert_rows (consumers)", err);
    }
    for (int i = 0; i < n; ++i) {
        const int rc = upload_row(t, expert_ids[i], spare[i], s);
        if (rc) return rc;
    }
    // publish: the uploaded experts become visible ...
    for (int i = 0; i < n; ++i) {
        t->slot_of[expert_ids[i]] = spare[i];
        t->expert_in[spare[i]] = expert_ids[i];
    }
    // ... and, above capacity, least recently used experts outside the current
    // step lose their device copy (ties: lower expert id)
    int published = 0;
    for (int e = 0; e < t->E; ++e) published += t->slot_of[e] >= 0;
    while (published > t->capacity) {
        const int victim = lru_outside_step(t);
        if (victim < 0) break;              // every published expert is in use this step
        t->expert_in[t->slot_of[victim]] = -1;
        t->slot_of[victim] = -1;
        t->ctr.evictions++;
        --published;
    }
    return publish(t, s);
}

int moe_table_record_consumers(moe_table *t, void *stream)
{
    moe::clear_error();
    if (!t) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_record_consumers: null table");
    hipError_t err = hipEventRecord(t->consumers, (hipStream_t)stream);
    if (err != hipSuccess) return moe::fail(MOE_ERR_HIP, "moe_table_record_consumers: %s", hipGetErrorString(err));
    t->consumers_recorded = true;
    return MOE_OK;
}

int moe_table_stats(const moe_table *t, moe_table_counters *out)
{
    moe::clear_error();
    if (!t || !out) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_stats: null pointer argument");
    *out = t->ctr;
    return MOE_OK;
}

int moe_table_published(const moe_table *t, int32_t *slot_map_host)
{
    moe::clear_error();
    if (!t || !slot_map_host) return moe::fail(MOE_ERR_INVALID_ARG, "moe_table_published: null pointer argument");
    for (int e = 0; e < t->E; ++e) slot_map_host[e] = t->slot_of[e];
    return MOE_OK;
}

}  // extern "C"
