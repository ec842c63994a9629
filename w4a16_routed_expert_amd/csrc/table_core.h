// Resident expert table: the host-side state machine behind moe_table_*.
//
// Plain C++ (no HIP types): every device action goes through a Transport, so
// the same code runs on the GPU (table.hip supplies a HIP transport) and in a
// host-only test build with a simulated transport, under address, undefined
// behaviour and thread sanitizers.  Not part of the C ABI.
//
// Contract ("Horizon RunMap - architecture", section "Immutable authority and
// miss lifecycle"; "Horizon technical notes — publication edition v1",
// section "Immutable cache — the scope of ADR 0009"):
//   * the host source holds every expert's row, belongs to the caller, and is
//     never written; its identity (a digest per row) and layout (every FP16
//     scale finite) are validated at creation, and can be re-checked later;
//   * a consumer captures a complete generation (a lease): the device map of
//     that generation and the rows it names stay valid until the lease is
//     released and the work it covers has finished;
//   * a miss transaction (serialized; one at a time per table) takes spare
//     rows that no generation a live lease can see still names, moves each
//     row host source -> bounded pinned staging -> spare row on the table's
//     copy stream (a staging buffer is refilled only after its previous copy
//     has retired), then publishes the new complete map as the next
//     generation, after the copies in stream order;
//   * eviction drops an expert from the next generation's map; its row
//     becomes reusable only after every lease on a generation that named it
//     has been released and its consumers have finished (the copy stream
//     waits for their events);
//   * a failure before publication leaves the previous generation
//     authoritative (nothing of the transaction becomes visible); an
//     ambiguous failure after publication faults the table;
//   * capacity is fixed at creation, which rejects too few spare rows or
//     staging buffers.
#pragma once

#include <condition_variable>
#include <cstdarg>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <system_error>
#include <thread>
#include <vector>

#include "../../include/moe_w4a16.h"

namespace tcore {

// Records a message for moe_last_error() and returns `code` (the embedding
// library defines it).
int fail(int code, const char *fmt, ...);

// Device actions the table needs.  Streams and events are opaque handles.
// Every call returns 0 on success or a non-zero error; message() describes
// the last error.
struct Transport {
    virtual ~Transport() {}
    virtual int alloc_device(void **p, size_t n) = 0;
    virtual void free_device(void *p) = 0;
    virtual int alloc_pinned(void **p, size_t n) = 0;
    virtual void free_pinned(void *p) = 0;
    virtual int create_event(void **ev) = 0;
    virtual void destroy_event(void *ev) = 0;
    virtual int create_stream(void **s) = 0;
    virtual void destroy_stream(void *s) = 0;
    // host (pinned) -> device, asynchronous on stream s
    virtual int h2d_async(void *dst, const void *src, size_t n, void *s) = 0;
    virtual int record(void *ev, void *s) = 0;
    virtual int event_sync(void *ev) = 0;
    // 1: done, 0: not yet, < 0: error
    virtual int event_done(void *ev) = 0;
    virtual int stream_wait(void *s, void *ev) = 0;
    virtual int stream_sync(void *s) = 0;
    // writes map_dev[e] = slots[e] for e < E, asynchronously on stream s
    virtual int publish(int32_t *map_dev, const int32_t *slots, int E, void *s) = 0;
    // one expert row (n host bytes in pinned staging) into device row dst,
    // asynchronously on s: a copy, or for FP16 execution slots a copy and a
    // dequantization into the slot
    virtual int row_upload(void *dst, const void *src, size_t n, void *s) { return h2d_async(dst, src, n, s); }
    // True when [p, p + n) is page-locked host memory the copy engine can read directly.
    virtual bool host_pinned(const void *p, size_t n) { (void)p; (void)n; return false; }
    virtual const char *message() = 0;
};

// 64-bit digest of a byte range (identity of a host row): 8-byte words mixed
// with a multiply-rotate step, then the length.
inline uint64_t digest(const void *p, size_t n)
{
    const uint8_t *b = static_cast<const uint8_t *>(p);
    uint64_t h = 0x243F6A8885A308D3ull ^ (uint64_t)n;
    size_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        std::memcpy(&w, b + i, 8);
        h = (h ^ w) * 0x9E3779B97F4A7C15ull;
        h = (h << 27) | (h >> 37);
    }
    uint64_t w = 0;
    for (size_t j = 0; i + j < n; ++j) w |= (uint64_t)b[i + j] << (8 * j);
    h = (h ^ w ^ (uint64_t)n) * 0xBF58476D1CE4E5B9ull;
    return h ^ (h >> 31);
}

// Host copy of one row into pinned staging, split over a few threads (one
// thread copying from pageable memory runs at about half the host-to-device
// link rate).  One pool per process, created on first use; calls from
// several tables are serialized.  If threads cannot be started the copies
// run on the calling thread.
class CopyPool {
public:
    // Worker threads besides the caller: MOE_COPY_THREADS - 1 if set (1..32
    // threads in all), else 3 (four threads copy a row; on the host of an
    // MI355X a decode stack's upload rate was the same with 4, 8 and 12).
    static CopyPool &get()
    {
        static CopyPool pool(configured_workers());
        return pool;
    }

    static int configured_workers()
    {
        const char *v = std::getenv("MOE_COPY_THREADS");
        if (v) {
            const int n = std::atoi(v);
            if (n >= 1 && n <= 32) return n - 1;
        }
        return 3;
    }

    void copy(uint8_t *dst, const uint8_t *src, size_t n)
    {
        std::lock_guard<std::mutex> one(call_);
        const int workers = (int)th_.size();
        if (n < kMinSplit || workers == 0) {
            std::memcpy(dst, src, n);
            return;
        }
        {
            std::lock_guard<std::mutex> lk(m_);
            dst_ = dst;
            src_ = src;
            n_ = n;
            pending_ = workers;
            ++gen_;
        }
        cv_.notify_all();
        part(workers, workers + 1, dst, src, n);   // the caller takes the last part
        std::unique_lock<std::mutex> lk(m_);
        done_.wait(lk, [this] { return pending_ == 0; });
    }

    int workers() const { return (int)th_.size(); }

    ~CopyPool()
    {
        {
            std::lock_guard<std::mutex> lk(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto &t : th_) t.join();
    }

private:
    static constexpr size_t kMinSplit = 256 * 1024;

    explicit CopyPool(int workers)
    {
        try {
            for (int i = 0; i < workers; ++i) th_.emplace_back([this, i] { run(i); });
        } catch (const std::system_error &) {
            // threads that did start keep serving; with none, copies run inline
        }
    }

    static void part(int i, int parts, uint8_t *dst, const uint8_t *src, size_t n)
    {
        const size_t chunk = (n / parts + 63) / 64 * 64;
        const size_t b = (size_t)i * chunk, e = b + chunk < n ? b + chunk : n;
        if (b < e) std::memcpy(dst + b, src + b, e - b);
    }

    void run(int i)
    {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(m_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            uint8_t *dst = dst_;
            const uint8_t *src = src_;
            const size_t n = n_;
            const int parts = (int)th_.size() + 1;
            lk.unlock();
            part(i, parts, dst, src, n);
            lk.lock();
            if (--pending_ == 0) done_.notify_one();
        }
    }

    std::vector<std::thread> th_;
    std::mutex call_, m_;
    std::condition_variable cv_, done_;
    uint8_t *dst_ = nullptr;
    const uint8_t *src_ = nullptr;
    size_t n_ = 0;
    int pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

// Layout of one qpacked expert row (byte offsets of the six sections and the
// row size; the same arithmetic as moe_expert_row_bytes).
inline size_t row_layout(int H, int I, size_t off[6])
{
    if (H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
    const size_t nbH = (size_t)(H + 255) / 256, nbI = (size_t)(I + 255) / 256;
    const size_t sz[6] = {(size_t)I * H / 2, (size_t)I * H / 2, (size_t)H * I / 2,
                          (size_t)I * nbH * 2, (size_t)I * nbH * 2, (size_t)H * nbI * 2};
    size_t o = 0;
    for (int i = 0; i < 6; ++i) {
        off[i] = o;
        o = (o + sz[i] + 255) / 256 * 256;
    }
    return o;
}

// Spare rows a table needs so that no step of at most max_tokens tokens ever
// lacks a free row: a step has at most A = min(E, max_tokens * k) active
// experts; after it at most max(capacity, A) experts stay published, so the
// next step's A misses need A + max(0, A - capacity) rows outside the
// published set, unless every expert fits (E - capacity).
inline int spare_needed(int E, int capacity, int k, int max_tokens)
{
    const long long a = (long long)max_tokens * k < E ? (long long)max_tokens * k : E;
    const long long need = a + (a > capacity ? a - capacity : 0);
    return (int)(need < E - capacity ? need : E - capacity);
}

class Table {
public:
    static constexpr int kMaps = 4;          // device maps of the last generations (a ring)
    static constexpr int kEvents = 64;       // consumer events per table

    // Creates the table, uploads the initial residents and publishes
    // generation 1 (waits for it).  On failure returns a code and *out = null.
    static int create(Transport *tr, const moe_table_desc *d, Table **out)
    {
        *out = nullptr;
        int rc = validate(d);
        if (rc) return rc;
        Table *t = new (std::nothrow) Table(tr);
        if (!t) return fail(MOE_ERR_CAPACITY, "moe_table_create: out of host memory");
        rc = t->init(d);
        if (rc) {
            delete t;
            return rc;
        }
        *out = t;
        return MOE_OK;
    }

    // Waits for the table's copies and for the consumers of released leases,
    // then frees everything.
    ~Table()
    {
        if (copy_) (void)tr_->stream_sync(copy_);
        if (copy2_) (void)tr_->stream_sync(copy2_);
        for (auto &g : gens_)
            for (auto &se : g.ev) (void)tr_->event_sync(se.ev);
        for (void *ev : recycle_) (void)tr_->event_sync(ev);
        for (void *ev : all_events_) tr_->destroy_event(ev);
        for (void *p : staging_) tr_->free_pinned(p);
        if (rows_) tr_->free_device(rows_);
        if (maps_) tr_->free_device(maps_);
        if (copy_) tr_->destroy_stream(copy_);
        if (copy2_) tr_->destroy_stream(copy2_);
    }

    int device(const void **rows, size_t *stride, const int32_t **map) const
    {
        *rows = rows_;
        *stride = row_stride_;
        *map = map_of(gen_);
        return MOE_OK;
    }

    // Starts a step: marks the active experts used now and lists those with no
    // published row.
    int misses(const int32_t *active, int n, int32_t *miss_out, int *n_miss)
    {
        if (faulted_) return fail(MOE_ERR_FAULTED, "moe_table_misses: the table faulted earlier");
        if (n < 0 || n > E_) return fail(MOE_ERR_INVALID_ARG, "moe_table_misses: n=%d outside [0, E]", n);
        for (int i = 0; i < n; ++i)
            if (active[i] < 0 || active[i] >= E_)
                return fail(MOE_ERR_INVALID_ARG, "moe_table_misses: expert id %d outside [0, E)", active[i]);
        step_++;
        std::fill(active_now_.begin(), active_now_.end(), 0);
        int m = 0;
        for (int i = 0; i < n; ++i) {
            const int e = active[i];
            if (active_now_[e]) continue;
            active_now_[e] = 1;
            last_use_[e] = step_;
            if (slot_of_[e] >= 0) {
                ctr_.hits++;
                if (prefetched_[e]) {
                    prefetched_[e] = 0;
                    ctr_.prefetch_hits++;
                }
            } else {
                ctr_.misses++;
                miss_out[m++] = e;
            }
        }
        ctr_.steps++;
        *n_miss = m;
        return MOE_OK;
    }

    // One miss transaction: copies the n experts' rows into free spare rows
    // and publishes the next generation; `consumer` is ordered after the
    // publication (a null handle is the default stream, as in HIP).
    int upload(const int32_t *ids, int n, void *consumer) { return transact(ids, n, consumer, true); }

    // Speculative load of experts a later step is expected to route: starts a
    // step with these ids as its active set (so the transaction's eviction
    // keeps them), and uploads those without a published row as one
    // transaction that no stream waits for (a later acquire orders its
    // consumer after the publication).  Counted as prefetches, not misses;
    // a prefetched expert that a later step routes counts a prefetch hit.
    int prefetch(const int32_t *ids, int n)
    {
        if (faulted_) return fail(MOE_ERR_FAULTED, "moe_table_prefetch: the table faulted earlier");
        if (n < 0 || n > E_) return fail(MOE_ERR_INVALID_ARG, "moe_table_prefetch: n=%d outside [0, E]", n);
        for (int i = 0; i < n; ++i)
            if (ids[i] < 0 || ids[i] >= E_)
                return fail(MOE_ERR_INVALID_ARG, "moe_table_prefetch: expert id %d outside [0, E)", ids[i]);
        step_++;
        std::fill(active_now_.begin(), active_now_.end(), 0);
        std::vector<int32_t> load;
        for (int i = 0; i < n; ++i) {
            const int e = ids[i];
            if (active_now_[e]) continue;
            active_now_[e] = 1;
            last_use_[e] = step_;
            if (slot_of_[e] < 0) load.push_back(e);
        }
        const int rc = transact(load.data(), (int)load.size(), nullptr, false);
        if (rc == MOE_OK) {
            for (int e : load) prefetched_[e] = 1;
            ctr_.prefetched += load.size();
        }
        return rc;
    }

private:
    int transact(const int32_t *ids, int n, void *consumer, bool order_consumer)
    {
        if (faulted_) return fail(MOE_ERR_FAULTED, "moe_upload_expert_rows: the table faulted earlier");
        if (n < 0 || n > E_) return fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: n=%d", n);
        std::vector<uint8_t> want(E_, 0);
        for (int i = 0; i < n; ++i) {
            const int e = ids[i];
            if (e < 0 || e >= E_) return fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: expert id %d", e);
            if (slot_of_[e] >= 0 || want[e])
                return fail(MOE_ERR_INVALID_ARG, "moe_upload_expert_rows: expert %d is published or listed twice", e);
            want[e] = 1;
        }
        if (n == 0) return MOE_OK;
        const uint64_t g_new = gen_ + 1;
        // the ring slot of the new map last served generation g_new - kMaps
        const uint64_t map_prev = g_new > (uint64_t)kMaps ? g_new - kMaps : 0;
        if (!retired(map_prev))
            return fail(MOE_ERR_CAPACITY, "moe_upload_expert_rows: a lease on generation %llu (or older) is still "
                        "open; its device map cannot be reused", (unsigned long long)map_prev);
        // target rows: not named by the current generation and not named by
        // any generation a live lease can still see
        std::vector<int> target;
        int held = 0;
        for (int sl = 0; sl < nslots_ && (int)target.size() < n; ++sl) {
            if (expert_in_[sl] >= 0) continue;
            if (retired(last_visible_[sl])) target.push_back(sl);
            else ++held;
        }
        if ((int)target.size() < n)
            return fail(MOE_ERR_CAPACITY, "moe_upload_expert_rows: %d misses but %d free spare rows (%d more held by "
                        "open leases)", n, (int)target.size(), held);
        uint64_t need = map_prev;
        for (int sl : target)
            if (last_visible_[sl] > need) need = last_visible_[sl];
        // the next generation's map: the misses in their rows, then, above
        // capacity, least recently used experts outside this step dropped
        // (ties: lower expert id)
        std::vector<int32_t> next(slot_of_);
        for (int i = 0; i < n; ++i) next[ids[i]] = target[i];
        std::vector<int> dropped;
        int published = 0;
        for (int e = 0; e < E_; ++e) published += next[e] >= 0;
        while (published > capacity_) {
            int v = -1;
            for (int e = 0; e < E_; ++e)
                if (next[e] >= 0 && !active_now_[e] && (v < 0 || last_use_[e] < last_use_[v])) v = e;
            if (v < 0) break;                    // every published expert is in use this step
            dropped.push_back(v);
            next[v] = -1;
            --published;
        }
        // ---- before publication: a failure leaves generation gen_ authoritative
        int rc = wait_consumers(need);
        if (rc) return rc;
        for (int i = 0; i < n; ++i) {
            rc = copy_row(ids[i], target[i], copy_stream(i));
            if (rc) return abandon(rc);
        }
        if (join_copies(n) != 0)
            return abandon(fail(MOE_ERR_HIP, "moe_upload_expert_rows (joining the copy streams): %s", tr_->message()));
        if (tr_->publish(map_of(g_new), next.data(), E_, copy_) != 0)
            return abandon(fail(MOE_ERR_HIP, "moe_upload_expert_rows (publish): %s", tr_->message()));
        if (tr_->record(published_[g_new % kMaps], copy_) != 0)
            return abandon(fail(MOE_ERR_HIP, "moe_upload_expert_rows (publication event): %s", tr_->message()));
        // ---- publication
        gen_ = g_new;
        for (int e : dropped) {
            const int sl = slot_of_[e];
            expert_in_[sl] = -1;
            last_visible_[sl] = g_new - 1;
            ctr_.evictions++;
            if (prefetched_[e]) {
                prefetched_[e] = 0;
                ctr_.prefetch_unused++;
            }
        }
        for (int i = 0; i < n; ++i) expert_in_[target[i]] = ids[i];
        slot_of_.swap(next);
        ctr_.generation = gen_;
        if (order_consumer && tr_->stream_wait(consumer, published_[gen_ % kMaps]) != 0) {
            faulted_ = true;
            return fail(MOE_ERR_FAULTED, "moe_upload_expert_rows: ordering the consumer stream after publication "
                        "failed (%s); the table is faulted", tr_->message());
        }
        return MOE_OK;
    }

public:
    // Captures the current generation for a consumer on `stream` (ordered
    // after its publication; a null handle is the default stream).
    int acquire(void *stream, moe_table_lease *out)
    {
        if (faulted_) return fail(MOE_ERR_FAULTED, "moe_table_acquire: the table faulted earlier");
        if (tr_->stream_wait(stream, published_[gen_ % kMaps]) != 0)
            return fail(MOE_ERR_HIP, "moe_table_acquire: %s", tr_->message());
        GenRec &g = rec(gen_);
        g.open++;
        out->generation = gen_;
        out->rows_dev = rows_;
        out->row_stride = row_stride_;
        out->slot_map_dev = map_of(gen_);
        ctr_.open_leases++;
        return MOE_OK;
    }

    // Ends a lease: the point on `stream` after which its consumers no longer
    // read the generation's rows or map.
    int release(const moe_table_lease *lease, void *stream)
    {
        GenRec *g = find(lease->generation);
        if (!g || g->open <= 0)
            return fail(MOE_ERR_INVALID_ARG, "moe_table_release: no open lease on generation %llu",
                        (unsigned long long)lease->generation);
        void *ev = take_event();
        if (!ev) return fail(MOE_ERR_HIP, "moe_table_release: no consumer event available: %s", tr_->message());
        if (tr_->record(ev, stream) != 0) {
            recycle_.push_back(ev);
            return fail(MOE_ERR_HIP, "moe_table_release: %s", tr_->message());
        }
        // a later event on the same stream covers an earlier one
        for (auto &se : g->ev)
            if (se.stream == stream) {
                recycle_.push_back(se.ev);
                se.ev = ev;
                ev = nullptr;
                break;
            }
        if (ev) g->ev.push_back({stream, ev});
        g->open--;
        ctr_.open_leases--;
        return MOE_OK;
    }

    // Re-checks the host source against the digests taken at creation.
    int verify_source()
    {
        int changed = 0;
        for (int e = 0; e < E_; ++e)
            if (digest(host_ + (size_t)e * host_stride_, row_bytes_) != digests_[e]) ++changed;
        if (changed) {
            ctr_.host_writes += (uint64_t)changed;
            return fail(MOE_ERR_SOURCE, "moe_table_verify_source: %d host rows changed since creation", changed);
        }
        return MOE_OK;
    }

    void stats(moe_table_counters *out) const { *out = ctr_; }

    void published(int32_t *map) const
    {
        for (int e = 0; e < E_; ++e) map[e] = slot_of_[e];
    }

    bool faulted() const { return faulted_; }

private:
    struct StreamEvent {
        void *stream;
        void *ev;
    };
    struct GenRec {
        uint64_t gen;
        int open;
        std::vector<StreamEvent> ev;         // consumer events of released leases
    };

    explicit Table(Transport *tr) : tr_(tr) {}

    static int validate(const moe_table_desc *d)
    {
        if (d->E < 1 || d->E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "moe_table_create: E=%d", d->E);
        size_t off[6];
        if (row_layout(d->H, d->I, off) == 0)
            return fail(MOE_ERR_UNSUPPORTED, "moe_table_create: H=%d, I=%d must be positive multiples of 128", d->H,
                        d->I);
        if (d->top_k < 1 || d->top_k > d->E || d->top_k > MOE_MAX_TOPK)
            return fail(MOE_ERR_UNSUPPORTED, "moe_table_create: top_k=%d", d->top_k);
        if (d->max_tokens < 1 || d->max_tokens > 65536)
            return fail(MOE_ERR_UNSUPPORTED, "moe_table_create: max_tokens=%d outside [1, 65536]", d->max_tokens);
        if (d->capacity < 1 || d->capacity > d->E)
            return fail(MOE_ERR_CAPACITY, "moe_table_create: capacity %d outside [1, E]", d->capacity);
        const int need = spare_needed(d->E, d->capacity, d->top_k, d->max_tokens);
        if (d->spare_rows < need || d->capacity + d->spare_rows > 4 * MOE_MAX_EXPERTS)
            return fail(MOE_ERR_CAPACITY, "moe_table_create: %d spare rows; steps of %d tokens x top-%d need %d "
                        "(at most %d rows in all)", d->spare_rows, d->max_tokens, d->top_k, need,
                        4 * MOE_MAX_EXPERTS);
        if (d->slot_format != MOE_SLOT_QPACKED && d->slot_format != MOE_SLOT_FP16)
            return fail(MOE_ERR_INVALID_ARG, "moe_table_create: slot_format %d", d->slot_format);
        if (d->staging_rows < 1 || d->staging_rows > 16)
            return fail(MOE_ERR_CAPACITY, "moe_table_create: staging_rows %d outside [1, 16]", d->staging_rows);
        const size_t rb = row_layout(d->H, d->I, off);
        if (!d->host_source || d->host_row_stride < rb)
            return fail(MOE_ERR_INVALID_ARG, "moe_table_create: host source missing or stride < %zu", rb);
        std::vector<uint8_t> seen(d->E, 0);
        for (int i = 0; i < d->capacity; ++i) {
            const int e = d->initial_resident ? d->initial_resident[i] : i;
            if (e < 0 || e >= d->E || seen[e])
                return fail(MOE_ERR_INVALID_ARG, "moe_table_create: initial resident list invalid at %d", i);
            seen[e] = 1;
        }
        return MOE_OK;
    }

    int init(const moe_table_desc *d)
    {
        E_ = d->E;
        capacity_ = d->capacity;
        nslots_ = d->capacity + d->spare_rows;
        size_t off[6];
        row_bytes_ = row_layout(d->H, d->I, off);
        // device rows: the qpacked row, or an FP16 execution slot (three FP16
        // matrices of I*H values each)
        const size_t dev_bytes = d->slot_format == MOE_SLOT_FP16 ? (size_t)3 * d->I * d->H * 2 : row_bytes_;
        row_stride_ = (dev_bytes + 255) / 256 * 256;
        host_stride_ = d->host_row_stride;
        host_ = static_cast<const uint8_t *>(d->host_source);
        // identity and layout of the host source
        digests_.resize(E_);
        for (int e = 0; e < E_; ++e) {
            const uint8_t *row = host_ + (size_t)e * host_stride_;
            digests_[e] = digest(row, row_bytes_);
            if (d->row_digests && d->row_digests[e] != digests_[e])
                return fail(MOE_ERR_SOURCE, "moe_table_create: host row of expert %d does not match its digest", e);
            for (int sec = 3; sec < 6; ++sec) {
                const size_t n = sec == 5 ? (size_t)d->H * ((d->I + 255) / 256) : (size_t)d->I * ((d->H + 255) / 256);
                for (size_t i = 0; i < n; ++i) {
                    uint16_t b;
                    std::memcpy(&b, row + off[sec] + 2 * i, 2);
                    if (((b >> 10) & 0x1f) == 0x1f)
                        return fail(MOE_ERR_SOURCE, "moe_table_create: expert %d has a non-finite FP16 scale", e);
                }
            }
        }
        slot_of_.assign(E_, -1);
        expert_in_.assign(nslots_, -1);
        last_visible_.assign(nslots_, 0);
        last_use_.assign(E_, 0);
        active_now_.assign(E_, 0);
        prefetched_.assign(E_, 0);
        if (tr_->create_stream(&copy_) != 0) return hip_fail("copy stream");
        // a page-locked source is read by the copy engine directly: no staging
        direct_ = tr_->host_pinned(host_, (size_t)(E_ - 1) * host_stride_ + row_bytes_);
        // direct qpacked copies alternate between two copy streams, so a row's
        // transfer overlaps the previous one's (3.2 MB rows from pinned memory
        // moved at 47.9 GB/s on one stream and 54.4 GB/s on two, measured on
        // the MI355X); staged copies keep one (there the host's staging copy,
        // not the link, sets the pace: measured no gain), and so do FP16
        // slots (their uploads share the transport's device staging row)
        if (direct_ && d->slot_format == MOE_SLOT_QPACKED) {
            if (tr_->create_stream(&copy2_) != 0) return hip_fail("copy stream");
            if (tr_->create_event(&join_) != 0) return hip_fail("events");
            all_events_.push_back(join_);
        }
        if (tr_->alloc_device(&rows_, (size_t)nslots_ * row_stride_) != 0) return hip_fail("device rows");
        if (tr_->alloc_device(reinterpret_cast<void **>(&maps_), sizeof(int32_t) * (size_t)E_ * kMaps) != 0)
            return hip_fail("device maps");
        for (int i = 0; i < (direct_ ? 0 : d->staging_rows); ++i) {
            void *p = nullptr, *ev = nullptr;
            if (tr_->alloc_pinned(&p, row_bytes_) != 0) return hip_fail("pinned staging");
            staging_.push_back(static_cast<uint8_t *>(p));
            if (tr_->create_event(&ev) != 0) return hip_fail("events");
            all_events_.push_back(ev);
            staging_done_.push_back(ev);
            staging_used_.push_back(0);
        }
        for (int i = 0; i < kMaps; ++i) {
            void *ev = nullptr;
            if (tr_->create_event(&ev) != 0) return hip_fail("events");
            all_events_.push_back(ev);
            published_[i] = ev;
        }
        for (int i = 0; i < kEvents; ++i) {
            void *ev = nullptr;
            if (tr_->create_event(&ev) != 0) return hip_fail("events");
            all_events_.push_back(ev);
            free_events_.push_back(ev);
        }
        // generation 1: the initial residents in rows 0..capacity-1
        std::vector<int32_t> first(E_, -1);
        for (int i = 0; i < capacity_; ++i) {
            const int e = d->initial_resident ? d->initial_resident[i] : i;
            int rc = copy_row(e, i, copy_stream(i));
            if (rc) return rc;
            first[e] = i;
        }
        if (join_copies(capacity_) != 0) return hip_fail("joining the copy streams");
        if (tr_->publish(map_of(1), first.data(), E_, copy_) != 0) return hip_fail("publish");
        if (tr_->record(published_[1 % kMaps], copy_) != 0) return hip_fail("publication event");
        if (tr_->stream_sync(copy_) != 0) return hip_fail("initial upload");
        gen_ = 1;
        for (int e = 0; e < E_; ++e)
            if (first[e] >= 0) expert_in_[first[e]] = e;
        slot_of_.swap(first);
        ctr_ = moe_table_counters{};         // creation traffic is not a miss
        ctr_.generation = gen_;
        return MOE_OK;
    }

    int hip_fail(const char *what) { return fail(MOE_ERR_CAPACITY, "moe_table_create (%s): %s", what, tr_->message()); }

    int32_t *map_of(uint64_t g) const { return maps_ + (size_t)(g % kMaps) * E_; }

    GenRec *find(uint64_t g)
    {
        for (auto &r : gens_)
            if (r.gen == g) return &r;
        return nullptr;
    }

    GenRec &rec(uint64_t g)
    {
        GenRec *r = find(g);
        if (r) return *r;
        gens_.push_back(GenRec{g, 0, {}});
        return gens_.back();
    }

    // No lease on generation x or older is open.
    bool retired(uint64_t x) const
    {
        for (const auto &r : gens_)
            if (r.gen <= x && r.open > 0) return false;
        return true;
    }

    // Orders the copy stream after the consumers of generations <= x.
    int wait_consumers(uint64_t x)
    {
        for (size_t i = 0; i < gens_.size();) {
            GenRec &r = gens_[i];
            if (r.gen > x) {
                ++i;
                continue;
            }
            for (auto &se : r.ev) {
                if (tr_->stream_wait(copy_, se.ev) != 0 || (copy2_ && tr_->stream_wait(copy2_, se.ev) != 0))
                    return fail(MOE_ERR_HIP, "moe_upload_expert_rows (consumer wait): %s", tr_->message());
            }
            for (auto &se : r.ev) recycle_.push_back(se.ev);
            gens_.erase(gens_.begin() + (long)i);
        }
        return MOE_OK;
    }

    void *take_event()
    {
        if (free_events_.empty()) {
            // events whose consumers have finished go back to the pool
            for (size_t i = 0; i < recycle_.size();) {
                if (tr_->event_done(recycle_[i]) == 1) {
                    free_events_.push_back(recycle_[i]);
                    recycle_.erase(recycle_.begin() + (long)i);
                } else {
                    ++i;
                }
            }
        }
        if (free_events_.empty() && !recycle_.empty()) {
            void *ev = recycle_.front();
            if (tr_->event_sync(ev) != 0) return nullptr;
            recycle_.erase(recycle_.begin());
            free_events_.push_back(ev);
        }
        if (free_events_.empty()) {
            // every event is attached to a generation that still has live
            // consumers: wait for the oldest attached one
            for (auto &r : gens_)
                for (size_t i = 0; i < r.ev.size(); ++i) {
                    if (tr_->event_sync(r.ev[i].ev) != 0) return nullptr;
                    free_events_.push_back(r.ev[i].ev);
                    r.ev.erase(r.ev.begin() + (long)i);
                    goto got;
                }
        }
    got:
        if (free_events_.empty()) return nullptr;
        void *ev = free_events_.back();
        free_events_.pop_back();
        return ev;
    }

    // A transaction failed before publication: its target rows stay free, so
    // with two copy streams the next transaction may write one of them on the
    // other stream while this one's copy is in flight - both streams are
    // drained first (one stream keeps its copies in order by itself).
    int abandon(int rc)
    {
        ctr_.failed_uploads++;
        if (copy2_ && (tr_->stream_sync(copy2_) != 0 || tr_->stream_sync(copy_) != 0)) {
            faulted_ = true;
            return fail(MOE_ERR_FAULTED, "moe_upload_expert_rows: copy state unknown after a failed transaction (%s)",
                        tr_->message());
        }
        return rc;
    }

    // Copy stream of the i-th row of a transaction (alternating when there are two).
    void *copy_stream(int i) const { return (copy2_ && (i & 1)) ? copy2_ : copy_; }

    // Orders the first copy stream after the second one's copies of a
    // transaction of n rows (publication runs on the first).
    int join_copies(int n)
    {
        if (!copy2_ || n < 2) return 0;
        if (tr_->record(join_, copy2_) != 0) return 1;
        return tr_->stream_wait(copy_, join_);
    }

    // Host row of expert e -> device row `slot` (through staging unless the
    // source is page-locked).
    int copy_row(int e, int slot, void *stream)
    {
        if (direct_) {
            // straight from the page-locked source (unchanged for the table's lifetime)
            if (tr_->row_upload(static_cast<uint8_t *>(rows_) + (size_t)slot * row_stride_, host_ + (size_t)e * host_stride_,
                                row_bytes_, stream) != 0)
                return fail(MOE_ERR_HIP, "moe_upload_expert_rows (copy): %s", tr_->message());
            ctr_.h2d_bytes += row_bytes_;
            ctr_.direct_copies++;
            return MOE_OK;
        }
        const size_t i = next_staging_;
        next_staging_ = (i + 1) % staging_.size();
        if (staging_used_[i]) {
            // staging is refilled only after its previous transfer has retired
            const int done = tr_->event_done(staging_done_[i]);
            if (done == 0) ctr_.staging_waits++;
            if (done < 0 || tr_->event_sync(staging_done_[i]) != 0)
                return fail(MOE_ERR_HIP, "moe_upload_expert_rows (staging): %s", tr_->message());
        }
        CopyPool::get().copy(staging_[i], host_ + (size_t)e * host_stride_, row_bytes_);
        if (tr_->row_upload(static_cast<uint8_t *>(rows_) + (size_t)slot * row_stride_, staging_[i], row_bytes_,
                            copy_) != 0)
            return fail(MOE_ERR_HIP, "moe_upload_expert_rows (copy): %s", tr_->message());
        staging_used_[i] = 1;
        if (tr_->record(staging_done_[i], copy_) != 0) {
            // the copy may be in flight without an event: wait for the stream
            // so the staging buffer is not refilled under it
            if (tr_->stream_sync(copy_) != 0) {
                faulted_ = true;
                return fail(MOE_ERR_FAULTED, "moe_upload_expert_rows: copy state unknown (%s)", tr_->message());
            }
            staging_used_[i] = 0;
            return fail(MOE_ERR_HIP, "moe_upload_expert_rows (copy event): %s", tr_->message());
        }
        ctr_.h2d_bytes += row_bytes_;
        return MOE_OK;
    }

    Transport *tr_;
    int E_ = 0, capacity_ = 0, nslots_ = 0;
    size_t row_bytes_ = 0, row_stride_ = 0, host_stride_ = 0;
    const uint8_t *host_ = nullptr;
    std::vector<uint64_t> digests_;
    void *copy_ = nullptr;                   // copy stream (publication runs here)
    void *copy2_ = nullptr;                  // second copy stream (direct qpacked copies), or null
    void *join_ = nullptr;                   // event: copy2_'s copies of a transaction
    bool direct_ = false;                    // the host source is page-locked: no staging
    void *rows_ = nullptr;
    int32_t *maps_ = nullptr;                // [kMaps][E]
    std::vector<int32_t> slot_of_;           // published map of generation gen_ (host mirror)
    std::vector<int32_t> expert_in_;         // slot -> expert named by generation gen_, -1 = none
    std::vector<uint64_t> last_visible_;     // slot -> last generation that named it before it was freed
    std::vector<uint64_t> last_use_;         // expert -> step of last use
    std::vector<uint8_t> active_now_;        // expert -> active in the current step
    std::vector<uint8_t> prefetched_;        // expert -> uploaded by a prefetch, not yet routed
    uint64_t step_ = 0, gen_ = 0;
    std::vector<uint8_t *> staging_;
    std::vector<void *> staging_done_;
    std::vector<uint8_t> staging_used_;
    size_t next_staging_ = 0;
    void *published_[kMaps] = {};
    std::vector<GenRec> gens_;               // generations with leases or pending consumer events
    std::vector<void *> free_events_, recycle_, all_events_;
    bool faulted_ = false;
    moe_table_counters ctr_{};
};

}  // namespace tcore
