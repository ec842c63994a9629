// Host-only checks of the resident expert table's state machine
// (w4a16_routed_expert_amd/csrc/table_core.h) over a simulated transport.
//
// The simulated device runs nothing when work is enqueued: each stream keeps
// its operations (copies, event records, waits, map writes, reads that stand
// for the expert FFN) and executes them only when something forces it (an
// event or stream synchronization, a wait of another stream, or the test).
// The tests run the table's copy stream as early as they can and consumer
// streams as late as they can, so a missing wait shows up as a consumer that
// reads overwritten bytes, and a refilled staging buffer as a wrong row.
// Failures are injected into chosen transport calls.
//
// Built with g++ by tests/test_table_cpu.py, under -fsanitize=address,undefined
// and separately -fsanitize=thread.  Usage: table_sim <scenario|all>.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "../../w4a16_routed_expert_amd/csrc/table_core.h"

static thread_local char g_msg[512];

int tcore::fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return code;
}

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                                                 \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);         \
            std::fprintf(stderr, __VA_ARGS__);                                           \
            std::fprintf(stderr, " [last message: %s]\n", g_msg);                        \
            ++g_failures;                                                                \
        }                                                                                \
    } while (0)

struct SimStream;

struct SimEvent {
    SimStream *owner = nullptr;   // stream of the latest record
    uint64_t recorded = 0;        // records issued
    uint64_t executed = 0;        // records executed
};

struct Op {
    enum Kind { COPY, RECORD, WAIT, PUBLISH, CALL } kind;
    void *dst = nullptr;
    const void *src = nullptr;
    size_t n = 0;
    SimEvent *ev = nullptr;
    uint64_t seq = 0;
    std::vector<int32_t> slots;
    std::function<void()> fn;
};

struct SimStream {
    std::vector<Op> ops;
    size_t next = 0;
};

void run_until(SimStream *s, SimEvent *ev, uint64_t seq);

// Executes the stream's operations in order; stops when `stop` returns true.
void run_stream(SimStream *s, const std::function<bool()> &stop)
{
    while (s->next < s->ops.size()) {
        if (stop && stop()) return;
        Op &op = s->ops[s->next];
        switch (op.kind) {
        case Op::COPY:
            std::memcpy(op.dst, op.src, op.n);
            break;
        case Op::RECORD:
            if (op.seq > op.ev->executed) op.ev->executed = op.seq;
            break;
        case Op::WAIT:
            if (op.ev->owner && op.ev->executed < op.seq) run_until(op.ev->owner, op.ev, op.seq);
            break;
        case Op::PUBLISH:
            std::memcpy(op.dst, op.slots.data(), op.slots.size() * sizeof(int32_t));
            break;
        case Op::CALL:
            op.fn();
            break;
        }
        s->next++;
    }
}

void run_until(SimStream *s, SimEvent *ev, uint64_t seq)
{
    run_stream(s, [&] { return ev->executed >= seq; });
}

class SimTransport final : public tcore::Transport {
public:
    // the n-th call (1-based) of a kind fails; 0 = never
    int fail_h2d_at = 0, fail_publish_at = 0, fail_wait_at = 0, fail_record_at = 0, fail_pinned_at = 0;
    bool pinned_source = false;          // host_pinned() answer: the source is page-locked
    int n_h2d = 0, n_publish = 0, n_wait = 0, n_record = 0, n_pinned = 0;
    std::vector<std::unique_ptr<SimStream>> streams;
    std::vector<std::unique_ptr<SimEvent>> events;

    ~SimTransport() override
    {
        for (void *p : live_) std::free(p);
    }

    int alloc_device(void **p, size_t n) override { return alloc(p, n); }
    void free_device(void *p) override { release(p); }
    int alloc_pinned(void **p, size_t n) override
    {
        if (++n_pinned == fail_pinned_at) return err("simulated pinned allocation failure");
        return alloc(p, n);
    }
    void free_pinned(void *p) override { release(p); }
    bool host_pinned(const void *, size_t) override { return pinned_source; }
    int create_event(void **ev) override
    {
        events.emplace_back(new SimEvent);
        *ev = events.back().get();
        return 0;
    }
    void destroy_event(void *) override {}
    int create_stream(void **s) override
    {
        streams.emplace_back(new SimStream);
        *s = streams.back().get();
        return 0;
    }
    void destroy_stream(void *) override {}
    int h2d_async(void *dst, const void *src, size_t n, void *s) override
    {
        if (++n_h2d == fail_h2d_at) return err("simulated copy failure");
        Op op{Op::COPY, nullptr, nullptr, 0, nullptr, 0, {}, {}};
        op.dst = dst;
        op.src = src;
        op.n = n;
        st(s)->ops.push_back(op);
        return 0;
    }
    int record(void *e, void *s) override
    {
        if (++n_record == fail_record_at) return err("simulated record failure");
        SimEvent *ev = static_cast<SimEvent *>(e);
        ev->owner = st(s);
        Op op{Op::RECORD, nullptr, nullptr, 0, nullptr, 0, {}, {}};
        op.ev = ev;
        op.seq = ++ev->recorded;
        st(s)->ops.push_back(op);
        return 0;
    }
    int event_sync(void *e) override
    {
        SimEvent *ev = static_cast<SimEvent *>(e);
        if (ev->owner) run_until(ev->owner, ev, ev->recorded);
        return 0;
    }
    int event_done(void *e) override
    {
        SimEvent *ev = static_cast<SimEvent *>(e);
        return ev->executed >= ev->recorded ? 1 : 0;
    }
    int stream_wait(void *s, void *e) override
    {
        if (++n_wait == fail_wait_at) return err("simulated wait failure");
        SimEvent *ev = static_cast<SimEvent *>(e);
        Op op{Op::WAIT, nullptr, nullptr, 0, nullptr, 0, {}, {}};
        op.ev = ev;
        op.seq = ev->recorded;               // the latest record at the time of the call
        st(s)->ops.push_back(op);
        return 0;
    }
    int stream_sync(void *s) override
    {
        run_stream(st(s), nullptr);
        return 0;
    }
    int publish(int32_t *map_dev, const int32_t *slots, int E, void *s) override
    {
        if (++n_publish == fail_publish_at) return err("simulated publish failure");
        Op op{Op::PUBLISH, nullptr, nullptr, 0, nullptr, 0, {}, {}};
        op.dst = map_dev;
        op.slots.assign(slots, slots + E);
        st(s)->ops.push_back(op);
        return 0;
    }
    const char *message() override { return msg_.c_str(); }

    // a consumer stream owned by the test
    SimStream *new_stream()
    {
        void *s;
        create_stream(&s);
        return static_cast<SimStream *>(s);
    }
    void call(SimStream *s, std::function<void()> fn)
    {
        Op op{Op::CALL, nullptr, nullptr, 0, nullptr, 0, {}, {}};
        op.fn = std::move(fn);
        st(s)->ops.push_back(op);
    }
    void run_all()
    {
        for (auto &s : streams) run_stream(s.get(), nullptr);
        run_stream(&default_stream, nullptr);
    }

    // the stream a null handle stands for (HIP's default stream)
    SimStream default_stream;

private:
    SimStream *st(void *s) { return s ? static_cast<SimStream *>(s) : &default_stream; }
    int alloc(void **p, size_t n)
    {
        *p = std::malloc(n ? n : 1);
        if (!*p) return err("out of memory");
        std::memset(*p, 0xA5, n);
        live_.push_back(*p);
        return 0;
    }
    void release(void *p)
    {
        for (size_t i = 0; i < live_.size(); ++i)
            if (live_[i] == p) {
                std::free(p);
                live_.erase(live_.begin() + (long)i);
                return;
            }
    }
    int err(const char *m)
    {
        msg_ = m;
        return 1;
    }
    std::vector<void *> live_;
    std::string msg_;
};

// ------------------------------------------------------------------ fixtures
struct Shape {
    int E, H, I;
};

struct Source {
    Shape sh;
    size_t row_bytes, stride;
    std::vector<uint8_t> bytes;
    std::vector<uint64_t> digests;
    Source(Shape s, uint32_t seed) : sh(s)
    {
        size_t off[6];
        row_bytes = tcore::row_layout(s.H, s.I, off);
        stride = row_bytes + 512;
        bytes.assign((size_t)s.E * stride, 0);
        std::mt19937 rng(seed);
        for (int e = 0; e < s.E; ++e) {
            uint8_t *row = bytes.data() + (size_t)e * stride;
            for (size_t i = 0; i < row_bytes; ++i) row[i] = (uint8_t)rng();
            // scales: finite FP16 values
            for (int sec = 3; sec < 6; ++sec) {
                const size_t n = sec == 5 ? (size_t)s.H * ((s.I + 255) / 256) : (size_t)s.I * ((s.H + 255) / 256);
                for (size_t i = 0; i < n; ++i) {
                    const uint16_t v = (uint16_t)(0x1000 + (rng() & 0x3fff));
                    std::memcpy(row + off[sec] + 2 * i, &v, 2);
                }
            }
            digests.push_back(tcore::digest(row, row_bytes));
        }
    }
    const uint8_t *row(int e) const { return bytes.data() + (size_t)e * stride; }
};

moe_table_desc desc_of(const Source &src, int capacity, int spare, int staging, int k, int max_tokens)
{
    moe_table_desc d{};
    d.E = src.sh.E;
    d.H = src.sh.H;
    d.I = src.sh.I;
    d.capacity = capacity;
    d.spare_rows = spare;
    d.staging_rows = staging;
    d.top_k = k;
    d.max_tokens = max_tokens;
    d.host_source = src.bytes.data();
    d.host_row_stride = src.stride;
    d.initial_resident = nullptr;
    d.row_digests = src.digests.data();
    return d;
}

// Device state of a generation, as a consumer reading it would see it: every
// expert its map names has the host row's bytes.
bool rows_match(const tcore::Table &t, const Source &src, const moe_table_lease &lease, std::string *why)
{
    (void)t;
    const int32_t *map = lease.slot_map_dev;
    for (int e = 0; e < src.sh.E; ++e) {
        const int sl = map[e];
        if (sl < 0) continue;
        const uint8_t *dev = static_cast<const uint8_t *>(lease.rows_dev) + (size_t)sl * lease.row_stride;
        if (std::memcmp(dev, src.row(e), src.row_bytes) != 0) {
            if (why) *why = "expert " + std::to_string(e) + " slot " + std::to_string(sl);
            return false;
        }
    }
    return true;
}

// One decode step as the layer runs it: misses, upload, lease, a deferred
// read of the lease's rows on the consumer stream, release.
struct Stepper {
    SimTransport &tr;
    tcore::Table &t;
    const Source &src;
    SimStream *consumer;
    SimStream *uploader = nullptr;            // stream passed to the upload (consumer if null)
    bool own_uploader = false;
    int bad_reads = 0, reads = 0;
    int step(const std::vector<int32_t> &active, bool run_consumer)
    {
        std::vector<int32_t> miss(active.size() + 1);
        int nm = 0;
        int rc = t.misses(active.data(), (int)active.size(), miss.data(), &nm);
        if (rc) return rc;
        rc = t.upload(miss.data(), nm, own_uploader ? uploader : consumer);
        if (rc) return rc;
        moe_table_lease lease;
        rc = t.acquire(consumer, &lease);
        if (rc) return rc;
        std::vector<int32_t> act(active);
        tr.call(consumer, [this, lease, act] {
            ++reads;
            std::string why;
            if (!rows_match(t, src, lease, &why)) {
                ++bad_reads;
                std::fprintf(stderr, "  consumer of generation %llu read a wrong row (%s)\n",
                             (unsigned long long)lease.generation, why.c_str());
            }
            for (int32_t e : act)
                if (lease.slot_map_dev[e] < 0) {
                    ++bad_reads;
                    std::fprintf(stderr, "  active expert %d not published in generation %llu\n", e,
                                 (unsigned long long)lease.generation);
                }
        });
        rc = t.release(&lease, consumer);
        if (rc) return rc;
        if (run_consumer) tr.stream_sync(consumer);
        return MOE_OK;
    }
};

std::vector<int32_t> random_active(std::mt19937 &rng, int E, int n, int skew)
{
    std::vector<int32_t> a;
    while ((int)a.size() < n) {
        int e = (int)(rng() % (uint32_t)E);
        if (skew && (rng() & 1)) e = (int)(rng() % (uint32_t)(E / 4 + 1));
        bool dup = false;
        for (int x : a) dup |= x == e;
        if (!dup) a.push_back(e);
    }
    return a;
}

// ---------------------------------------------------------------- scenarios
void scenario_steps()
{
    // Random steps with the copy stream run eagerly and consumers lazily: every
    // consumer sees intact rows of its generation; counters add up.
    const Source src({16, 256, 512}, 1);
    for (int max_tokens : {1, 2, 4}) {
        const int k = 2, capacity = 5;
        const int spare = tcore::spare_needed(16, capacity, k, max_tokens);
        SimTransport tr;
        moe_table_desc d = desc_of(src, capacity, spare, 2, k, max_tokens);
        tcore::Table *t = nullptr;
        CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create (max_tokens %d)", max_tokens);
        if (!t) continue;
        Stepper st{tr, *t, src, tr.new_stream()};
        std::mt19937 rng(7 + max_tokens);
        uint64_t active_total = 0;
        for (int s = 0; s < 300; ++s) {
            const int n = 1 + (int)(rng() % (uint32_t)(max_tokens * k));
            auto act = random_active(rng, 16, n, s & 1);
            active_total += act.size();
            // either the consumer runs at once and the copy stream only when
            // forced, or the copy stream runs ahead of a lazy consumer
            const bool consumer_first = rng() & 1;
            const int rc = st.step(act, consumer_first);
            CHECK(rc == MOE_OK, "step %d rc %d", s, rc);
            if (rc) break;
            if (!consumer_first) tr.stream_sync(tr.streams[0].get());
        }
        tr.run_all();
        CHECK(st.bad_reads == 0, "%d bad reads of %d", st.bad_reads, st.reads);
        moe_table_counters c;
        t->stats(&c);
        CHECK(c.hits + c.misses == active_total, "hits %llu + misses %llu != %llu", (unsigned long long)c.hits,
              (unsigned long long)c.misses, (unsigned long long)active_total);
        CHECK(c.h2d_bytes == c.misses * src.row_bytes, "h2d bytes");
        CHECK(c.expert_d2h_bytes == 0 && c.host_writes == 0, "no d2h, no host writes");
        CHECK(c.open_leases == 0, "leases left open");
        CHECK(t->verify_source() == MOE_OK, "source unchanged");
        int32_t map[64];
        t->published(map);
        int pub = 0;
        for (int e = 0; e < 16; ++e) pub += map[e] >= 0;
        CHECK(pub <= (capacity > max_tokens * k ? capacity : max_tokens * k), "published %d", pub);
        delete t;
    }
}

void scenario_default_stream_consumer()
{
    // The consumer passes the null handle (the default stream): it must still
    // be ordered after each publication and its reads covered by its release.
    const Source src({16, 256, 512}, 9);
    SimTransport tr;
    moe_table_desc d = desc_of(src, 5, 7, 2, 2, 3);
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    // the transactions order another stream; the lease alone must order
    // the default stream after the publication
    Stepper st{tr, *t, src, nullptr, tr.new_stream(), true};
    std::mt19937 rng(3);
    for (int s = 0; s < 100; ++s) {
        // the consumer runs as soon as it is enqueued, the copy stream only
        // when a wait forces it (or every third step)
        const int rc = st.step(random_active(rng, 16, 1 + (int)(rng() % 6u), 1), true);
        CHECK(rc == MOE_OK, "step %d rc %d", s, rc);
        if (rc) break;
        if (s % 3 == 2) tr.stream_sync(tr.streams[0].get());
    }
    tr.run_all();
    CHECK(st.bad_reads == 0 && st.reads == 100, "%d bad reads of %d", st.bad_reads, st.reads);
    delete t;
}

void scenario_prefetch()
{
    // Before each step, a speculative load of a guess of its active set (some
    // right, some wrong); the step's consumer still reads intact rows under
    // either schedule, and every prefetched row is counted once as a hit, as
    // unused (evicted first), or is still waiting.
    const Source src({16, 256, 512}, 11);
    SimTransport tr;
    moe_table_desc d = desc_of(src, 5, 7, 2, 2, 3);
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    Stepper st{tr, *t, src, tr.new_stream()};
    std::mt19937 rng(5);
    for (int s = 0; s < 200; ++s) {
        auto act = random_active(rng, 16, 1 + (int)(rng() % 6u), 1);
        std::vector<int32_t> guess;
        for (int32_t e : act)
            if (rng() % 4u) guess.push_back(e);                  // most of the real set
        if (rng() & 1) guess.push_back((int32_t)(rng() % 16u));    // and a wrong one
        std::vector<int32_t> uniq;
        for (int32_t e : guess) {
            bool dup = false;
            for (int32_t u : uniq) dup |= u == e;
            if (!dup) uniq.push_back(e);
        }
        const int rc0 = t->prefetch(uniq.data(), (int)uniq.size());
        CHECK(rc0 == MOE_OK, "prefetch %d rc %d", s, rc0);
        const bool consumer_first = rng() & 1;
        if (!consumer_first && (rng() & 1)) tr.stream_sync(tr.streams[0].get());
        const int rc = st.step(act, consumer_first);
        CHECK(rc == MOE_OK, "step %d rc %d", s, rc);
        if (rc0 || rc) break;
        if (!consumer_first) tr.stream_sync(tr.streams[0].get());
    }
    tr.run_all();
    CHECK(st.bad_reads == 0, "%d bad reads of %d", st.bad_reads, st.reads);
    moe_table_counters c;
    t->stats(&c);
    CHECK(c.prefetched > 0 && c.prefetch_hits > 0, "prefetched %llu, hits %llu", (unsigned long long)c.prefetched,
          (unsigned long long)c.prefetch_hits);
    CHECK(c.prefetch_hits + c.prefetch_unused <= c.prefetched, "prefetch accounting");
    CHECK(c.h2d_bytes == (c.misses + c.prefetched) * src.row_bytes, "h2d bytes");
    delete t;
}

void scenario_staging_reuse()
{
    // One staging buffer, three misses: each refill waits for the previous
    // copy out of it; the rows arrive intact.
    const Source src({8, 256, 512}, 2);
    SimTransport tr;
    moe_table_desc d = desc_of(src, 2, 6, 1, 2, 8);
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    SimStream *c = tr.new_stream();
    std::vector<int32_t> act = {0, 3, 5, 6}, miss(4);
    int nm = 0;
    CHECK(t->misses(act.data(), 4, miss.data(), &nm) == MOE_OK && nm == 3, "misses %d", nm);
    CHECK(t->upload(miss.data(), nm, c) == MOE_OK, "upload");
    moe_table_counters k;
    t->stats(&k);
    CHECK(k.staging_waits == 2, "staging waits %llu", (unsigned long long)k.staging_waits);
    moe_table_lease l;
    CHECK(t->acquire(c, &l) == MOE_OK, "acquire");
    tr.run_all();
    std::string why;
    CHECK(rows_match(*t, src, l, &why), "rows after staged copies: %s", why.c_str());
    CHECK(t->release(&l, c) == MOE_OK, "release");
    delete t;
}

void scenario_direct_from_pinned_source()
{
    // A page-locked source: no staging buffer is allocated, every miss is one
    // copy straight from the source; random steps with lazy consumers still
    // see intact rows of their generation.
    const Source src({16, 256, 512}, 11);
    SimTransport tr;
    tr.pinned_source = true;
    moe_table_desc d = desc_of(src, 5, tcore::spare_needed(16, 5, 2, 2), 2, 2, 2);
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    CHECK(tr.n_pinned == 0, "staging allocated: %d pinned buffers", tr.n_pinned);
    Stepper st{tr, *t, src, tr.new_stream()};
    std::mt19937 rng(17);
    const int h2d_before = tr.n_h2d;
    for (int s = 0; s < 100; ++s) {
        const int n = 1 + (int)(rng() % 4u);
        const bool consumer_first = rng() & 1;
        const int rc = st.step(random_active(rng, 16, n, s & 1), consumer_first);
        CHECK(rc == MOE_OK, "step %d rc %d", s, rc);
        if (rc) break;
        if (!consumer_first) tr.stream_sync(tr.streams[0].get());
    }
    tr.run_all();
    CHECK(st.bad_reads == 0, "%d bad reads of %d", st.bad_reads, st.reads);
    moe_table_counters k;
    t->stats(&k);
    CHECK(k.direct_copies == k.misses && k.misses > 0, "direct copies %llu of %llu misses",
          (unsigned long long)k.direct_copies, (unsigned long long)k.misses);
    CHECK((uint64_t)(tr.n_h2d - h2d_before) == k.misses, "one copy per miss");
    int copies[2] = {0, 0};
    for (int i = 0; i < 2; ++i)
        for (const Op &op : tr.streams[i]->ops) copies[i] += op.kind == Op::COPY;
    CHECK(copies[0] > 0 && copies[1] > 0, "copies on the two copy streams: %d, %d", copies[0], copies[1]);
    CHECK(k.staging_waits == 0, "staging waits");
    delete t;
}

void scenario_open_lease_holds_rows()
{
    // A lease that is never released keeps the rows its generation names
    // (and, kMaps generations later, its map) out of reach.
    const Source src({8, 256, 512}, 3);
    SimTransport tr;
    moe_table_desc d = desc_of(src, 2, 6, 2, 2, 4);       // 8 rows: everything fits
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    SimStream *c = tr.new_stream();
    moe_table_lease held;
    CHECK(t->acquire(c, &held) == MOE_OK, "acquire generation 1");
    Stepper st{tr, *t, src, c};
    int rc = MOE_OK, s = 0;
    // each step publishes a new generation; the 4th would reuse generation 1's map
    for (; s < 3 && rc == MOE_OK; ++s) rc = st.step({(int32_t)(2 + 2 * s), (int32_t)(3 + 2 * s)}, false);
    CHECK(rc == MOE_OK, "three generations with a lease on the first (rc %d at %d)", rc, s);
    std::vector<int32_t> act = {0, 1}, miss(2);
    int nm = 0;
    t->misses(act.data(), 2, miss.data(), &nm);
    // 0 and 1 were dropped above capacity in generation 2; reloading them needs rows and map
    rc = nm ? t->upload(miss.data(), nm, c) : MOE_OK;
    CHECK(nm == 2 && rc == MOE_ERR_CAPACITY, "upload while generation 1 is leased: nm %d rc %d", nm, rc);
    moe_table_counters k;
    t->stats(&k);
    CHECK(k.generation == 4 && k.open_leases == 1, "generation %llu, open %llu", (unsigned long long)k.generation,
          (unsigned long long)k.open_leases);
    CHECK(t->release(&held, c) == MOE_OK, "release");
    CHECK(t->upload(miss.data(), nm, c) == MOE_OK, "upload after release");
    tr.run_all();
    CHECK(st.bad_reads == 0, "bad reads %d", st.bad_reads);
    delete t;
}

void scenario_failure_before_publication()
{
    // A copy fails in the middle of a transaction: the previous generation
    // stays current and intact, the table is not faulted, the next
    // transaction succeeds.  Cases 3-6 copy from a page-locked source over
    // two copy streams (no staging records; the first record joins them).
    const Source src({8, 256, 512}, 4);
    for (int which = 0; which < 7; ++which) {
        SimTransport tr;
        tr.pinned_source = which >= 3;
        moe_table_desc d = desc_of(src, 3, 5, 2, 2, 2);
        tcore::Table *t = nullptr;
        CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
        if (!t) continue;
        SimStream *c = tr.new_stream();
        moe_table_lease old;
        CHECK(t->acquire(c, &old) == MOE_OK, "acquire");
        int32_t before[64];
        t->published(before);
        if (which == 0) tr.fail_h2d_at = tr.n_h2d + 2;          // second copy of the transaction
        if (which == 1) tr.fail_publish_at = tr.n_publish + 1;  // the map write
        if (which == 2) tr.fail_record_at = tr.n_record + 4;    // the publication event (after 3 staging records)
        if (which == 3) tr.fail_h2d_at = tr.n_h2d + 3;          // third copy (the second is in flight on stream 2)
        if (which == 4) tr.fail_record_at = tr.n_record + 1;    // joining the copy streams
        if (which == 5) tr.fail_publish_at = tr.n_publish + 1;
        if (which == 6) tr.fail_record_at = tr.n_record + 2;    // the publication event
        std::vector<int32_t> act = {4, 5, 6}, miss(3);
        int nm = 0;
        t->misses(act.data(), 3, miss.data(), &nm);
        const int rc = t->upload(miss.data(), nm, c);
        CHECK(rc == MOE_ERR_HIP, "case %d: rc %d", which, rc);
        CHECK(!t->faulted(), "case %d: faulted", which);
        // two copy streams: the failed transaction's copies are drained before
        // the call returns (the retry may write its rows on the other stream)
        if (tr.pinned_source)
            for (int i = 0; i < 2; ++i)
                CHECK(tr.streams[i]->next == tr.streams[i]->ops.size(), "case %d: copy stream %d not drained", which,
                      i);
        int32_t after[64];
        t->published(after);
        CHECK(std::memcmp(before, after, sizeof(int32_t) * 8) == 0, "case %d: map changed", which);
        moe_table_counters k;
        t->stats(&k);
        CHECK(k.generation == 1 && k.failed_uploads == 1, "case %d: generation %llu", which,
              (unsigned long long)k.generation);
        tr.run_all();
        std::string why;
        CHECK(rows_match(*t, src, old, &why), "case %d: generation 1 damaged: %s", which, why.c_str());
        CHECK(t->release(&old, c) == MOE_OK, "release");
        CHECK(t->upload(miss.data(), nm, c) == MOE_OK, "case %d: retry", which);
        moe_table_lease nl;
        CHECK(t->acquire(c, &nl) == MOE_OK, "acquire new");
        tr.run_all();
        CHECK(rows_match(*t, src, nl, &why), "case %d: new generation: %s", which, why.c_str());
        t->release(&nl, c);
        delete t;
    }
}

void scenario_failure_after_publication()
{
    // Ordering the consumer after the new generation fails: ambiguous, so the
    // table faults and refuses further work.
    const Source src({8, 256, 512}, 5);
    SimTransport tr;
    moe_table_desc d = desc_of(src, 3, 5, 2, 2, 2);
    tcore::Table *t = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK, "create");
    if (!t) return;
    SimStream *c = tr.new_stream();
    std::vector<int32_t> act = {6, 7}, miss(2);
    int nm = 0;
    t->misses(act.data(), 2, miss.data(), &nm);
    tr.fail_wait_at = tr.n_wait + 1;
    CHECK(t->upload(miss.data(), nm, c) == MOE_ERR_FAULTED, "faulted upload");
    CHECK(t->faulted(), "faulted flag");
    CHECK(t->misses(act.data(), 2, miss.data(), &nm) == MOE_ERR_FAULTED, "misses after fault");
    moe_table_lease l;
    CHECK(t->acquire(c, &l) == MOE_ERR_FAULTED, "acquire after fault");
    tr.run_all();
    delete t;
}

void scenario_create_checks()
{
    const Source src({8, 256, 512}, 6);
    SimTransport tr;
    tcore::Table *t = nullptr;
    // spare rows below what steps of max_tokens need
    moe_table_desc d = desc_of(src, 3, 4, 2, 2, 2);       // needs min(5, 4 + 1) = 5
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_ERR_CAPACITY && !t, "too few spares");
    d = desc_of(src, 3, 5, 0, 2, 2);
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_ERR_CAPACITY && !t, "no staging");
    d = desc_of(src, 3, 5, 2, 2, 2);
    std::vector<uint64_t> wrong(src.digests);
    wrong[5] ^= 1;
    d.row_digests = wrong.data();
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_ERR_SOURCE && !t, "digest mismatch");
    Source bad({8, 256, 512}, 6);
    size_t off[6];
    tcore::row_layout(256, 512, off);
    const uint16_t inf = 0x7c00;
    std::memcpy(bad.bytes.data() + 3 * bad.stride + off[4] + 10, &inf, 2);
    d = desc_of(bad, 3, 5, 2, 2, 2);
    d.row_digests = nullptr;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_ERR_SOURCE && !t, "non-finite scale");
    d = desc_of(src, 3, 5, 2, 2, 2);
    tr.fail_pinned_at = tr.n_pinned + 2;
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_ERR_CAPACITY && !t, "pinned allocation failure");
    // identity re-check after a host rewrite
    Source mut({8, 256, 512}, 8);
    d = desc_of(mut, 3, 5, 2, 2, 2);
    CHECK(tcore::Table::create(&tr, &d, &t) == MOE_OK && t, "create");
    if (t) {
        CHECK(t->verify_source() == MOE_OK, "unchanged source");
        mut.bytes[2 * mut.stride + 100] ^= 0x10;
        CHECK(t->verify_source() == MOE_ERR_SOURCE, "rewrite found");
        moe_table_counters k;
        t->stats(&k);
        CHECK(k.host_writes == 1, "host_writes %llu", (unsigned long long)k.host_writes);
        delete t;
    }
    // the spare-row rule: every step of max_tokens tokens finds rows
    CHECK(tcore::spare_needed(64, 40, 8, 32) == 24, "OLMoE stack");
    CHECK(tcore::spare_needed(64, 40, 8, 1) == 8, "OLMoE stack T=1");
    CHECK(tcore::spare_needed(60, 39, 4, 1) == 4, "Qwen T=1");
    CHECK(tcore::spare_needed(60, 39, 4, 16) == 21, "Qwen T=16");
    CHECK(tcore::spare_needed(64, 2, 8, 1) == 14, "small capacity");
}

void scenario_threads()
{
    // Several tables on several threads share the process-wide copy pool
    // (rows above its split size): run under the thread sanitizer.
    const Shape sh{12, 1024, 512};
    std::vector<std::thread> th;
    std::vector<int> bad(4, 0), errs(4, 0);
    for (int w = 0; w < 4; ++w)
        th.emplace_back([&, w] {
            const Source src(sh, 100 + w);
            SimTransport tr;
            moe_table_desc d = desc_of(src, 4, 8, 2, 2, 4);
            tcore::Table *t = nullptr;
            if (tcore::Table::create(&tr, &d, &t) != MOE_OK) {
                errs[w]++;
                return;
            }
            Stepper st{tr, *t, src, tr.new_stream()};
            std::mt19937 rng(w);
            for (int s = 0; s < 60; ++s) {
                if (st.step(random_active(rng, sh.E, 1 + (int)(rng() % 8u), 1), s % 3 == 0) != MOE_OK) errs[w]++;
                tr.stream_sync(tr.streams[0].get());
            }
            tr.run_all();
            bad[w] = st.bad_reads;
            delete t;
        });
    for (auto &t : th) t.join();
    for (int w = 0; w < 4; ++w) CHECK(bad[w] == 0 && errs[w] == 0, "thread %d: %d bad reads, %d errors", w, bad[w],
                                      errs[w]);
    CHECK(tcore::CopyPool::get().workers() == tcore::CopyPool::configured_workers(), "copy pool workers");
}

}  // namespace

int main(int argc, char **argv)
{
    const std::string which = argc > 1 ? argv[1] : "all";
    const std::pair<const char *, void (*)()> all[] = {
        {"steps", scenario_steps},
        {"default_stream", scenario_default_stream_consumer},
        {"prefetch", scenario_prefetch},
        {"staging", scenario_staging_reuse},
        {"direct", scenario_direct_from_pinned_source},
        {"lease", scenario_open_lease_holds_rows},
        {"fail_before", scenario_failure_before_publication},
        {"fail_after", scenario_failure_after_publication},
        {"create", scenario_create_checks},
        {"threads", scenario_threads},
    };
    int ran = 0;
    for (const auto &s : all)
        if (which == "all" || which == s.first) {
            const int before = g_failures;
            s.second();
            std::printf("%s: %s\n", s.first, g_failures == before ? "ok" : "FAILED");
            ++ran;
        }
    if (!ran) {
        std::fprintf(stderr, "unknown scenario %s\n", which.c_str());
        return 2;
    }
    return g_failures ? 1 : 0;
}
