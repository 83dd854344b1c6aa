// workspace_selftest.cpp -- the scratch pool of gemm_tiled_amd/csrc/
// workspace.hpp under a mock device, on the CPU.
//
// The mock device keeps one FIFO of operations per stream (allocations,
// frees, event records, and the "launches" of the simulated calls) and runs
// them in a random interleaving of the streams, in order within each stream,
// as a GPU would.  It reports:
//   - a launch that runs on a buffer already freed, or before its allocation
//     has run on another stream (use after free / before allocation);
//   - a free that runs while a launch of the buffer is still queued on some
//     stream (the buffer freed under pending work);
//   - two calls whose launches on one buffer interleave (between the first
//     and the last launch of one call, another call's launch on the buffer);
//   - more slots kept than the cap;
//   - an allocation or event query while the stream is being captured, and a
//     withdrawn buffer that is reused or freed.
// Exit status 0 and "ok" when every scenario passes.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <map>
#include <mutex>
#include <random>
#include <set>
#include <string>
#include <thread>
#include <vector>

#include "workspace.hpp"

namespace {

int g_fail = 0;
std::mutex g_fail_mu;
void fail(const std::string& what) {
    std::lock_guard<std::mutex> lock(g_fail_mu);
    if (g_fail < 20) std::fprintf(stderr, "FAIL: %s\n", what.c_str());
    ++g_fail;
}

struct Op {
    enum Kind { Alloc, Free, Record, Use } kind;
    uintptr_t buf;
    int ev;
    long call;   // Use: the simulated call
};

struct MockDevice {
    using Stream = int;
    using Event = int;
    std::mutex mu;
    std::map<int, std::deque<Op>> q;           // per stream
    std::set<uintptr_t> live;                  // allocation has run, free has not
    std::set<uintptr_t> freed;
    std::set<uintptr_t> withdrawn;             // must never be freed or reused
    std::map<int, int> pending_records;        // event -> records not yet run
    std::set<int> capturing_streams;
    uintptr_t next = 0x10000;
    int next_ev = 1;
    long allocs = 0, frees = 0, queries_in_capture = 0;
    bool fail_next_alloc = false;
    std::map<uintptr_t, long> active_call;     // buffer -> call in the middle of its launches
    std::map<uintptr_t, std::string> kind_of;

    // Backend interface
    int alloc(void** p, size_t bytes, Stream s) {
        std::lock_guard<std::mutex> lock(mu);
        if (capturing_streams.count(s)) fail("allocation during capture");
        if (fail_next_alloc) {
            fail_next_alloc = false;
            return 2;   // out of memory
        }
        if (bytes == 0) fail("zero-byte allocation");
        const uintptr_t b = next;
        next += 0x10000;
        ++allocs;
        q[s].push_back(Op{Op::Alloc, b, 0, 0});
        *p = reinterpret_cast<void*>(b);
        return 0;
    }
    int release(void* p, Stream s) {
        std::lock_guard<std::mutex> lock(mu);
        const uintptr_t b = reinterpret_cast<uintptr_t>(p);
        if (withdrawn.count(b)) fail("a withdrawn buffer is freed");
        ++frees;
        q[s].push_back(Op{Op::Free, b, 0, 0});
        return 0;
    }
    int zero_u32(unsigned* p, size_t, Stream s) {
        std::lock_guard<std::mutex> lock(mu);
        q[s].push_back(Op{Op::Use, reinterpret_cast<uintptr_t>(p), 0, -1});
        return 0;
    }
    int event_create(Event* e) {
        std::lock_guard<std::mutex> lock(mu);
        *e = next_ev++;
        return 0;
    }
    void event_destroy(Event) {}
    int record(Event e, Stream s) {
        std::lock_guard<std::mutex> lock(mu);
        if (capturing_streams.count(s)) fail("event recorded on a capturing stream");
        ++pending_records[e];
        q[s].push_back(Op{Op::Record, 0, e, 0});
        return 0;
    }
    bool idle(Event e) {
        std::lock_guard<std::mutex> lock(mu);
        if (!capturing_streams.empty()) ++queries_in_capture;
        return pending_records[e] == 0;
    }
    bool capturing(Stream s) {
        std::lock_guard<std::mutex> lock(mu);
        return capturing_streams.count(s) != 0;
    }

    // The simulated calls' launches.  A buffer may have queued launches on
    // one stream at a time: on two, their order is unknown (a race).
    void launch(uintptr_t b, Stream s, long call) {
        std::lock_guard<std::mutex> lock(mu);
        for (auto& kv : q)
            if (kv.first != s)
                for (const Op& o : kv.second)
                    if (o.kind == Op::Use && o.buf == b)
                        fail("a buffer has queued launches on two streams");
        q[s].push_back(Op{Op::Use, b, 0, call});
    }
    // Host-side bracket of one call's launches on a buffer: no other call
    // may enqueue a launch on it in between.
    void begin_call(uintptr_t b, long call) {
        std::lock_guard<std::mutex> lock(mu);
        auto it = active_call.find(b);
        if (it != active_call.end() && it->second != call)
            fail("two calls interleave launches on one buffer");
        active_call[b] = call;
    }
    void end_call(uintptr_t b, long call) {
        std::lock_guard<std::mutex> lock(mu);
        auto it = active_call.find(b);
        if (it == active_call.end() || it->second != call) fail("call bracket mismatch");
        else active_call.erase(it);
    }

    // Run one queued operation of a random non-empty stream.
    bool step(std::mt19937& rng) {
        std::lock_guard<std::mutex> lock(mu);
        std::vector<int> ready;
        for (auto& kv : q)
            if (!kv.second.empty()) ready.push_back(kv.first);
        if (ready.empty()) return false;
        const int s = ready[rng() % ready.size()];
        const Op op = q[s].front();
        q[s].pop_front();
        switch (op.kind) {
            case Op::Alloc:
                live.insert(op.buf);
                break;
            case Op::Free: {
                if (!live.count(op.buf)) fail("free of a buffer that is not live");
                for (auto& kv : q)
                    for (const Op& o : kv.second)
                        if (o.kind == Op::Use && o.buf == op.buf)
                            fail("buffer freed while a launch on it is still queued");
                live.erase(op.buf);
                freed.insert(op.buf);
                break;
            }
            case Op::Record:
                --pending_records[op.ev];
                break;
            case Op::Use:
                if (freed.count(op.buf)) fail("launch on a freed buffer");
                else if (!live.count(op.buf)) fail("launch before the buffer's allocation ran");
                break;
        }
        return true;
    }
    void drain(std::mt19937& rng) {
        while (step(rng)) {
        }
    }
};

using Pool = g355::ScratchPool<MockDevice>;

// One simulated library call: lease, ask for scratch (workspace and/or
// counters), enqueue 1-3 launches on each buffer, end.
void one_call(Pool& pool, MockDevice& dev, int s, long call, size_t bytes, size_t ncnt,
              int launches, bool expect_ok = true) {
    Pool::Lease l = pool.lease(s);
    void* ws = nullptr;
    unsigned* cnt = nullptr;
    if (bytes) {
        const int e = l.workspace(bytes, &ws);
        if (e) {
            if (expect_ok) fail("workspace request failed: " + std::to_string(e));
            return;
        }
        if (l.slot()->ws_bytes < bytes) fail("workspace smaller than asked");
    }
    if (ncnt) {
        const int e = l.counters(ncnt, &cnt);
        if (e) {
            if (expect_ok) fail("counters request failed");
            return;
        }
    }
    std::vector<uintptr_t> bufs;
    if (ws) bufs.push_back(reinterpret_cast<uintptr_t>(ws));
    if (cnt) bufs.push_back(reinterpret_cast<uintptr_t>(cnt));
    for (uintptr_t b : bufs) dev.begin_call(b, call);
    for (int i = 0; i < launches; ++i) {
        for (uintptr_t b : bufs) dev.launch(b, s, call);
        std::this_thread::yield();
    }
    for (uintptr_t b : bufs) dev.end_call(b, call);
}

// Random calls on several streams with random sizes, the device running a
// random interleaving in between.
void scenario_random(unsigned seed) {
    MockDevice dev;
    std::mt19937 rng(seed);
    {
        Pool pool(dev, 3);
        for (long call = 0; call < 4000; ++call) {
            const int s = static_cast<int>(rng() % 6);
            const size_t bytes = (rng() % 4) ? (size_t{1} << (10 + rng() % 14)) * (1 + rng() % 5) : 0;
            const size_t ncnt = (rng() % 3) ? 0 : 1 + rng() % 20000;
            one_call(pool, dev, s, call, bytes, ncnt, 1 + static_cast<int>(rng() % 3));
            const Pool::Stats st = pool.stats();
            if (st.kept > pool.cap()) fail("more slots kept than the cap");
            if (st.leased != 0) fail("a slot stays leased after its call");
            const int steps = static_cast<int>(rng() % 12);
            for (int i = 0; i < steps; ++i) dev.step(rng);
            if (rng() % 200 == 0) dev.drain(rng);
        }
        dev.drain(rng);
        if (dev.allocs == 0 || dev.frees == 0) fail("the random scenario never grew a buffer");
    }
}

// Calls on one stream and on two streams from many threads at once.
void scenario_threads() {
    MockDevice dev;
    Pool pool(dev, 4);
    std::atomic<long> ids{0};
    std::atomic<bool> stop{false};
    std::thread device([&] {
        std::mt19937 rng(7);
        while (!stop.load()) {
            if (!dev.step(rng)) std::this_thread::yield();
        }
        dev.drain(rng);
    });
    std::vector<std::thread> ts;
    for (int t = 0; t < 8; ++t)
        ts.emplace_back([&, t] {
            std::mt19937 rng(100 + t);
            for (int i = 0; i < 3000; ++i) {
                const int s = (t % 2 == 0) ? 0 : static_cast<int>(1 + rng() % 2);
                const size_t bytes = size_t{1} << (12 + rng() % 12);
                one_call(pool, dev, s, ids.fetch_add(1), bytes, (rng() % 2) ? 64 : 0, 3);
            }
        });
    for (auto& th : ts) th.join();
    stop.store(true);
    device.join();
    if (pool.stats().leased != 0) fail("threads: a slot stays leased");
}

// Stream capture: no allocation, no event query, no record; a slot of the
// capturing stream that is large enough is used and then withdrawn.
void scenario_capture() {
    MockDevice dev;
    std::mt19937 rng(3);
    Pool pool(dev, 4);
    // nothing yet on stream 5: a capture that needs scratch fails cleanly
    dev.capturing_streams.insert(5);
    {
        Pool::Lease l = pool.lease(5);
        void* p = nullptr;
        if (l.workspace(1 << 20, &p) != Pool::kNeedsAlloc) fail("capture without a slot must fail");
    }
    dev.capturing_streams.clear();
    // eager call creates the stream's slot, then a capture uses it
    one_call(pool, dev, 5, 1, 8 << 20, 100, 2);
    const long allocs = dev.allocs;
    dev.capturing_streams.insert(5);
    Pool::Stats before = pool.stats();
    uintptr_t captured = 0;
    {
        Pool::Lease l = pool.lease(5);
        void* p = nullptr;
        if (l.workspace(4 << 20, &p) != 0) fail("capture with a large-enough slot must succeed");
        captured = reinterpret_cast<uintptr_t>(p);
        dev.launch(captured, 5, 2);
        void* q = nullptr;
        if (l.workspace(64 << 20, &q) != Pool::kNeedsAlloc) fail("growth during capture must fail");
    }
    if (dev.allocs != allocs) fail("allocation during capture");
    if (dev.queries_in_capture) fail("event query during capture");
    Pool::Stats after = pool.stats();
    if (after.withdrawn != before.withdrawn + 1) fail("the captured slot is not withdrawn");
    dev.capturing_streams.clear();
    {
        std::lock_guard<std::mutex> lock(dev.mu);
        dev.withdrawn.insert(captured);
    }
    // later eager calls of every size never get the withdrawn buffer
    for (long c = 10; c < 200; ++c) {
        Pool::Lease l = pool.lease(static_cast<int>(c % 3) + 4);
        void* p = nullptr;
        if (l.workspace(size_t{1} << (12 + c % 16), &p) != 0) fail("eager call after capture");
        if (reinterpret_cast<uintptr_t>(p) == captured) fail("a withdrawn buffer is reused");
        dev.launch(reinterpret_cast<uintptr_t>(p), static_cast<int>(c % 3) + 4, c);
        dev.step(rng);
    }
    dev.drain(rng);
    // a capture lease that hands out no buffer withdraws nothing
    one_call(pool, dev, 6, 300, 1 << 12, 0, 1);
    dev.capturing_streams.insert(6);
    const size_t w = pool.stats().withdrawn;
    { Pool::Lease l = pool.lease(6); }
    if (pool.stats().withdrawn != w) fail("an unused capture lease withdrew its slot");
    dev.capturing_streams.clear();
    dev.drain(rng);
}

// An allocation that fails leaves the pool usable and nothing dangling.
void scenario_alloc_failure() {
    MockDevice dev;
    std::mt19937 rng(5);
    Pool pool(dev, 2);
    one_call(pool, dev, 0, 1, 1 << 20, 0, 1);
    dev.fail_next_alloc = true;
    {
        Pool::Lease l = pool.lease(0);
        void* p = nullptr;
        if (l.workspace(64 << 20, &p) == 0) fail("injected allocation failure not reported");
    }
    for (long c = 2; c < 50; ++c) one_call(pool, dev, static_cast<int>(c % 2), c, 1 << (16 + c % 8), 0, 1);
    dev.drain(rng);
    if (pool.stats().leased) fail("alloc failure: slot stays leased");
}

// The cap holds when more streams than slots are busy at once: transient
// slots are freed stream-ordered when their call ends.
void scenario_cap() {
    MockDevice dev;
    std::mt19937 rng(9);
    Pool pool(dev, 2);
    std::vector<Pool::Lease> held;
    for (int s = 0; s < 6; ++s) {
        held.push_back(pool.lease(s));
        void* p = nullptr;
        if (held.back().workspace(1 << 20, &p) != 0) fail("cap: request failed");
        dev.launch(reinterpret_cast<uintptr_t>(p), s, s);
    }
    held.clear();
    if (pool.stats().kept > 2) fail("cap: more slots kept than the cap");
    dev.drain(rng);
    if (dev.frees < 4) fail("cap: transient slots not freed");
}

// Events are recorded only while the pool is full: one stream, or fewer
// streams than the cap, records none (each stream keeps its own slot); at
// the cap, leases record events and idle slots move between streams.
void scenario_events() {
    std::mt19937 rng(11);
    {
        MockDevice dev;
        Pool pool(dev, 4);
        for (long c = 0; c < 200; ++c) one_call(pool, dev, 0, c, 1 << (12 + c % 10), c % 3 ? 0 : 50, 2);
        for (long c = 200; c < 400; ++c) one_call(pool, dev, static_cast<int>(c % 3), c, 1 << 16, 0, 1);
        dev.drain(rng);
        const Pool::Stats st = pool.stats();
        if (st.records != 0) fail("events recorded below the cap");
        if (st.kept != 3) fail("three streams below the cap should keep three slots");
    }
    {
        MockDevice dev;
        Pool pool(dev, 2);
        {
        // events recorded at the cap, then a capture withdraws a slot (the pool
        // drops below the cap and later leases record no event): the older
        // event of the other slot must not make it look idle to a third stream
        MockDevice dev;
        Pool pool(dev, 2);
        for (long c = 0; c < 10; ++c) one_call(pool, dev, static_cast<int>(c % 2), c, 1 << 20, 0, 1);
        dev.drain(rng);
        dev.capturing_streams.insert(1);
        {
            Pool::Lease l = pool.lease(1);
            void* p = nullptr;
            if (l.workspace(1 << 20, &p) != 0) fail("events: capture lease");
            dev.launch(reinterpret_cast<uintptr_t>(p), 1, 50);
        }
        dev.capturing_streams.clear();
        dev.drain(rng);
        one_call(pool, dev, 0, 60, 1 << 20, 0, 2);   // queued, not run: below the cap, no event
        one_call(pool, dev, 5, 61, 1 << 20, 0, 1);   // must not take stream 0's slot
        dev.drain(rng);
    }
    // fill the pool: two streams, then calls that record
        for (long c = 0; c < 40; ++c) one_call(pool, dev, static_cast<int>(c % 2), c, 1 << 20, 0, 1);
        if (pool.stats().records == 0) fail("no events recorded at the cap");
        dev.drain(rng);
        // a third stream finds an idle slot of another stream and reuses it
        const long allocs = dev.allocs;
        one_call(pool, dev, 7, 100, 1 << 20, 0, 1);
        if (dev.allocs != allocs) fail("an idle slot at the cap was not reused across streams");
        if (pool.stats().kept != 2) fail("cap: kept slots");
        dev.drain(rng);
    }
}

}  // namespace

int main() {
    for (unsigned seed = 1; seed <= 4; ++seed) scenario_random(seed);
    scenario_threads();
    scenario_capture();
    scenario_alloc_failure();
    scenario_cap();
    scenario_events();
    if (g_fail) {
        std::fprintf(stderr, "%d failure(s)\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
