// workspace.hpp -- the device scratch of the library's calls (the packed
// binary16 operands of the f16r mode, the partial tiles of the calls that
// split K over workgroups, and their arrival counters), kept in a pool per
// device.
//
// Plain C++ with no HIP header: the device operations come from a Backend
// class, so the same pool runs on the GPU (the HIP backend in gemm355.cpp)
// and under a mock backend in a CPU test.
//
// The rules that make it safe:
//   * A call holds one slot of the pool (a lease) from its first request for
//     scratch until its last launch is enqueued.  No other call touches the
//     slot meanwhile, so two calls never interleave launches on one buffer,
//     whichever threads and streams they come from.
//   * A slot is leased again only when that use is ordered after the work of
//     its last lease: by a call on the same stream (stream order), or, on
//     another stream, once the event recorded when the last lease ended has
//     completed.  That event is recorded only while the pool holds `cap`
//     slots (an event in the stream costs each call a few microseconds of GPU
//     time): below the cap a call on a new stream gets a slot of its own, and
//     a slot whose last lease recorded no event is never handed to another
//     stream.
//   * Buffers are allocated and freed stream-ordered on the stream of the
//     call that leases them (the stream of their last use, or any stream
//     once they are idle), so nothing waits on the host.
//   * The pool keeps at most `cap` slots per device.  A call that finds no
//     reusable slot when the pool is full gets a transient slot, freed
//     stream-ordered when the call ends.  Memory kept is thus at most cap
//     times the largest request, plus the slots withdrawn below.
//   * Under stream capture nothing is allocated or queried: a call may only
//     take a slot of its own stream that is already large enough (otherwise
//     it fails with kNeedsAlloc), and that slot is then withdrawn from the
//     pool for good, because the graph may replay its launches at any time
//     (it is never reused, grown or freed).
//
// Backend interface (all int results: 0 = success, else an error code):
//   using Stream, Event;
//   int  alloc(void** p, size_t bytes, Stream s);   stream-ordered allocation
//   int  release(void* p, Stream s);                stream-ordered free
//   int  zero_u32(unsigned* p, size_t n, Stream s); p[0..n) = 0 on s
//   int  event_create(Event* e);  void event_destroy(Event e);
//   int  record(Event e, Stream s);
//   bool idle(Event e);       the work before the last record has completed
//   bool capturing(Stream s); s is being captured into a graph
#ifndef GEMM355_WORKSPACE_HPP
#define GEMM355_WORKSPACE_HPP

#include <cstddef>
#include <atomic>
#include <cstdint>
#include <list>
#include <memory>
#include <mutex>
#include <vector>

namespace g355 {

template <class Backend>
class ScratchPool {
public:
    using Stream = typename Backend::Stream;
    using Event = typename Backend::Event;

    // Returned by Lease::workspace / Lease::counters when the buffer would
    // have to be allocated while the stream is being captured.
    static constexpr int kNeedsAlloc = -1;
    // Buffers grow in steps of this many bytes.
    static constexpr size_t kGrain = size_t{2} << 20;

    struct Stats {
        size_t kept = 0;        // slots in the pool
        size_t withdrawn = 0;   // slots a captured call withdrew
        size_t leased = 0;      // slots leased now
        size_t bytes = 0;       // device bytes held by kept and withdrawn slots
        uint64_t leases = 0;    // leases ended (outside capture)
        uint64_t records = 0;   // of which recorded an event
    };

    ScratchPool(Backend& b, size_t cap) : b_(b), cap_(cap ? cap : 1) {}
    ~ScratchPool() {
        // The process is ending (the pool is a static object) or a test
        // owns it: give events back; device memory goes with the context.
        for (auto& s : slots_)
            if (s->has_event) b_.event_destroy(s->ev);
        for (auto& s : withdrawn_)
            if (s->has_event) b_.event_destroy(s->ev);
    }
    ScratchPool(const ScratchPool&) = delete;
    ScratchPool& operator=(const ScratchPool&) = delete;

    struct Slot {
        void* ws = nullptr;
        size_t ws_bytes = 0;
        unsigned* cnt = nullptr;
        size_t cnt_n = 0;
        Stream last{};          // stream of the last lease
        bool used = false;      // `last` is meaningful
        Event ev{};
        bool has_event = false;
        bool recorded = false;  // ev was recorded after the last lease
        bool leased = false;
        bool transient = false;
        uint64_t tick = 0;
    };

    class Lease {
    public:
        Lease() = default;
        Lease(Lease&& o) noexcept { *this = std::move(o); }
        Lease& operator=(Lease&& o) noexcept {
            end();
            pool_ = o.pool_;
            slot_ = o.slot_;
            s_ = o.s_;
            capture_ = o.capture_;
            handed_ = o.handed_;
            status_ = o.status_;
            o.pool_ = nullptr;
            o.slot_ = nullptr;
            return *this;
        }
        Lease(const Lease&) = delete;
        Lease& operator=(const Lease&) = delete;
        ~Lease() { end(); }

        // 0, or why no slot could be leased (kNeedsAlloc under capture).
        int status() const { return status_; }
        const Slot* slot() const { return slot_; }

        // A device buffer of at least `bytes` bytes for the launches of this
        // call (its contents are whatever the last call left).
        int workspace(size_t bytes, void** out) {
            if (status_) return status_;
            Slot& sl = *slot_;
            if (sl.ws_bytes < bytes) {
                if (capture_) return kNeedsAlloc;
                const size_t grown = (bytes + kGrain - 1) / kGrain * kGrain;
                if (sl.ws) {
                    // stream-ordered: runs after every earlier launch on s_,
                    // which is the stream of the buffer's last use or the
                    // buffer is idle
                    if (const int e = pool_->b_.release(sl.ws, s_)) return e;
                    pool_->account(-static_cast<int64_t>(sl.ws_bytes));
                    sl.ws = nullptr;
                    sl.ws_bytes = 0;
                }
                void* p = nullptr;
                if (const int e = pool_->b_.alloc(&p, grown, s_)) return e;
                sl.ws = p;
                sl.ws_bytes = grown;
                pool_->account(static_cast<int64_t>(grown));
            }
            *out = sl.ws;
            handed_ = true;
            return 0;
        }

        // n zeroed arrival counters.  Every kernel that counts arrivals
        // leaves the counters it used at zero, so they are zeroed only when
        // allocated.
        int counters(size_t n, unsigned** out) {
            if (status_) return status_;
            Slot& sl = *slot_;
            if (sl.cnt_n < n) {
                if (capture_) return kNeedsAlloc;
                const size_t grown = n < 4096 ? 4096 : (n + 4095) / 4096 * 4096;
                if (sl.cnt) {
                    if (const int e = pool_->b_.release(sl.cnt, s_)) return e;
                    pool_->account(-static_cast<int64_t>(sl.cnt_n * sizeof(unsigned)));
                    sl.cnt = nullptr;
                    sl.cnt_n = 0;
                }
                void* p = nullptr;
                if (const int e = pool_->b_.alloc(&p, grown * sizeof(unsigned), s_)) return e;
                sl.cnt = static_cast<unsigned*>(p);
                sl.cnt_n = grown;
                pool_->account(static_cast<int64_t>(grown * sizeof(unsigned)));
                if (const int e = pool_->b_.zero_u32(sl.cnt, grown, s_)) return e;
            }
            *out = sl.cnt;
            handed_ = true;
            return 0;
        }

    private:
        friend class ScratchPool;
        void end() {
            if (pool_ && slot_) pool_->give_back(slot_, s_, capture_, handed_);
            pool_ = nullptr;
            slot_ = nullptr;
        }
        ScratchPool* pool_ = nullptr;
        Slot* slot_ = nullptr;
        Stream s_{};
        bool capture_ = false;
        bool handed_ = false;   // a buffer went to a launch of this call
        int status_ = 0;
    };

    // Lease a slot for one call on stream s (see the rules above).
    Lease lease(Stream s) {
        Lease l;
        l.pool_ = this;
        l.s_ = s;
        l.capture_ = b_.capturing(s);
        std::lock_guard<std::mutex> lock(mu_);
        Slot* pick = nullptr;
        // 1. a free slot whose last lease was on this stream (stream order),
        //    the largest
        for (auto& sp : slots_) {
            Slot* x = sp.get();
            if (!x->leased && x->used && x->last == s && (!pick || size_of(*x) > size_of(*pick)))
                pick = x;
        }
        if (!pick && l.capture_) {
            // under capture: no event query, no allocation
            l.status_ = kNeedsAlloc;
            l.pool_ = nullptr;
            return l;
        }
        // 2. a free slot that is idle: never used, or its event completed
        //    (the largest)
        if (!pick)
            for (auto& sp : slots_) {
                Slot* x = sp.get();
                if (x->leased || (x->used && !(x->recorded && b_.idle(x->ev)))) continue;
                if (!pick || size_of(*x) > size_of(*pick)) pick = x;
            }
        // 3. a new slot, transient when the pool is full
        if (!pick) {
            slots_.push_back(std::unique_ptr<Slot>(new Slot()));
            pick = slots_.back().get();
            pick->transient = slots_.size() > cap_ + transients_;
            if (pick->transient) ++transients_;
        }
        pick->leased = true;
        pick->tick = ++tick_;
        l.slot_ = pick;
        return l;
    }

    Stats stats() {
        std::lock_guard<std::mutex> lock(mu_);
        Stats st;
        for (auto& sp : slots_) {
            if (sp->transient) continue;
            ++st.kept;
            st.leased += sp->leased ? 1 : 0;
        }
        for (auto& sp : slots_)
            if (sp->transient && sp->leased) ++st.leased;
        st.withdrawn = withdrawn_.size();
        st.bytes = bytes_.load();
        st.leases = leases_;
        st.records = records_;
        return st;
    }
    size_t cap() const { return cap_; }

private:
    static size_t size_of(const Slot& x) { return x.ws_bytes + x.cnt_n * sizeof(unsigned); }

    void account(int64_t delta) {
        bytes_.fetch_add(static_cast<size_t>(delta));   // modular: adds a negative delta too
    }

    void give_back(Slot* sl, Stream s, bool capture, bool handed) {
        std::lock_guard<std::mutex> lock(mu_);
        auto it = slots_.begin();
        while (it != slots_.end() && it->get() != sl) ++it;
        if (it == slots_.end()) return;   // cannot happen: leased slots stay listed
        if (capture && !handed) {
            // nothing of the slot went into the graph: leave it as it was
            // (no event may be recorded on a capturing stream)
            sl->leased = false;
            return;
        }
        if (capture) {
            // a graph holds these buffers now: never reuse, grow or free them
            if (sl->transient) --transients_;
            sl->leased = false;
            withdrawn_.push_back(std::move(*it));
            slots_.erase(it);
            return;
        }
        if (sl->transient) {
            // stream-ordered frees after this call's launches on s
            if (sl->ws) b_.release(sl->ws, s);
            if (sl->cnt) b_.release(sl->cnt, s);
            bytes_.fetch_sub(sl->ws_bytes + sl->cnt_n * sizeof(unsigned));
            if (sl->has_event) b_.event_destroy(sl->ev);
            --transients_;
            slots_.erase(it);
            return;
        }
        sl->last = s;
        sl->used = sl->ws || sl->cnt;   // a slot without buffers is idle for any stream
        sl->recorded = false;           // an older event says nothing about this lease
        ++leases_;
        if (sl->used && slots_.size() - transients_ >= cap_) {
            if (!sl->has_event && b_.event_create(&sl->ev) == 0) sl->has_event = true;
            if (sl->has_event && b_.record(sl->ev, s) == 0) {
                sl->recorded = true;
                ++records_;
            }
        }
        sl->leased = false;
    }

    Backend& b_;
    const size_t cap_;
    std::mutex mu_;
    std::list<std::unique_ptr<Slot>> slots_;
    std::vector<std::unique_ptr<Slot>> withdrawn_;
    size_t transients_ = 0;
    std::atomic<size_t> bytes_{0};
    uint64_t leases_ = 0, records_ = 0;
    uint64_t tick_ = 0;
};

}  // namespace g355

#endif  // GEMM355_WORKSPACE_HPP
