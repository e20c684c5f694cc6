// Co-resident capacity shared by lean launches on several streams of one
// device (host only).
//
// A lean launch is correct only if every peer its hosts wait for gets to run:
// the grid is capped at the kernel's co-resident capacity so that all of it
// fits on the device at once. Launches on several streams run concurrently,
// and the hardware may interleave the dispatch of their workgroups; if their
// grids together exceed the capacity, each can end up partly resident, its
// hosts spinning on peers that cannot start until another launch's hosts stop
// spinning. The budget keeps the unfinished lean launches of a device within
// the capacity: a launch's share is grid / capacity of its kernel (the
// single-head and grouped kernels fit different numbers of workgroups on a
// CU), and a new launch gets the largest grid whose share fits beside the
// unfinished launches of other streams -- or, when not even one workgroup
// fits, waits for the oldest of them. Earlier launches on the same stream are
// ordered before the new one and do not count.
//
// `Ops` supplies the completion events: `event record(void* stream)` (marks
// the work enqueued on the stream so far), `bool done(event)`, `void
// wait(event)` and `void release(event)`.
#pragma once

#include <vector>

namespace la {

template <class Ops>
class LaunchBudget {
public:
    using event = typename Ops::event;

    explicit LaunchBudget(Ops ops) : ops_(ops) {}

    // Grid for a launch of `want` workgroups (>= 1) of a kernel that fits
    // `cap` workgroups on the device, on `stream`: `want` if it fits beside the
    // unfinished launches of other streams, else the largest grid that does
    // (>= 1), waiting for the oldest of them while none fits.
    int admit(void* stream, int want, int cap) {
        for (;;) {
            retire();
            double used = 0.0;
            for (const Entry& e : live_)
                if (e.stream != stream) used += e.share;
            const double room = 1.0 - used;
            // the largest grid g <= want with g / cap <= room (within rounding)
            int g = want;
            if ((double)g / cap > room + 1e-12) g = (int)((room + 1e-12) * cap);
            if (g >= 1) return g;
            wait_oldest_other(stream);
        }
    }

    // A launch of `grid` workgroups of a kernel with capacity `cap` was just
    // enqueued on `stream`.
    void record(void* stream, int grid, int cap) {
        live_.push_back(Entry{ops_.record(stream), stream, (double)grid / cap});
    }

    // Launches still tracked (unfinished when last looked at).
    size_t live() const { return live_.size(); }

    // Forget every launch (their events released), e.g. before the streams
    // are destroyed.
    void clear() {
        for (Entry& e : live_) ops_.release(e.ev);
        live_.clear();
    }

private:
    struct Entry {
        event ev;
        void* stream;
        double share;
    };

    void retire() {
        size_t k = 0;
        for (size_t i = 0; i < live_.size(); ++i) {
            if (ops_.done(live_[i].ev))
                ops_.release(live_[i].ev);
            else
                live_[k++] = live_[i];
        }
        live_.resize(k);
    }

    void wait_oldest_other(void* stream) {
        for (Entry& e : live_) {
            if (e.stream != stream) {
                ops_.wait(e.ev);
                return;
            }
        }
    }

    Ops ops_;
    std::vector<Entry> live_;
};

}  // namespace la
