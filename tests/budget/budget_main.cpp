// Host test of the lean launch budget (csrc/budget.h) with fake events that
// the test completes by hand. Prints "ok" and exits 0 when every check holds.
// Test infrastructure: built and run by tests/test_budget.py.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "budget.h"

namespace {

struct Fake {
    std::vector<int> state;    // per event: 0 pending, 1 done
    std::vector<int> waited;   // events waited for, in order
    int released = 0;
};
Fake g;

struct FakeOps {
    using event = int;
    event record(void*) {
        g.state.push_back(0);
        return (int)g.state.size() - 1;
    }
    bool done(event e) { return g.state[e] == 1; }
    void wait(event e) {
        g.waited.push_back(e);
        g.state[e] = 1;
    }
    void release(event) { ++g.released; }
};

int failures = 0;
void check(bool ok, const char* what) {
    if (!ok) {
        std::printf("FAIL: %s\n", what);
        ++failures;
    }
}

}  // namespace

int main() {
    la::LaunchBudget<FakeOps> b{FakeOps{}};
    void* s1 = (void*)0x1;
    void* s2 = (void*)0x2;
    void* s3 = (void*)0x3;
    const int cap = 1024;

    // one stream: its own unfinished launches never count
    check(b.admit(s1, 512, cap) == 512, "first launch keeps its grid");
    b.record(s1, 512, cap);
    check(b.admit(s1, 1024, cap) == 1024, "same stream: earlier launches do not count");
    b.record(s1, 1024, cap);

    // a second stream fits beside half of the device...
    g.state[1] = 1;   // the 1024-workgroup launch on s1 finished
    check(b.admit(s2, 512, cap) == 512, "two halves fit");
    b.record(s2, 512, cap);
    check(b.live() == 2, "finished launch retired");
    // ... a third launch gets only what is left of the device: nothing, so it
    // waits for the oldest launch of another stream (s1's), then fits
    check(b.admit(s3, 512, cap) == 512, "third launch after waiting");
    check(g.waited.size() == 1 && g.waited[0] == 0, "waited for the oldest other launch");
    b.record(s3, 512, cap);

    // a partial room shrinks the grid: s2 and s3 hold 512 each of 1024 ->
    // after s2's launch finishes, 512 are free for s1 however many it asks
    g.state[2] = 1;
    check(b.admit(s1, 1024, cap) == 512, "shrunk to the room left");
    b.record(s1, 512, cap);

    // kernels of different capacities share by fraction: a grouped launch of
    // 256 of 512 (one half) beside s3's 512 of 1024 (one half) and s1's 512 of
    // 1024 (one half) does not fit -> waits for the oldest other (s3's), fits
    check(b.admit(s2, 256, 512) == 256, "mixed capacities: wait then fit");
    check(g.waited.size() == 2 && g.waited[1] == 3, "waited for s3's launch");
    b.record(s2, 256, 512);
    // now s1 (1/2) + s2 (1/2) are live: a 100-workgroup launch of capacity
    // 1024 on s1 ignores s1's own and fits beside s2's half
    check(b.admit(s1, 100, cap) == 100, "own stream ignored in the sum");

    // rounding: three thirds fill the device exactly
    la::LaunchBudget<FakeOps> c{FakeOps{}};
    c.record(s1, 341, 1023);
    c.record(s2, 341, 1023);
    check(c.admit(s3, 341, 1023) == 341, "exact fill within rounding");
    check(c.admit(s3, 342, 1023) == 341, "one more than the room is shrunk");

    b.clear();
    check(b.live() == 0, "clear forgets every launch");
    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
