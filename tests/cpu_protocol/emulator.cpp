// CPU emulator of the two cross-workgroup exchange protocols of the decode
// kernels, for tests: one std::thread per workgroup, fp64 arithmetic, random
// delays, C++ atomics in place of the device's agent-scope ones.
//
//   lean  the static stream-K schedule (xllm-io paper review of arXiv
//         2405.10480, §3.5): the real tables from the library's host
//         scheduler; a peer publishes its partial (m, l, Obar) and raises its
//         flag to the launch's epoch (after the first step of its
//         workgroup's next segment, or once the workgroup is done, as the
//         kernel does); a head's host waits for its peers'
//         flags to hold that epoch (bounded, like the kernel's watchdog),
//         folds their partials in workgroup order with f (§3.2) and
//         normalises. Several launches run back to back on one exchange
//         (flags, partials, control words), as on one stream: the last
//         workgroup out of a launch makes its epoch the completed one.
//   pull  chunks of the same tile order pulled from a counter by a pool of
//         threads (siliconandsystems digest, "Exact softmax can be reduced in
//         pieces"); a head spread over chunks is merged by the two-level tree
//         of the pull kernels (groups of 16 chunks, then the groups), each
//         level completed by whoever brings its arrival counter to the total.
//
// The device publishes with completion-ordered stores (a drain before the
// flag or counter); release/acquire is the C++ analogue used here, so the
// ThreadSanitizer build checks that every record is published before it is
// read. Test infrastructure: built and run by tests/test_cpu_protocol.py.
//
// Input file (little endian): int32 mode (0 lean, 1 pull), B, H, d, L, G
// (lean grid, or pull threads), C (pull chunk tiles), drop (lean: a peer
// workgroup that raises its flag only after twice the wait bound in the
// first launch, and after a quarter of it in later ones; -1 none), wait_ms,
// seed, launches (lean: launches in a row); int32 ctx[B]; float64 scale,
// q[B*H*d], k[H*sum(n)*d], v[same]. Output file: int32 status (0 ok, 4 a
// wait gave up in some launch, 5 the control words were left inconsistent),
// then float64 out[B*H*d], m[B*H], l[B*H] of the last launch (NaN for a head
// whose host gave up).

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "sched.h"

namespace {

// Built with -DEMU_UNORDERED_PUBLISH, flags and counters carry no ordering
// (relaxed): a planted mistake that the ThreadSanitizer test must catch.
#ifdef EMU_UNORDERED_PUBLISH
constexpr std::memory_order kRelease = std::memory_order_relaxed;
constexpr std::memory_order kAcquire = std::memory_order_relaxed;
constexpr std::memory_order kAcqRel = std::memory_order_relaxed;
#else
constexpr std::memory_order kRelease = std::memory_order_release;
constexpr std::memory_order kAcquire = std::memory_order_acquire;
constexpr std::memory_order kAcqRel = std::memory_order_acq_rel;
#endif

// Built with -DEMU_UNEPOCHED, the lean exchange is the earlier protocol that
// the epochs replaced: flags hold 1 and hosts lower them after merging, and
// once any wait has given up every later wait gives up at once. A late peer
// then leaves its flag raised into the next launch: a planted mistake that
// the tests must catch.

struct Rec {
    double m = -INFINITY, l = 0.0;
    std::vector<double> o;
};

struct Problem {
    int B, H, d, L;
    std::vector<int32_t> ctx;
    std::vector<int64_t> row0;   // first K/V row of head u
    double scale;
    std::vector<double> q, k, v;
};

// f on (m, l, Obar): a side with m = -inf weighs nothing.
void merge(Rec& acc, const Rec& x) {
    const double m = std::max(acc.m, x.m);
    if (m == -INFINITY) return;
    const double a = acc.m == -INFINITY ? 0.0 : std::exp(acc.m - m);
    const double b = x.m == -INFINITY ? 0.0 : std::exp(x.m - m);
    acc.l = a * acc.l + b * x.l;
    for (size_t i = 0; i < acc.o.size(); ++i) acc.o[i] = a * acc.o[i] + b * x.o[i];
    acc.m = m;
}

// Partial of head u over tiles [t0, t1): online softmax one tile at a time.
Rec partial(const Problem& P, int u, int t0, int t1) {
    const int b = u / P.H, n = P.ctx[b];
    Rec acc;
    acc.o.assign(P.d, 0.0);
    const double* q = &P.q[(size_t)u * P.d];
    for (int t = t0; t < t1; ++t) {
        const int a = t * P.L, e = std::min(n, (t + 1) * P.L);
        Rec tile;
        tile.o.assign(P.d, 0.0);
        std::vector<double> s(e - a);
        for (int j = a; j < e; ++j) {
            const double* kr = &P.k[(size_t)(P.row0[u] + j) * P.d];
            double x = 0.0;
            for (int i = 0; i < P.d; ++i) x += q[i] * kr[i];
            s[j - a] = P.scale * x;
            tile.m = std::max(tile.m, s[j - a]);
        }
        for (int j = a; j < e; ++j) {
            const double p = std::exp(s[j - a] - tile.m);
            tile.l += p;
            const double* vr = &P.v[(size_t)(P.row0[u] + j) * P.d];
            for (int i = 0; i < P.d; ++i) tile.o[i] += p * vr[i];
        }
        merge(acc, tile);
    }
    return acc;
}

void finish(const Problem& P, int u, const Rec& r, double* out, double* mo, double* lo) {
    for (int i = 0; i < P.d; ++i) out[(size_t)u * P.d + i] = r.o[i] / r.l;
    mo[u] = r.m;
    lo[u] = r.l;
}

void nap(std::mt19937& rng) {
    std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
}

int run_lean(const Problem& P, int grid, int drop, int wait_ms, int launches, unsigned seed,
             double* out, double* mo, double* lo) {
    const int BH = P.B * P.H;
    int64_t I = 0;
    int G = 0, rows = 0;
    const char* why = "";
    if (la::schedule_dims(P.ctx.data(), P.B, P.H, P.L, grid, &I, &G, &rows, &why) != 0) return 1;
    std::vector<int32_t> cta_begin(G + 1), cta_seg(G + 1), seg((size_t)rows * 6), host(BH), last(BH);
    la::build_schedule(P.ctx.data(), P.B, P.H, P.L, G, I, cta_begin.data(), cta_seg.data(),
                       seg.data(), nullptr, host.data(), last.data());
    // the exchange, kept across launches
    std::vector<Rec> part(G);
    std::vector<std::atomic<uint32_t>> flag(G);
    for (auto& f : flag) f.store(0);
    std::atomic<uint32_t> err{0}, epoch{0}, exited{0}, aborted{0};
    for (int launch = 0; launch < launches; ++launch) {
        for (int u = 0; u < BH; ++u) {
            for (int i = 0; i < P.d; ++i) out[(size_t)u * P.d + i] = NAN;
            mo[u] = lo[u] = NAN;
        }
        auto cta = [&](int c) {
            std::mt19937 rng(seed * 7919u + c + 104729u * (unsigned)launch);
            uint32_t e = epoch.load(std::memory_order_relaxed) + 1u;
            if (e == 0u) e = 1u;
            // A peer's flag goes up after the first step of its workgroup's
            // next segment, as in the kernel, or when the workgroup is done.
            bool pending = false;
            auto raise = [&]() {
                if (!pending) return;
                pending = false;
                if (c == drop)
                    std::this_thread::sleep_for(
                        std::chrono::milliseconds(launch == 0 ? 2 * wait_ms : wait_ms / 4));
#ifdef EMU_UNEPOCHED
                flag[c].store(1, kRelease);
#else
                flag[c].store(e, kRelease);
#endif
            };
            for (int si = cta_seg[c]; si < cta_seg[c + 1]; ++si) {
                const int32_t* r = &seg[(size_t)si * 6];
                const int u = r[1], t0 = r[2], t1 = r[3], is_host = r[4], is_fin = r[5];
                nap(rng);       // the segment's first step
                raise();
                Rec acc = partial(P, u, t0, t1);
                if (!is_host) {
                    part[c] = acc;
                    nap(rng);
                    pending = true;
                    continue;
                }
                bool gave_up = false;
                if (!is_fin) {
                    const auto t_end =
                        std::chrono::steady_clock::now() + std::chrono::milliseconds(wait_ms);
                    for (int p = c + 1; p <= last[u] && !gave_up; ++p) {
#ifdef EMU_UNEPOCHED
                        while (flag[p].load(kAcquire) == 0) {
                            if (err.load() != 0 || std::chrono::steady_clock::now() > t_end) {
#else
                        while (flag[p].load(kAcquire) != e) {
                            if (aborted.load() == e || std::chrono::steady_clock::now() > t_end) {
                                aborted.store(e);
#endif
                                err.fetch_or(1u);
                                gave_up = true;
                                break;
                            }
                            std::this_thread::yield();
                        }
                    }
                    if (!gave_up)
                        for (int p = c + 1; p <= last[u]; ++p) merge(acc, part[p]);
#ifdef EMU_UNEPOCHED
                    for (int p = c + 1; p <= last[u]; ++p) flag[p].store(0, std::memory_order_relaxed);
#endif
                }
                if (!gave_up) finish(P, u, acc, out, mo, lo);
            }
            raise();
            if (exited.fetch_add(1, std::memory_order_relaxed) == (uint32_t)G - 1) {
                exited.store(0, std::memory_order_relaxed);
                epoch.store(e, std::memory_order_relaxed);
            }
        };
        std::vector<std::thread> th;
        for (int c = 0; c < G; ++c) th.emplace_back(cta, c);
        for (auto& t : th) t.join();
    }
    if (exited.load() != 0 || epoch.load() != (uint32_t)launches) return 5;
    return err.load() != 0 ? 4 : 0;
}

int run_pull(const Problem& P, int threads, int C, unsigned seed, double* out, double* mo,
             double* lo) {
    constexpr int kFanIn = 16;
    const int BH = P.B * P.H;
    std::vector<int32_t> S(BH + 1);
    int64_t acc_t = 0;
    for (int u = 0; u < BH; ++u) {
        S[u] = (int32_t)acc_t;
        acc_t += (P.ctx[u / P.H] + P.L - 1) / P.L;
    }
    S[BH] = (int32_t)acc_t;
    const int I = (int)acc_t;
    const int nchunks = (I + C - 1) / C;
    std::vector<Rec> l0(2 * (size_t)nchunks), l1(2 * (size_t)nchunks);
    std::vector<std::atomic<uint32_t>> gcount(2 * (size_t)nchunks), arrive(BH);
    for (auto& x : gcount) x.store(0);
    for (auto& x : arrive) x.store(0);
    std::atomic<int> next{0};
    auto slot = [&](int ch, int Su) { return ch * 2 + (std::max(Su, ch * C) == ch * C ? 0 : 1); };
    auto fold = [&](const std::vector<Rec>& recs, int ch0, int cnt, int step, int Su) {
        Rec r;
        r.o.assign(P.d, 0.0);
        for (int i = 0; i < cnt; ++i) merge(r, recs[slot(ch0 + i * step, Su)]);
        return r;
    };
    auto worker = [&](int w) {
        std::mt19937 rng(seed * 104729u + w);
        for (;;) {
            const int k = next.fetch_add(1);
            if (k >= nchunks) return;
            const int c0 = k * C, c1 = std::min(c0 + C, I);
            int u = 0;
            while (S[u + 1] <= c0) ++u;
            for (int it = c0; it < c1; ++u) {
                const int Su = S[u], Se = S[u + 1], t1 = std::min(Se, c1);
                nap(rng);
                Rec r = partial(P, u, it - Su, t1 - Su);
                const int side = it == c0 ? 0 : 1;
                it = t1;
                const int kf = Su / C, kl = (Se - 1) / C;
                if (kf != kl) {
                    const int g0 = kf + (k - kf) / kFanIn * kFanIn;
                    const int g1 = std::min(g0 + kFanIn - 1, kl);
                    const int ngroups = (kl - kf) / kFanIn + 1;
                    const int gs = slot(g0, Su);
                    if (g1 > g0) {
                        l0[(size_t)k * 2 + side] = r;
                        nap(rng);
                        if (gcount[gs].fetch_add(1, kAcqRel) != (uint32_t)(g1 - g0))
                            continue;
                        r = fold(l0, g0, g1 - g0 + 1, 1, Su);
                        gcount[gs].store(0, std::memory_order_relaxed);
                    }
                    if (ngroups > 1) {
                        l1[gs] = r;
                        nap(rng);
                        if (arrive[u].fetch_add(1, kAcqRel) != (uint32_t)(ngroups - 1))
                            continue;
                        r = fold(l1, kf, ngroups, kFanIn, Su);
                        arrive[u].store(0, std::memory_order_relaxed);
                    }
                }
                finish(P, u, r, out, mo, lo);
            }
        }
    };
    std::vector<std::thread> th;
    for (int w = 0; w < threads; ++w) th.emplace_back(worker, w);
    for (auto& t : th) t.join();
    for (auto& x : gcount)
        if (x.load() != 0) return 5;
    for (auto& x : arrive)
        if (x.load() != 0) return 5;
    return 0;
}

template <typename T>
bool rd(FILE* f, T* p, size_t n) { return fread(p, sizeof(T), n, f) == n; }

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 2;
    }
    FILE* f = fopen(argv[1], "rb");
    if (!f) return 2;
    int32_t h[11];
    Problem P;
    if (!rd(f, h, 11)) return 2;
    const int mode = h[0];
    P.B = h[1];
    P.H = h[2];
    P.d = h[3];
    P.L = h[4];
    const int G = h[5], C = h[6], drop = h[7], wait_ms = h[8];
    const unsigned seed = (unsigned)h[9];
    const int launches = h[10] > 0 ? h[10] : 1;
    P.ctx.resize(P.B);
    if (!rd(f, P.ctx.data(), P.B)) return 2;
    int64_t N = 0;
    P.row0.resize((size_t)P.B * P.H);
    for (int b = 0; b < P.B; ++b) {
        for (int hh = 0; hh < P.H; ++hh) P.row0[(size_t)b * P.H + hh] = (int64_t)P.H * N + (int64_t)hh * P.ctx[b];
        N += P.ctx[b];
    }
    P.q.resize((size_t)P.B * P.H * P.d);
    P.k.resize((size_t)P.H * N * P.d);
    P.v.resize(P.k.size());
    if (!rd(f, &P.scale, 1) || !rd(f, P.q.data(), P.q.size()) || !rd(f, P.k.data(), P.k.size()) ||
        !rd(f, P.v.data(), P.v.size()))
        return 2;
    fclose(f);
    const size_t BH = (size_t)P.B * P.H;
    std::vector<double> out(BH * P.d, NAN), mo(BH, NAN), lo(BH, NAN);
    const int st = mode == 0 ? run_lean(P, G, drop, wait_ms, launches, seed, out.data(), mo.data(), lo.data())
                             : run_pull(P, G, C, seed, out.data(), mo.data(), lo.data());
    FILE* g = fopen(argv[2], "wb");
    if (!g) return 2;
    const int32_t s32 = st;
    fwrite(&s32, 4, 1, g);
    fwrite(out.data(), 8, out.size(), g);
    fwrite(mo.data(), 8, mo.size(), g);
    fwrite(lo.data(), 8, lo.size(), g);
    fclose(g);
    return 0;
}
