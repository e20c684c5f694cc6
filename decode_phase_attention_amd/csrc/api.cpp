// C-ABI entry points of libla_decode (declared in include/la_decode.h).
//
// Per call: validate, build the tables the kind needs (the stream-K schedule,
// the chunk tables of the pull kinds, or only the per-request lengths and
// offsets), copy them through a pinned staging slot to the workspace's device
// buffer on the caller's stream -- unless the buffer already holds the same
// bytes -- and launch. Workspaces are per (device, stream) so that concurrent
// streams never share partials, flags or counters.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "la_decode.h"
#include "budget.h"
#include "kernels.h"
#include "sched.h"
#include "noalloc.h"
#include "select.h"

namespace {

thread_local char g_msg[512] = "";

la_status fail(la_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return st;
}

#define HIP_TRY(expr)                                                                     \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess)                                                             \
            return fail(LA_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
    } while (0)

constexpr int kRing = 4;                    // pinned staging slots per workspace
constexpr uint32_t kDefaultWaitUs = 2000000;  // bound on one device-side wait: 2 s

struct Staging {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
};

struct Workspace {
    int device = 0;
    hipStream_t stream = nullptr;
    float* part = nullptr;          // lean partial records
    size_t part_cap = 0;            // bytes
    uint32_t* flags = nullptr;      // one per lean workgroup (epochs; zero-filled when allocated)
    size_t flags_cap = 0;
    uint32_t* ctl = nullptr;        // lean control block: error word, epoch, exit count, abort
    float* split_part = nullptr;    // fixed-split partial records
    size_t split_cap = 0;
    float* pull_part = nullptr;     // dynamic-pull partial records, two per chunk
    size_t pull_part_cap = 0;
    uint32_t* arrive = nullptr;     // dynamic pull: pieces arrived per head, zero between launches
    size_t arrive_cap = 0;
    uint32_t* pull_ctr = nullptr;   // dynamic pull: next chunk, workgroups done; zero between launches
    size_t pull_ctr_cap = 0;
    uint32_t* gcount = nullptr;     // dynamic pull: pieces arrived per group, zero between launches
    size_t gcount_cap = 0;
    void* tables = nullptr;         // device copy of the schedule tables
    size_t tables_cap = 0;
    std::vector<char> last_tables;  // host copy of what `tables` holds (valid while non-empty)
    Staging ring[kRing];
    int next = 0;
    bool capturing = false;         // the current call is being captured: nothing may be allocated
    bool captured = false;          // a graph may hold the buffers: growing keeps the old ones
    std::vector<void*> retired;     // buffers replaced after a capture, freed at shutdown
    int last_lean_grid = 0;         // the last lean launch on the stream (for the budget)
    int last_lean_cap = 1;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace*> g_ws;

// Completion events for the lean launch budget (budget.h), from a per-device
// pool of timing-free events. An error of the runtime counts as done, so that
// no wait can block on an event that will never complete.
struct HipEventOps {
    using event = hipEvent_t;
    std::vector<hipEvent_t>* pool;
    hipEvent_t record(void* stream) {
        hipEvent_t e = nullptr;
        if (!pool->empty()) {
            e = pool->back();
            pool->pop_back();
        } else if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            return nullptr;
        }
        if (hipEventRecord(e, (hipStream_t)stream) != hipSuccess) {
            pool->push_back(e);
            return nullptr;
        }
        return e;
    }
    bool done(hipEvent_t e) { return e == nullptr || hipEventQuery(e) != hipErrorNotReady; }
    void wait(hipEvent_t e) {
        if (e != nullptr) (void)hipEventSynchronize(e);
    }
    void release(hipEvent_t e) {
        if (e != nullptr) pool->push_back(e);
    }
};

// Per device: how many streams have a workspace, and -- once there are two
// or more -- the budget that keeps their unfinished lean launches within the
// co-resident capacity. With one stream every lean launch is ordered after the
// previous one and nothing is tracked.
struct DeviceState {
    int streams = 0;
    std::vector<hipEvent_t> pool;
    la::LaunchBudget<HipEventOps>* budget = nullptr;
};
std::map<int, DeviceState> g_dev;
struct Capacity {
    int coresident;   // occupancy per CU x CUs: the largest grid a launch may use
    int preferred;    // default grid: kWgPerCu workgroups on every CU
    int cus;          // compute units of the device
    int per_cu;       // workgroups of the kernel one CU holds at once
};
std::map<std::pair<int, const void*>, Capacity> g_capacity;

// One lean workgroup per CU by default. Each workgroup already keeps
// 2*kRows 16-byte loads per lane in flight; more workgroups per CU add
// concurrent sequential streams without adding bandwidth (measured on MI355X:
// 1 per CU streams fastest on the long-context and ragged workloads).
constexpr int kWgPerCu = 1;
constexpr int kMaxQTokens = 64;
constexpr int kMaxPullGrid = 65536;
constexpr int kMinChunkTiles = 32;   // 2 MiB of K and V at either head dim
uint32_t g_wait_us = kDefaultWaitUs;

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// LeanTiles of a context of n tokens (n >= 1, any L >= 1 without overflow).
int tiles_of(int32_t n, int L) { return (int)(((int64_t)n + L - 1) / L); }

// Grows a device buffer. The old one may still be read by work queued on the
// stream, so the stream is drained before it is freed.
la_status grow(Workspace& w, void** p, size_t* cap, size_t need_bytes, bool zero) {
    if (need_bytes <= *cap) return LA_OK;
    if (w.capturing)
        return fail(LA_EUNSUPPORTED, "the stream's workspace must grow, which a captured call "
                                     "cannot do: make a call of this size (grid, head dim) on the "
                                     "stream before capturing");
    if (*p != nullptr) {
        if (w.captured) {
            w.retired.push_back(*p);   // a captured graph's replays may still use it
        } else {
            HIP_TRY(hipStreamSynchronize(w.stream));
            HIP_TRY(hipFree(*p));
        }
        *p = nullptr;
        *cap = 0;
    }
    size_t bytes = need_bytes + need_bytes / 2;
    if (hipMalloc(p, bytes) != hipSuccess) {
        *p = nullptr;
        return fail(LA_ENOMEM, "hipMalloc of %zu bytes failed", bytes);
    }
    if (zero) HIP_TRY(hipMemsetAsync(*p, 0, bytes, w.stream));
    *cap = bytes;
    return LA_OK;
}

la_status get_workspace(hipStream_t stream, Workspace** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    auto key = std::make_pair(dev, stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        *out = it->second;
        return LA_OK;
    }
    Workspace* w = new Workspace();
    w->device = dev;
    w->stream = stream;
    size_t cap = 0;
    la_status st = grow(*w, (void**)&w->ctl, &cap, sizeof(uint32_t) * la::kCtlWords, true);
    if (st != LA_OK) {
        delete w;
        return st;
    }
    for (auto& s : w->ring) {
        if (hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) {
            s.ev = nullptr;
            for (auto& r : w->ring)
                if (r.ev != nullptr) (void)hipEventDestroy(r.ev);
            (void)hipStreamSynchronize(stream);   // the control block's clear may be queued
            (void)hipFree(w->ctl);
            delete w;
            return fail(LA_EHIP, "hipEventCreate failed");
        }
    }
    g_ws[key] = w;
    DeviceState& ds = g_dev[dev];
    if (++ds.streams == 2) {
        // from now on lean launches are tracked; the other stream's last lean
        // launch may still run, so it is counted from here on
        ds.budget = new la::LaunchBudget<HipEventOps>(HipEventOps{&ds.pool});
        for (auto& kv : g_ws)
            if (kv.first.first == dev && kv.second != w && kv.second->last_lean_grid > 0)
                ds.budget->record(kv.second->stream, kv.second->last_lean_grid,
                                  kv.second->last_lean_cap);
    }
    *out = w;
    return LA_OK;
}

la_status capacity(int dtype, int d, bool grouped, Capacity* out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    // the smallest occupancy of the three instantiations (schedule from the
    // tables, the kernel arguments or device lengths): the same grid limits
    const void* fn[3];
    for (int src = 0; src < 3; ++src)
        fn[src] = grouped ? la::lean_gqa_kernel_ptr(dtype, d, src) : la::lean_kernel_ptr(dtype, d, src);
    auto key = std::make_pair(dev, fn[0]);
    auto it = g_capacity.find(key);
    if (it != g_capacity.end()) {
        *out = it->second;
        return LA_OK;
    }
    int per_cu = 1 << 30, cus = 0;
    for (int src = 0; src < 3; ++src) {
        int p = 0;
        HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&p, fn[src], la::kThreads, 0));
        per_cu = p < per_cu ? p : per_cu;
    }
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    if (per_cu < 1 || cus < 1) return fail(LA_EHIP, "lean kernel does not fit on this device");
    Capacity c;
    c.coresident = per_cu * cus;
    c.preferred = (per_cu < kWgPerCu ? per_cu : kWgPerCu) * cus;
    c.cus = cus;
    c.per_cu = per_cu;
    g_capacity[key] = c;
    *out = c;
    return LA_OK;
}

// The CUs a stream's kernels may run on: all of the device's, unless the
// stream was created with a CU mask (hipExtStreamCreateWithCUMask), whose set
// bits are counted. Asked on every call (a host-side lookup, well under a
// microsecond), so a stream handle reused for a stream with another mask is
// never answered from a stale copy.
int stream_cus(hipStream_t stream, int cus) {
    constexpr int kMaxWords = 64;
    uint32_t mask[kMaxWords];
    const int words = (cus + 31) / 32;
    if (words > kMaxWords) return cus;
    if (hipExtStreamGetCUMask(stream, (uint32_t)words, mask) != hipSuccess) {
        (void)hipGetLastError();   // leave no error for the caller's next check
        return cus;
    }
    int n = 0;
    for (int i = 0; i < words; ++i) n += __builtin_popcount(mask[i]);
    return n >= 1 && n < cus ? n : cus;
}

// A lean kernel's limits on the CUs of one stream. Its hosts wait for their
// peers, so every workgroup of a launch must be resident at once on the CUs
// the stream may use: on a CU-masked stream that is per_cu times the masked
// CUs, not the device's capacity. The default grid there is one workgroup per
// CU of the stream, except for single heads on under 70% of the CUs, which
// keep the device's default (capped at what the stream's CUs hold): one
// single-head workgroup per CU reads at most ~34.6 GB/s with K in 16-row
// blocks, while two on a CU switch to whole rows and reach ~48 GB/s, so with
// n CUs one per CU takes bytes / (n * 34.6 GB/s) and the device grid about
// bytes / (128 * 48 GB/s) on a 256-CU device: equal near n = 178 (measured on
// 512k: 1254 against 1557 us at 224 CUs, 1597 against 1526 at 160). Grouped
// heads were fastest on one per CU of the stream at every count measured.
struct StreamCap {
    int cus, coresident, preferred;
};
StreamCap on_stream(const Capacity& cap, hipStream_t stream, bool grouped) {
    const int n = stream_cus(stream, cap.cus);
    int preferred = (cap.per_cu < kWgPerCu ? cap.per_cu : kWgPerCu) * n;
    if (!grouped && n < cap.cus && 10 * n < 7 * cap.cus)
        preferred = std::min(cap.preferred, cap.per_cu * n);
    return {n, cap.per_cu * n, preferred};
}

// Pinned staging slot with room for `bytes`; waits until its previous copy is done.
la_status staging(Workspace& w, size_t bytes, Staging** out) {
    Staging& s = w.ring[w.next];
    w.next = (w.next + 1) % kRing;
    HIP_TRY(hipEventSynchronize(s.ev));
    if (s.cap < bytes) {
        if (s.host != nullptr) HIP_TRY(hipHostFree(s.host));
        s.host = nullptr;
        s.cap = 0;
        size_t b = bytes + bytes / 2;
        if (hipHostMalloc(&s.host, b, hipHostMallocDefault) != hipSuccess) {
            s.host = nullptr;
            return fail(LA_ENOMEM, "hipHostMalloc of %zu bytes failed", b);
        }
        s.cap = b;
    }
    *out = &s;
    return LA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ctx_lens may be null when the lengths are read on the device.
la_status validate(const void* q, const void* k, const void* v, const int32_t* ctx_lens,
                   bool host_lens, int B, int H, int d, float scale, const float* out, int dtype) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr ||
        (host_lens && ctx_lens == nullptr))
        return fail(LA_EINVAL, "null pointer argument");
    if (B < 1 || H < 1) return fail(LA_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
    if (d != 64 && d != 128) return fail(LA_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (dtype != LA_F16 && dtype != LA_BF16) return fail(LA_EINVAL, "unknown dtype %d", dtype);
    if (!isfinite(scale)) return fail(LA_EINVAL, "scale must be finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(LA_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned");
    for (int b = 0; b < B && host_lens; ++b) {
        if (ctx_lens[b] < 1) return fail(LA_EINVAL, "ctx_lens[%d] = %d; must be >= 1", b, ctx_lens[b]);
        // kernels address one head's rows with 32-bit byte offsets
        if ((int64_t)ctx_lens[b] * d * 2 > (int64_t)UINT32_MAX)
            return fail(LA_EUNSUPPORTED, "ctx_lens[%d] = %d: one head's cache exceeds 4 GiB", b,
                        ctx_lens[b]);
    }
    if ((int64_t)B * H > INT32_MAX / 2) return fail(LA_EUNSUPPORTED, "too many heads");
    return LA_OK;
}

// Request tables every kernel kind needs: n_b and the token prefix sums.
struct ReqLayout {
    size_t off_tok, off_ctx, bytes;
};

ReqLayout req_layout(size_t start, int B) {
    ReqLayout r;
    r.off_tok = align16(start);
    r.off_ctx = align16(r.off_tok + sizeof(int64_t) * B);
    r.bytes = align16(r.off_ctx + sizeof(int32_t) * B);
    return r;
}

void fill_req(char* base, const ReqLayout& r, const int32_t* ctx_lens, int B) {
    int64_t* tok = (int64_t*)(base + r.off_tok);
    int32_t* ctx = (int32_t*)(base + r.off_ctx);
    int64_t acc = 0;
    for (int b = 0; b < B; ++b) {
        tok[b] = acc;
        ctx[b] = ctx_lens[b];
        acc += ctx_lens[b];
    }
}

// Copies the tables built in `host` (bytes long) to the workspace's device
// buffer on its stream -- unless the buffer already holds exactly these bytes
// (repeated calls with the same lengths, heads, tile and grid), in which case
// nothing is enqueued. The copy goes through a pinned staging slot.
la_status upload(Workspace& w, const char* host, size_t bytes) {
    if (w.last_tables.size() == bytes && memcmp(w.last_tables.data(), host, bytes) == 0)
        return LA_OK;
    const void* old = w.tables;
    la_status st = grow(w, &w.tables, &w.tables_cap, bytes, false);
    if (st != LA_OK) return st;
    if (w.tables != old) w.last_tables.clear();
    Staging* s = nullptr;
    if ((st = staging(w, bytes, &s)) != LA_OK) return st;
    memcpy(s->host, host, bytes);
    HIP_TRY(hipMemcpyAsync(w.tables, s->host, bytes, hipMemcpyHostToDevice, w.stream));
    HIP_TRY(hipEventRecord(s->ev, w.stream));
    w.last_tables.assign(host, host + bytes);
    return LA_OK;
}

// Host scratch for building tables before they are compared and uploaded.
thread_local std::vector<char> g_build;

// Query columns of a call: H query heads over Hk K/V heads, times Nq new
// tokens per request. With more than one column per K/V head (g * Nq > 1) the
// grouped kernels run and the schedule unit is (request, K/V head, block of
// up to 16 columns); otherwise the unit is (request, head).
struct Heads {
    int H, Hk, g, Nq, cols, QB;
    bool grouped;
    int units_per_req() const { return grouped ? Hk * QB : H; }
};

Heads heads_of(int H, int kv_heads, int q_tokens) {
    Heads h;
    h.H = H;
    h.Hk = kv_heads > 0 ? kv_heads : H;
    h.g = H / h.Hk;
    h.Nq = q_tokens > 0 ? q_tokens : 1;
    h.cols = h.g * h.Nq;
    h.QB = (h.cols + 15) / 16;
    h.grouped = h.cols > 1;
    return h;
}

void fill_gqa(la::GqaArgs& a, const void* q, const void* k, const void* v, float* out,
              const la_opts& o, const Heads& hd, int L, float scale) {
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.out = out;
    a.m_out = o.m_out;
    a.l_out = o.l_out;
    a.tile_owner = o.tile_owner;
    a.ts = o.cta_timestamps;
    a.H = hd.H;
    a.Hk = hd.Hk;
    a.g = hd.g;
    a.Nq = hd.Nq;
    a.cols = hd.cols;
    a.QB = hd.QB;
    a.L = L;
    a.kv_stride = o.kv_stride;
    a.splits = 1;
    a.sl2e = scale * 1.4426950408889634f;
    a.wait_ticks = (uint64_t)g_wait_us * 100u;   // realtime clock runs at 100 MHz
}

// Whether a single-head launch whose workgroups take at most ceil(I / G)
// tiles of L tokens each (at d) can stream a range long enough for the
// 16-row K blocks, and so for the per-CU crowding watch: shorter ranges read
// by whole rows anyway, and the watch's two counter atomics per workgroup
// would be its only effect (tiny: 0.4 us of 9 us).
bool watch_cus(int64_t I, int64_t G, int L, int d) {
    const int64_t tiles = (I + G - 1) / G;
    return tiles * (int64_t)L >= (int64_t)la::kBlockMinSteps * la::chunk_rows(d);
}

// Whether a lean call with host lengths derives its segments in the launch
// (prefix sums in the kernel arguments) rather than from uploaded tables.
bool in_launch_schedule(const int32_t* ctx_lens, int B, const la_opts& o) {
    if (B > la::kInlineB || o.host_tables != 0) return false;
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += ctx_lens[b];
    return total <= (int64_t)UINT32_MAX;
}

// The buffers of a lean exchange: a stream's workspace, or a device's fixed
// scratch array (allocation-free entry point).
struct Exchange {
    float* part;
    size_t part_bytes;
    uint32_t* flags;
    uint32_t* ctl;
    int max_grid;     // workgroups the flags hold
};

// After a lean launch through a workspace: remember it on the stream, and
// count it in the device's budget when one is kept.
void lean_launched(Workspace* w, la::LaunchBudget<HipEventOps>* budget, int G, int cap) {
    if (w == nullptr || w->capturing) return;
    w->last_lean_grid = G;
    w->last_lean_cap = cap;
    if (budget != nullptr) budget->record(w->stream, G, cap);
}

// A lean call. With `fixed` the exchange is that fixed scratch and nothing is
// allocated or copied: the schedule must be derived in the launch, and the
// grid and records must fit the scratch. Otherwise `w` is the stream's
// workspace, grown as needed.
la_status run_lean(Workspace* w, const Exchange* fixed, hipStream_t stream, const void* q,
                   const void* k, const void* v, const int32_t* ctx_lens, int B, const Heads& hd,
                   int d, float scale, float* out, const la_opts& o) {
    Capacity cap;
    la_status st = capacity(o.dtype, d, hd.grouped, &cap);
    if (st != LA_OK) return st;
    const StreamCap sc = on_stream(cap, stream, hd.grouped);
    if (o.grid < 0 || o.grid > sc.coresident)
        return fail(LA_EINVAL, "grid %d outside [1, %d] (co-resident capacity on the %d CUs "
                    "the stream may use)", o.grid, sc.coresident, sc.cus);
    const int L = o.tile_tokens > 0 ? o.tile_tokens : la::chunk_rows(d);
    const int U = hd.units_per_req();
    int64_t I = 0;
    int G = 0, max_rows = 0;
    const bool dev_lens = o.ctx_lens_device != nullptr;
    if (dev_lens) {
        // The lengths are known only in the launch: the grid is the requested
        // (or default) one, and workgroups beyond the iterations stay empty.
        G = o.grid > 0 ? o.grid : sc.preferred;
    } else {
        const char* why = "";
        const int rc = la::schedule_dims(ctx_lens, B, U, L, o.grid > 0 ? o.grid : sc.preferred,
                                         &I, &G, &max_rows, &why);
        if (rc != 0) return fail(rc == 1 ? LA_EINVAL : LA_EUNSUPPORTED, "%s", why);
    }

    // With lean launches on several streams of the device, their unfinished
    // grids together stay within the co-resident capacity (budget.h): this
    // launch may get a smaller grid, or wait for another stream's launch.
    la::LaunchBudget<HipEventOps>* budget = nullptr;
    if (fixed == nullptr && !w->capturing) {
        auto it = g_dev.find(w->device);
        if (it != g_dev.end()) budget = it->second.budget;
    }
    if (budget != nullptr) {
        const int g = budget->admit(w->stream, G, sc.coresident);
        if (g < G) {
            if (dev_lens) {
                G = g;
            } else {
                const char* why = "";
                const int rc = la::schedule_dims(ctx_lens, B, U, L, g, &I, &G, &max_rows, &why);
                if (rc != 0) return fail(rc == 1 ? LA_EINVAL : LA_EUNSUPPORTED, "%s", why);
            }
        }
    }

    const size_t records = (size_t)G * (hd.grouped ? 16 : 1);
    const size_t rec_bytes = sizeof(float) * records * la::part_stride(d);
    Exchange x;
    if (fixed != nullptr) {
        if (G > fixed->max_grid)
            return fail(LA_EUNSUPPORTED, "grid %d exceeds the %d workgroups of the "
                        "allocation-free scratch", G, fixed->max_grid);
        if (rec_bytes > fixed->part_bytes)
            return fail(LA_EUNSUPPORTED, "%zu bytes of partial records (grid %d) exceed the "
                        "%zu bytes of the allocation-free scratch", rec_bytes, G, fixed->part_bytes);
        x = *fixed;
    } else {
        if ((st = grow(*w, (void**)&w->part, &w->part_cap, rec_bytes, false)) != LA_OK) return st;
        if ((st = grow(*w, (void**)&w->flags, &w->flags_cap, sizeof(uint32_t) * (size_t)G, true)) !=
            LA_OK)
            return st;
        x = {w->part, w->part_cap, w->flags, w->ctl, (int)(w->flags_cap / sizeof(uint32_t))};
    }

    // Where the workgroups find their segments. Up to kInlineB requests: the
    // prefix sums of tiles and tokens travel in the kernel arguments and each
    // workgroup derives its own segments (nothing is copied on the stream,
    // which matters when the lengths change every decode step). Up to
    // kMaxDeviceB: only the lengths are copied and the launch derives the
    // same segments from them. Beyond that, or on request, the host builds
    // the tables and uploads them.
    la::SchedArgs sa{};
    sa.B = B;
    sa.U = U;
    sa.G = G;
    if (dev_lens) {
        sa.src = la::kSrcDevice;
        sa.dlens = o.ctx_lens_device;
        sa.L = L;
        sa.n_min = hd.Nq;
        sa.n_max = o.kv_stride;
    } else if (in_launch_schedule(ctx_lens, B, o)) {
        sa.src = la::kSrcArgs;
        int32_t tp = 0;
        uint32_t tk = 0;
        for (int b = 0; b < B; ++b) {
            sa.tp[b] = tp;
            sa.tok[b] = tk;
            tp += tiles_of(ctx_lens[b], L);
            tk += (uint32_t)ctx_lens[b];
        }
        sa.tp[B] = tp;
        sa.tok[B] = tk;
    } else if (fixed != nullptr) {
        return fail(LA_EUNSUPPORTED, "the allocation-free entry point derives the schedule in "
                    "the launch: up to %d host-side requests and 2^32 - 1 tokens in all, no "
                    "host_tables, or lengths on the device (ctx_lens_device)", la::kInlineB);
    } else if (o.host_tables == 0 && B <= la::kMaxDeviceB) {
        // More requests than the kernel arguments hold: copy the B lengths
        // (4 B each) and let the launch derive the partition from them, as
        // with lengths kept on the device; G is the host's min(grid, I), so
        // the partition is the tables' one.
        if ((st = upload(*w, (const char*)ctx_lens, sizeof(int32_t) * (size_t)B)) != LA_OK) return st;
        sa.src = la::kSrcDevice;
        sa.dlens = (const int32_t*)w->tables;
        sa.L = L;
        sa.n_min = 1;
        sa.n_max = o.kv_stride > 0 ? o.kv_stride : INT32_MAX;
    } else {
        const int BU = B * U;
        const size_t off_seg = 0;
        const size_t off_cta_seg = align16(off_seg + 16 * (size_t)max_rows);
        const size_t off_cta_begin = align16(off_cta_seg + 4 * (size_t)(G + 1));
        const size_t off_last = align16(off_cta_begin + 4 * (size_t)(G + 1));
        const size_t off_host = align16(off_last + 4 * (size_t)BU);
        const ReqLayout rl = req_layout(off_host + 4 * (size_t)BU, B);
        g_build.assign(rl.bytes, 0);
        char* hb = g_build.data();
        la::build_schedule(ctx_lens, B, U, L, G, I, (int32_t*)(hb + off_cta_begin),
                           (int32_t*)(hb + off_cta_seg), nullptr, (int32_t*)(hb + off_seg),
                           (int32_t*)(hb + off_host), (int32_t*)(hb + off_last));
        fill_req(hb, rl, ctx_lens, B);
        if ((st = upload(*w, hb, rl.bytes)) != LA_OK) return st;
        const char* db = (const char*)w->tables;
        sa.src = la::kSrcTables;
        sa.seg = (const int4*)(db + off_seg);
        sa.cta_seg = (const int32_t*)(db + off_cta_seg);
        sa.cta_begin = (const int32_t*)(db + off_cta_begin);
        sa.last_cta = (const int32_t*)(db + off_last);
        sa.ctx = (const int32_t*)(db + rl.off_ctx);
        sa.tok_off = (const int64_t*)(db + rl.off_tok);
    }

    const bool coop = o.cooperative != 0;
    if (hd.grouped) {
        la::GqaArgs a{};
        fill_gqa(a, q, k, v, out, o, hd, L, scale);
        a.sched = sa;
        a.part = x.part;
        a.part_bytes = x.part_bytes > (size_t)INT32_MAX ? (uint32_t)INT32_MAX : (uint32_t)x.part_bytes;
        a.flags = x.flags;
        a.ctl = x.ctl;
        if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, stream));
        HIP_TRY(la::launch_lean_gqa(o.dtype, d, a, G, stream, coop));
        if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, stream));
        lean_launched(w, budget, G, sc.coresident);
        return LA_OK;
    }
    la::LeanArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.out = out;
    a.m_out = o.m_out;
    a.l_out = o.l_out;
    a.sched = sa;
    a.part = x.part;
    a.flags = x.flags;
    a.ctl = x.ctl;
    a.tile_owner = o.tile_owner;
    a.ts = o.cta_timestamps;
    a.H = hd.H;
    a.L = L;
    a.kv_stride = o.kv_stride;
    a.sl2e = scale * 1.4426950408889634f;
    a.wait_ticks = (uint64_t)g_wait_us * 100u;   // realtime clock runs at 100 MHz
    // lengths on the device: the ranges are known only in the launch
    a.cu_fair = dev_lens || watch_cus(I, G, L, d) ? (G + cap.cus - 1) / cap.cus : 0;
    // uniform host lengths: every range starts at the same phase in its head,
    // and the kernel staggers where each workgroup's long ranges begin
    a.rotate = 0;
    if (!dev_lens) {
        bool uniform = true;
        for (int b = 1; b < B && uniform; ++b) uniform = ctx_lens[b] == ctx_lens[0];
        a.rotate = uniform ? 1 : 0;
    }
    if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, stream));
    HIP_TRY(la::launch_lean(o.dtype, d, a, G, stream, coop));
    if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, stream));
    lean_launched(w, budget, G, sc.coresident);
    return LA_OK;
}

la_status run_split_or_head(Workspace& w, const void* q, const void* k, const void* v,
                            const int32_t* ctx_lens, int B, const Heads& hd, int d, float scale,
                            float* out, const la_opts& o) {
    const int BU = B * hd.units_per_req();
    const int L = o.tile_tokens > 0 ? o.tile_tokens : la::chunk_rows(d);
    int splits = 1;
    if (o.kind == LA_KIND_FIXED_SPLIT) {
        if (o.num_splits < 0) return fail(LA_EINVAL, "num_splits must be >= 0");
        splits = o.num_splits;
        if (splits == 0) {
            Capacity cap;
            la_status st = capacity(o.dtype, d, hd.grouped, &cap);
            if (st != LA_OK) return st;
            splits = 1;
            while ((int64_t)BU * splits < cap.coresident && splits < 64) splits *= 2;
        }
        if ((int64_t)BU * splits > INT32_MAX / 32) return fail(LA_EUNSUPPORTED, "too many splits");
    }
    const ReqLayout rl = req_layout(0, B);
    la_status st = LA_OK;
    g_build.assign(rl.bytes, 0);
    fill_req(g_build.data(), rl, ctx_lens, B);
    const size_t records = (size_t)BU * splits * (hd.grouped ? 16 : 1);
    if (o.kind == LA_KIND_FIXED_SPLIT &&
        (st = grow(w, (void**)&w.split_part, &w.split_cap,
                   sizeof(float) * records * la::part_stride(d), false)) != LA_OK)
        return st;
    if ((st = upload(w, g_build.data(), rl.bytes)) != LA_OK) return st;

    char* db = (char*)w.tables;
    if (hd.grouped) {
        la::GqaArgs a{};
        fill_gqa(a, q, k, v, out, o, hd, L, scale);
        a.ctx = (const int32_t*)(db + rl.off_ctx);
        a.tok_off = (const int64_t*)(db + rl.off_tok);
        a.part = w.split_part;
        a.part_bytes = 0;   // the split kernels use plain accesses
        a.splits = splits;
        if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, w.stream));
        if (o.kind == LA_KIND_PER_HEAD) {
            HIP_TRY(la::launch_per_head_gqa(o.dtype, d, a, BU, w.stream));
        } else {
            HIP_TRY(la::launch_split_gqa(o.dtype, d, a, BU * splits, w.stream));
            a.ts = nullptr;
            HIP_TRY(la::launch_combine_gqa(d, a, BU, w.stream));
        }
        if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, w.stream));
        return LA_OK;
    }
    la::SplitArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.out = out;
    a.m_out = o.m_out;
    a.l_out = o.l_out;
    a.ctx = (const int32_t*)(db + rl.off_ctx);
    a.tok_off = (const int64_t*)(db + rl.off_tok);
    a.part = w.split_part;
    a.ts = o.cta_timestamps;
    a.H = hd.H;
    a.L = L;
    a.kv_stride = o.kv_stride;
    a.splits = splits;
    a.sl2e = scale * 1.4426950408889634f;
    if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, w.stream));
    if (o.kind == LA_KIND_PER_HEAD) {
        HIP_TRY(la::launch_per_head(o.dtype, d, a, BU, w.stream));
    } else {
        HIP_TRY(la::launch_split(o.dtype, d, a, BU * splits, w.stream));
        la::CombineArgs c{};
        c.part = w.split_part;
        c.out = out;
        c.m_out = o.m_out;
        c.l_out = o.l_out;
        c.splits = splits;
        HIP_TRY(la::launch_combine(d, c, BU, w.stream));
    }
    if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, w.stream));
    return LA_OK;
}

// Dynamic tile pull (LA_KIND_PULL) and one chunk per workgroup
// (LA_KIND_CHUNKS): the tile sequence of the lean schedule cut into fixed
// chunks; heads spanning chunks are merged by their last piece's workgroup.
la_status run_pull(Workspace& w, const void* q, const void* k, const void* v,
                   const int32_t* ctx_lens, int B, const Heads& hd, int d, float scale,
                   float* out, const la_opts& o) {
    Capacity cap;
    la_status st = capacity(o.dtype, d, hd.grouped, &cap);
    if (st != LA_OK) return st;
    const int L = o.tile_tokens > 0 ? o.tile_tokens : la::chunk_rows(d);
    const int U = hd.units_per_req();
    const int BU = B * U;
    int64_t I = 0;
    for (int b = 0; b < B; ++b) I += (int64_t)U * tiles_of(ctx_lens[b], L);
    if (I > INT32_MAX / 2) return fail(LA_EUNSUPPORTED, "%lld tile iterations do not fit", (long long)I);
    const bool dynamic = o.kind == LA_KIND_PULL;
    // Default chunk: about eight chunks per workgroup of a one-per-CU grid
    // (four for grouped units), and at least kMinChunkTiles tiles (or one
    // chunk per workgroup). Measured on MI355X with part of the CUs taken
    // away (a CU-masked stream): eight to sixteen chunks per workgroup keep a
    // 512k-token decode within 6% of its full-GPU time with 7/8 of the CUs,
    // where a static split of the same grid loses a third, and four lose
    // another 8%; chunks of less than about 2 MiB spend too large a share in
    // the per-chunk fold, publish and merge. The grouped kernels' per-chunk
    // costs are higher (16 records per piece): four chunks per workgroup ran
    // 2.6-3.2% faster than eight on the grouped ragged batches on all of the
    // CUs, on 7/8 and on half of them.
    const int G0 = dynamic && o.grid > 0 ? o.grid : cap.preferred;
    int C = o.chunk_tiles;
    if (C == 0) {
        const int64_t per_wg = (I + G0 - 1) / G0;   // never fewer chunks than workgroups
        const int64_t chunks_per_wg = hd.grouped ? 4 : 8;
        C = (int)std::max<int64_t>(std::min<int64_t>(kMinChunkTiles, per_wg),
                                   (I + chunks_per_wg * G0 - 1) / (chunks_per_wg * G0));
    }
    const int64_t nchunks = (I + C - 1) / C;
    if (nchunks > kMaxPullGrid * 64) return fail(LA_EUNSUPPORTED, "too many chunks (%lld)", (long long)nchunks);
    const int grid = dynamic ? (int)std::min<int64_t>(G0, nchunks) : (int)nchunks;

    const size_t off_start = 0;
    const size_t off_chunk = align16(off_start + 4 * ((size_t)BU + 1));
    const ReqLayout rl = req_layout(off_chunk + 4 * (size_t)nchunks, B);
    g_build.assign(rl.bytes, 0);
    char* hb = g_build.data();
    int32_t* S = (int32_t*)(hb + off_start);
    int32_t* CH = (int32_t*)(hb + off_chunk);
    {
        int64_t acc = 0;
        int u = 0;
        for (int b = 0; b < B; ++b) {
            const int T = tiles_of(ctx_lens[b], L);
            for (int h = 0; h < U; ++h, ++u) {
                S[u] = (int32_t)acc;
                acc += T;
            }
        }
        S[BU] = (int32_t)acc;
        int head = 0;
        for (int64_t c = 0; c < nchunks; ++c) {
            while (S[head + 1] <= c * C) ++head;
            CH[c] = head;
        }
    }
    fill_req(hb, rl, ctx_lens, B);

    // two levels of records (pieces, then groups of pieces), two slots per chunk
    const size_t part_bytes =
        sizeof(float) * 4 * (size_t)nchunks * (hd.grouped ? 16 : 1) * la::part_stride(d);
    if (hd.grouped && part_bytes > (size_t)INT32_MAX)
        return fail(LA_EUNSUPPORTED, "%lld chunks of 16 records exceed the 2 GiB exchange buffer",
                    (long long)nchunks);
    if ((st = grow(w, (void**)&w.pull_part, &w.pull_part_cap, part_bytes, false)) != LA_OK)
        return st;
    if ((st = grow(w, (void**)&w.arrive, &w.arrive_cap, sizeof(uint32_t) * (size_t)BU, true)) != LA_OK)
        return st;
    if ((st = grow(w, (void**)&w.gcount, &w.gcount_cap, sizeof(uint32_t) * 2 * (size_t)nchunks,
                   true)) != LA_OK)
        return st;
    if ((st = grow(w, (void**)&w.pull_ctr, &w.pull_ctr_cap, 2 * sizeof(uint32_t), true)) != LA_OK)
        return st;
    if ((st = upload(w, hb, rl.bytes)) != LA_OK) return st;
    char* db = (char*)w.tables;
    if (hd.grouped) {
        la::GqaArgs a{};
        fill_gqa(a, q, k, v, out, o, hd, L, scale);
        a.ctx = (const int32_t*)(db + rl.off_ctx);
        a.tok_off = (const int64_t*)(db + rl.off_tok);
        a.part = w.pull_part;
        a.part_bytes = (uint32_t)std::min<size_t>(w.pull_part_cap, (size_t)INT32_MAX);
        a.head_start = (const int32_t*)(db + off_start);
        a.chunk_head = (const int32_t*)(db + off_chunk);
        a.arrive = w.arrive;
        a.gcount = w.gcount;
        a.pull = w.pull_ctr;
        a.C = C;
        a.I = (int)I;
        a.nchunks = (int)nchunks;
        a.dynamic = dynamic ? 1 : 0;
        if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, w.stream));
        HIP_TRY(la::launch_pull_gqa(o.dtype, d, a, grid, w.stream));
        if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, w.stream));
        return LA_OK;
    }
    la::PullArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.out = out;
    a.m_out = o.m_out;
    a.l_out = o.l_out;
    a.ctx = (const int32_t*)(db + rl.off_ctx);
    a.tok_off = (const int64_t*)(db + rl.off_tok);
    a.head_start = (const int32_t*)(db + off_start);
    a.chunk_head = (const int32_t*)(db + off_chunk);
    a.part = w.pull_part;
    a.arrive = w.arrive;
    a.gcount = w.gcount;
    a.pull = w.pull_ctr;
    a.tile_owner = o.tile_owner;
    a.ts = o.cta_timestamps;
    a.H = hd.H;
    a.L = L;
    a.kv_stride = o.kv_stride;
    a.C = C;
    a.I = (int)I;
    a.nchunks = (int)nchunks;
    a.dynamic = dynamic ? 1 : 0;
    a.sl2e = scale * 1.4426950408889634f;
    // the stream's lean control block: launches on one stream never overlap,
    // so its per-CU counters are free while a pull launch runs
    a.ctl = w.ctl;
    a.cu_fair = dynamic && watch_cus(C, 1, L, d) ? (grid + cap.cus - 1) / cap.cus : 0;
    if (o.ev_start != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_start, w.stream));
    HIP_TRY(la::launch_pull(o.dtype, d, a, grid, w.stream));
    if (o.ev_stop != nullptr) HIP_TRY(hipEventRecord((hipEvent_t)o.ev_stop, w.stream));
    return LA_OK;
}

// la_select_for with the current device's CU count and lean capacity.
la_status select_on_device(const int32_t* ctx_lens, int B, const Heads& hd, int d,
                           const la_opts& o, hipStream_t stream, int* kind, int* grid) {
    Capacity cap;
    la_status st = capacity(o.dtype, d, hd.grouped, &cap);
    if (st != LA_OK) return st;
    const StreamCap sc = on_stream(cap, stream, hd.grouped);
    const int L = o.tile_tokens > 0 ? o.tile_tokens : la::chunk_rows(d);
    const char* why = "";
    const int rc = la::select_kind(ctx_lens, B, hd.units_per_req(), L, d, hd.grouped, sc.cus,
                                   sc.coresident, kind, grid, &why);
    if (rc != 0) return fail(rc == 1 ? LA_EINVAL : LA_EUNSUPPORTED, "%s", why);
    // Other work on the device (stated by the caller), or single heads on a
    // stream confined to part of the CUs: chunks pulled as CUs free up rather
    // than a static split. Grouped heads on such a stream keep lean on a grid
    // of the stream's CUs, which measured faster than pull there.
    if (*kind == LA_KIND_LEAN && (o.shared_gpu != 0 || (sc.cus < cap.cus && !hd.grouped))) {
        *kind = LA_KIND_PULL;
        *grid = cap.preferred;
    }
    return LA_OK;
}

// Best effort at shutdown: errors are ignored (there is no caller to report
// them to, and freeing continues with the next buffer).
void free_workspace(Workspace* w) {
    (void)hipSetDevice(w->device);
    (void)hipDeviceSynchronize();
    for (void* p : {(void*)w->part, (void*)w->flags, (void*)w->ctl, (void*)w->split_part,
                    (void*)w->pull_part, (void*)w->arrive, (void*)w->pull_ctr, (void*)w->gcount,
                    w->tables})
        if (p != nullptr) (void)hipFree(p);
    for (void* p : w->retired) (void)hipFree(p);
    for (auto& s : w->ring) {
        if (s.host != nullptr) (void)hipHostFree(s.host);
        if (s.ev != nullptr) (void)hipEventDestroy(s.ev);
    }
    delete w;
}

// The exchange of the allocation-free entry point on the current device:
// its fixed scratch array. The first call on a device looks the array up and
// clears its control words (la::scratch_setup), and caches the co-resident
// capacity of both lean kernels at every head dim and dtype, so that later
// calls only read cached values.
la_status noalloc_exchange(hipStream_t stream, Exchange* x) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    void* base = la::scratch_base(dev);
    if (base == nullptr) {
        Capacity c;
        for (int dt = 0; dt < 2; ++dt)
            for (int d : {64, 128})
                for (bool grouped : {false, true}) {
                    la_status st = capacity(dt, d, grouped, &c);
                    if (st != LA_OK) return st;
                }
        HIP_TRY(la::scratch_setup(dev, stream, &base));
    }
    char* p = static_cast<char*>(base);
    x->ctl = reinterpret_cast<uint32_t*>(p);
    x->flags = reinterpret_cast<uint32_t*>(p + la::kScratchFlagsOff);
    x->part = reinterpret_cast<float*>(p + la::kScratchPartOff);
    x->part_bytes = la::kScratchPartBytes;
    x->max_grid = la::kScratchMaxGrid;
    return LA_OK;
}

// Argument checks shared by la_decode_ex and la_decode_noalloc. `o` holds
// the caller's options (kind auto already mapped to lean with device
// lengths); `hd` receives the query columns of the call.
la_status prepare(const void* q, const void* k, const void* v, const int32_t* ctx_lens, int B,
                  int H, int d, float scale, const float* out, la_opts& o, Heads& hd) {
    const bool dev_lens = o.ctx_lens_device != nullptr;
    // lengths on the device are known only in the launch: auto means lean,
    // the one kind that reads them there
    if (dev_lens && o.kind == LA_KIND_AUTO) o.kind = LA_KIND_LEAN;
    la_status st = validate(q, k, v, ctx_lens, !dev_lens, B, H, d, scale, out, o.dtype);
    if (st != LA_OK) return st;
    if (o.kind != LA_KIND_LEAN && o.kind != LA_KIND_FIXED_SPLIT && o.kind != LA_KIND_PER_HEAD &&
        o.kind != LA_KIND_AUTO && o.kind != LA_KIND_PULL && o.kind != LA_KIND_CHUNKS)
        return fail(LA_EINVAL, "unknown kind %d", o.kind);
    if (o.kind == LA_KIND_AUTO && (o.tile_owner != nullptr || o.cta_timestamps != nullptr))
        return fail(LA_EINVAL, "tile_owner and cta_timestamps need an explicit kind");
    if (o.tile_tokens < 0) return fail(LA_EINVAL, "tile_tokens must be >= 0");
    if (o.kind != LA_KIND_LEAN && o.kind != LA_KIND_PULL && o.kind != LA_KIND_CHUNKS &&
        o.tile_owner != nullptr)
        return fail(LA_EINVAL, "tile_owner applies to the lean and pull kinds only");
    if (o.kind == LA_KIND_FIXED_SPLIT && o.cta_timestamps != nullptr && o.num_splits < 1)
        return fail(LA_EINVAL, "cta_timestamps with fixed_split needs an explicit num_splits");
    if (o.chunk_tiles < 0) return fail(LA_EINVAL, "chunk_tiles must be >= 0");
    if ((o.kind == LA_KIND_PULL || o.kind == LA_KIND_CHUNKS) && (o.grid < 0 || o.grid > kMaxPullGrid))
        return fail(LA_EINVAL, "grid %d outside [0, %d]", o.grid, kMaxPullGrid);
    if (o.kind == LA_KIND_PULL && o.cta_timestamps != nullptr && o.grid < 1)
        return fail(LA_EINVAL, "cta_timestamps with pull needs an explicit grid");
    if (o.kind == LA_KIND_CHUNKS && o.cta_timestamps != nullptr && o.chunk_tiles < 1)
        return fail(LA_EINVAL, "cta_timestamps with chunks needs an explicit chunk_tiles");
    if (o.kv_heads < 0 || (o.kv_heads > 0 && H % o.kv_heads != 0))
        return fail(LA_EINVAL, "kv_heads %d must divide H = %d", o.kv_heads, H);
    if (o.kv_stride < 0) return fail(LA_EINVAL, "kv_stride must be >= 0");
    if (o.q_tokens < 0 || o.q_tokens > kMaxQTokens)
        return fail(LA_EINVAL, "q_tokens %d outside [0, %d]", o.q_tokens, kMaxQTokens);
    if (dev_lens) {
        // lengths read in the launch: the lean kind on a [B, Hk, kv_stride, d]
        // cache, whose size bounds every read; lengths outside
        // [max(1, q_tokens), kv_stride] are reported by la_sync_check
        if (o.kind != LA_KIND_LEAN)
            return fail(LA_EINVAL, "ctx_lens_device needs kind lean");
        if (o.kv_stride < 1)
            return fail(LA_EINVAL, "ctx_lens_device needs a cache with kv_stride rows per head");
        if ((int64_t)o.kv_stride * d * 2 > (int64_t)UINT32_MAX)
            return fail(LA_EUNSUPPORTED, "kv_stride %d: one head's cache exceeds 4 GiB", o.kv_stride);
        if (o.q_tokens > o.kv_stride)
            return fail(LA_EINVAL, "q_tokens %d exceeds kv_stride %d", o.q_tokens, o.kv_stride);
        if (B > la::kMaxDeviceB)
            return fail(LA_EUNSUPPORTED, "ctx_lens_device takes up to %d requests", la::kMaxDeviceB);
        if (o.host_tables != 0) return fail(LA_EINVAL, "host_tables needs host lengths");
        if (o.tile_owner != nullptr)
            return fail(LA_EINVAL, "tile_owner needs host lengths (its size is the tile count)");
        if (((uintptr_t)o.ctx_lens_device & 3u) != 0)
            return fail(LA_EINVAL, "ctx_lens_device must be 4-byte aligned");
    }
    for (int b = 0; b < B && o.kv_stride > 0 && !dev_lens; ++b)
        if (ctx_lens[b] > o.kv_stride)
            return fail(LA_EINVAL, "ctx_lens[%d] = %d exceeds kv_stride = %d", b, ctx_lens[b],
                        o.kv_stride);
    for (int b = 0; b < B && o.q_tokens > 1 && !dev_lens; ++b)
        if (ctx_lens[b] < o.q_tokens)
            return fail(LA_EINVAL, "ctx_lens[%d] = %d is shorter than the %d new tokens it must hold",
                        b, ctx_lens[b], o.q_tokens);
    hd = heads_of(H, o.kv_heads, o.q_tokens);
    if ((int64_t)B * hd.units_per_req() > INT32_MAX / 32) return fail(LA_EUNSUPPORTED, "too many heads");
    return LA_OK;
}

}  // namespace

extern "C" {

void la_opts_init(la_opts* o) {
    if (o != nullptr) memset(o, 0, sizeof(*o));
}

la_status la_decode_ex(const void* q, const void* k, const void* v, const int32_t* ctx_lens,
                       int B, int H, int d, float scale, float* out, void* stream,
                       const la_opts* opts) {
    g_msg[0] = 0;
    la_opts o;
    la_opts_init(&o);
    if (opts != nullptr) o = *opts;
    Heads hd;
    la_status st = prepare(q, k, v, ctx_lens, B, H, d, scale, out, o, hd);
    if (st != LA_OK) return st;
    const bool dev_lens = o.ctx_lens_device != nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    // Stream capture: only a lean launch whose schedule needs nothing copied
    // (lengths on the device, or prefix sums in the kernel arguments), into a
    // workspace that already exists and need not grow. Table uploads and the
    // other kinds' tables go through staging buffers that later calls reuse,
    // and growing would allocate and clear memory inside the graph.
    hipStreamCaptureStatus cap_status = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing((hipStream_t)stream, &cap_status));
    const bool capturing = cap_status != hipStreamCaptureStatusNone;
    if (capturing) {
        if (o.kind != LA_KIND_LEAN || (!dev_lens && !in_launch_schedule(ctx_lens, B, o)))
            return fail(LA_EUNSUPPORTED, "stream capture takes only the lean kind with the "
                                         "schedule derived in the launch");
        if (o.cooperative != 0)
            return fail(LA_EUNSUPPORTED, "stream capture takes ordinary launches only "
                                         "(cooperative = 0)");
        int dev = 0;
        HIP_TRY(hipGetDevice(&dev));
        if (g_ws.find(std::make_pair(dev, (hipStream_t)stream)) == g_ws.end())
            return fail(LA_EUNSUPPORTED, "stream capture needs the stream's workspace: make a "
                                         "call on the stream before capturing");
    }
    if (o.kind == LA_KIND_AUTO) {
        int kind = 0, grid = 0;
        if ((st = select_on_device(ctx_lens, B, hd, d, o, (hipStream_t)stream, &kind, &grid)) !=
            LA_OK)
            return st;
        o.kind = kind;
        if (o.grid == 0) o.grid = grid;
    }
    Workspace* w = nullptr;
    if ((st = get_workspace((hipStream_t)stream, &w)) != LA_OK) return st;
    if (o.kind == LA_KIND_LEAN) {
        w->capturing = capturing;
        st = run_lean(w, nullptr, w->stream, q, k, v, ctx_lens, B, hd, d, scale, out, o);
        w->capturing = false;
        if (capturing && st == LA_OK) w->captured = true;
        return st;
    }
    if (o.kind == LA_KIND_PULL || o.kind == LA_KIND_CHUNKS)
        return run_pull(*w, q, k, v, ctx_lens, B, hd, d, scale, out, o);
    return run_split_or_head(*w, q, k, v, ctx_lens, B, hd, d, scale, out, o);
}

la_status la_decode_noalloc(const void* q, const void* k, const void* v,
                            const int32_t* ctx_lens, int B, int H, int d, float scale, float* out,
                            void* stream, const la_opts* opts) {
    g_msg[0] = 0;
    la_opts o;
    la_opts_init(&o);
    if (opts != nullptr) o = *opts;
    if (o.kind != LA_KIND_LEAN)
        return fail(LA_EINVAL, "the allocation-free entry point runs the lean kind only (kind %d)",
                    o.kind);
    Heads hd;
    la_status st = prepare(q, k, v, ctx_lens, B, H, d, scale, out, o, hd);
    if (st != LA_OK) return st;
    if (o.ctx_lens_device == nullptr && !in_launch_schedule(ctx_lens, B, o))
        return fail(LA_EUNSUPPORTED, "the allocation-free entry point derives the schedule in "
                    "the launch: up to %d host-side requests and 2^32 - 1 tokens in all, no "
                    "host_tables, or lengths on the device (ctx_lens_device)", la::kInlineB);
    std::lock_guard<std::mutex> lock(g_mu);
    hipStreamCaptureStatus cap_status = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing((hipStream_t)stream, &cap_status));
    if (cap_status != hipStreamCaptureStatusNone) {
        if (o.cooperative != 0)
            return fail(LA_EUNSUPPORTED, "stream capture takes ordinary launches only "
                                         "(cooperative = 0)");
        int dev = 0;
        HIP_TRY(hipGetDevice(&dev));
        if (la::scratch_base(dev) == nullptr)
            return fail(LA_EUNSUPPORTED, "the first allocation-free call on a device sets up its "
                                         "scratch array and must not be captured");
    }
    Exchange x;
    if ((st = noalloc_exchange((hipStream_t)stream, &x)) != LA_OK) return st;
    return run_lean(nullptr, &x, (hipStream_t)stream, q, k, v, ctx_lens, B, hd, d, scale, out, o);
}

la_status la_decode(const void* q, const void* k, const void* v, const int32_t* ctx_lens, int B,
                    int H, int d, float scale, float* out, void* stream, int dtype) {
    la_opts o;
    la_opts_init(&o);
    o.dtype = dtype;
    return la_decode_ex(q, k, v, ctx_lens, B, H, d, scale, out, stream, &o);
}

la_status la_decode_bf16(const void* q, const void* k, const void* v, const int32_t* ctx_lens,
                         int B, int H, int d, float scale, float* out, void* stream) {
    return la_decode(q, k, v, ctx_lens, B, H, d, scale, out, stream, LA_BF16);
}

la_status la_decode_f16(const void* q, const void* k, const void* v, const int32_t* ctx_lens,
                        int B, int H, int d, float scale, float* out, void* stream) {
    return la_decode(q, k, v, ctx_lens, B, H, d, scale, out, stream, LA_F16);
}

la_status la_schedule_dims(const int32_t* ctx_lens, int B, int H, int tile_tokens, int grid,
                           int64_t* iters, int* grid_used, int* max_rows) {
    g_msg[0] = 0;
    if (iters == nullptr || grid_used == nullptr || max_rows == nullptr)
        return fail(LA_EINVAL, "null output pointer");
    const char* why = "";
    const int rc = la::schedule_dims(ctx_lens, B, H, tile_tokens, grid, iters, grid_used, max_rows,
                                     &why);
    if (rc != 0) return fail(rc == 1 ? LA_EINVAL : LA_EUNSUPPORTED, "%s", why);
    return LA_OK;
}

la_status la_schedule(const int32_t* ctx_lens, int B, int H, int tile_tokens, int grid,
                      int32_t* cta_begin, int32_t* cta_seg, int32_t* seg, int max_rows,
                      int* n_seg, int32_t* host_cta, int32_t* last_cta) {
    int64_t I = 0;
    int G = 0, rows = 0;
    la_status st = la_schedule_dims(ctx_lens, B, H, tile_tokens, grid, &I, &G, &rows);
    if (st != LA_OK) return st;
    if (cta_begin == nullptr || cta_seg == nullptr || seg == nullptr || n_seg == nullptr ||
        host_cta == nullptr || last_cta == nullptr)
        return fail(LA_EINVAL, "null output pointer");
    if (max_rows < rows) return fail(LA_EINVAL, "max_rows %d < required %d", max_rows, rows);
    *n_seg = la::build_schedule(ctx_lens, B, H, tile_tokens, G, I, cta_begin, cta_seg, seg,
                                nullptr, host_cta, last_cta);
    return LA_OK;
}

la_status la_select_for(const int32_t* ctx_lens, int B, int H, int d, int kv_heads, int q_tokens,
                        int tile_tokens, int cus, int coresident, int* kind, int* grid) {
    g_msg[0] = 0;
    if (ctx_lens == nullptr || kind == nullptr || grid == nullptr)
        return fail(LA_EINVAL, "null pointer argument");
    if (B < 1 || H < 1) return fail(LA_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
    if (d != 64 && d != 128) return fail(LA_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (kv_heads < 0 || (kv_heads > 0 && H % kv_heads != 0))
        return fail(LA_EINVAL, "kv_heads %d must divide H = %d", kv_heads, H);
    if (q_tokens < 0 || q_tokens > kMaxQTokens)
        return fail(LA_EINVAL, "q_tokens %d outside [0, %d]", q_tokens, kMaxQTokens);
    if (tile_tokens < 0) return fail(LA_EINVAL, "tile_tokens must be >= 0");
    const Heads hd = heads_of(H, kv_heads, q_tokens);
    const int L = tile_tokens > 0 ? tile_tokens : la::chunk_rows(d);
    const char* why = "";
    const int rc = la::select_kind(ctx_lens, B, hd.units_per_req(), L, d, hd.grouped, cus,
                                   coresident, kind, grid, &why);
    if (rc != 0) return fail(rc == 1 ? LA_EINVAL : LA_EUNSUPPORTED, "%s", why);
    return LA_OK;
}

la_status la_select(const int32_t* ctx_lens, int B, int H, int d, const la_opts* opts, int* kind,
                    int* grid) {
    g_msg[0] = 0;
    la_opts o;
    la_opts_init(&o);
    if (opts != nullptr) o = *opts;
    if (ctx_lens == nullptr || kind == nullptr || grid == nullptr)
        return fail(LA_EINVAL, "null pointer argument");
    if (B < 1 || H < 1) return fail(LA_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
    if (d != 64 && d != 128) return fail(LA_EUNSUPPORTED, "head dim %d not supported (64, 128)", d);
    if (o.dtype != LA_F16 && o.dtype != LA_BF16) return fail(LA_EINVAL, "unknown dtype %d", o.dtype);
    if (o.kv_heads < 0 || (o.kv_heads > 0 && H % o.kv_heads != 0))
        return fail(LA_EINVAL, "kv_heads %d must divide H = %d", o.kv_heads, H);
    if (o.kv_stride < 0) return fail(LA_EINVAL, "kv_stride must be >= 0");
    for (int b = 0; b < B && o.kv_stride > 0; ++b)
        if (ctx_lens[b] > o.kv_stride)
            return fail(LA_EINVAL, "ctx_lens[%d] = %d exceeds kv_stride = %d", b, ctx_lens[b],
                        o.kv_stride);
    if (o.q_tokens < 0 || o.q_tokens > kMaxQTokens)
        return fail(LA_EINVAL, "q_tokens %d outside [0, %d]", o.q_tokens, kMaxQTokens);
    if (o.tile_tokens < 0) return fail(LA_EINVAL, "tile_tokens must be >= 0");
    std::lock_guard<std::mutex> lock(g_mu);
    return select_on_device(ctx_lens, B, heads_of(H, o.kv_heads, o.q_tokens), d, o, nullptr, kind,
                            grid);
}

int la_default_tile(int d) { return (d == 64 || d == 128) ? la::chunk_rows(d) : 0; }

int la_max_grid(int d, int dtype) {
    if ((d != 64 && d != 128) || (dtype != LA_F16 && dtype != LA_BF16)) {
        fail(LA_EINVAL, "unsupported d/dtype");
        return -1;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Capacity cap;
    if (capacity(dtype, d, false, &cap) != LA_OK) return -1;
    return cap.coresident;
}

int la_max_grid_grouped(int d, int dtype) {
    if ((d != 64 && d != 128) || (dtype != LA_F16 && dtype != LA_BF16)) {
        fail(LA_EINVAL, "unsupported d/dtype");
        return -1;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Capacity cap;
    if (capacity(dtype, d, true, &cap) != LA_OK) return -1;
    return cap.coresident;
}

int la_default_grid(int d, int dtype) {
    if ((d != 64 && d != 128) || (dtype != LA_F16 && dtype != LA_BF16)) {
        fail(LA_EINVAL, "unsupported d/dtype");
        return -1;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Capacity cap;
    if (capacity(dtype, d, false, &cap) != LA_OK) return -1;
    return cap.preferred;
}

la_status la_sync_check(void* stream) {
    g_msg[0] = 0;
    std::lock_guard<std::mutex> lock(g_mu);
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    // the stream's workspace, and the device's allocation-free scratch
    uint32_t* words[2] = {nullptr, nullptr};
    auto it = g_ws.find(std::make_pair(dev, (hipStream_t)stream));
    if (it != g_ws.end()) words[0] = it->second->ctl + la::kCtlErr;
    if (void* base = la::scratch_base(dev)) words[1] = static_cast<uint32_t*>(base) + la::kCtlErr;
    uint32_t err = 0;
    for (uint32_t* word : words) {
        if (word == nullptr) continue;
        uint32_t e = 0;
        HIP_TRY(hipMemcpy(&e, word, sizeof(e), hipMemcpyDeviceToHost));
        if (e == 0) continue;
        // only the sticky report is cleared: a wait that gave up affected its
        // own launch alone (flags carry epochs), so nothing else needs resetting
        HIP_TRY(hipMemsetAsync(word, 0, sizeof(uint32_t), (hipStream_t)stream));
        err |= e;
    }
    if (err == 0) return LA_OK;
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    if (err & la::kErrLengths)
        return fail(LA_EINVAL, "context lengths read on the device were outside "
                               "[max(1, q_tokens), kv_stride], or their tiles overflowed "
                               "(error word 0x%x)", err);
    return fail(LA_ETIMEOUT, "a device-side wait exceeded its bound (error word 0x%x)", err);
}

la_status la_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream,
                         size_t* bytes_read) {
    g_msg[0] = 0;
    if (src == nullptr || sink == nullptr || bytes_read == nullptr)
        return fail(LA_EINVAL, "null pointer");
    if (((uintptr_t)src & 15u) != 0) return fail(LA_EINVAL, "src must be 16-byte aligned");
    int dev = 0, cus = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    if (grid == 0) grid = cus;
    if (grid < 1 || grid > 65535) return fail(LA_EINVAL, "grid %d outside [1, 65535]", grid);
    const uint64_t unit = la::stream_read_unit();
    const uint64_t chunk = (uint64_t)bytes / (uint64_t)grid / unit * unit;
    if (chunk == 0)
        return fail(LA_EINVAL, "%zu bytes is less than %llu per workgroup", bytes,
                    (unsigned long long)unit);
    HIP_TRY(la::launch_stream_read(src, chunk, grid, sink, (hipStream_t)stream));
    *bytes_read = (size_t)(chunk * (uint64_t)grid);
    return LA_OK;
}

const char* la_last_error(void) { return g_msg; }

void la_shutdown(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto& kv : g_ws) free_workspace(kv.second);
    g_ws.clear();
    for (auto& kv : g_dev) {
        if (kv.second.budget != nullptr) {
            kv.second.budget->clear();
            delete kv.second.budget;
        }
        for (hipEvent_t e : kv.second.pool) (void)hipEventDestroy(e);
    }
    g_dev.clear();
    g_capacity.clear();
}

// Bound on one device-side wait in microseconds (0 restores the default).
// A small bound makes waits give up early; tests use it to force that path.
void la_set_wait_limit_us(uint32_t us) { g_wait_us = us == 0 ? kDefaultWaitUs : us; }

}  // extern "C"
