// Device helpers shared by the decode-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"
#include "seg_walk.h"

namespace la {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load with the non-temporal hint: K and V are streamed exactly once,
// so they should not displace other lines in the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const char* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Butterflies across the 16-lane rows of a wave on gfx950's row-swap
// instructions, without the LDS round trip of a lane shuffle. A swap of x with
// itself leaves both lanes of every pair (l, l ^ 16), or (l, l ^ 32), with the
// lower lane's value first and the upper lane's second (checked on MI355X), so
// combining the two gives the same bits in both lanes.
__device__ __forceinline__ float2 pair16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float2 pair32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// x summed over lanes (l, l ^ 16, l ^ 32, l ^ 48) as (x_l + x_l^16) + (...),
// and the maximum over the same four lanes; every one of them gets the same bits.
__device__ __forceinline__ float sum_xor16_32(float x) {
    float2 p = pair16(x);
    p = pair32(p.x + p.y);
    return p.x + p.y;
}
__device__ __forceinline__ float max_xor16_32(float x) {
    float2 p = pair16(x);
    p = pair32(fmaxf(p.x, p.y));
    return fmaxf(p.x, p.y);
}

// f applied to a running (M, Ls, O) and one more record (pm, pl, po).
template <int N>
__device__ __forceinline__ void merge_into(float& M, float& Ls, float (&O)[N], float pm, float pl,
                                           const float (&po)[N]) {
    const float mn = fmaxf(M, pm);
    const float mu = (mn == kNegInf) ? 0.f : mn;
    const float a = fexp2(M - mu), b = fexp2(pm - mu);
    Ls = a * Ls + b * pl;
#pragma unroll
    for (int k = 0; k < N; ++k) O[k] = a * O[k] + b * po[k];
    M = mn;
}

// Cross-workgroup exchange. Peers and hosts run on different XCDs, whose L2
// caches are not coherent with each other. Instead of release/acquire fences
// (which write back / invalidate a whole L2 and stall every other workgroup
// on that XCD), every access to the exchange buffers is an agent-scope atomic
// (stores write through to the device coherence point, loads bypass stale
// lines), and ordering comes from completion: a peer waits until its data
// stores have completed (s_waitcnt vmcnt(0)) before it stores its flag, and a
// host loads a peer's data only after it has observed the flag.
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_flag(uint32_t* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16- and 8-byte exchange accesses with the same device-scope coherence
// (cache policy sc1), through a raw buffer resource over the exchange buffer
// (offsets in bytes; the resource also bounds every access to `bytes`).
constexpr int kCoherentPolicy = 16;   // sc1
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t exchange_rsrc(float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
    const u32x4_t x = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                       __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)off, 0, kCoherentPolicy);
}
__device__ __forceinline__ void store8_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b) {
    const u32x2_t x = {__float_as_uint(a), __float_as_uint(b)};
    __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)off, 0, kCoherentPolicy);
}
__device__ __forceinline__ float4 load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t x = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherentPolicy));
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                       __uint_as_float(x.w));
}
__device__ __forceinline__ float2 load8_agent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2_t x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCoherentPolicy));
    return make_float2(__uint_as_float(x.x), __uint_as_float(x.y));
}

__device__ __forceinline__ void drain_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // every memory operation of this wave has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Row of the first key of head h (of Hx per request) of request b in the K/V
// cache: packed per request (stride 0: request b's block [Hx, n_b, d] starts
// at row Hx * tok_off) or a cache of `stride` rows per head ([B, Hx, stride,
// d]).
__device__ __forceinline__ int64_t head_row0(int stride, int Hx, int b, int h, int64_t tok_off,
                                             int n) {
    return stride > 0 ? ((int64_t)b * Hx + h) * stride : (int64_t)Hx * tok_off + (int64_t)h * n;
}

// Epoch of this launch on a lean exchange: one more than the last completed
// launch's, never 0 (zero-filled flags never match).
__device__ __forceinline__ uint32_t launch_epoch(uint32_t* ctl) {
    const uint32_t e = __builtin_amdgcn_readfirstlane(load_flag(&ctl[kCtlEpoch])) + 1u;
    return e == 0u ? 1u : e;
}

// One thread per workgroup, after its last access to the exchange: the last
// workgroup out resets the exit count and makes this launch's epoch the
// completed one, which the next launch starts from.
__device__ __forceinline__ void launch_exit(uint32_t* ctl, uint32_t epoch) {
    const uint32_t n = __hip_atomic_fetch_add(&ctl[kCtlExit], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (n == gridDim.x - 1) {
        __hip_atomic_store(&ctl[kCtlExit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kCtlEpoch], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wait until a peer's flag holds this launch's epoch. Gives up after `limit`
// ticks of the 100 MHz realtime clock, or at once when a wait of the same
// launch has given up; then it raises the sticky error bit and marks the
// launch aborted. A missing peer cannot hang the launch, and a give-up does
// not reach later launches.
__device__ __forceinline__ void wait_flag(uint32_t* f, uint32_t epoch, uint64_t limit,
                                          uint32_t* ctl) {
    if (load_flag(f) == epoch) return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (load_flag(f) != epoch) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - t0 > limit || load_flag(&ctl[kCtlAbort]) == epoch) {
            atomicOr(&ctl[kCtlErr], kErrTimeout);
            __hip_atomic_store(&ctl[kCtlAbort], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
}

// The schedule prefix sums carried in the kernel arguments (Args::sched.tp
// and .tok), read in place through the kernarg segment with scalar loads.
// Args must be the kernel's only argument (offset 0).
typedef const __attribute__((address_space(4))) int32_t* ktp_t;
typedef const __attribute__((address_space(4))) uint32_t* ktok_t;
typedef const __attribute__((address_space(4))) SchedArgs* ksa_t;
struct KSched {
    ktp_t tp;
    ktok_t tok;
    ksa_t sa;
};
template <class Args>
__device__ __forceinline__ KSched kernarg_sched() {
    typedef const __attribute__((address_space(4))) char* kchar_t;
    const kchar_t base = (kchar_t)__builtin_amdgcn_kernarg_segment_ptr();
    return {(ktp_t)(base + offsetof(Args, sched) + offsetof(SchedArgs, tp)),
            (ktok_t)(base + offsetof(Args, sched) + offsetof(SchedArgs, tok)),
            (ksa_t)(base + offsetof(Args, sched))};
}

// LDS for the segment walk over lengths read from device memory.
struct SchedLds {
    int32_t tp[kMaxDeviceB + 1];   // tiles of the requests before b (exclusive prefix)
    int64_t tok[kMaxDeviceB + 1];  // tokens of the requests before b
    int bad;                    // a length was out of range, or the tiles overflow
    int uniform;                // every request has the same length
};

// Walks a workgroup's segments in order: derived here (SegWalk over prefix
// sums from the kernel arguments, or computed by the first wave from lengths
// in device memory), or read from the host's tables. The tests compare every
// source with the executed tile map. One type per source and kernel
// instantiation keeps the cursor state in scalar registers.
template <int kSrc>
struct SegCursor;

template <>
struct SegCursor<kSrcArgs> {
    SegWalk<ktp_t, ktok_t> w;

    __device__ SegCursor(const SchedArgs& a, KSched k, SchedLds&, int c) {
        w.init(k.tp, k.tok, a.B, a.U, a.G, c);
    }
    __device__ bool bad() const { return false; }
    __device__ bool uniform() const { return false; }   // host lengths: the host knows
    __device__ bool next(LeanSeg& s) { return w.next(s); }
};

template <>
struct SegCursor<kSrcDevice> {
    SegWalk<const int32_t*, const int64_t*> w;
    int bad_;
    int uniform_;               // every request has the same length

    // Every thread constructs it (a barrier inside). The first wave reads the
    // lengths once (up to 16 consecutive requests per lane), checks them, and
    // scans tiles and tokens across the wave into LDS. Each length is read
    // from device memory once and kept in the lane's own LDS entries, so the
    // checked values are the ones the walk uses.
    __device__ SegCursor(const SchedArgs& a, KSched, SchedLds& l, int c) {
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            const int per = (a.B + 63) >> 6;
            const int x0 = min(lane * per, a.B), x1 = min(x0 + per, a.B);
            int bad = 0;
            int64_t tp = 0, tk = 0;
            int32_t nlo = 0x7fffffff, nhi = -0x7fffffff - 1;
            for (int x = x0; x < x1; ++x) {
                const int32_t n = a.dlens[x];
                l.tp[x] = n;
                bad |= n < a.n_min || n > a.n_max;
                tp += ((int64_t)n + a.L - 1) / a.L;
                tk += n;
                nlo = min(nlo, n);
                nhi = max(nhi, n);
            }
            for (int o = 1; o < 64; o <<= 1) {
                nlo = min(nlo, __shfl_xor(nlo, o, 64));
                nhi = max(nhi, __shfl_xor(nhi, o, 64));
            }
            int64_t tpi = tp, tki = tk;
            for (int o = 1; o < 64; o <<= 1) {
                const int64_t t2 = __shfl_up(tpi, o, 64);
                const int64_t k2 = __shfl_up(tki, o, 64);
                if (lane >= o) {
                    tpi += t2;
                    tki += k2;
                }
            }
            tp = tpi - tp;
            tk = tki - tk;
            for (int x = x0; x < x1; ++x) {
                const int32_t n = l.tp[x];
                l.tp[x] = (int32_t)tp;
                l.tok[x] = tk;
                tp += ((int64_t)n + a.L - 1) / a.L;
                tk += n;
            }
            // the total must leave U * tiles < 2^31 (the schedule's 32-bit iterations)
            const int64_t total = __shfl(tpi, 63, 64);
            bad |= total * a.U > (int64_t)0x7fffffff;
            bad = __any(bad);
            if (lane == 63) {
                l.tp[a.B] = (int32_t)total;
                l.tok[a.B] = tki;
            }
            if (lane == 0) {
                l.bad = bad;
                l.uniform = nlo == nhi;
            }
        }
        __syncthreads();
        bad_ = __builtin_amdgcn_readfirstlane(l.bad);
        uniform_ = __builtin_amdgcn_readfirstlane(l.uniform);
        if (!bad_) w.init(l.tp, l.tok, a.B, a.U, a.G, c);
    }
    __device__ bool bad() const { return bad_ != 0; }
    __device__ bool uniform() const { return uniform_ != 0; }
    __device__ bool next(LeanSeg& s) { return bad_ ? false : w.next(s); }
};

template <>
struct SegCursor<kSrcTables> {
    ksa_t ka;
    int si, s1;                 // next segment, end
    int iter;                   // linear iteration of the next segment

    __device__ SegCursor(const SchedArgs& a_, KSched k, SchedLds&, int c)
        : ka(k.sa), si(a_.cta_seg[c]), s1(a_.cta_seg[c + 1]), iter(a_.cta_begin[c]) {}
    __device__ bool bad() const { return false; }
    __device__ bool uniform() const { return false; }   // host lengths: the host knows

    // The table pointers are read from the kernel arguments at every segment
    // (an opaque copy of the kernarg pointer keeps them from being hoisted):
    // kept live across the grouped kernel's step loop they pushed it past its
    // scalar registers and into scratch.
    __device__ bool next(LeanSeg& s) {
        if (si >= s1) return false;
        ksa_t p = ka;
        asm volatile("" : "+s"(p));
        const auto& a = *p;
        const int4 sg = a.seg[si++];
        s.u = sg.x;
        s.t0 = sg.y;
        s.t1 = sg.z;
        s.host = (sg.w & 1) != 0;
        s.fin = (sg.w & 2) != 0;
        s.b = s.u / a.U;
        s.unit = s.u - s.b * a.U;
        s.n = a.ctx[s.b];
        s.tok_off = a.tok_off[s.b];
        s.last = (s.host && !s.fin) ? a.last_cta[s.u] : 0;
        s.iter0 = iter;
        iter += s.t1 - s.t0;
        return true;
    }
};

// This workgroup's CU slot in the control block's per-CU counters.
__device__ __forceinline__ uint32_t cu_slot() {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
    return ((xcc & 15u) << 8) | ((hw >> 8) & 0xFFu);
}
__device__ __forceinline__ void cu_add(uint32_t* ctl, uint32_t slot, int delta) {
    __hip_atomic_fetch_add(ctl + kCtlCu + slot, (uint32_t)delta, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t cu_count(const uint32_t* ctl, uint32_t slot) {
    return __hip_atomic_load(ctl + kCtlCu + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t hwreg_ids() {
    // HW_ID (register 4) and XCC_ID (register 20), all 32 bits of each
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
    return ((uint64_t)xcc << 32) | hw;
}

// Per-workgroup trace: realtime clock at entry and exit plus the hardware
// ids of the CU it ran on (thread 0 only). Returns the entry clock.
__device__ __forceinline__ uint64_t stamp_start(uint64_t* ts, int blk) {
    const uint64_t t = ts != nullptr ? __builtin_amdgcn_s_memrealtime() : 0;
    if (ts != nullptr && threadIdx.x == 0) {
        ts[blk * 4 + 0] = t;
        ts[blk * 4 + 2] = hwreg_ids();
        ts[blk * 4 + 3] = 0;
    }
    return t;
}
__device__ __forceinline__ uint64_t stamp_now(const uint64_t* ts) {
    return ts != nullptr ? __builtin_amdgcn_s_memrealtime() : 0;
}
// A lean host's wait for its peers began at w0 and ends now: the fourth word
// holds both as clock ticks after entry t_in, (end << 32) | begin.
__device__ __forceinline__ void stamp_wait(uint64_t* ts, int blk, uint64_t t_in, uint64_t w0) {
    if (ts != nullptr && threadIdx.x == 0) {
        const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
        ts[blk * 4 + 3] = ((w1 - t_in) << 32) | ((w0 - t_in) & 0xffffffffull);
    }
}
__device__ __forceinline__ void stamp_end(uint64_t* ts, int blk) {
    if (ts != nullptr && threadIdx.x == 0) ts[blk * 4 + 1] = __builtin_amdgcn_s_memrealtime();
}

}  // namespace
}  // namespace la
