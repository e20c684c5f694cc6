// A lean workgroup's segments, derived from the per-request prefix sums of
// tiles and tokens (xllm-io paper review of arXiv 2405.10480, §3.4 linear
// mapping and §3.5 equal partition / host and finishing detection): the I
// tile iterations laid end to end in the order request -> unit -> tile, the
// first I mod G of the G workgroups one iteration more than the others, each
// range cut at unit boundaries; the segment with a unit's first tile is its
// host, the one with its last tile its finishing segment.
//
// Plain C++ with no HIP dependency (LA_HD marks the functions host+device),
// so the same code also builds on the host for checking.
#pragma once

#include <stdint.h>

#ifndef LA_HD
#define LA_HD __host__ __device__
#endif

namespace la {

// The walk's values are the same in every lane. Read from LDS they would sit
// in vector registers for the whole streaming loop; on the device they are
// moved to scalar registers instead.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
    const uint64_t u = (uint64_t)x;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
#else
inline int uniform(int x) { return x; }
inline int64_t uniform(int64_t x) { return x; }
#endif

// One segment of a lean workgroup's range: tiles [t0, t1) of unit u.
struct LeanSeg {
    int u, b, unit;            // unit, its request, its index within the request
    int t0, t1;
    bool host, fin;            // holds the unit's first / last tile
    int last;                  // host and not finishing: the unit's last workgroup
    int n;                     // n_b
    int64_t tok_off;           // sum of the earlier requests' n
    int iter0;                 // linear iteration of tile t0
};

struct SegWalk {
    const int32_t* tp;         // [B+1] tiles of the earlier requests (exclusive prefix)
    const int64_t* tok;        // [B+1] tokens of the earlier requests
    int U;
    int64_t q, r;              // I = q*G + r
    int i, i1, b;              // next iteration, end of the range, request of i

    // Workgroup c of G; every request has at least one tile.
    LA_HD void init(const int32_t* tp_, const int64_t* tok_, int B, int U_, int G, int c) {
        tp = tp_;
        tok = tok_;
        U = U_;
        const int64_t I = (int64_t)U * uniform(tp[B]);
        q = I / G;
        r = I - q * G;
        const int64_t lo = (int64_t)c * q + (c < r ? c : r);
        i = (int)lo;
        i1 = (int)(lo + q + (c < r ? 1 : 0));
        int x = 0, y = B;   // U * tp[x] <= i < U * tp[y]
        while (y - x > 1) {
            const int mid = (x + y) >> 1;
            if ((int64_t)U * uniform(tp[mid]) <= i) x = mid; else y = mid;
        }
        b = x;
    }

    // Workgroup whose range holds linear iteration it.
    LA_HD int cta_of(int64_t it) const {
        const int64_t big = r * (q + 1);
        return (int)(it < big ? it / (q + 1) : r + (it - big) / q);
    }

    LA_HD bool next(LeanSeg& s) {
        if (i >= i1) return false;
        int p1 = uniform(tp[b + 1]);
        while ((int64_t)U * p1 <= i) p1 = uniform(tp[++b + 1]);
        const int p0 = uniform(tp[b]);
        const int T = p1 - p0;
        const int j = i - U * p0;
        const int h = j / T;
        s.t0 = j - h * T;
        s.t1 = s.t0 + (i1 - i) < T ? s.t0 + (i1 - i) : T;
        s.b = b;
        s.unit = h;
        s.u = b * U + h;
        s.host = s.t0 == 0;
        s.fin = s.t1 == T;
        s.tok_off = uniform(tok[b]);
        s.n = (int)(uniform(tok[b + 1]) - s.tok_off);
        s.last = (s.host && !s.fin) ? cta_of((int64_t)i - s.t0 + T - 1) : 0;
        s.iter0 = i;
        i += s.t1 - s.t0;
        return true;
    }
};

}  // namespace la
