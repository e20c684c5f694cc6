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

// The walk's values are the same in every lane; on the device they are kept
// in scalar registers.
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

// TpPtr / TokPtr: pointers (or any indexable) to the [B+1] exclusive prefix
// sums of tiles and tokens per request.
template <class TpPtr, class TokPtr>
struct SegWalk {
    TpPtr tp;
    TokPtr tok;
    int U;
    int q, r;                  // I = q*Ge + r, Ge = min(G, I) workgroups with work (I < 2^31)
    int i, i1, b;              // next iteration, end of the range, request of i

    // Workgroup c of a grid of G; every request has at least one tile. A grid
    // larger than the I iterations splits them over its first I workgroups
    // (one each) and leaves the others empty.
    LA_HD void init(TpPtr tp_, TokPtr tok_, int B, int U_, int G, int c) {
        tp = tp_;
        tok = tok_;
        U = U_;
        const int I = U * uniform((int)tp[B]);
        const int Ge = G < I ? G : I;
        q = I / Ge;
        r = I - q * Ge;
        if (c >= Ge) {
            i = i1 = b = 0;
            return;
        }
        i = c * q + (c < r ? c : r);
        i1 = i + q + (c < r ? 1 : 0);
        int x = 0, y = B;   // U * tp[x] <= i < U * tp[y]
        while (y - x > 1) {
            const int mid = (x + y) >> 1;
            if (U * uniform((int)tp[mid]) <= i) x = mid; else y = mid;
        }
        b = x;
    }

    // Workgroup whose range holds linear iteration it.
    LA_HD int cta_of(int it) const {
        const int big = r * (q + 1);
        return it < big ? it / (q + 1) : r + (it - big) / q;
    }

    LA_HD bool next(LeanSeg& s) {
        if (i >= i1) return false;
        int p1 = uniform((int)tp[b + 1]);
        while (U * p1 <= i) p1 = uniform((int)tp[++b + 1]);
        const int p0 = uniform((int)tp[b]);
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
        s.tok_off = uniform((int64_t)tok[b]);
        s.n = (int)(uniform((int64_t)tok[b + 1]) - s.tok_off);
        s.last = (s.host && !s.fin) ? cta_of(i - s.t0 + T - 1) : 0;
        s.iter0 = i;
        i += s.t1 - s.t0;
        return true;
    }
};

}  // namespace la
