// Host-side stream-K scheduler (xllm-io paper review of arXiv 2405.10480,
// §3.4 linear mapping and §3.5 execution flow).
//
// The LeanTile iterations of every (request, head) are laid end to end --
// request-major, then head, then tile -- and the resulting line of I
// iterations is cut into G contiguous ranges whose sizes differ by at most one
// (the first I mod G ranges are one longer). Each range is then cut at head
// boundaries into segments; the segment that holds a head's first tile marks
// that CTA as the head's host, the one holding its last tile as the finishing
// CTA. One forward sweep over the CTAs with a head cursor that only moves
// forward: O(G + B*H) work.

#include "sched.h"

#include <limits.h>

namespace la {

int schedule_dims(const int32_t* ctx_lens, int B, int H, int L, int grid, int64_t* iters,
                  int* grid_used, int* max_rows, const char** why) {
    if (ctx_lens == nullptr) { *why = "ctx_lens is null"; return 1; }
    if (B < 1 || H < 1) { *why = "B and H must be >= 1"; return 1; }
    if (L < 1) { *why = "tile_tokens must be >= 1"; return 1; }
    if (grid < 1) { *why = "grid must be >= 1"; return 1; }
    int64_t I = 0;
    for (int b = 0; b < B; ++b)
        if (ctx_lens[b] < 1) { *why = "every context length must be >= 1"; return 1; }
    for (int b = 0; b < B; ++b) {
        I += (int64_t)H * ((ctx_lens[b] + (int64_t)L - 1) / L);
        if (I > INT32_MAX) { *why = "too many tile iterations for int32 tables"; return 2; }
    }
    const int64_t rows = (I < grid ? I : grid) + (int64_t)B * H;
    if (rows > INT32_MAX) { *why = "schedule too large"; return 2; }
    *iters = I;
    *grid_used = (int)(I < grid ? I : grid);
    *max_rows = (int)rows;
    return 0;
}

int build_schedule(const int32_t* ctx_lens, int B, int H, int L, int G, int64_t I,
                   int32_t* cta_begin, int32_t* cta_seg, int32_t* rows6, int32_t* rows4,
                   int32_t* host_cta, int32_t* last_cta) {
    (void)B;   // the head cursor stops at I, within the B * H heads
    const int64_t base = I / G;
    const int64_t extra = I % G;
    // head cursor: head u covers iterations [head_lo, head_lo + Tu)
    int u = 0;
    int64_t head_lo = 0;
    int64_t Tu = (ctx_lens[0] + (int64_t)L - 1) / L;
    int nseg = 0;
    int64_t lo = 0;
    for (int c = 0; c < G; ++c) {
        const int64_t hi = lo + base + (c < extra ? 1 : 0);
        cta_begin[c] = (int32_t)lo;
        cta_seg[c] = nseg;
        int64_t i = lo;
        while (i < hi) {
            while (i >= head_lo + Tu) {          // move to the head that holds i
                head_lo += Tu;
                ++u;
                Tu = (ctx_lens[u / H] + (int64_t)L - 1) / L;
            }
            const int64_t stop = (hi < head_lo + Tu) ? hi : head_lo + Tu;
            const int32_t t0 = (int32_t)(i - head_lo);
            const int32_t t1 = (int32_t)(stop - head_lo);
            const int host = (t0 == 0);
            const int fin = (t1 == Tu);
            if (host) host_cta[u] = c;
            if (fin) last_cta[u] = c;
            if (rows6 != nullptr) {
                int32_t* r = rows6 + 6 * (int64_t)nseg;
                r[0] = c; r[1] = u; r[2] = t0; r[3] = t1; r[4] = host; r[5] = fin;
            }
            if (rows4 != nullptr) {
                int32_t* r = rows4 + 4 * (int64_t)nseg;
                r[0] = u; r[1] = t0; r[2] = t1; r[3] = host | (fin << 1);
            }
            ++nseg;
            i = stop;
        }
        lo = hi;
    }
    cta_begin[G] = (int32_t)lo;
    cta_seg[G] = nseg;
    return nseg;
}

}  // namespace la
