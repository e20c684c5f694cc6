// Shape-driven selection among the decompositions (siliconandsystems digest,
// "A useful control policy": pick a FlashAttention-style, fixed-split or
// stream-K schedule from the actual shape; xllm-io paper review §4.3: the
// stream-K schedule reduces to the per-head one when every workgroup holds
// whole heads, and to a fixed split of K = G / (B H) pieces when the lengths
// are uniform and B H divides G).
//
// The choice, from measurements of all three kernels over shapes from one
// 512k-token head to thousands of 256-token heads:
//   1. Grid. One lean workgroup per CU keeps a CU's loads in flight from a
//      single stream, which is fastest while a workgroup's range holds few
//      heads. With at least two heads per CU, every workgroup switches heads,
//      and the fixed costs of a switch (loading q, the cross-wave fold, the
//      epilogue) stall a CU that runs one workgroup; two per CU hide them --
//      unless the heads average kLongUnitTiles tiles or more, where a
//      workgroup switches heads a few times in a long range and one per CU
//      is faster again (measured on three draws of the 16-request ragged
//      batch, 178-423 tiles per head on average: 0.2-1.6%).
//   2. Kind. If the lean schedule on that grid splits no head, every
//      workgroup holds whole heads: the per-head decomposition (review §4.3's
//      FlashAttention-2 case) does the same work with no tables, partials or
//      flags, and the hardware dispatcher balances it, so per head is chosen.
//      Single-head kernels take it for any head length (measured on 4096
//      to 65536 whole heads of 1-8 tiles: per head 20% faster at one tile, 9%
//      at two, 2% at four, 1.5% at eight: several per-head workgroups on a CU
//      hide the latency of a short head's few steps, which a lean workgroup
//      walking its heads one after the other does not). Grouped units take it
//      from kMinTilesPerUnitGrouped tiles on average (measured: 2-tile units
//      4% faster on lean, 4- and 8-tile units 3% faster per head). Otherwise
//      lean. A fixed split is never chosen: on uniform
//      lengths the lean schedule already is the best fixed split, in one
//      launch instead of two, and on ragged lengths its balance is better.
//   3. Short heads. When every head's K and V fit in kShortUnitBytes and all
//      heads run at once on one workgroup per CU, the launch is bound by
//      latency, not bandwidth: the few workgroups of the per-head kernel
//      stream their head without contention, while the lean schedule would
//      split the heads into one-tile pieces and add a merge. Per head is
//      chosen (measured on 4 to 256 heads of 128-256 KiB: 12-19% faster than
//      lean; heads of 512 KiB already favour lean). Single-head kernels
//      only: the grouped per-head kernel, whose waves step through a short
//      unit in few long-latency steps, measured 27% slower than lean on 64
//      units of 256 KiB.
#include "select.h"

#include <stddef.h>

#include <vector>

#include "sched.h"

namespace la {

constexpr int64_t kMinTilesPerUnitGrouped = 4;
constexpr int64_t kLongUnitTiles = 128;
constexpr int64_t kShortUnitBytes = 256 * 1024;

int select_kind(const int32_t* ctx_lens, int B, int units, int L, int d, bool grouped, int cus,
                int coresident, int* kind, int* grid, const char** why) {
    if (cus < 1 || coresident < 1 || B < 1 || units < 1 || d < 1) {
        *why = "select: cus, coresident, B, units and d must be >= 1";
        return 1;
    }
    const int64_t U = (int64_t)B * units;
    int32_t n_max = 0;
    int64_t tiles = 0;   // tiles of one unit of every request
    for (int b = 0; b < B; ++b) {
        if (ctx_lens[b] < 1) {
            *why = "select: every context length must be >= 1";
            return 1;
        }
        n_max = ctx_lens[b] > n_max ? ctx_lens[b] : n_max;
        tiles += ((int64_t)ctx_lens[b] + L - 1) / L;
    }
    const bool long_units = tiles >= kLongUnitTiles * (int64_t)B;
    int G = U >= 2 * (int64_t)cus && !long_units ? 2 * cus : cus;
    if (G > coresident) G = coresident;
    if (!grouped && U <= cus && (int64_t)n_max * 4 * d <= kShortUnitBytes) {
        *kind = 2;
        *grid = G;
        return 0;
    }
    int64_t I = 0;
    int Gu = 0, rows = 0;
    const int rc = schedule_dims(ctx_lens, B, units, L, G, &I, &Gu, &rows, why);
    if (rc != 0) return rc;
    thread_local std::vector<int32_t> cb, cs, host, last;
    cb.resize((size_t)Gu + 1);
    cs.resize((size_t)Gu + 1);
    host.resize((size_t)U);
    last.resize((size_t)U);
    build_schedule(ctx_lens, B, units, L, Gu, I, cb.data(), cs.data(), nullptr, nullptr,
                   host.data(), last.data());
    bool split = false;
    for (int64_t u = 0; u < U && !split; ++u) split = host[u] != last[u];
    *kind = (split || (grouped && I < kMinTilesPerUnitGrouped * U)) ? 0 : 2;
    *grid = G;
    return 0;
}

}  // namespace la
