// Host-side stream-K scheduler for LeanTile decode attention.
#pragma once

#include <stdint.h>

namespace la {

// Sizes of the tables for one batch. Returns 0 on success, 1 for invalid
// arguments, 2 when the iteration count does not fit in int32 (and sets *why).
int schedule_dims(const int32_t* ctx_lens, int B, int H, int L, int grid, int64_t* iters,
                   int* grid_used, int* max_rows, const char** why);

// Writes the tables for one batch (sizes from schedule_dims):
//   cta_begin[G+1], cta_seg[G+1], host_cta[B*H], last_cta[B*H], and the
//   segments, either as 6-int rows (cta, u, t0, t1, host, finishing) into
//   `rows6` or as 4-int device rows (u, t0, t1, host | finishing << 1) into
//   `rows4` (either may be null). Returns the number of segments.
int build_schedule(const int32_t* ctx_lens, int B, int H, int L, int G, int64_t I,
                   int32_t* cta_begin, int32_t* cta_seg, int32_t* rows6, int32_t* rows4,
                   int32_t* host_cta, int32_t* last_cta);

}  // namespace la
