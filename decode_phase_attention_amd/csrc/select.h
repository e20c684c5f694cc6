// Shape-driven choice between the lean, fixed-split and per-head kernels.
#pragma once

#include <stdint.h>

namespace la {

// Picks the kernel kind (0 lean, 2 per head) and the lean grid for a batch of
// B requests with `units` schedule units each, tiles of L tokens, head dim d
// (a token of one K/V head is 4 d bytes of K and V), `grouped` when the units
// run on the grouped (MFMA) kernels, on a device with `cus` compute units and
// room for `coresident` lean workgroups. ctx_lens[b] >= 1.
// Returns 0 on success, 1/2 as schedule_dims (and sets *why).
int select_kind(const int32_t* ctx_lens, int B, int units, int L, int d, bool grouped, int cus,
                int coresident, int* kind, int* grid, const char** why);

}  // namespace la
