"""Exact decode-phase attention over a KV cache for MI355X (gfx950).

LeanAttention-style stream-K decomposition: LeanTiles along the context, an
even split of all (request, head, tile) iterations over a persistent grid, and
in-launch merging of partial (m, l, Obar) results with the softmax-rescaling
reduction. The computation lives in the HIP library ``libla_decode.so``; this
package only binds it (``binding``) and builds it (``build``).
"""
from .binding import (LA_BF16, LA_F16, LA_KIND_AUTO, LA_KIND_CHUNKS, LA_KIND_FIXED_SPLIT,
                      LA_KIND_LEAN, LA_KIND_PER_HEAD, LA_KIND_PULL, LaError, decode_attention,
                      la_decode, la_decode_bf16, la_decode_ex, la_decode_f16, la_default_grid,
                      la_default_tile, la_last_error, la_max_grid, la_max_grid_grouped,
                      la_schedule, la_schedule_dims, la_select, la_select_for,
                      la_set_wait_limit_us, la_shutdown, la_sync_check, lib)

__all__ = [
    "LA_BF16", "LA_F16", "LA_KIND_AUTO", "LA_KIND_CHUNKS", "LA_KIND_FIXED_SPLIT", "LA_KIND_LEAN",
    "LA_KIND_PER_HEAD", "LA_KIND_PULL",
    "LaError", "decode_attention", "la_decode", "la_decode_bf16", "la_decode_ex", "la_decode_f16",
    "la_default_grid", "la_default_tile", "la_last_error", "la_max_grid", "la_max_grid_grouped",
    "la_schedule",
    "la_schedule_dims", "la_select", "la_select_for", "la_set_wait_limit_us", "la_shutdown",
    "la_sync_check", "lib",
]
