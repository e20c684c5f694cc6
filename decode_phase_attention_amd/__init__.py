"""Exact decode-phase attention over a KV cache for MI355X (gfx950).

LeanAttention-style stream-K decomposition: LeanTiles along the context, an
even split of all (request, head, tile) iterations over a persistent grid, and
in-launch merging of partial (m, l, Obar) results with the softmax-rescaling
reduction. The computation lives in the HIP library ``libla_decode.so``; this
package only binds it (``binding``) and builds it (``build``).
"""
from . import binding
from .binding import *  # noqa: F401,F403 -- exactly the names in binding.__all__

__all__ = list(binding.__all__)
