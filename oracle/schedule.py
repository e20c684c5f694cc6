"""Stream-K LeanTile schedule, in plain Python integers (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg use this module; the product's scheduler is separate
native code whose tables must equal these field for field.

Steps, in the order of the xllm-io paper review of arXiv 2405.10480:

1. LeanTiles (§3.3): the context of each (request, head) is cut into tiles of
   ``L`` tokens. A request of n tokens has ``T = ceil(n / L)`` tiles; the last
   one may be partly filled and still counts as one iteration.
2. Linear mapping (§3.4): the tile iterations of all heads are laid end to end
   along the context, crossing head and request boundaries. Order: request
   first, then head, then tile. Head ``u = b*H + h`` starts at iteration
   ``S_u``; ``I`` is the total.
3. Equal partition (§3.5, initialisation and parallel execution): a grid of
   ``G = min(G_req, I)`` CTAs; each runs ``I/G`` consecutive iterations. When G
   does not divide I, the first ``I mod G`` CTAs run one more (sizes differ by
   at most one, the "equal-sized chunks" of the LeanAttention talk summary,
   "Technical Deep Dive").
4. Host / finishing detection (§3.5): each CTA's range is cut at head
   boundaries into segments. The segment holding a head's first tile is that
   head's host; the one holding its last tile is its finishing segment.
   ``host_cta[u]`` and ``last_cta[u]`` are the CTAs holding those segments;
   the CTAs in between (and ``last_cta``) are the peers whose partial results
   the host merges, in ascending CTA order.

Segment rows are 6 integers: (cta, u, t0, t1, host, finishing), with tiles
``t0 <= t < t1`` of head u, ``host = (t0 == 0)``, ``finishing = (t1 == T_u)``.
"""
from __future__ import annotations

from bisect import bisect_right

__all__ = ["tiles_per_request", "lean_schedule", "cta_of_iteration"]


def tiles_per_request(ctx_lens, L: int) -> list[int]:
    if L < 1:
        raise ValueError("tile size must be at least one token")
    out = []
    for n in ctx_lens:
        n = int(n)
        if n < 1:
            raise ValueError("every request needs a context of at least one token")
        out.append((n + L - 1) // L)
    return out


def cta_of_iteration(i: int, I: int, G: int) -> int:
    """CTA whose range holds iteration i under the equal partition of step 3."""
    q, r = divmod(I, G)
    big = r * (q + 1)               # iterations owned by the first r (larger) CTAs
    if i < big:
        return i // (q + 1)
    return r + (i - big) // q


def lean_schedule(ctx_lens, H: int, L: int, G_req: int) -> dict:
    """Build the stream-K tables for one decode step.

    Returns a dict with ``I``, ``G``, ``T`` (tiles per request), ``S`` (start
    iteration of each head, length B*H+1), ``cta_begin`` (G+1 iteration
    bounds), ``cta_seg`` (G+1 bounds into ``seg``), ``seg`` (list of 6-tuples),
    ``host_cta`` and ``last_cta`` (per head).
    """
    if H < 1:
        raise ValueError("need at least one head")
    if G_req < 1:
        raise ValueError("need at least one CTA")
    T = tiles_per_request(ctx_lens, L)
    B = len(T)
    S = []
    pos = 0
    for b in range(B):
        for _h in range(H):
            S.append(pos)
            pos += T[b]
    S.append(pos)
    I = pos
    if I < 1:
        raise ValueError("empty batch")
    G = min(int(G_req), I)
    q, r = divmod(I, G)
    cta_begin = [c * q + min(c, r) for c in range(G + 1)]

    seg = []
    cta_seg = []
    for c in range(G):
        cta_seg.append(len(seg))
        i, end = cta_begin[c], cta_begin[c + 1]
        while i < end:
            u = bisect_right(S, i) - 1          # head whose tiles contain iteration i
            Tu = T[u // H]
            j = min(end, S[u] + Tu)
            t0, t1 = i - S[u], j - S[u]
            seg.append((c, u, t0, t1, int(t0 == 0), int(t1 == Tu)))
            i = j
    cta_seg.append(len(seg))

    host_cta = [cta_of_iteration(S[u], I, G) for u in range(B * H)]
    last_cta = [cta_of_iteration(S[u] + T[u // H] - 1, I, G) for u in range(B * H)]
    return {
        "I": I, "G": G, "T": T, "S": S,
        "cta_begin": cta_begin, "cta_seg": cta_seg, "seg": seg,
        "host_cta": host_cta, "last_cta": last_cta,
    }
