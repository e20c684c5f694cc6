"""CPU oracle for decode-phase attention and its stream-K schedule.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything here. The product
(``decode_phase_attention_amd``) shares no code with this package and never
imports it.

``attention``: fp64 two-pass softmax attention (the plain definition), the
per-range statistics (m, l, Obar) and the rescaling reduction f.
``schedule``: the LeanTile linearisation, equal partition over a grid and
host/finishing detection, in Python integers.
"""
from .attention import (attend_fp64, attend_head, decode_half, identity, normalise,
                        partial_stats, rescale_merge)
from .schedule import cta_of_iteration, lean_schedule, tiles_per_request

__all__ = [
    "attend_fp64", "attend_head", "decode_half", "identity", "normalise",
    "partial_stats", "rescale_merge", "cta_of_iteration", "lean_schedule",
    "tiles_per_request",
]
