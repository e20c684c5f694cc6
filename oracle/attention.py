"""fp64 CPU oracle for decode-phase attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use this module. The product path never imports it.

What it computes is the plain definition of scaled dot-product attention for a
single query row per (request, head) -- the decode shape Nq = 1 (xllm-io paper
review of arXiv 2405.10480, §2.1 and §3.1; LeanAttention talk summary,
"Background") -- and, for several new tokens per request, the same definition
over each token's causally visible prefix (see ``attend_fp64``). LeanAttention
reaches this result exactly, up to floating-point rounding order (xllm-io paper review, §4.1; siliconandsystems digest,
"Exactness and numerical qualification"), so the oracle is the definition
itself, not the tiled algorithm:

    s_j = scale * sum_i q_i K[j, i]          (§3.1; scale placed inside, see below)
    m   = max_j s_j                          (§3.2, rowmax)
    l   = sum_j exp(s_j - m)                 (§3.2, rowsum)
    O   = (sum_j exp(s_j - m) V[j, :]) / l   (§3.2, normalised by diag(l)^-1)

Reading taken where the pages differ: §3.1 applies 1/sqrt(d) inside the
softmax while §3.2 writes S = Q K^T with no factor. Here the caller's
``scale`` multiplies the dot product, so ``m`` and ``l`` are statistics of the
scaled logits.

The partial statistics of one context range (§3.2, "first part") and the
softmax-rescaling reduction f (§3.2, "second part"; restated in §8.4) are also
here, as separate functions, so tests can check the associativity claim of
§3.2/§4.1 against the two-pass definition.

Precision: fp16/bf16 inputs are decoded exactly to fp64 (``decode_half``); all
arithmetic is fp64; sums use numpy's pairwise summation.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "decode_half",
    "attend_head",
    "partial_stats",
    "rescale_merge",
    "identity",
    "normalise",
    "attend_fp64",
    "visible_rows",
]

_CHUNK = 65536  # tokens decoded to fp64 at a time, to bound memory per head


def decode_half(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of raw 16-bit floating-point patterns.

    ``dtype`` is ``"f16"`` (IEEE binary16) or ``"bf16"`` (bfloat16: the top
    16 bits of an IEEE binary32). Both widen to fp64 without rounding.
    """
    b = np.ascontiguousarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected raw uint16 bit patterns")
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        with np.errstate(invalid="ignore"):     # NaN patterns stay NaN
            return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def attend_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Two-pass softmax attention of one query row over n >= 1 context rows.

    ``q`` is [d], ``K`` and ``V`` are [n, d], all fp64. Returns (O[d], m, l).
    Pass 1 finds the maximum scaled logit; pass 2 forms exp(s - m), its sum
    and the weighted sum of V rows; the result is divided by that sum.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] < 1:
        raise ValueError("attention over an empty context is undefined")
    s = scale * (K @ q)
    m = float(np.max(s))
    p = np.exp(s - m)
    l = float(np.sum(p))
    O = (p @ V) / l
    return O, m, l


def partial_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Statistics of one context range: (m, l, Obar) with Obar unnormalised.

    m = rowmax(S), l = rowsum(exp(S - m)), Obar = exp(S - m) V, for
    S = scale * K q over the rows of this range (xllm-io paper review, §3.2,
    first part). An empty range gives the identity element of ``rescale_merge``.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = V.shape[1]
    if K.shape[0] == 0:
        return (-math.inf, 0.0, np.zeros(d))
    s = scale * (K @ np.asarray(q, dtype=np.float64))
    m = float(np.max(s))
    p = np.exp(s - m)
    return (m, float(np.sum(p)), p @ V)


def identity(d: int):
    """Identity of f: a range with no rows, (m, l, Obar) = (-inf, 0, 0)."""
    return (-math.inf, 0.0, np.zeros(d))


def rescale_merge(x, y):
    """The softmax-rescaling reduction f(x, y) on (m, l, Obar) triples.

    m  = max(m_x, m_y)
    l  = exp(m_x - m) l_x + exp(m_y - m) l_y
    Ob = exp(m_x - m) Ob_x + exp(m_y - m) Ob_y
    (xllm-io paper review, §3.2 second part and §8.4). A side whose m is -inf
    (an empty range) gets weight 0, so (-inf, 0, 0) is the identity and no
    -inf - (-inf) is formed.
    """
    mx, lx, ox = x
    my, ly, oy = y
    m = max(mx, my)
    if m == -math.inf:
        return (m, 0.0, np.zeros_like(np.asarray(ox, dtype=np.float64)))
    ax = 0.0 if mx == -math.inf else math.exp(mx - m)
    ay = 0.0 if my == -math.inf else math.exp(my - m)
    return (m, ax * lx + ay * ly,
            ax * np.asarray(ox, dtype=np.float64) + ay * np.asarray(oy, dtype=np.float64))


def normalise(t):
    """O = diag(l)^-1 Obar (xllm-io paper review, §3.2 and §3.5 final step)."""
    m, l, o = t
    if not l > 0.0:
        raise ValueError("cannot normalise an empty range")
    return np.asarray(o, dtype=np.float64) / l


def visible_rows(n: int, Nq: int, t: int) -> int:
    """Rows of an n-row cache that new token t of Nq sees: the token sits at
    position n - Nq + t and attends causally to positions 0 .. n - Nq + t."""
    return n - Nq + 1 + t


def _head_from_packed(kbits, vbits, row0: int, n: int, q: np.ndarray, scale: float,
                      dtype: str):
    """Two-pass attention for one head whose rows are kbits[row0:row0+n]."""
    if n < 1:
        raise ValueError("every request needs a context of at least one token")
    s = np.empty(n, dtype=np.float64)
    for a in range(0, n, _CHUNK):
        e = min(n, a + _CHUNK)
        s[a:e] = scale * (decode_half(kbits[row0 + a:row0 + e], dtype) @ q)
    m = float(np.max(s))
    p = np.exp(s - m)
    l = float(np.sum(p))
    acc = np.zeros(q.shape[0], dtype=np.float64)
    for a in range(0, n, _CHUNK):
        e = min(n, a + _CHUNK)
        acc += p[a:e] @ decode_half(vbits[row0 + a:row0 + e], dtype)
    return acc / l, m, l


def attend_fp64(qbits: np.ndarray, kbits: np.ndarray, vbits: np.ndarray, ctx_lens,
                scale: float, dtype: str, heads=None, workers: int | None = None,
                kv_heads: int | None = None):
    """Decode attention for a packed batch, in fp64.

    ``qbits`` [B, H, d] and ``kbits``/``vbits`` [Hk * sum(n_b), d] hold raw
    fp16/bf16 patterns, with Hk = ``kv_heads`` (default H). Request b's K
    block is [Hk, n_b, d] starting at row Hk * sum(n_{b'} for b' < b) (layout
    (batch, heads, seq_len, head_dim), xllm-io paper review §7.4, with
    requests packed back to back).

    Grouped-query attention (named as a direction in the review, §7.4, and as
    a qualification case in the siliconandsystems digest, "Exactness and
    numerical qualification"): with g = H / Hk, query head h attends over KV
    head h // g, so each run of g consecutive query heads shares one KV head;
    Hk = 1 is multi-query attention. The arithmetic per query head is the
    plain definition above.

    Several new tokens per request (the review, §7.4, names combining the
    method with speculative decoding as a direction; the digest lists masked
    tokens among the cases to qualify): ``qbits`` [B, Nq, H, d] holds Nq
    query tokens per request. They occupy the last Nq of the request's n_b
    cached positions (their own K/V rows end the cache), and token t
    (0-based) attends causally, to the first n_b - Nq + 1 + t rows of its K/V
    head: exactly the rows a one-token decode at that position would see.
    Then every n_b must be >= Nq.

    ``heads`` optionally restricts the work to a list of (b, h) pairs --
    (b, t, h) triples with several tokens; other entries of the outputs are
    NaN. Returns (O[B,H,d], m[B,H], l[B,H]) in fp64, or O[B,Nq,H,d],
    m[B,Nq,H], l[B,Nq,H] with several tokens.
    """
    qbits = np.asarray(qbits)
    multi = qbits.ndim == 4
    if multi:
        B, Nq, H, d = qbits.shape
    else:
        B, H, d = qbits.shape
        Nq = 1
    Hk = H if kv_heads is None else int(kv_heads)
    if Hk < 1 or H % Hk:
        raise ValueError("kv_heads must divide the number of query heads")
    g = H // Hk
    lens = [int(n) for n in ctx_lens]
    if len(lens) != B:
        raise ValueError("ctx_lens must have one entry per request")
    if Nq < 1 or any(n < Nq for n in lens):
        raise ValueError("every context must hold the request's new tokens (n_b >= Nq)")
    if kbits.shape != (Hk * sum(lens), d) or vbits.shape != kbits.shape:
        raise ValueError("packed K/V shape does not match ctx_lens, kv_heads and d")
    q64 = decode_half(qbits.reshape(B * Nq * H, d), dtype).reshape(B, Nq, H, d)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64) * Hk
    if heads is None:
        work = [(b, t, h) for b in range(B) for t in range(Nq) for h in range(H)]
    elif multi:
        work = [tuple(x) for x in heads]
    else:
        work = [(b, 0, h) for b, h in heads]
    O = np.full((B, Nq, H, d), np.nan)
    M = np.full((B, Nq, H), np.nan)
    L = np.full((B, Nq, H), np.nan)

    def one(bth):
        b, t, h = bth
        n = lens[b]
        r0 = int(starts[b]) + (h // g) * n
        return bth, _head_from_packed(kbits, vbits, r0, visible_rows(n, Nq, t), q64[b, t, h],
                                      scale, dtype)

    if workers is None:
        workers = max(1, min(len(work), len(os.sched_getaffinity(0))))
    if workers > 1:
        # one BLAS thread per worker; the heads are the parallel axis
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(one, work))
    else:
        results = [one(x) for x in work]
    for (b, t, h), (o, m, l) in results:
        O[b, t, h] = o
        M[b, t, h] = m
        L[b, t, h] = l
    if not multi:
        return O[:, 0], M[:, 0], L[:, 0]
    return O, M, L
