"""Seeded synthetic decode-attention workloads.

This module only draws inputs. It holds none of the attention arithmetic, so
the CPU oracle (``oracle/``) and the HIP path (``decode_phase_attention_amd``)
can both be fed from it without sharing any code with each other.

Workload shapes follow the pages' evaluation axes: single long-context decodes
and ragged batches of unequal context lengths (LeanAttention talk summary,
"Experimental Setup & Results", Workloads; xllm-io paper review, §5.2), over a
KV cache laid out per request as (heads, seq_len, head_dim) (xllm-io paper
review, §7.4).

Packed layout. For request ``b`` with context ``n_b`` the K block is
``[H, n_b, d]``; blocks follow each other in request order, so the whole cache
is a 2-D ``[H * sum(n_b), d]`` tensor and request ``b`` starts at row
``H * sum(n_{b'} for b' < b)``. For equal lengths this equals
``[B, H, n, d]``. V uses the same layout.

Values are i.i.d. N(0, 1), drawn in fp32 from torch generators seeded per
(seed, tensor, request) and rounded to fp16/bf16 (round to nearest even).
The draws do not depend on the order in which requests are generated.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "CONFIGS",
    "Workload",
    "Inputs",
    "context_lengths",
    "make_inputs",
    "make_custom",
    "to_bits",
    "kv_bytes",
    "algorithmic_bytes",
]

_TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}

# tensor ids used in seed mixing
_TID_Q, _TID_K, _TID_V, _TID_SHIFT = 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    dtype: str                    # "f16" or "bf16"
    ctx: int | None = None        # uniform context length, or None for ragged
    ctx_lo: int = 0               # ragged: log-uniform range [ctx_lo, ctx_hi]
    ctx_hi: int = 0
    shift_frac: float = 0.0       # fraction of keys shifted toward q
    shift_norm: float = 0.0       # length of that shift
    kv_heads: int | None = None   # K/V heads per request (None: H, plain multi-head)
    q_tokens: int = 1             # new tokens per request decoded together (speculative verification)
    note: str = ""


CONFIGS: dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, H=4, d=64, dtype="f16", ctx=1024,
                     shift_frac=0.01, shift_norm=8.0,
                     note="1% of keys per head shifted by 8*q/|q| to stress max tracking"),
    "65k": Workload("65k", B=1, H=32, d=128, dtype="bf16", ctx=65536),
    "512k": Workload("512k", B=1, H=32, d=128, dtype="bf16", ctx=524288),
    "ragged": Workload("ragged", B=16, H=32, d=128, dtype="bf16",
                       ctx_lo=1024, ctx_hi=262144,
                       note="per-request context log-uniform in [1024, 262144]"),
    "many-heads": Workload("many-heads", B=8, H=128, d=64, dtype="f16", ctx=16384),
    # grouped-query layouts: g = H / kv_heads query heads share each K/V head
    "gqa-512k": Workload("gqa-512k", B=1, H=32, d=128, dtype="bf16", ctx=524288, kv_heads=8,
                         note="32 query heads over 8 K/V heads (g = 4)"),
    "gqa8-ragged": Workload("gqa8-ragged", B=16, H=64, d=128, dtype="bf16", ctx_lo=1024,
                            ctx_hi=262144, kv_heads=8,
                            note="64 query heads over 8 K/V heads (g = 8), log-uniform lengths"),
    "mqa-32k": Workload("mqa-32k", B=8, H=16, d=64, dtype="f16", ctx=32768, kv_heads=1,
                        note="16 query heads over one K/V head (g = 16)"),
    # several new tokens per request (draft tokens under verification); the
    # last q_tokens positions of each cache are those tokens' own K/V rows
    "spec4-ragged": Workload("spec4-ragged", B=16, H=32, d=128, dtype="bf16", ctx_lo=1024,
                             ctx_hi=262144, kv_heads=8, q_tokens=4,
                             note="4 new tokens per request, 32 query heads over 8 K/V heads"),
    "spec8-64k": Workload("spec8-64k", B=4, H=32, d=128, dtype="bf16", ctx=65536, q_tokens=8,
                          note="8 new tokens per request, plain multi-head"),
    # one GPU's share of 512k when its 32 heads are sharded over 8 GPUs
    "512k-h4": Workload("512k-h4", B=1, H=4, d=128, dtype="bf16", ctx=524288,
                        note="4 of 512k's 32 heads: one GPU's share under 8-way head sharding"),
}


@dataclass
class Inputs:
    q: torch.Tensor               # [B, H, d], or [B, Nq, H, d] with several new tokens
    k: torch.Tensor               # [H * sum(n_b), d] packed per request
    v: torch.Tensor               # same layout as k
    ctx_lens: list[int]
    H: int
    d: int
    dtype: str
    scale: float
    seed: int
    name: str = "custom"
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.ctx_lens)

    @property
    def Hk(self) -> int:
        """K/V heads per request (H for plain multi-head attention)."""
        return int(self.meta.get("kv_heads", self.H))

    @property
    def Nq(self) -> int:
        """New tokens per request (1 for plain decode)."""
        return int(self.meta.get("q_tokens", 1))


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from a tuple of small integers."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h ^= (int(p) + 0x632BE59BD9B4E019 + ((h << 6) & 0xFFFFFFFFFFFFFFFF) + (h >> 2))
        h &= 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device: str, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


def context_lengths(w: Workload, seed: int = 0) -> list[int]:
    """Context length per request.

    Ragged batches draw ``n_b = floor(exp(ln lo + u_b * ln(hi/lo)))`` with
    ``u_b ~ U[0, 1)`` from ``numpy.random.default_rng(seed)``, clipped to
    ``[lo, hi]``: log-uniform lengths, so the batch mixes short and long
    requests the way the pages' ragged workloads do.
    """
    if w.ctx is not None:
        return [int(w.ctx)] * w.B
    u = np.random.default_rng(seed).random(w.B)
    lo, hi = w.ctx_lo, w.ctx_hi
    n = np.floor(np.exp(math.log(lo) + u * math.log(hi / lo))).astype(np.int64)
    return [int(x) for x in np.clip(n, lo, hi)]


def _draw_request(gq_row: torch.Tensor | None, H: int, n: int, d: int, seed: int,
                  tid: int, b: int, device: str, w: Workload | None) -> torch.Tensor:
    g = _gen(device, seed, tid, b)
    x = torch.randn((H, n, d), generator=g, device=device, dtype=torch.float32)
    if w is not None and tid == _TID_K and w.shift_frac > 0.0 and gq_row is not None:
        cnt = max(1, int(round(w.shift_frac * n)))
        for h in range(H):
            gs = _gen("cpu", seed, _TID_SHIFT, b, h)
            idx = torch.randperm(n, generator=gs)[:cnt].to(device)
            qh = gq_row[h]
            x[h, idx, :] += w.shift_norm * qh / torch.linalg.vector_norm(qh)
    return x


def make_custom(ctx_lens: list[int], H: int, d: int, dtype: str = "bf16", seed: int = 0,
                device: str = "cpu", q_std: float = 1.0, scale: float | None = None,
                workload: Workload | None = None, name: str = "custom",
                kv_heads: int | None = None, q_tokens: int = 1) -> Inputs:
    """Draw q, K, V for arbitrary request lengths.

    ``q_std`` widens the score range (adversarial inputs): scores grow in
    proportion to it. ``kv_heads`` (default H) sets the number of K/V heads
    per request for grouped-query layouts: K and V are then
    [kv_heads * sum(n_b), d] while q keeps H heads. ``q_tokens`` > 1 draws
    that many query tokens per request, q then being [B, q_tokens, H, d]
    (token-major, as a batch of new tokens arrives); every n_b must be at
    least q_tokens, since the new tokens' own K/V rows end each cache.
    """
    Hk = H if kv_heads is None else int(kv_heads)
    if Hk < 1 or H % Hk:
        raise ValueError("kv_heads must divide H")
    if any(int(n) < 0 for n in ctx_lens):
        raise ValueError("context lengths must be >= 0")
    Nq = int(q_tokens)
    if Nq < 1 or (Nq > 1 and any(int(n) < Nq for n in ctx_lens)):
        raise ValueError("q_tokens must be >= 1 and at most every context length")
    tdt = _TORCH_DTYPE[dtype]
    B = len(ctx_lens)
    qs = []
    for b in range(B):
        g = _gen(device, seed, _TID_Q, b)
        qs.append(torch.randn((Nq * H, d), generator=g, device=device, dtype=torch.float32) * q_std)
    q32 = torch.stack(qs) if B else torch.empty((0, Nq * H, d), device=device)
    if Nq > 1:
        q32 = q32.view(B, Nq, H, d)
    N = int(sum(ctx_lens))
    k = torch.empty((Hk * N, d), dtype=tdt, device=device)
    v = torch.empty((Hk * N, d), dtype=tdt, device=device)
    row = 0
    for b, n in enumerate(ctx_lens):
        n = int(n)
        if n == 0:
            continue
        kb = _draw_request(q32[b] if Hk == H and Nq == 1 else None, Hk, n, d, seed, _TID_K, b,
                           device, workload)
        k[row:row + Hk * n] = kb.reshape(Hk * n, d).to(tdt)
        del kb
        vb = _draw_request(None, Hk, n, d, seed, _TID_V, b, device, None)
        v[row:row + Hk * n] = vb.reshape(Hk * n, d).to(tdt)
        del vb
        row += Hk * n
    sc = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    inp = Inputs(q=q32.to(tdt).contiguous(), k=k, v=v, ctx_lens=[int(n) for n in ctx_lens],
                 H=H, d=d, dtype=dtype, scale=sc, seed=seed, name=name)
    inp.meta["kv_heads"] = Hk
    inp.meta["q_tokens"] = Nq
    return inp


def make_inputs(name: str, seed: int = 0, device: str = "cpu") -> Inputs:
    """Inputs for one of the named workloads in ``CONFIGS``."""
    w = CONFIGS[name]
    lens = context_lengths(w, seed)
    inp = make_custom(lens, w.H, w.d, w.dtype, seed=seed, device=device, workload=w, name=name,
                      kv_heads=w.kv_heads, q_tokens=w.q_tokens)
    inp.meta["workload"] = w
    return inp


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of an fp16/bf16 tensor as a host numpy uint16 array."""
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"expected fp16/bf16, got {t.dtype}")
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def kv_bytes(ctx_lens: list[int], H: int, d: int, elem: int = 2) -> int:
    return 2 * int(sum(ctx_lens)) * H * d * elem


def algorithmic_bytes(ctx_lens: list[int], H: int, d: int, elem: int = 2,
                      kv_heads: int | None = None, q_tokens: int = 1) -> int:
    """Bytes one decode step must move: K and V once (kv_heads heads), q once
    and the fp32 output once (q_tokens x H query rows per request)."""
    B = len(ctx_lens)
    Hk = H if kv_heads is None else kv_heads
    rows = B * q_tokens * H
    return kv_bytes(ctx_lens, Hk, d, elem) + rows * d * elem + rows * d * 4
