"""Pins for the oracle's chunked path: heads longer than one decode chunk.

``attend_fp64`` decodes a head's K and V rows to fp64 a chunk at a time
(``_CHUNK`` tokens) in two loops: the scores chunk by chunk, then the
weighted sum of V accumulated chunk by chunk. Heads of the 512k and ragged
workloads span several chunks, so both loops -- their row offsets and the
accumulation across chunks -- are pinned here against references that never
go through them:
- brute force at 50 digits on small heads, with the chunk shrunk to 7 tokens
  so every head spans several chunks and the last one is partial;
- torch's CPU scaled_dot_product_attention in fp64 on a real-size head of
  more than two chunks (140,000 tokens), in a batch of two requests of two
  heads each so that the checked heads start at a non-zero row;
- the closed forms of a dominant logit and of a constant V, with the
  dominant key placed past the first chunk.
Planted mistakes in the real source of the chunked function (an accumulation
that overwrites, a dropped row offset in either loop) are caught by these
pins, and the unmodified function passes them.
"""
from __future__ import annotations

import inspect
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention as att


def bits_and_vals(x64: np.ndarray, dtype: str):
    """Round fp64 values to the 16-bit type: (raw bits, exact fp64 values)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    x = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(tdt)
    return x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy()


def brute_mp(q, K, V, scale, dps=50):
    """O, m, l by the direct formula (no max shift), at ``dps`` digits."""
    with mpmath.workdps(dps):
        n, d = K.shape
        sc = mpmath.mpf(float(scale))
        s = [sc * mpmath.fsum(mpmath.mpf(float(q[i])) * mpmath.mpf(float(K[j, i])) for i in range(d))
             for j in range(n)]
        e = [mpmath.exp(x) for x in s]
        Z = mpmath.fsum(e)
        O = [mpmath.fsum(e[j] * mpmath.mpf(float(V[j, i])) for j in range(n)) / Z for i in range(d)]
        m = max(s)
        return np.array([float(x) for x in O]), float(m), float(Z / mpmath.exp(m))


def make_batch(lens, H, d, dtype, seed):
    """Per-request [H, n_b, d] blocks of N(0,1) draws, packed back to back.
    Returns q bits/values [B, H, d], per-request K/V values, packed K/V bits."""
    rng = np.random.default_rng(seed)
    qb, qv = bits_and_vals(rng.standard_normal((len(lens), H, d)), dtype)
    kv_bits, kv_vals = [], []
    for n in lens:
        kb, kvv = bits_and_vals(rng.standard_normal((H, n, d)), dtype)
        vb, vvv = bits_and_vals(rng.standard_normal((H, n, d)), dtype)
        kv_bits.append((kb, vb))
        kv_vals.append((kvv, vvv))
    kp = np.concatenate([kb.reshape(-1, d) for kb, _ in kv_bits])
    vp = np.concatenate([vb.reshape(-1, d) for _, vb in kv_bits])
    return qb, qv, kv_vals, kp, vp


def sdpa64(q, K, V, scale):
    d = q.shape[0]
    n = K.shape[0]
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).view(1, 1, 1, d), torch.from_numpy(np.ascontiguousarray(K)).view(1, 1, n, d),
        torch.from_numpy(np.ascontiguousarray(V)).view(1, 1, n, d), scale=scale)
    s = scale * (torch.from_numpy(np.ascontiguousarray(K)) @ torch.from_numpy(q))
    m = float(s.max())
    l = float(torch.exp(s - m).sum())
    return t.view(d).numpy(), m, l


# ----------------------------------------------------------------- the pins

def pin_small_chunks(monkeypatch):
    """Chunks of 7 tokens, brute force on every head of a 2-request batch."""
    monkeypatch.setattr(att, "_CHUNK", 7)
    lens, H, d, scale = [23, 17], 2, 4, 0.45
    for dtype in ("bf16", "f16"):
        qb, qv, kv_vals, kp, vp = make_batch(lens, H, d, dtype, seed=3)
        O, M, L = att.attend_fp64(qb, kp, vp, lens, scale, dtype, workers=1)
        for b in range(len(lens)):
            for h in range(H):
                Ob, mb, lb = brute_mp(qv[b, h], kv_vals[b][0][h], kv_vals[b][1][h], scale)
                np.testing.assert_allclose(O[b, h], Ob, rtol=1e-12, atol=1e-12)
                assert abs(M[b, h] - mb) <= 1e-12 * max(1.0, abs(mb))
                assert abs(L[b, h] - lb) <= 1e-12 * lb


LONG = [140_000, 70_001]      # 3 chunks (the last partial) and 2 chunks (one row in the second)


def pin_long_heads(dtype):
    """Real chunk size; heads of more than two chunks against torch sdpa."""
    assert LONG[0] > 2 * att._CHUNK and LONG[1] > att._CHUNK
    H, d = 2, 8
    scale = 1.0 / math.sqrt(d)
    qb, qv, kv_vals, kp, vp = make_batch(LONG, H, d, dtype, seed=17)
    O, M, L = att.attend_fp64(qb, kp, vp, LONG, scale, dtype, workers=1)
    for b in range(len(LONG)):
        for h in range(H):
            Or, mr, lr = sdpa64(qv[b, h], kv_vals[b][0][h], kv_vals[b][1][h], scale)
            np.testing.assert_allclose(O[b, h], Or, rtol=1e-11, atol=1e-12)
            assert abs(M[b, h] - mr) <= 1e-12 * max(1.0, abs(mr))
            assert abs(L[b, h] - lr) <= 1e-10 * lr


def pin_closed_forms_past_first_chunk(dtype):
    """Head (1, 1) of a 2-request batch: a dominant key at token 100,000
    gives that token's V row; a constant V gives the constant."""
    lens, H, d = [1000, 140_000], 2, 8
    rng = np.random.default_rng(23)
    q = rng.standard_normal((len(lens), H, d))
    K = [rng.standard_normal((H, n, d)) for n in lens]
    V = [rng.standard_normal((H, n, d)) for n in lens]
    scale = 1.0 / math.sqrt(d)
    qb, qv = bits_and_vals(q, dtype)
    j = 100_000
    u = qv[1, 1] / np.linalg.norm(qv[1, 1])
    others = scale * np.max(np.abs(K[1][1] @ qv[1, 1]))
    # scores of the other keys are at most `others`; this one is >= 70 above
    K[1][1][j] = (others + 70.0) / (scale * np.linalg.norm(qv[1, 1])) * u
    c = rng.standard_normal(d)
    for const_v in (False, True):
        Vx = [v.copy() for v in V]
        if const_v:
            Vx[1][1][:] = c
        kbits, kvals, vbits, vvals = [], [], [], []
        for b in range(len(lens)):
            kb, kv = bits_and_vals(K[b], dtype)
            vb, vv = bits_and_vals(Vx[b], dtype)
            kbits.append(kb.reshape(-1, d))
            vbits.append(vb.reshape(-1, d))
            kvals.append(kv)
            vvals.append(vv)
        O, M, L = att.attend_fp64(qb, np.concatenate(kbits), np.concatenate(vbits), lens, scale,
                                  dtype, heads=[(1, 1)], workers=1)
        s = scale * (kvals[1][1] @ qv[1, 1])
        assert int(np.argmax(s)) == j and s[j] - np.max(np.delete(s, j)) >= 60.0
        if const_v:
            np.testing.assert_allclose(O[1, 1], vvals[1][1][0], rtol=1e-13, atol=1e-13)
        else:
            np.testing.assert_allclose(O[1, 1], vvals[1][1][j], rtol=1e-14, atol=1e-14)
            assert abs(L[1, 1] - 1.0) <= 1e-20 * lens[1] + 1e-15
        assert abs(M[1, 1] - s[j]) <= 1e-12 * abs(s[j])


# ----------------------------------------------------------------- tests

def test_small_chunks_against_brute_force(monkeypatch):
    pin_small_chunks(monkeypatch)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_long_heads_against_torch_sdpa(dtype):
    pin_long_heads(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_closed_forms_past_first_chunk(dtype):
    pin_closed_forms_past_first_chunk(dtype)


# Each mutant is the chunked function's own source with one plausible mistake.
MUTANTS = {
    "accumulate_overwrites": ("acc += ", "acc = "),
    "k_loop_drops_row0": ("kbits[row0 + a:row0 + e]", "kbits[a:e]"),
    "v_loop_drops_row0": ("vbits[row0 + a:row0 + e]", "vbits[a:e]"),
    "v_loop_reads_first_chunk": ("vbits[row0 + a:row0 + e]", "vbits[row0:row0 + e - a]"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(att._head_from_packed)
    assert src.count(old) == 1, f"{name}: the planted spot is not in the source any more"
    # the mutant's globals are the module's own, so it sees a patched _CHUNK
    local = {}
    exec(compile(src.replace(old, new), att.__file__, "exec"), vars(att), local)
    return local["_head_from_packed"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_chunk_mistakes_are_caught(monkeypatch, name):
    monkeypatch.setattr(att, "_head_from_packed", _mutant(name))
    # caught at the real chunk size (the branch the long workloads take) ...
    with pytest.raises(AssertionError):
        pin_long_heads("bf16")
    # ... and with small chunks against brute force
    with pytest.raises(AssertionError):
        with monkeypatch.context() as mp:
            pin_small_chunks(mp)
