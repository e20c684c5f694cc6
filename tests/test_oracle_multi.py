"""Pins for the oracle's several-new-tokens path (speculative verification).

Reading taken (the pages name combining the method with speculative decoding
as a direction, xllm-io paper review §7.4, and list masked tokens among the
cases to qualify, siliconandsystems digest "Exactness and numerical
qualification", but fix no mask): the Nq new tokens of a request are the last
Nq of its n_b cached positions, and token t attends causally to positions
0 .. n_b - Nq + t.

The pins are independent of the oracle's prefix slicing:
- brute force at 50 digits over the whole head with an explicit mask from
  query and key positions;
- torch's scaled_dot_product_attention with is_causal=True when every cached
  position is new (Nq = n, where top-left and bottom-right alignment agree),
  with and without grouped K/V heads;
- the same routine with a boolean mask built from positions for Nq < n;
- planted mistakes in the visible-row count are caught.
"""
from __future__ import annotations

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as att


def bits_and_vals(rng, shape, dtype="bf16"):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    x = x.to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy()


def brute_masked(q, K, V, scale, qpos, dps=50):
    """Attention of one query at position qpos over all n rows of K/V, rows at
    positions > qpos weighted zero, at ``dps`` digits."""
    with mpmath.workdps(dps):
        n, d = K.shape
        sc = mpmath.mpf(float(scale))
        s = [sc * mpmath.fsum(mpmath.mpf(float(q[i])) * mpmath.mpf(float(K[j, i])) for i in range(d))
             for j in range(n)]
        allowed = [j <= qpos for j in range(n)]
        e = [mpmath.exp(s[j]) if allowed[j] else mpmath.mpf(0) for j in range(n)]
        Z = mpmath.fsum(e)
        O = [mpmath.fsum(e[j] * mpmath.mpf(float(V[j, i])) for j in range(n)) / Z for i in range(d)]
        m = max(s[j] for j in range(n) if allowed[j])
        return np.array([float(x) for x in O]), float(m), float(Z / mpmath.exp(m))


def make_case(rng, lens, Nq, H, Hk, d, dtype="bf16"):
    qb, qv = bits_and_vals(rng, (len(lens), Nq, H, d), dtype)
    kbl = [bits_and_vals(rng, (Hk, n, d), dtype) for n in lens]
    vbl = [bits_and_vals(rng, (Hk, n, d), dtype) for n in lens]
    kp = np.concatenate([k.reshape(-1, d) for k, _ in kbl])
    vp = np.concatenate([v.reshape(-1, d) for v, _ in vbl])
    return qb, qv, kbl, vbl, kp, vp


@pytest.mark.parametrize("H,Hk", [(2, 2), (4, 2), (6, 1)])
def test_multi_token_against_masked_brute_force(H, Hk):
    rng = np.random.default_rng(100 + H * 10 + Hk)
    lens, Nq, d, scale = [3, 9, 14], 3, 8, 0.45
    g = H // Hk
    qb, qv, kbl, vbl, kp, vp = make_case(rng, lens, Nq, H, Hk, d)
    O, M, L = oracle.attend_fp64(qb, kp, vp, lens, scale, "bf16", workers=1, kv_heads=Hk)
    assert O.shape == (3, Nq, H, d) and M.shape == (3, Nq, H)
    for b, n in enumerate(lens):
        for t in range(Nq):
            for h in range(H):
                Ob, mb, lb = brute_masked(qv[b, t, h], kbl[b][1][h // g], vbl[b][1][h // g], scale,
                                          qpos=n - Nq + t)
                np.testing.assert_allclose(O[b, t, h], Ob, rtol=1e-12, atol=1e-12)
                assert abs(M[b, t, h] - mb) <= 1e-12 * max(1.0, abs(mb))
                assert abs(L[b, t, h] - lb) <= 1e-12 * lb


@pytest.mark.parametrize("H,Hk,n,d", [(4, 4, 37, 16), (8, 2, 64, 32), (4, 1, 5, 8)])
def test_all_new_tokens_is_causal_self_attention(H, Hk, n, d):
    """Nq = n: every cached position is a new token, so the result is ordinary
    causal self-attention over n positions (torch SDPA, is_causal=True)."""
    rng = np.random.default_rng(7 + n)
    qb, qv, kbl, vbl, kp, vp = make_case(rng, [n], n, H, Hk, d, "f16")
    O, _, _ = oracle.attend_fp64(qb, kp, vp, [n], 0.3, "f16", workers=2, kv_heads=Hk)
    q = torch.from_numpy(qv[0]).permute(1, 0, 2).unsqueeze(0)          # [1, H, n, d]
    k = torch.from_numpy(kbl[0][1]).unsqueeze(0)                       # [1, Hk, n, d]
    v = torch.from_numpy(vbl[0][1]).unsqueeze(0)
    t = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.3, is_causal=True,
                                                         enable_gqa=Hk != H)
    np.testing.assert_allclose(O[0], t[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_fewer_new_tokens_against_sdpa_position_mask():
    rng = np.random.default_rng(11)
    H, Hk, d, lens, Nq = 6, 3, 16, [40, 8], 5
    qb, qv, kbl, vbl, kp, vp = make_case(rng, lens, Nq, H, Hk, d)
    O, _, _ = oracle.attend_fp64(qb, kp, vp, lens, 0.2, "bf16", workers=2, kv_heads=Hk)
    for b, n in enumerate(lens):
        qpos = torch.arange(n - Nq, n).view(Nq, 1)
        kpos = torch.arange(n).view(1, n)
        mask = kpos <= qpos                                            # [Nq, n]
        q = torch.from_numpy(qv[b]).permute(1, 0, 2).unsqueeze(0)
        k = torch.from_numpy(kbl[b][1]).unsqueeze(0)
        v = torch.from_numpy(vbl[b][1]).unsqueeze(0)
        t = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=0.2,
                                                             enable_gqa=True)
        np.testing.assert_allclose(O[b], t[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_one_new_token_in_four_d_layout_equals_plain_decode():
    rng = np.random.default_rng(12)
    qb, _, _, _, kp, vp = make_case(rng, [20, 3], 1, 4, 2, 8)
    a = oracle.attend_fp64(qb, kp, vp, [20, 3], 0.5, "bf16", workers=1, kv_heads=2)
    b = oracle.attend_fp64(qb[:, 0], kp, vp, [20, 3], 0.5, "bf16", workers=1, kv_heads=2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x[:, 0], y)


def test_context_must_hold_the_new_tokens():
    rng = np.random.default_rng(13)
    qb, _, _, _, kp, vp = make_case(rng, [4, 2], 3, 2, 2, 8)
    with pytest.raises(ValueError):
        oracle.attend_fp64(qb, kp, vp, [4, 2], 0.5, "bf16", workers=1)
    # n_b == Nq is allowed: the first new token then sees a single row
    qb, qv, kbl, vbl, kp, vp = make_case(rng, [3], 3, 1, 1, 8)
    O, M, L = oracle.attend_fp64(qb, kp, vp, [3], 0.5, "bf16", workers=1)
    np.testing.assert_array_equal(O[0, 0, 0], vbl[0][1][0, 0])
    assert L[0, 0, 0] == 1.0


@pytest.mark.parametrize("mistake", ["one_future_row", "no_mask", "one_row_short"])
def test_planted_mask_mistakes_are_caught(monkeypatch, mistake):
    wrong = {
        "one_future_row": lambda n, Nq, t: min(n, n - Nq + 2 + t),
        "no_mask": lambda n, Nq, t: n,
        "one_row_short": lambda n, Nq, t: max(1, n - Nq + t),
    }[mistake]
    monkeypatch.setattr(att, "visible_rows", wrong)
    caught = 0
    for fn in (test_all_new_tokens_is_causal_self_attention, ):
        try:
            fn(4, 2, 12, 8)
        except AssertionError:
            caught += 1
    try:
        test_fewer_new_tokens_against_sdpa_position_mask()
    except AssertionError:
        caught += 1
    assert caught == 2
