"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself:
- hand-derived worked examples with rational answers (tests/golden);
- brute force at 50 digits with mpmath, through a different formula
  (no max shift: O = sum e^{s_j} V_j / sum e^{s_j});
- torch's CPU scaled_dot_product_attention in fp64 (a library special case);
- associativity/commutativity/identity of the reduction f over every
  contiguous partition and every bracketing;
- closed forms (constant V, one token, q = 0, dominant logit, 1 <= l <= n);
- the exact 16-bit decoders, against torch's conversions for all 65536 patterns.
Mutation tests at the end plant plausible mistakes in copies of the oracle's
functions and check that these pins catch them.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def brute_mp(q, K, V, scale, dps=50):
    """O, m, l by the direct formula, at ``dps`` digits."""
    with mpmath.workdps(dps):
        n, d = K.shape
        sc = mpmath.mpf(float(scale))
        s = [sc * mpmath.fsum(mpmath.mpf(float(q[i])) * mpmath.mpf(float(K[j, i])) for i in range(d))
             for j in range(n)]
        e = [mpmath.exp(x) for x in s]
        Z = mpmath.fsum(e)
        O = [mpmath.fsum(e[j] * mpmath.mpf(float(V[j, i])) for j in range(n)) / Z for i in range(d)]
        m = max(s)
        l = Z / mpmath.exp(m)
        return np.array([float(x) for x in O]), float(m), float(l)


def _val(x):
    if isinstance(x, dict):
        return x.get("mul", 1.0) * math.log(x["ln"])
    return float(x)


def _arr(rows):
    return np.array([[_val(x) for x in r] for r in rows], dtype=np.float64)


def fold(parts, merge=None):
    merge = merge or oracle.rescale_merge
    acc = parts[0]
    for p in parts[1:]:
        acc = merge(acc, p)
    return acc


def all_bracketings(items, merge):
    """Every way to parenthesise merge over ``items`` in order."""
    if len(items) == 1:
        return [items[0]]
    out = []
    for k in range(1, len(items)):
        for a in all_bracketings(items[:k], merge):
            for b in all_bracketings(items[k:], merge):
                out.append(merge(a, b))
    return out


def max_partition_error(q, K, V, scale, merge=None, stats=None):
    """Largest deviation from the two-pass result over all contiguous partitions."""
    merge = merge or oracle.rescale_merge
    stats = stats or oracle.partial_stats
    O, m, l = oracle.attend_head(q, K, V, scale)
    n = K.shape[0]
    worst = 0.0
    for mask in range(1 << (n - 1)):
        cuts = [0] + [i + 1 for i in range(n - 1) if mask >> i & 1] + [n]
        parts = [stats(q, K[a:b], V[a:b], scale) for a, b in zip(cuts[:-1], cuts[1:])]
        t = fold(parts, merge)
        err = max(np.max(np.abs(oracle.normalise(t) - O)) / max(1.0, np.max(np.abs(O))),
                  abs(t[1] - l) / l, abs(t[0] - m) / max(1.0, abs(m)))
        worst = max(worst, err)
    return worst


def rand_case(rng, n, d, q_std=1.0):
    q = rng.standard_normal(d) * q_std
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    return q, K, V


# ----------------------------------------------------------------- golden

def test_worked_examples_golden():
    cases = json.load(open(os.path.join(GOLDEN, "attention_worked.json")))["cases"]
    assert len(cases) >= 4
    for c in cases:
        q = np.array([_val(x) for x in c["q"]])
        K, V = _arr(c["K"]), _arr(c["V"])
        O, m, l = oracle.attend_head(q, K, V, c["scale"])
        np.testing.assert_allclose(O, c["O"], rtol=1e-14, atol=1e-14, err_msg=c["name"])
        assert abs(m - _val(c["m"])) <= 1e-14 * max(1.0, abs(m)), c["name"]
        assert abs(l - c["l"]) <= 1e-14 * l, c["name"]
        if "partition" in c:
            p = c["partition"]
            k = p["cut"]
            left = oracle.partial_stats(q, K[:k], V[:k], c["scale"])
            right = oracle.partial_stats(q, K[k:], V[k:], c["scale"])
            for got, want in ((left, p["left"]), (right, p["right"])):
                assert abs(got[0] - _val(want["m"])) < 1e-14
                assert abs(got[1] - want["l"]) < 1e-14
                np.testing.assert_allclose(got[2], want["Obar"], rtol=1e-14, atol=1e-14)
            mg = oracle.rescale_merge(left, right)
            assert abs(mg[0] - _val(p["merged"]["m"])) < 1e-14
            assert abs(mg[1] - p["merged"]["l"]) < 1e-14
            np.testing.assert_allclose(mg[2], p["merged"]["Obar"], rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(oracle.normalise(mg), c["O"], rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_random(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    d = int(rng.integers(1, 9))
    q, K, V = rand_case(rng, n, d)
    scale = float(rng.uniform(0.1, 2.0))
    O, m, l = oracle.attend_head(q, K, V, scale)
    Ob, mb, lb = brute_mp(q, K, V, scale)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12 * np.max(np.abs(V)))
    assert abs(m - mb) <= 1e-12 * max(1.0, abs(mb))
    assert abs(l - lb) <= 1e-12 * lb


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_adversarial_scores(seed):
    """Scores spread over about +-60: exp(s) without a shift spans 1e-26..1e26."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 65))
    d = int(rng.integers(1, 9))
    s_target = rng.uniform(-60, 60, size=n)
    q = np.zeros(d)
    q[0] = 1.0
    K = rng.standard_normal((n, d))
    K[:, 0] = s_target
    V = rng.standard_normal((n, d)) * 10
    O, m, l = oracle.attend_head(q, K, V, 1.0)
    Ob, mb, lb = brute_mp(q, K, V, 1.0)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12 * np.max(np.abs(V)))
    assert abs(m - mb) <= 1e-12 * max(1.0, abs(mb))
    assert abs(l - lb) <= 1e-12 * lb


def _pack(blocks):
    """Pack per-request [H, n_b, d] blocks back to back: rows [H * sum n_b, d]."""
    return np.concatenate([b.reshape(-1, b.shape[-1]) for b in blocks], axis=0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_packed_batch_against_brute_force(dtype):
    """attend_fp64's request/head offsets, checked head by head against brute
    force on the per-head source arrays (which never go through its indexing)."""
    rng = np.random.default_rng(7)
    H, d = 3, 8
    lens = [5, 1, 17, 2]
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16

    def bits_and_vals(shape):
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(tdt)
        return (x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy())

    qb, qv = bits_and_vals((len(lens), H, d))
    kblocks, vblocks = [], []
    for n in lens:
        kblocks.append(bits_and_vals((H, n, d)))
        vblocks.append(bits_and_vals((H, n, d)))
    kp = _pack([kb for kb, _ in kblocks])
    vp = _pack([vb for vb, _ in vblocks])
    scale = 0.37
    O, M, L = oracle.attend_fp64(qb, kp, vp, lens, scale, dtype, workers=2)
    for b, n in enumerate(lens):
        for h in range(H):
            Ob, mb, lb = brute_mp(qv[b, h], kblocks[b][1][h], vblocks[b][1][h], scale)
            np.testing.assert_allclose(O[b, h], Ob, rtol=1e-12, atol=1e-12)
            assert abs(M[b, h] - mb) <= 1e-12 * max(1.0, abs(mb))
            assert abs(L[b, h] - lb) <= 1e-12 * lb
    # the restricted form computes only the requested heads
    O2, _, _ = oracle.attend_fp64(qb, kp, vp, lens, scale, dtype, heads=[(2, 1)], workers=1)
    np.testing.assert_array_equal(O2[2, 1], O[2, 1])
    assert np.isnan(O2[0, 0]).all()


# ----------------------------------------------------------------- library special case

@pytest.mark.parametrize("n,d", [(1, 64), (257, 64), (4096, 128), (8000, 128)])
def test_against_torch_sdpa_fp64(n, d):
    rng = np.random.default_rng(n + d)
    q, K, V = rand_case(rng, n, d)
    scale = 1.0 / math.sqrt(d)
    O, m, l = oracle.attend_head(q, K, V, scale)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).view(1, 1, 1, d), torch.from_numpy(K).view(1, 1, n, d),
        torch.from_numpy(V).view(1, 1, n, d), scale=scale)
    np.testing.assert_allclose(O, t.view(d).numpy(), rtol=1e-12, atol=1e-12)
    s = scale * (torch.from_numpy(K) @ torch.from_numpy(q))
    assert abs(m - float(s.max())) <= 1e-12 * max(1.0, abs(m))
    assert abs(l - float(torch.logsumexp(s, 0).sub(s.max()).exp())) <= 1e-12 * l


# ----------------------------------------------------------------- reduction f

@pytest.mark.parametrize("n,seed", [(6, 0), (9, 1), (12, 2)])
def test_every_contiguous_partition(n, seed):
    rng = np.random.default_rng(seed)
    q, K, V = rand_case(rng, n, 5, q_std=4.0)
    assert max_partition_error(q, K, V, 0.8) < 1e-12


def test_every_bracketing_and_permutation():
    rng = np.random.default_rng(3)
    q, K, V = rand_case(rng, 11, 4, q_std=3.0)
    O, m, l = oracle.attend_head(q, K, V, 0.5)
    cuts = [0, 1, 3, 4, 7, 9, 11]          # 6 unequal parts
    parts = [oracle.partial_stats(q, K[a:b], V[a:b], 0.5) for a, b in zip(cuts[:-1], cuts[1:])]
    trees = all_bracketings(parts, oracle.rescale_merge)
    assert len(trees) == 42                  # Catalan(5)
    for t in trees:
        np.testing.assert_allclose(oracle.normalise(t), O, rtol=1e-12, atol=1e-12)
        assert abs(t[1] - l) <= 1e-12 * l and abs(t[0] - m) <= 1e-15 * max(1, abs(m))
    for perm in itertools.islice(itertools.permutations(range(6)), 0, 720, 37):
        t = fold([parts[i] for i in perm])
        np.testing.assert_allclose(oracle.normalise(t), O, rtol=1e-12, atol=1e-12)
    # the identity (an empty range) can be inserted anywhere
    e = oracle.identity(4)
    for k in range(len(parts) + 1):
        t = fold(parts[:k] + [e] + parts[k:])
        np.testing.assert_allclose(oracle.normalise(t), O, rtol=1e-12, atol=1e-12)
    assert oracle.rescale_merge(e, e)[0] == -math.inf
    assert oracle.partial_stats(q, K[:0], V[:0], 0.5)[1] == 0.0


def test_merge_adversarial_max_gap():
    """Ranges whose maxima differ by ~1400: one side's weight underflows to 0
    in fp64, and the merged result must still equal the two-pass one."""
    rng = np.random.default_rng(11)
    n, d = 8, 3
    q = np.array([1.0, 0.0, 0.0])
    K = rng.standard_normal((n, d))
    K[:4, 0] = rng.uniform(-700, -690, 4)
    K[4:, 0] = rng.uniform(690, 700, 4)
    V = rng.standard_normal((n, d))
    assert max_partition_error(q, K, V, 1.0) < 1e-12


# ----------------------------------------------------------------- closed forms

def test_closed_forms():
    rng = np.random.default_rng(5)
    n, d = 300, 16
    q, K, V = rand_case(rng, n, d, q_std=2.0)
    # constant V gives that constant
    c = rng.standard_normal(d)
    O, m, l = oracle.attend_head(q, K, np.tile(c, (n, 1)), 0.3)
    np.testing.assert_allclose(O, c, rtol=1e-13, atol=1e-13)
    assert 1.0 <= l <= n
    # one token gives V_0, l = 1, m = s_0
    O, m, l = oracle.attend_head(q, K[:1], V[:1], 0.3)
    np.testing.assert_allclose(O, V[0], rtol=0, atol=0)
    assert l == 1.0 and abs(m - 0.3 * float(K[0] @ q)) <= 1e-15 * max(1, abs(m))
    # q = 0 gives the mean of V, m = 0 and l = n
    O, m, l = oracle.attend_head(np.zeros(d), K, V, 0.3)
    np.testing.assert_allclose(O, np.mean(V, axis=0), rtol=1e-12, atol=1e-14)
    assert m == 0.0 and abs(l - n) <= 1e-12 * n
    # a dominant logit (60 above every other score) gives its V row
    j = 123
    qq = q / np.linalg.norm(q)
    K2 = K.copy()
    K2[j] = 0.0
    others = np.max(np.abs(K2 @ qq))
    K2[j] = (others + 60.0) * qq
    O, m, l = oracle.attend_head(qq, K2, V, 1.0)
    np.testing.assert_allclose(O, V[j], rtol=1e-15, atol=1e-15 * np.max(np.abs(V)) * 10)
    assert abs(l - 1.0) < 1e-20 * n + 1e-15


# ----------------------------------------------------------------- 16-bit decoding

@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_decode_half_all_patterns(dtype, tdt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_half(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    one = 0x3C00 if dtype == "f16" else 0x3F80
    assert oracle.decode_half(np.array([one, 0xC000], dtype=np.uint16), dtype).tolist() == [1.0, -2.0]


# ----------------------------------------------------------------- mutation tests

def _bad_merge_drop_term(x, y):
    mx, lx, ox = x
    my, ly, oy = y
    m = max(mx, my)
    ax = 0.0 if mx == -math.inf else math.exp(mx - m)
    ay = 0.0 if my == -math.inf else math.exp(my - m)
    return (m, ax * lx + ly, ax * ox + ay * oy)          # weight of l_y dropped


def _bad_merge_sign(x, y):
    mx, lx, ox = x
    my, ly, oy = y
    m = max(mx, my)
    ax = 0.0 if mx == -math.inf else math.exp(m - mx)    # sign flipped
    ay = 0.0 if my == -math.inf else math.exp(m - my)
    return (m, ax * lx + ay * ly, ax * ox + ay * oy)


def _bad_stats_noscale(q, K, V, scale):
    return oracle.partial_stats(q, K, V, 1.0)


def test_pins_catch_planted_mistakes():
    rng = np.random.default_rng(9)
    q, K, V = rand_case(rng, 7, 3, q_std=3.0)
    assert max_partition_error(q, K, V, 0.6) < 1e-12
    assert max_partition_error(q, K, V, 0.6, merge=_bad_merge_drop_term) > 1e-3
    assert max_partition_error(q, K, V, 0.6, merge=_bad_merge_sign) > 1e-3
    assert max_partition_error(q, K, V, 0.6, stats=_bad_stats_noscale) > 1e-3

    # a transposed operand or a missing scale in the attention itself
    Ob, _, _ = brute_mp(q, K, V, 0.6)
    q3, K3, V3 = rand_case(rng, 3, 3)
    Ob3, _, _ = brute_mp(q3, K3, V3, 0.6)
    assert np.max(np.abs(oracle.attend_head(q3, K3.T, V3, 0.6)[0] - Ob3)) > 1e-3
    assert np.max(np.abs(oracle.attend_head(q, K, V, 1.0)[0] - Ob)) > 1e-3
    assert np.max(np.abs(oracle.attend_head(q, K, V, 0.6)[0] - Ob)) < 1e-12


# ----------------------------------------------------------------- grouped-query heads

@pytest.mark.parametrize("H,Hk", [(4, 2), (6, 1), (8, 8)])
def test_grouped_query_against_brute_force(H, Hk):
    """Query head h reads K/V head h // (H / Hk); checked head by head against
    brute force on the K/V head's own source arrays."""
    rng = np.random.default_rng(H * 10 + Hk)
    d = 8
    lens = [4, 1, 13]
    g = H // Hk

    def bits_and_vals(shape):
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
        return (x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy())

    qb, qv = bits_and_vals((len(lens), H, d))
    kbl = [bits_and_vals((Hk, n, d)) for n in lens]
    vbl = [bits_and_vals((Hk, n, d)) for n in lens]
    kp = np.concatenate([k.reshape(-1, d) for k, _ in kbl])
    vp = np.concatenate([v.reshape(-1, d) for v, _ in vbl])
    O, M, L = oracle.attend_fp64(qb, kp, vp, lens, 0.4, "bf16", workers=1, kv_heads=Hk)
    for b in range(len(lens)):
        for h in range(H):
            Ob, mb, lb = brute_mp(qv[b, h], kbl[b][1][h // g], vbl[b][1][h // g], 0.4)
            np.testing.assert_allclose(O[b, h], Ob, rtol=1e-12, atol=1e-12)
            assert abs(M[b, h] - mb) <= 1e-12 * max(1.0, abs(mb))
            assert abs(L[b, h] - lb) <= 1e-12 * lb


def test_grouped_query_against_torch_sdpa():
    """torch's scaled_dot_product_attention with enable_gqa (fp64, CPU)."""
    rng = np.random.default_rng(77)
    H, Hk, d, n = 16, 4, 64, 3000
    q = torch.from_numpy(rng.standard_normal((1, H, 1, d)).astype(np.float32)).to(torch.float16)
    k = torch.from_numpy(rng.standard_normal((1, Hk, n, d)).astype(np.float32)).to(torch.float16)
    v = torch.from_numpy(rng.standard_normal((1, Hk, n, d)).astype(np.float32)).to(torch.float16)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    O, _, _ = oracle.attend_fp64(bits(q).reshape(1, H, d), bits(k).reshape(Hk * n, d),
                                 bits(v).reshape(Hk * n, d), [n], 0.125, "f16", workers=2,
                                 kv_heads=Hk)
    t = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), scale=0.125, enable_gqa=True)
    np.testing.assert_allclose(O[0], t[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.attend_fp64(bits(q).reshape(1, H, d), bits(k).reshape(Hk * n, d),
                           bits(v).reshape(Hk * n, d), [n], 0.125, "f16", kv_heads=3)


def test_grouping_mistake_is_caught():
    """A plausible slip -- query head h reading K/V head h % Hk instead of
    h // g -- disagrees with torch's grouped-query attention."""
    rng = np.random.default_rng(78)
    H, Hk, d, n = 8, 2, 16, 50
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((Hk, n, d))
    v = rng.standard_normal((Hk, n, d))
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).view(1, H, 1, d), torch.from_numpy(k).view(1, Hk, n, d),
        torch.from_numpy(v).view(1, Hk, n, d), scale=0.3, enable_gqa=True)[0, :, 0].numpy()
    good = np.stack([oracle.attend_head(q[h], k[h // (H // Hk)], v[h // (H // Hk)], 0.3)[0]
                     for h in range(H)])
    bad = np.stack([oracle.attend_head(q[h], k[h % Hk], v[h % Hk], 0.3)[0] for h in range(H)])
    np.testing.assert_allclose(good, t, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(bad - t)) > 1e-3
