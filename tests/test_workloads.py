"""The seeded input generator: shapes, determinism and the drawn structure."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W


def test_named_configs_shapes():
    assert {"tiny", "65k", "512k", "ragged", "many-heads"} <= set(W.CONFIGS)
    for name, w in W.CONFIGS.items():
        assert w.kv_heads is None or w.H % w.kv_heads == 0, name
    inp = W.make_inputs("tiny", seed=0)
    assert inp.q.shape == (1, 4, 64) and inp.q.dtype == torch.float16
    assert inp.k.shape == (4 * 1024, 64) and inp.v.shape == inp.k.shape
    assert inp.ctx_lens == [1024] and abs(inp.scale - 1 / 8) < 1e-15


def test_deterministic_and_order_independent():
    a = W.make_custom([7, 3, 11], H=2, d=8, dtype="bf16", seed=5)
    b = W.make_custom([7, 3, 11], H=2, d=8, dtype="bf16", seed=5)
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    # request 1's block does not depend on the requests around it
    c = W.make_custom([3], H=2, d=8, dtype="bf16", seed=5)
    blk_a = a.v[2 * 7:2 * 7 + 2 * 3]
    d1 = W._draw_request(None, 2, 3, 8, 5, W._TID_V, 1, "cpu", None)
    assert torch.equal(blk_a.float(), d1.reshape(6, 8).to(torch.bfloat16).float())
    assert not torch.equal(c.v.view(torch.int16), blk_a.view(torch.int16))  # b differs (0 vs 1)


def test_ragged_lengths_loguniform():
    w = W.CONFIGS["ragged"]
    for seed in range(4):
        lens = W.context_lengths(w, seed)
        assert len(lens) == 16
        assert all(1024 <= n <= 262144 for n in lens)
    u = np.random.default_rng(0).random(16)
    want = np.floor(np.exp(math.log(1024) + u * math.log(256))).astype(int)
    assert W.context_lengths(w, 0) == list(want)


def test_tiny_shifted_keys_present():
    """Ten keys per head lie 8 units along q/|q| above the N(0,1) cloud."""
    inp = W.make_inputs("tiny", seed=0)
    q = inp.q.float()[0]
    K = inp.k.float().view(4, 1024, 64)
    for h in range(4):
        proj = K[h] @ (q[h] / q[h].norm())
        top = torch.topk(proj, 10).values
        assert float(top.min()) > 4.0
        assert int((proj > 4.5).sum()) <= 12


def test_bits_roundtrip():
    inp = W.make_custom([4], H=1, d=8, dtype="f16", seed=1)
    bits = W.to_bits(inp.k)
    assert bits.dtype == np.uint16 and bits.shape == (4, 8)
    assert np.array_equal(bits.view(np.float16).astype(np.float32), inp.k.float().numpy())


def test_grouped_query_shapes():
    inp = W.make_custom([5, 9], H=8, d=16, dtype="bf16", seed=2, kv_heads=2)
    assert inp.q.shape == (2, 8, 16) and inp.k.shape == (2 * 14, 16) and inp.Hk == 2
    assert W.algorithmic_bytes([5, 9], 8, 16, kv_heads=2) == 2 * 14 * 2 * 16 * 2 + 2 * 8 * 16 * 6
    with pytest.raises(ValueError):
        W.make_custom([4], H=6, d=16, kv_heads=4)


def test_several_new_tokens_shapes():
    a = W.make_custom([6, 3], H=4, d=8, dtype="bf16", seed=2, kv_heads=2, q_tokens=3)
    assert a.q.shape == (2, 3, 4, 8) and a.Nq == 3 and a.Hk == 2
    assert a.k.shape == (2 * 9, 8)
    # token 0 of the batch is the single-token draw: the token axis extends it
    b = W.make_custom([6, 3], H=4, d=8, dtype="bf16", seed=2, kv_heads=2)
    assert torch.equal(a.q[:, 0].view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    with pytest.raises(ValueError):
        W.make_custom([6, 2], H=4, d=8, q_tokens=3)
    assert W.algorithmic_bytes([6, 3], 4, 8, kv_heads=2, q_tokens=3) == \
        2 * 9 * 2 * 8 * 2 + 2 * 3 * 4 * 8 * (2 + 4)
    for name in ("spec4-ragged", "spec8-64k"):
        w = W.CONFIGS[name]
        assert w.q_tokens > 1 and min(W.context_lengths(w)) >= w.q_tokens
