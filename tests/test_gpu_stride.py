"""GPU parity for a K/V cache with a per-head capacity ([B, Hk, S, d], only
the first n_b rows of each head valid): every kind against the fp64 oracle
on the packed rows, with the unused rows of the cache filled with NaN, so
that reading a single row past a head's context would poison its output;
and a decode loop that appends one token per step to the same cache."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fullsize_ref import full_reference

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def strided(inp, S):
    """The packed K and V of `inp` copied into [B, Hk, S, d] caches whose rows
    past each head's context hold NaN."""
    B, Hk, d = inp.B, inp.Hk, inp.d
    caches = []
    for t in (inp.k, inp.v):
        c = torch.full((B, Hk, S, d), float("nan"), dtype=t.dtype, device=t.device)
        row = 0
        for b, n in enumerate(inp.ctx_lens):
            c[b, :, :n, :] = t[row:row + Hk * n].view(Hk, n, d)
            row += Hk * n
        caches.append(c)
    return caches


CASES = [([700, 1, 5000, 129], 4, 4, 1, 128, "bf16"),
         ([3000, 17, 256], 8, 2, 1, 64, "f16"),
         ([900, 4100], 16, 1, 1, 64, "f16"),
         ([515, 1030], 8, 2, 4, 128, "bf16")]


@pytest.mark.parametrize("lens,H,Hk,Nq,d,dtype", CASES)
@pytest.mark.parametrize("kind,opts", [("lean", {}), ("lean", {"host_tables": True}),
                                       ("lean", {"grid": 7}), ("fixed_split", {"num_splits": 3}),
                                       ("per_head", {}), ("pull", {"grid": 5}),
                                       ("chunks", {"chunk_tiles": 2}), ("auto", {})])
def test_strided_cache_parity(la, lens, H, Hk, Nq, d, dtype, kind, opts):
    S = max(lens) + 77
    say(f"[stride] lens={lens} H={H} Hk={Hk} Nq={Nq} d={d} {dtype} S={S} {kind} {opts}")
    inp = W.make_custom(lens, H, d, dtype, seed=len(lens) + H + Nq, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    kc, vc = strided(inp, S)
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, dtype, workers=8, kv_heads=Hk)[0]
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, kc, vc, lens, len(lens), H, d, inp.scale, out, kind=kind,
                    kv_heads=Hk, q_tokens=Nq, kv_stride=S, **opts)
    la.la_sync_check()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert float(np.max(np.abs(got - ref))) <= 1e-3


def test_decode_loop_appends_in_place(la):
    """Twelve decode steps on one [B, Hk, S, d] cache: each step writes the new
    token's K/V row at position n_b and attends over n_b + 1 rows; all steps
    queued without synchronisation, each checked against the oracle."""
    H, Hk, d, S = 8, 2, 128, 2048
    lens0 = [1000, 37, 1500]
    steps = 12
    final = [n + steps for n in lens0]
    inp = W.make_custom(final, H, d, "bf16", seed=91, device="cuda", kv_heads=Hk)
    kc, vc = strided(inp, S)
    full_k, full_v = kc.clone(), vc.clone()
    # start with only the first lens0 rows of each head valid
    for b, n in enumerate(lens0):
        kc[b, :, n:, :] = float("nan")
        vc[b, :, n:, :] = float("nan")
    outs = []
    for i in range(steps):
        lens = [n + i + 1 for n in lens0]
        for b, n in enumerate(lens):                  # append the step's token
            kc[b, :, n - 1, :] = full_k[b, :, n - 1, :]
            vc[b, :, n - 1, :] = full_v[b, :, n - 1, :]
        out = torch.empty((len(lens), H, d), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, kc, vc, lens, len(lens), H, d, inp.scale, out, kv_heads=Hk,
                        kv_stride=S)
        outs.append((lens, out))
    la.la_sync_check()
    fk = full_k.cpu()
    fv = full_v.cpu()
    for lens, out in outs:
        pk = torch.cat([fk[b, :, :n, :].reshape(Hk * n, d) for b, n in enumerate(lens)])
        pv = torch.cat([fv[b, :, :n, :].reshape(Hk * n, d) for b, n in enumerate(lens)])
        ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(pk), W.to_bits(pv), lens, inp.scale,
                                 "bf16", workers=8, kv_heads=Hk)[0]
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        assert err <= 1e-3, (lens, err)


def test_wrapper_takes_a_4d_cache(la):
    lens = [300, 4000]
    inp = W.make_custom(lens, 8, 64, "f16", seed=92, device="cuda", kv_heads=2)
    kc, vc = strided(inp, 4096)
    out = la.decode_attention(inp.q, kc, vc, lens, kind="auto")
    la.la_sync_check()
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "f16", workers=8, kv_heads=2)[0]
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= 1e-3


@pytest.mark.parametrize("name", ["512k", "gqa8-ragged"])
def test_full_size_strided(la, name):
    """Full-size workloads in a [B, Hk, S, d] cache with S = the longest
    context (gqa8-ragged: heads up to 5.9 GB into the cache, past 32-bit
    offsets), lean and pull, and lean with the lengths read on the device
    (the same bits as with host lengths), on every head against the
    oracle."""
    inp = W.make_inputs(name, seed=0, device="cuda")
    S = max(inp.ctx_lens)
    say(f"[stride full {name}] S={S}")
    kc, vc = strided(inp, S)
    ref = full_reference(name, 0, inp)[0]      # every query row
    del inp.k, inp.v
    outs = {}
    dl = torch.tensor(inp.ctx_lens, dtype=torch.int32, device="cuda")
    for kind in ("lean", "pull", "device"):
        out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
        if kind == "device":
            la.la_decode_ex(inp.q, kc, vc, None, inp.B, inp.H, inp.d, inp.scale, out,
                            kv_heads=inp.Hk, kv_stride=S, ctx_lens_device=dl)
        else:
            la.la_decode_ex(inp.q, kc, vc, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out,
                            kind=kind, kv_heads=inp.Hk, kv_stride=S)
        la.la_sync_check()
        outs[kind] = out.cpu().numpy()
        err = float(np.max(np.abs(outs[kind] - ref)))
        say(f"[stride full {name}] {kind} max|dO|={err:.2e}")
        assert err <= 1e-3
    np.testing.assert_array_equal(outs["lean"], outs["device"])
    del kc, vc, inp
    torch.cuda.empty_cache()
