"""The allocation-free entry point, la_decode_noalloc, against la_decode_ex.

la_decode_noalloc runs the same lean kernels with their exchange (partial
records, flags, control words) in a fixed device array instead of a
per-stream workspace. Through the C ABI, on two calls in a row of which the
second is smaller, its outputs must equal la_decode_ex's with the same
options bit for bit, and the fp64 oracle within the parity bar (max |dO| <=
1e-3; l within 1e-5 relative after rescaling to the oracle's m; |dm| <=
1e-5 max(1, |m|)). Also: lengths on the device with a captured graph
replayed over growing lengths, the grid and size limits refused before any
launch, and a wait forced to give up staying inside its launch.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

O_TOL, L_RTOL, M_RTOL = 1e-3, 1e-5, 1e-5
LA_EINVAL, LA_EUNSUPPORTED, LA_ETIMEOUT = 1, 2, 4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def call(la, fn, inp, **opts):
    """One call of `fn` (la_decode_ex or la_decode_noalloc) on fresh NaN-filled
    outputs; returns (O, m, l) as numpy arrays after la_sync_check."""
    rows = int(np.prod(tuple(inp.q.shape)[:-1]))
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    fn(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out, m_out=m, l_out=l,
       kv_heads=inp.Hk, q_tokens=inp.Nq, **opts)
    la.la_sync_check()
    return out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()


def oracle_of(inp):
    qb = W.to_bits(inp.q)
    O, M, L = oracle.attend_fp64(qb, W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens, inp.scale,
                                 inp.dtype, workers=8, kv_heads=inp.Hk)
    return O, M.reshape(-1), L.reshape(-1)


def check_oracle(got, ref, tag):
    O, m, l = got
    Or, mr, lr = ref
    err = float(np.max(np.abs(O - Or.reshape(O.shape))))
    assert err <= O_TOL, f"{tag}: max |dO| = {err}"
    assert np.all(np.abs(m - mr) <= M_RTOL * np.maximum(1.0, np.abs(mr))), tag
    lrel = np.abs(l * np.exp(m.astype(np.float64) - mr) - lr) / lr
    assert float(np.max(lrel)) <= L_RTOL, f"{tag}: l rel err {float(np.max(lrel))}"


# name, first lengths, second (smaller) lengths, H, Hk, Nq, d, dtype, grid
CASES = [
    ("mha-bf16-d128", [3000, 17, 60000, 129], [1000, 5], 4, 4, 1, 128, "bf16", 0),
    ("mha-f16-d64", [1, 700, 256, 2049, 9000], [300, 12], 8, 8, 1, 64, "f16", 97),
    ("gqa-bf16-d128", [5000, 40000, 77], [2000], 8, 2, 1, 128, "bf16", 0),
    ("spec3-f16-d64", [515, 4000, 1030], [300, 64], 8, 2, 3, 64, "f16", 0),
    ("mqa-f16-d64", [32768, 32768], [4096], 16, 1, 1, 64, "f16", 0),
    ("mha-bf16-d128-maxgrid", [70000, 3, 9000], [20000], 4, 4, 1, 128, "bf16", "max"),
    ("gqa-bf16-d128-maxgrid", [70000, 3, 9000], [20000], 8, 2, 1, 128, "bf16", "max"),
]


@pytest.mark.parametrize("name,first,second,H,Hk,Nq,d,dtype,grid", CASES)
def test_same_bits_as_la_decode_ex(la, name, first, second, H, Hk, Nq, d, dtype, grid):
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
    if grid == "max":
        cap = la.la_max_grid_grouped(d, dt) if (Hk < H or Nq > 1) else la.la_max_grid(d, dt)
        # the scratch holds 2048 workgroups, and 992 grouped ones at d = 128
        grid = min(cap, 992 if (Hk < H or Nq > 1) else 2048)
    for i, lens in enumerate((first, second)):
        say(f"[noalloc {name} call {i}] lens={lens} H={H} Hk={Hk} Nq={Nq} d={d} grid={grid}")
        inp = W.make_custom(lens, H, d, dtype, seed=len(lens) + i, device="cuda", kv_heads=Hk,
                            q_tokens=Nq)
        want = call(la, la.la_decode_ex, inp, grid=grid)
        got = call(la, la.la_decode_noalloc, inp, grid=grid)
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b)
        check_oracle(got, oracle_of(inp), f"{name}/{i}")


def strided(inp, S):
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


def test_device_lengths_in_a_captured_graph(la):
    """A step with the lengths on the device, captured into a graph and
    replayed while eager work grows every context: each replay equals
    la_decode_ex on the same lengths bit for bit."""
    lens0 = [1000, 37, 1500]
    steps = 6
    final = [n + steps for n in lens0]
    S, H, Hk, d = 2048, 8, 2, 128
    inp = W.make_custom(final, H, d, "bf16", seed=5, device="cuda", kv_heads=Hk)
    kc, vc = strided(inp, S)
    dl = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
    eager = torch.empty_like(out)
    kw = dict(kv_heads=Hk, kv_stride=S, grid=64)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):            # an eager call first: the device's set-up
        la.la_decode_noalloc(inp.q, kc, vc, None, 3, H, d, inp.scale, out, ctx_lens_device=dl,
                             stream=s.cuda_stream, **kw)
    s.synchronize()
    la.la_sync_check(s.cuda_stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        la.la_decode_noalloc(inp.q, kc, vc, None, 3, H, d, inp.scale, out, ctx_lens_device=dl,
                             stream=s.cuda_stream, **kw)
    for i in range(steps):
        lens = [n + i + 1 for n in lens0]
        say(f"[noalloc graph step {i}] lens={lens}")
        with torch.cuda.stream(s):
            dl.add_(1)
            g.replay()
        s.synchronize()
        la.la_sync_check(s.cuda_stream)
        la.la_decode_ex(inp.q, kc, vc, lens, 3, H, d, inp.scale, eager, **kw)
        la.la_sync_check()
        np.testing.assert_array_equal(out.cpu().numpy(), eager.cpu().numpy())
    del g


def test_limits_refused_before_any_launch(la):
    """Requests beyond the scratch or outside the in-launch schedule are
    refused with a clear error, and a correct call right after still works."""
    inp = W.make_custom([3000, 500], 8, 128, "bf16", seed=9, device="cuda", kv_heads=2)
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
    args = (inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out)
    with pytest.raises(la.LaError) as e:
        la.la_decode_noalloc(*args, kv_heads=2, kind="fixed_split")
    assert e.value.status == LA_EINVAL
    cap = la.la_max_grid_grouped(128, la.LA_BF16)
    if cap >= 993:                    # 993 grouped records of d = 128 exceed the 8 MiB
        with pytest.raises(la.LaError) as e:
            la.la_decode_noalloc(*args, kv_heads=2, grid=993)
        assert e.value.status == LA_EUNSUPPORTED and "scratch" in str(e.value)
    # 257 host-side requests: the schedule cannot travel in the kernel arguments
    many = W.make_custom([1] * 257, 2, 64, "f16", seed=3, device="cuda")
    out2 = torch.empty(tuple(many.q.shape), dtype=torch.float32, device="cuda")
    with pytest.raises(la.LaError) as e:
        la.la_decode_noalloc(many.q, many.k, many.v, many.ctx_lens, 257, 2, 64, many.scale, out2)
    assert e.value.status == LA_EUNSUPPORTED
    got = call(la, la.la_decode_noalloc, inp)
    check_oracle(got, oracle_of(inp), "after refusals")


def test_timeout_stays_in_its_launch(la):
    """Waits forced to give up (1 us bound) in three allocation-free
    launches; with the bound restored and no la_sync_check in between, the
    next launches are exact, and la_sync_check reports the timeout once.
    Request 0's one-token tile puts its host's wait a full 8192-token tile
    ahead of its first peer's publish, so the bound always runs out."""
    lens, opts = [1, 8192 * 5], dict(tile_tokens=8192, grid=3)
    H, Hk, d = 4, 1, 128
    inp = W.make_custom(lens, H, d, "bf16", seed=12, device="cuda", kv_heads=Hk)
    ref = oracle_of(inp)
    la.la_sync_check()
    out = torch.empty((inp.B, H, d), dtype=torch.float32, device="cuda")
    try:
        la.la_set_wait_limit_us(1)
        for _ in range(3):
            la.la_decode_noalloc(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, H, d, inp.scale, out,
                                 kv_heads=Hk, **opts)
    finally:
        la.la_set_wait_limit_us(0)
    for i in range(2):
        rows = inp.B * H
        o = torch.full((inp.B, H, d), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_noalloc(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, H, d, inp.scale, o,
                             kv_heads=Hk, m_out=m, l_out=l, **opts)
        torch.cuda.synchronize()
        check_oracle((o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()), ref, f"after {i}")
    with pytest.raises(la.LaError) as e:
        la.la_sync_check()
    assert e.value.status == LA_ETIMEOUT
    la.la_sync_check()
