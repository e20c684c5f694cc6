"""Context lengths read on the device (la_opts.ctx_lens_device) and lean
launches captured into HIP graphs.

With device lengths the lean kernels compute the stream-K partition in the
launch from a device array, so a captured decode step stays valid while the
lengths grow: the same tile map and output bits as host lengths on the same
grid, out-of-range lengths reported by la_sync_check (nothing computed), and
a captured step replayed as a decode loop matches the oracle and the eager
call at every step."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

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


def run(la, inp, kc, vc, S, lens=None, dlens=None, **opts):
    rows = int(np.prod(tuple(inp.q.shape)[:-1]))
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, kc, vc, lens, inp.B, inp.H, inp.d, inp.scale, out, m_out=m, l_out=l,
                    kv_heads=inp.Hk, q_tokens=inp.Nq, kv_stride=S, ctx_lens_device=dlens, **opts)
    la.la_sync_check()
    return out.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()


CASES = [([3000, 17, 60000, 129], 4, 4, 1, 128, "bf16"),
         ([1, 700, 256, 2049], 8, 2, 1, 64, "f16"),
         ([515, 4, 1030], 8, 2, 3, 128, "bf16"),
         ([int(x) for x in np.random.default_rng(3).integers(1, 400, 256)], 2, 2, 1, 64, "f16"),
         ([int(x) for x in np.random.default_rng(4).integers(1, 300, 600)], 4, 4, 1, 128, "bf16"),
         ([int(x) for x in np.random.default_rng(5).integers(2, 300, 1024)], 2, 1, 2, 64, "f16"),
         ([300, 64, 1000], 2, 1, 64, 64, "f16")]      # 64 new tokens: 8 column blocks per K/V head


@pytest.mark.parametrize("lens,H,Hk,Nq,d,dtype", CASES)
@pytest.mark.parametrize("grid", [0, 37, "max"])
def test_device_lengths_match_host_lengths(la, lens, H, Hk, Nq, d, dtype, grid):
    """Same grid, same partition: the device-length launch gives the host-length
    launch's output, m and l bit for bit, and both meet the oracle. A grid
    larger than the tile iterations leaves the extra workgroups idle. Above 256
    requests the host lengths go through the host-built tables, so those cases
    also compare the tables with the partition computed in the launch."""
    inp = W.make_custom(lens, H, d, dtype, seed=len(lens) + H + Nq, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
    grouped = H // Hk * Nq > 1
    if grid == "max":
        grid = la.la_max_grid_grouped(d, dt) if grouped else la.la_max_grid(d, dt)
    S = max(lens) + 5
    say(f"[device lens] B={len(lens)} H={H} Hk={Hk} Nq={Nq} d={d} grid={grid}")
    kc, vc = strided(inp, S)
    host = run(la, inp, kc, vc, S, lens=lens, grid=grid)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dev = run(la, inp, kc, vc, S, dlens=dl, grid=grid)
    for x, y in zip(host, dev):
        np.testing.assert_array_equal(x, y)
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, dtype, workers=16, kv_heads=Hk)[0]
    assert float(np.max(np.abs(dev[0] - ref))) <= 1e-3


def test_out_of_range_device_lengths(la):
    """A zero length, one past the cache and one shorter than the new tokens:
    the kernel computes nothing and la_sync_check reports LA_EINVAL; the next
    good call is unaffected."""
    lens = [300, 40]
    inp = W.make_custom(lens, 4, 64, "f16", seed=9, device="cuda", kv_heads=2, q_tokens=2)
    S = 512
    kc, vc = strided(inp, S)
    for bad in ([0, 40], [S + 1, 40], [300, 1]):
        say(f"[bad device lens] {bad}")
        dl = torch.tensor(bad, dtype=torch.int32, device="cuda")
        out = torch.full(tuple(inp.q.shape), 7.0, dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, kc, vc, None, 2, 4, 64, inp.scale, out, kv_heads=2, q_tokens=2,
                        kv_stride=S, ctx_lens_device=dl)
        with pytest.raises(la.LaError) as e:
            la.la_sync_check()
        assert e.value.status == 1 and "lengths" in str(e.value)
        assert bool((out == 7.0).all())          # nothing written
    got = run(la, inp, kc, vc, S, dlens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "f16", workers=8, kv_heads=2)[0]
    assert float(np.max(np.abs(got[0] - ref))) <= 1e-3


def packed_prefix(bits, final, lens, Hk, d):
    """Rows of a packed [Hk * sum(final), d] K or V holding, per request, the
    first lens[b] rows of each head: the packed cache of the shorter contexts."""
    parts, row = [], 0
    for nf, n in zip(final, lens):
        parts.append(bits[row:row + Hk * nf].reshape(Hk, nf, d)[:, :n].reshape(-1, d))
        row += Hk * nf
    return np.concatenate(parts)


@pytest.mark.parametrize("H,Hk,Nq,d,dtype", [(8, 2, 1, 128, "bf16"), (16, 16, 1, 64, "f16"),
                                              (8, 1, 2, 64, "f16")])
def test_graph_captured_decode_loop(la, H, Hk, Nq, d, dtype):
    """One lean decode step captured into a graph with the lengths on the
    device; eager work between replays grows every context by one token.
    Each replay equals the eager call on the same lengths bit for bit and
    meets the oracle. A call on the capturing stream that grows its
    workspace in the middle of the loop leaves the graph valid."""
    lens0 = [1000, 37, 1500]
    steps = 8
    final = [n + steps for n in lens0]
    S = 2048
    inp = W.make_custom(final, H, d, dtype, seed=H + Nq, device="cuda", kv_heads=Hk, q_tokens=Nq)
    kc, vc = strided(inp, S)
    dl = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
    eager = torch.empty_like(out)
    big = torch.empty_like(out)
    kw = dict(kv_heads=Hk, q_tokens=Nq, kv_stride=S, grid=64)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):            # sizes the stream's workspace
        la.la_decode_ex(inp.q, kc, vc, None, 3, H, d, inp.scale, out, ctx_lens_device=dl,
                        stream=s.cuda_stream, **kw)
    s.synchronize()
    la.la_sync_check(s.cuda_stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        la.la_decode_ex(inp.q, kc, vc, None, 3, H, d, inp.scale, out, ctx_lens_device=dl,
                        stream=s.cuda_stream, **kw)
    kb, vb, qb = W.to_bits(inp.k), W.to_bits(inp.v), W.to_bits(inp.q)
    for i in range(steps):
        lens = [n + i + 1 for n in lens0]
        say(f"[graph step {i}] H={H} Hk={Hk} Nq={Nq} d={d} lens={lens}")
        with torch.cuda.stream(s):
            dl.add_(1)                          # eager: the step's new token
            g.replay()
        s.synchronize()
        la.la_sync_check(s.cuda_stream)
        la.la_decode_ex(inp.q, kc, vc, lens, 3, H, d, inp.scale, eager, **kw)
        la.la_sync_check()
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got, eager.cpu().numpy())
        ref = oracle.attend_fp64(qb, packed_prefix(kb, final, lens, Hk, d),
                                 packed_prefix(vb, final, lens, Hk, d), lens, inp.scale, dtype,
                                 workers=8, kv_heads=Hk)[0]
        assert float(np.max(np.abs(got - ref))) <= 1e-3, i
        if i == 3:
            # a larger grid on the capturing stream grows its workspace
            la.la_decode_ex(inp.q, kc, vc, None, 3, H, d, inp.scale, big, ctx_lens_device=dl,
                            stream=s.cuda_stream, **dict(kw, grid=256))
            s.synchronize()
            la.la_sync_check(s.cuda_stream)
            assert float(np.max(np.abs(big.cpu().numpy() - ref))) <= 1e-3
    del g


def test_capture_refusals(la):
    """Refused before anything is enqueued: capture on a stream with no
    workspace yet, capture that would have to grow the workspace, capture of
    a kind that uploads tables, a cooperative launch. The stream works
    normally afterwards."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    hip.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    lens = [300, 40]
    inp = W.make_custom(lens, 4, 64, "f16", seed=12, device="cuda")
    S = 512
    kc, vc = strided(inp, S)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((2, 4, 64), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    ptr = ctypes.c_void_p(s.cuda_stream)

    def captured(**opts):
        torch.cuda.synchronize()
        assert hip.hipStreamBeginCapture(ptr, 2) == 0            # relaxed mode
        try:
            with pytest.raises(la.LaError) as e:
                la.la_decode_ex(inp.q, kc, vc, opts.pop("lens", None), 2, 4, 64, inp.scale, out,
                                stream=s.cuda_stream, kv_stride=S, **opts)
        finally:
            graph = ctypes.c_void_p()
            assert hip.hipStreamEndCapture(ptr, ctypes.byref(graph)) == 0
            if graph.value:
                hip.hipGraphDestroy(graph)
        assert e.value.status == 2, str(e.value)
        return str(e.value)

    assert "workspace" in captured(ctx_lens_device=dl)          # no workspace on s yet
    la.la_decode_ex(inp.q, kc, vc, None, 2, 4, 64, inp.scale, out, stream=s.cuda_stream,
                    kv_stride=S, ctx_lens_device=dl, grid=16)
    s.synchronize()
    assert "grow" in captured(ctx_lens_device=dl, grid=512)     # more workgroups than sized for
    assert "lean" in captured(lens=lens, kind="pull")           # tables through staging
    assert "lean" in captured(lens=lens, host_tables=True)
    assert "cooperative" in captured(ctx_lens_device=dl, grid=16, cooperative=True)
    la.la_decode_ex(inp.q, kc, vc, lens, 2, 4, 64, inp.scale, out, stream=s.cuda_stream,
                    kv_stride=S)
    s.synchronize()
    la.la_sync_check(s.cuda_stream)
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "f16", workers=8)[0]
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= 1e-3


def test_random_device_lengths(la):
    """Random shapes (head dims, dtypes, grouped heads, new tokens, up to 1024
    requests, lengths at tile edges), random grids and tiles on capacity-strided
    caches: device lengths give the host-length bits and meet the oracle."""
    rng = np.random.default_rng(4242)
    worst = 0.0
    for i in range(30):
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        H = int(rng.choice([1, 2, 4, 8, 16]))
        Hk = int(rng.choice([h for h in (1, 2, 4, 8, 16) if H % h == 0]))
        Nq = int(rng.choice([1, 1, 2, 5]))
        B = int(rng.choice([1, 3, 8, 64, 256, 700, 1024]))
        L = 128 if d == 128 else 256
        hi = 20000 if B <= 8 else 600
        lens = []
        for _ in range(B):
            if rng.random() < 0.25:
                n = int(rng.integers(1, 4)) * L + int(rng.integers(-1, 2))
            else:
                n = int(np.exp(rng.uniform(0, np.log(hi))))
            lens.append(max(n, Nq))
        grouped = H // Hk * Nq > 1
        dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
        cap = la.la_max_grid_grouped(d, dt) if grouped else la.la_max_grid(d, dt)
        grid = int(rng.choice([0, 1, int(rng.integers(1, cap + 1)), cap]))
        tile = int(rng.choice([0, 16, 64, 300]))
        S = max(lens) + int(rng.integers(0, 50))
        say(f"[random device lens {i}] d={d} {dtype} H={H} Hk={Hk} Nq={Nq} B={B} grid={grid} "
            f"tile={tile} S={S} max_len={max(lens)}")
        inp = W.make_custom(lens, H, d, dtype, seed=500 + i, device="cuda", kv_heads=Hk,
                            q_tokens=Nq)
        kc, vc = strided(inp, S)
        host = run(la, inp, kc, vc, S, lens=lens, grid=grid, tile_tokens=tile)
        dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        dev = run(la, inp, kc, vc, S, dlens=dl, grid=grid, tile_tokens=tile)
        for x, y in zip(host, dev):
            np.testing.assert_array_equal(x, y)
        ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                                 inp.scale, dtype, workers=16, kv_heads=Hk)[0]
        err = float(np.max(np.abs(dev[0] - ref)))
        assert err <= 1e-3, (i, err)
        worst = max(worst, err)
        del inp, kc, vc
    say(f"30 random device-length launches, worst max|dO| = {worst:.2e}")


def test_wrapper_takes_device_lengths(la):
    """decode_attention with an int32 device tensor of lengths and a 4-D cache
    gives the host-length call's bits; with a packed cache it is refused."""
    lens = [700, 33, 2049]
    inp = W.make_custom(lens, 8, 128, "bf16", seed=71, device="cuda", kv_heads=2)
    S = 2100
    kc, vc = strided(inp, S)
    host = la.decode_attention(inp.q, kc, vc, lens)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dev = la.decode_attention(inp.q, kc, vc, dl)
    auto = la.decode_attention(inp.q, kc, vc, dl, kind="auto")   # lean: the one kind that reads them
    la.la_sync_check()
    np.testing.assert_array_equal(host.cpu().numpy(), dev.cpu().numpy())
    np.testing.assert_array_equal(dev.cpu().numpy(), auto.cpu().numpy())
    with pytest.raises(ValueError, match="cache"):
        la.decode_attention(inp.q, inp.k, inp.v, dl)


def test_graph_captured_with_host_lengths(la):
    """A lean launch with host lengths within the in-launch limits (prefix sums
    in the kernel arguments) can be captured too: each replay repeats those
    lengths and equals the eager call bit for bit, with eager work between
    replays."""
    lens = [900, 17, 3000]
    inp = W.make_custom(lens, 8, 64, "f16", seed=91, device="cuda", kv_heads=2)
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
    eager = torch.empty_like(out)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, 3, 8, 64, inp.scale, out, kv_heads=2,
                        stream=s.cuda_stream)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, 3, 8, 64, inp.scale, out, kv_heads=2,
                        stream=s.cuda_stream)
    la.la_decode_ex(inp.q, inp.k, inp.v, lens, 3, 8, 64, inp.scale, eager, kv_heads=2)
    la.la_sync_check()
    ref = eager.cpu().numpy()
    for i in range(4):
        out.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        la.la_sync_check(s.cuda_stream)
        np.testing.assert_array_equal(out.cpu().numpy(), ref)
    del g


@pytest.mark.parametrize("lens", [[262144, 262144], [262144, 262143]],
                         ids=["uniform", "one-token-apart"])
def test_staggered_starts_same_bits_from_host_and_device(la, lens):
    """Long ranges of a launch whose lengths are all equal start at a staggered
    step in each workgroup (the single-head lean kernel). The host decides that
    from its lengths and the launch from the lengths it reads itself, so the
    two sources must give the same bits whether the lengths are equal (ranges
    of 64 steps here, staggered) or one token apart (not staggered); both
    meet the oracle."""
    H, d = 4, 128
    inp = W.make_custom(lens, H=H, d=d, dtype="bf16", seed=sum(lens) % 997, device="cuda")
    S = max(lens)
    kc, vc = strided(inp, S)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    say(f"[staggered starts] lens={lens}")
    host = run(la, inp, kc, vc, S, lens=lens)
    dev = run(la, inp, kc, vc, S, dlens=dl)
    for x, y in zip(host, dev):
        np.testing.assert_array_equal(x, y)
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "bf16", workers=16)
    err = float(np.max(np.abs(host[0] - ref[0])))
    assert err <= 1e-3, err
    del inp, kc, vc
    torch.cuda.empty_cache()
