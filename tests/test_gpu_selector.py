"""GPU parity of kind="auto" (the shape-driven choice among the kernels):
whichever kernel and grid it picks, the output meets the oracle bar (max |dO|
<= 1e-3, l within 1e-5 relative, m within 1e-5), and the pick is the one
la_select reports."""
from __future__ import annotations

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


CASES = [
    # (lens, H, Hk, Nq, d, dtype, expected pick on a 256-CU device)
    ([3000, 17, 60000], 8, 8, 1, 128, "bf16", "lean"),
    ([1024] * 64, 8, 8, 1, 128, "bf16", "per_head"),     # 512 whole heads on 512 workgroups
    ([256] * 128, 32, 32, 1, 64, "f16", "per_head"),       # whole heads of one tile each
    ([256] * 256, 32, 8, 1, 128, "bf16", "lean"),          # whole grouped units of 2 tiles
    ([2048] * 128, 32, 32, 1, 64, "f16", "per_head"),
    ([5000, 900, 33], 32, 8, 1, 128, "bf16", "lean"),
    ([2048] * 64, 64, 8, 1, 128, "bf16", "per_head"),    # grouped units: 512 whole units
    ([700, 4000], 16, 4, 4, 64, "f16", "lean"),          # several new tokens
]


@pytest.mark.parametrize("lens,H,Hk,Nq,d,dtype,want", CASES)
def test_auto_parity(la, lens, H, Hk, Nq, d, dtype, want):
    say(f"[auto] B={len(lens)} H={H} Hk={Hk} Nq={Nq} d={d} {dtype}")
    inp = W.make_custom(lens, H, d, dtype, seed=len(lens) + H, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
    pick, grid = la.la_select(lens, H, d, dt, kv_heads=Hk, q_tokens=Nq)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        assert pick == want
    shape = tuple(inp.q.shape)
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    rows = int(np.prod(shape[:-1]))
    m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out, kind="auto",
                    m_out=m, l_out=l, kv_heads=Hk, q_tokens=Nq)
    la.la_sync_check()
    Or, mr, lr = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                                    inp.scale, dtype, workers=16, kv_heads=Hk)
    O = out.cpu().numpy()
    M = m.cpu().numpy().reshape(mr.shape)
    L = l.cpu().numpy().reshape(lr.shape)
    err = float(np.max(np.abs(O - Or)))
    assert err <= 1e-3, err
    assert np.all(np.abs(M - mr) <= 1e-5 * np.maximum(1.0, np.abs(mr)))
    assert float(np.max(np.abs(L * np.exp(M.astype(np.float64) - mr) - lr) / lr)) <= 1e-5
    say(f"[auto] picked {pick}@{grid}, max|dO|={err:.2e}")


def test_decode_attention_wrapper(la):
    """The convenience wrapper: shapes from the tensors, 4-D q for several new
    tokens, grouped K/V heads, kind auto."""
    lens = [900, 37]
    inp = W.make_custom(lens, 8, 64, "f16", seed=5, device="cuda", kv_heads=2, q_tokens=3)
    out = la.decode_attention(inp.q, inp.k, inp.v, lens, kind="auto", kv_heads=2)
    la.la_sync_check()
    assert tuple(out.shape) == (2, 3, 8, 64) and out.dtype == torch.float32
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                             inp.scale, "f16", workers=8, kv_heads=2)[0]
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= 1e-3
    with pytest.raises(ValueError):       # K/V sized for 2 heads, called as 8
        la.decode_attention(inp.q, inp.k, inp.v, lens)


SHARED = [
    # (lens, H, Hk, Nq, d, dtype): lean picks become pull; a per-head pick stays
    ([3000, 17, 60000], 8, 8, 1, 128, "bf16"),
    ([5000, 900, 33], 32, 8, 1, 128, "bf16"),
    ([700, 4000], 16, 4, 4, 64, "f16"),
    ([1024] * 64, 8, 8, 1, 128, "bf16"),
]


@pytest.mark.parametrize("lens,H,Hk,Nq,d,dtype", SHARED)
def test_shared_gpu(la, lens, H, Hk, Nq, d, dtype):
    """shared_gpu: kind auto takes the dynamic pull on one workgroup per CU
    wherever it would take lean, and the call gives the explicit pull's bits
    (pull output does not depend on the grid or on which workgroup took a
    chunk), within the oracle bar."""
    say(f"[shared] B={len(lens)} H={H} Hk={Hk} Nq={Nq} d={d} {dtype}")
    dt = la.LA_BF16 if dtype == "bf16" else la.LA_F16
    base = la.la_select(lens, H, d, dt, kv_heads=Hk, q_tokens=Nq)
    pick, grid = la.la_select(lens, H, d, dt, kv_heads=Hk, q_tokens=Nq, shared_gpu=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if base[0] == "lean":
        assert (pick, grid) == ("pull", cus)
    else:
        assert (pick, grid) == base
    inp = W.make_custom(lens, H, d, dtype, seed=len(lens) + 3 * H, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    shape = tuple(inp.q.shape)
    rows = int(np.prod(shape[:-1]))
    outs = []
    for opts in ({"kind": "auto", "shared_gpu": True}, {"kind": pick, "grid": grid}):
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        la.la_decode_ex(inp.q, inp.k, inp.v, lens, len(lens), H, d, inp.scale, out, m_out=m,
                        l_out=l, kv_heads=Hk, q_tokens=Nq, **opts)
        la.la_sync_check()
        outs.append([t.cpu().numpy() for t in (out, m, l)])
    for x, y in zip(*outs):
        np.testing.assert_array_equal(x, y)
    Or = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), lens,
                            inp.scale, dtype, workers=16, kv_heads=Hk)[0]
    err = float(np.max(np.abs(outs[0][0] - Or)))
    assert err <= 1e-3, err
    say(f"[shared] {base[0]} -> {pick}@{grid}, max|dO|={err:.2e}")
