"""GPU parity for several new tokens per request (causal verification of a
draft): the grouped MFMA kernels with query columns = (query head, token),
through the C ABI, against the fp64 oracle. Same bar as the other kernels:
max |dO| <= 1e-3, l within 1e-5 relative after rescaling to the oracle's max,
m within 1e-5, and the executed tile-to-workgroup map bit-exact."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fullsize_ref import full_reference
from oracle.schedule import lean_schedule

pytestmark = pytest.mark.gpu

O_TOL = 1e-3
L_RTOL = 1e-5
M_RTOL = 1e-5
KINDS = ["lean", "fixed_split", "per_head"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def run(la, inp, kind="lean", **opts):
    B, H, d, Nq = inp.B, inp.H, inp.d, inp.Nq
    out = torch.full((B, Nq, H, d), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((B * Nq * H,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((B * Nq * H,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                    m_out=m, l_out=l, kv_heads=inp.Hk, q_tokens=Nq, **opts)
    la.la_sync_check()
    return (out.cpu().numpy(), m.view(B, Nq, H).cpu().numpy(), l.view(B, Nq, H).cpu().numpy())


def reference(inp, heads=None):
    return oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                              inp.scale, inp.dtype, heads=heads, workers=16, kv_heads=inp.Hk)


def check(got, ref, heads=None, tag=""):
    O, m, l = got
    Or, mr, lr = ref
    if heads is not None:
        idx = tuple(np.array(heads).T)
        O, m, l, Or, mr, lr = O[idx], m[idx], l[idx], Or[idx], mr[idx], lr[idx]
    assert np.isfinite(O).all(), tag
    err = float(np.max(np.abs(O - Or)))
    assert err <= O_TOL, f"{tag}: max |dO| = {err}"
    assert np.all(np.abs(m - mr) <= M_RTOL * np.maximum(1.0, np.abs(mr))), f"{tag}: m"
    lrel = np.abs(l * np.exp(m.astype(np.float64) - mr) - lr) / lr
    assert float(np.max(lrel)) <= L_RTOL, f"{tag}: l rel err {float(np.max(lrel))}"
    return err


def units_per_req(H, Hk, Nq):
    return Hk * ((H // Hk * Nq + 15) // 16)


# lengths that put the masked keys of the last tokens in awkward places: a
# cache of exactly Nq rows, a last tile of one key (whole tiles masked for
# early tokens), masked keys straddling a tile and a 128-key step boundary
def edge_lengths(Nq, L):
    return [Nq, L + 1, 2 * L + Nq - 1, 3 * L - 1, 5 * L + 2, 700, 1111]


@pytest.mark.parametrize("Nq", [2, 3, 4, 8])
@pytest.mark.parametrize("H,Hk", [(4, 4), (8, 2), (16, 1), (12, 4)])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_tokens_ragged(la, Nq, H, Hk, dtype, d):
    L = la.la_default_tile(d)
    lens = edge_lengths(Nq, L)
    say(f"[multi ragged] Nq={Nq} H={H} Hk={Hk} {dtype} d={d} lens={lens}")
    inp = W.make_custom(lens, H, d, dtype, seed=Nq * 100 + H + Hk, device="cuda", kv_heads=Hk,
                        q_tokens=Nq)
    ref = reference(inp)
    for kind in KINDS:
        check(run(la, inp, kind), ref, tag=f"{kind} Nq={Nq} H={H} Hk={Hk} {dtype} d={d}")


@pytest.mark.parametrize("host_tables", [False, True])
@pytest.mark.parametrize("grid,tile", [(1, 128), (7, 128), (64, 32), (300, 256), (512, 128)])
def test_schedule_invariance_and_tile_map(la, grid, tile, host_tables):
    H, Hk, Nq, d = 8, 2, 4, 128
    lens = [515, 4, 1030, 129, 2000]
    say(f"[multi sched] grid={grid} tile={tile}")
    inp = W.make_custom(lens, H, d, "bf16", seed=21, device="cuda", kv_heads=Hk, q_tokens=Nq)
    ref = reference(inp)
    U = units_per_req(H, Hk, Nq)
    sch = lean_schedule(lens, U, tile, grid)
    owner = torch.full((sch["I"],), -1, dtype=torch.int32, device="cuda")
    got = run(la, inp, "lean", grid=grid, tile_tokens=tile, tile_owner=owner,
              host_tables=host_tables)
    check(got, ref, tag=f"grid={grid} tile={tile}")
    want = np.repeat(np.arange(sch["G"]), np.diff(sch["cta_begin"]))
    np.testing.assert_array_equal(owner.cpu().numpy(), want)


@pytest.mark.parametrize("H,Hk,Nq", [(8, 1, 4), (16, 2, 8), (4, 4, 16), (2, 1, 64)])
def test_several_column_blocks(la, H, Hk, Nq):
    """More than 16 columns per K/V head: the head is cut into blocks of 16
    columns, which may split a query head's tokens across blocks."""
    lens = [Nq, 300, 901]
    say(f"[multi blocks] H={H} Hk={Hk} Nq={Nq}")
    inp = W.make_custom(lens, H, 64, "f16", seed=31 + Nq, device="cuda", kv_heads=Hk, q_tokens=Nq)
    ref = reference(inp)
    for kind in KINDS:
        check(run(la, inp, kind), ref, tag=f"{kind} H={H} Hk={Hk} Nq={Nq}")
    check(run(la, inp, "lean", grid=97, tile_tokens=64), ref, tag="lean grid 97")


def test_one_token_in_four_d_layout_matches_plain_call(la):
    """q_tokens = 1 with grouped heads is the plain grouped decode."""
    inp = W.make_custom([300, 77], 8, 128, "bf16", seed=41, device="cuda", kv_heads=2)
    out1 = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    out2 = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, 2, 8, 128, inp.scale, out1, kv_heads=2)
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, 2, 8, 128, inp.scale, out2, kv_heads=2,
                    q_tokens=1)
    la.la_sync_check()
    assert torch.equal(out1, out2)


def _truncated_cache(inp, keep):
    """Packed K/V of the same requests with request b cut to keep[b] rows."""
    Hk, d = inp.Hk, inp.d
    ks, vs = [], []
    row = 0
    for n, kb in zip(inp.ctx_lens, keep):
        blk_k = inp.k[row:row + Hk * n].view(Hk, n, d)[:, :kb]
        blk_v = inp.v[row:row + Hk * n].view(Hk, n, d)[:, :kb]
        ks.append(blk_k.reshape(Hk * kb, d))
        vs.append(blk_v.reshape(Hk * kb, d))
        row += Hk * n
    return torch.cat(ks).contiguous(), torch.cat(vs).contiguous()


@pytest.mark.parametrize("H,Hk", [(4, 4), (8, 2)])
def test_equals_one_token_decodes_of_the_prefix(la, H, Hk):
    """Token t of Nq gives what a one-token decode over the first
    n_b - Nq + 1 + t rows gives (the one-token kernels: a different path)."""
    Nq, d = 5, 128
    lens = [5, 260, 1500]
    inp = W.make_custom(lens, H, d, "bf16", seed=51, device="cuda", kv_heads=Hk, q_tokens=Nq)
    multi = run(la, inp, "lean")[0]
    for t in range(Nq):
        keep = [n - Nq + 1 + t for n in lens]
        k, v = _truncated_cache(inp, keep)
        q1 = inp.q[:, t].contiguous()
        out = torch.empty((len(lens), H, d), dtype=torch.float32, device="cuda")
        la.la_decode_ex(q1, k, v, keep, len(lens), H, d, inp.scale, out, kv_heads=Hk)
        la.la_sync_check()
        err = float(np.max(np.abs(out.cpu().numpy() - multi[:, t])))
        assert err <= O_TOL, f"token {t}: {err}"


def test_determinism(la):
    inp = W.make_custom([3000, 40], 16, 128, "bf16", seed=61, device="cuda", kv_heads=4,
                        q_tokens=4)
    a = run(la, inp, "lean")
    for _ in range(3):
        b = run(la, inp, "lean")
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name,seed", [("spec4-ragged", 0), ("spec4-ragged", 3), ("spec8-64k", 0)])
def test_full_size(la, name, seed):
    """Every kind on the full workload (the ragged one also at a second draw
    of its lengths), every (request, new token, query head) against the
    oracle."""
    say(f"[multi full {name} seed {seed}]")
    inp = W.make_inputs(name, seed=seed, device="cuda")
    ref = full_reference(name, seed, inp)
    for k in KINDS:
        err = check(run(la, inp, k), ref, tag=f"{name}/{k}")
        say(f"[multi full {name}] {k} max|dO|={err:.2e}")
    del inp
    torch.cuda.empty_cache()
