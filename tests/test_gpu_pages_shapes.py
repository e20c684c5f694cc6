"""GPU parity on the shapes of the pages' evaluation sweeps that bench.py
--pages-sweep times (xllm-io paper review, §5.2 and §5.4: context at 56 heads,
heads at 64k tokens, batch at 56 heads, the extremes the pages quote, head
dim 128; and few heads at long contexts, review §4.3): every kind the sweep
times, every query row against the fp64 oracle, to the same bar as
tests/test_gpu_parity.py (max |dO| <= 1e-3; m and rescaled l within 1e-5).
Shapes whose K/V exceed ~4 GB (copied to the host for the oracle) are left to
the sweep's timing alone."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

O_TOL = 1e-3
L_RTOL = 1e-5
M_RTOL = 1e-5
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

# (sweep, B, H, d, n): d = 64 in fp16, d = 128 in bf16, as the sweep runs them
SHAPES = [
    ("context", 1, 56, 64, 1024),
    ("context", 1, 56, 64, 8192),
    ("context", 1, 56, 64, 65536),
    ("heads", 1, 24, 64, 65536),
    ("heads", 1, 192, 64, 65536),
    ("batch", 4, 56, 64, 65536),
    ("extremes", 1, 16, 64, 524288),
    ("extremes", 1, 24, 64, 1024),
    ("head_dim_128", 1, 56, 128, 1024),
    ("few_heads", 1, 1, 128, 524288),
    ("few_heads", 1, 2, 128, 524288),
    ("few_heads", 1, 4, 128, 32768),
]
KINDS = ["lean", "auto", "pull", "fixed_split", "per_head"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def run(la, inp, kind):
    B, H, d = inp.B, inp.H, inp.d
    out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((B * H,), float("nan"), dtype=torch.float32, device="cuda")
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                    m_out=m, l_out=l)
    la.la_sync_check()
    return out.cpu().numpy(), m.view(B, H).cpu().numpy(), l.view(B, H).cpu().numpy()


def check(got, ref, tag):
    O, m, l = got
    Or, mr, lr = ref
    assert np.isfinite(O).all(), tag
    err = float(np.max(np.abs(O - Or)))
    assert err <= O_TOL, f"{tag}: max |dO| = {err}"
    assert np.all(np.abs(m - mr) <= M_RTOL * np.maximum(1.0, np.abs(mr))), f"{tag}: m"
    lrel = np.abs(l * np.exp(m.astype(np.float64) - mr) - lr) / lr
    assert float(np.max(lrel)) <= L_RTOL, f"{tag}: l rel err {float(np.max(lrel))}"
    return err


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}-B{s[1]}-H{s[2]}-d{s[3]}-n{s[4]}")
def test_pages_sweep_shape(la, shape):
    sweep, B, H, d, n = shape
    dt = "f16" if d == 64 else "bf16"
    tag = f"{sweep} B={B} H={H} d={d} n={n}"
    say(f"[pages {tag}] generating")
    inp = W.make_custom([n] * B, H, d, dt, seed=B * 1000 + H + n, device="cuda")
    res = {kind: run(la, inp, kind) for kind in KINDS}
    say(f"[pages {tag}] kernels done")
    ref = oracle.attend_fp64(W.to_bits(inp.q), W.to_bits(inp.k), W.to_bits(inp.v), inp.ctx_lens,
                             inp.scale, inp.dtype, workers=WORKERS)
    for kind in KINDS:
        err = check(res[kind], ref, f"{tag}/{kind}")
        say(f"[pages {tag}] {kind} max|dO|={err:.2e}")
    del inp
    torch.cuda.empty_cache()
