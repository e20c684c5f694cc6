"""The C ABI from a plain C program (tests/c_abi/decode_from_c.c): it builds
against include/la_decode.h with a C compiler and links libla_decode.so (CPU
test), and on the GPU its calls -- la_decode_bf16 with the plain argument
list, la_decode_ex with kind auto over grouped K/V heads, and a decode step
with the lengths in device memory captured into a HIP graph and replayed over
growing lengths -- match the fp64 oracle on the bits it wrote out."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "decode_from_c.c")
LIBDIR = os.path.join(ROOT, "decode_phase_attention_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libla_decode.so")):
        pytest.skip("libla_decode.so not built")
    exe = str(tmp_path / "decode_from_c")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC, f"-L{ROCM}/lib", "-lamdhip64",
           f"-L{LIBDIR}", "-lla_decode", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_builds_and_links(tmp_path):
    exe = build(tmp_path)
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_c_program_matches_oracle(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build(tmp_path)
    out = tmp_path / "result.bin"
    r = subprocess.run([exe, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(out, "rb").read()
    B, H, HK, D = np.frombuffer(raw[:16], np.int32)
    lens = np.frombuffer(raw[16:16 + 4 * B], np.int32).tolist()
    n = sum(lens)
    off = 16 + 4 * B
    q = np.frombuffer(raw, np.uint16, B * H * D, off).reshape(B, H, D)
    off += 2 * B * H * D
    k = np.frombuffer(raw, np.uint16, H * n * D, off).reshape(H * n, D)
    off += 2 * H * n * D
    v = np.frombuffer(raw, np.uint16, H * n * D, off).reshape(H * n, D)
    off += 2 * H * n * D
    out1 = np.frombuffer(raw, np.float32, B * H * D, off).reshape(B, H, D)
    off += 4 * B * H * D
    out2 = np.frombuffer(raw, np.float32, B * H * D, off).reshape(B, H, D)
    scale = float(np.float32(0.08838834764831845))
    ref1 = oracle.attend_fp64(q, k, v, lens, scale, "bf16", workers=8)[0]
    ref2 = oracle.attend_fp64(q, k[:HK * n], v[:HK * n], lens, scale, "bf16", workers=8,
                              kv_heads=int(HK))[0]
    assert float(np.max(np.abs(out1 - ref1))) <= 1e-3
    assert float(np.max(np.abs(out2 - ref2))) <= 1e-3
    off += 4 * B * H * D
    S, steps = 1024, 3
    ks = np.frombuffer(raw, np.uint16, B * H * S * D, off).reshape(B, H, S, D)
    off += 2 * B * H * S * D
    vs = np.frombuffer(raw, np.uint16, B * H * S * D, off).reshape(B, H, S, D)
    off += 2 * B * H * S * D
    out3 = np.frombuffer(raw, np.float32, steps * B * H * D, off).reshape(steps, B, H, D)
    assert off + 4 * steps * B * H * D == len(raw)
    for i in range(steps):
        ln = [x + i + 1 for x in lens]
        kp = np.concatenate([ks[b, :, :x].reshape(-1, D) for b, x in enumerate(ln)])
        vp = np.concatenate([vs[b, :, :x].reshape(-1, D) for b, x in enumerate(ln)])
        ref3 = oracle.attend_fp64(q, kp, vp, ln, scale, "bf16", workers=8)[0]
        assert float(np.max(np.abs(out3[i] - ref3))) <= 1e-3, i
