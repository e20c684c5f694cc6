"""The C-ABI library on the host (no GPU): it loads, exports every function
include/la_decode.h declares, and its host-side scheduler produces the same
tables as the schedule oracle, field for field. Argument validation is checked
through calls that fail before any device work."""
from __future__ import annotations

import ctypes
import json
import os
import random
import re

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_decode.h")

la = pytest.importorskip("decode_phase_attention_amd")
if not os.path.exists(la.binding.LIB_PATH):
    pytest.skip("libla_decode.so not built", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    h = ctypes.CDLL(la.binding.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n
    # the binding wraps each of them under the same name
    assert set(names) - {"la_opts_init"} <= set(la.binding.__all__)


def compare_tables(lens, H, L, G):
    want = oracle.lean_schedule(lens, H, L, G)
    got = la.la_schedule(lens, H, L, G)
    assert got["I"] == want["I"] and got["G"] == want["G"]
    for key in ("cta_begin", "cta_seg", "host_cta", "last_cta"):
        assert got[key].tolist() == want[key], key
    assert [tuple(r) for r in got["seg"].tolist()] == want["seg"]


def test_schedule_golden_cases():
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "schedule_cases.json")))["cases"]
    for c in cases:
        got = la.la_schedule(c["ctx_lens"], c["H"], c["L"], c["G_req"])
        assert got["cta_begin"].tolist() == c["cta_begin"], c["name"]
        assert got["seg"].tolist() == c["seg"], c["name"]
        assert got["host_cta"].tolist() == c["host_cta"] and got["last_cta"].tolist() == c["last_cta"]


def test_schedule_random_bit_exact():
    rng = random.Random(2024)
    for _ in range(3000):
        B = rng.randint(1, 8)
        H = rng.randint(1, 6)
        L = rng.choice([1, 2, 5, 16, 64, 128, 256])
        lens = [rng.randint(1, 3000) for _ in range(B)]
        G = rng.randint(1, 1200)
        compare_tables(lens, H, L, G)


@pytest.mark.parametrize("name", ["tiny", "65k", "512k", "ragged", "many-heads"])
@pytest.mark.parametrize("G", [1, 3, 255, 256, 1024, 1280, 2048])
def test_schedule_bench_shapes(name, G):
    w = W.CONFIGS[name]
    for seed in ([0, 1, 2] if name == "ragged" else [0]):
        lens = W.context_lengths(w, seed)
        L = 128 if w.d == 128 else 256
        compare_tables(lens, w.H, L, G)


def test_default_tile():
    assert la.la_default_tile(128) == 128
    assert la.la_default_tile(64) == 256
    assert la.la_default_tile(96) == 0


def test_schedule_validation():
    with pytest.raises(la.LaError) as e:
        la.la_schedule([4, 0], 2, 4, 3)
    assert e.value.status == 1 and "context" in str(e.value)
    for args in (([4], 0, 4, 3), ([4], 1, 0, 3), ([4], 1, 4, 0)):
        with pytest.raises(la.LaError) as e:
            la.la_schedule(*args)
        assert e.value.status == 1
    with pytest.raises(la.LaError) as e:      # 2^31 tiles do not fit the int32 tables
        la.la_schedule([2 ** 30, 2 ** 30], 2, 1, 64)
    assert e.value.status == 2
    # max_rows below the bound is rejected rather than overrun
    lens = (ctypes.c_int32 * 2)(8, 8)
    buf = (ctypes.c_int32 * 64)()
    n = ctypes.c_int()
    st = la.lib().la_schedule(lens, 2, 1, 4, 3, buf, buf, buf, 1, ctypes.byref(n), buf, buf)
    assert st == 1


def test_decode_validation_before_device_work():
    """These calls fail in argument checking, before any HIP call."""
    L = la.lib()
    lens = (ctypes.c_int32 * 2)(16, 16)
    fake = 1 << 20                       # aligned, never dereferenced
    cases = [
        (dict(q=None), 1),
        (dict(B=0), 1),
        (dict(H=0), 1),
        (dict(d=96), 2),
        (dict(scale=float("inf")), 1),
        (dict(scale=float("nan")), 1),
        (dict(k=fake + 8), 1),           # misaligned
        (dict(dtype=7), 1),
    ]
    for over, want in cases:
        a = dict(q=fake, k=fake, v=fake, B=2, H=4, d=128, scale=0.1, out=fake, dtype=1)
        a.update(over)
        st = L.la_decode(a["q"], a["k"], a["v"], lens, a["B"], a["H"], a["d"], a["scale"],
                         a["out"], None, a["dtype"])
        assert st == want, (over, st, la.la_last_error())
    bad = (ctypes.c_int32 * 2)(16, 0)
    assert L.la_decode(fake, fake, fake, bad, 2, 4, 128, 0.1, fake, None, 1) == 1
    huge = (ctypes.c_int32 * 1)(1 << 24)        # one head's cache > 4 GiB at d = 128
    assert L.la_decode(fake, fake, fake, huge, 1, 1, 128, 0.1, fake, None, 1) == 2
    o = la.binding.LaOpts()
    L.la_opts_init(ctypes.byref(o))
    o.kind = 9
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    o.kind = 1
    o.tile_owner = fake
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "lean" in la.la_last_error()
    o.tile_owner = None
    o.cta_timestamps = fake            # fixed split with timestamps needs num_splits
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "num_splits" in la.la_last_error()
    o.cta_timestamps = None
    o.kind = 0
    o.q_tokens = 65                    # more new tokens than supported
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "q_tokens" in la.la_last_error()
    o.q_tokens = 17                    # contexts of 16 cannot hold 17 new tokens
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "new tokens" in la.la_last_error()
    o.q_tokens = -1
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1


def test_pull_kinds_validation():
    L = la.lib()
    lens = (ctypes.c_int32 * 2)(16, 16)
    fake = 1 << 20
    o = la.binding.LaOpts()
    L.la_opts_init(ctypes.byref(o))
    o.kind = la.LA_KIND_PULL
    o.chunk_tiles = -1
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    o.chunk_tiles = 0
    o.cta_timestamps = fake               # needs an explicit grid
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "grid" in la.la_last_error()
    o.kind = la.LA_KIND_CHUNKS            # needs an explicit chunk size
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "chunk_tiles" in la.la_last_error()


def test_binding_rejects_tensors_too_small_for_the_call():
    """The library sees pointers only; the binding checks torch tensors against
    the sizes the call implies (here on CPU tensors, before any device use)."""
    import torch
    q = torch.zeros(2, 8, 64, dtype=torch.float16)
    kv = torch.zeros(2 * 300, 64, dtype=torch.float16)      # 2 K/V heads x 300 tokens
    out = torch.zeros(2, 8, 64)
    with pytest.raises(ValueError, match="k_cache"):
        la.la_decode_ex(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out)        # as if 8 K/V heads
    with pytest.raises(ValueError, match="q "):
        la.la_decode_ex(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out, kv_heads=2, q_tokens=2)
    with pytest.raises(ValueError, match="out"):
        la.la_decode_ex(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out.half(), kv_heads=2)
    with pytest.raises(ValueError, match="device tensors"):        # sizes fine: then the device check
        la.la_decode_ex(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out, kv_heads=2)


def test_binding_rejects_mixed_input_types():
    """q, K and V must all be of the call's input type: the kernels read every
    input with it, so a bf16 cache under an fp16 query would be decoded as fp16
    bits (checked on CPU tensors, before any device use)."""
    import torch
    q = torch.zeros(2, 8, 64, dtype=torch.float16)
    kv = torch.zeros(8 * 300, 64, dtype=torch.float16)
    kvb = kv.bfloat16()
    out = torch.zeros(2, 8, 64)
    with pytest.raises(ValueError, match="k_cache is torch.bfloat16"):
        la.la_decode_ex(q, kvb, kv, [100, 200], 2, 8, 64, 0.125, out)
    with pytest.raises(ValueError, match="v_cache is torch.bfloat16"):
        la.la_decode(q, kv, kvb, [100, 200], 2, 8, 64, 0.125, out)
    with pytest.raises(ValueError, match="q is torch.float16"):
        la.la_decode_bf16(q, kvb, kvb, [100, 200], 2, 8, 64, 0.125, out)
    with pytest.raises(ValueError, match="q is torch.float16"):
        la.la_decode_ex(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out, dtype=la.LA_BF16)
    with pytest.raises(ValueError, match="device tensors"):        # types agree: the device check
        la.la_decode_f16(q, kv, kv, [100, 200], 2, 8, 64, 0.125, out)


def test_stream_read_validation_before_device_work():
    L = la.lib()
    n = ctypes.c_size_t()
    sink = 1 << 20
    assert L.la_stream_read(None, 1 << 20, 0, sink, None, ctypes.byref(n)) == 1
    assert L.la_stream_read(1 << 20, 1 << 20, 0, None, None, ctypes.byref(n)) == 1
    assert L.la_stream_read((1 << 20) + 8, 1 << 20, 0, sink, None, ctypes.byref(n)) == 1
    assert "aligned" in la.la_last_error()
    assert L.la_stream_read(1 << 20, 1 << 20, 0, sink, None, None) == 1


def test_package_exports_the_binding():
    assert set(la.binding.__all__) <= set(dir(la))
    assert "la_stream_read" in la.__all__


def test_kv_stride_validation_and_sizes():
    """A [B, Hk, kv_stride, d] cache: a negative stride or a context longer than
    the stride fails in argument checking; the binding sizes the cache as
    B * Hk * kv_stride rows."""
    import torch
    L = la.lib()
    lens = (ctypes.c_int32 * 2)(16, 40)
    fake = 1 << 20
    o = la.binding.LaOpts()
    L.la_opts_init(ctypes.byref(o))
    o.kv_stride = -1
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "kv_stride" in la.la_last_error()
    o.kv_stride = 32                   # the second context (40) does not fit
    assert L.la_decode_ex(fake, fake, fake, lens, 2, 4, 128, 0.1, fake, None, ctypes.byref(o)) == 1
    assert "exceeds kv_stride" in la.la_last_error()
    q = torch.zeros(2, 8, 64, dtype=torch.float16)
    out = torch.zeros(2, 8, 64)
    kv = torch.zeros(2 * 2 * 64 - 1, 64, dtype=torch.float16)   # one row short of [2, 2, 64, 64]
    with pytest.raises(ValueError, match="k_cache"):
        la.la_decode_ex(q, kv, kv, [16, 40], 2, 8, 64, 0.125, out, kv_heads=2, kv_stride=64)
    cache = torch.zeros(2, 2, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="cache"):
        la.decode_attention(q, cache, cache[:1], [16, 40])


def test_device_lengths_validation():
    """ctx_lens_device: refused in argument checking (before any device call)
    without a kv_stride cache, for any kind but lean, above 1024 requests, with
    host tables or a tile map, or misaligned; the binding wants an int32 tensor."""
    import torch
    L = la.lib()
    fake = 1 << 20
    o = la.binding.LaOpts()

    def call(B=2, **kw):
        L.la_opts_init(ctypes.byref(o))
        o.ctx_lens_device = fake
        o.kv_stride = 64
        for k, v in kw.items():
            setattr(o, k, v)
        st = L.la_decode_ex(fake, fake, fake, None, B, 4, 128, 0.1, fake, None, ctypes.byref(o))
        return st, la.la_last_error()

    st, msg = call(kv_stride=0)
    assert st == 1 and "kv_stride" in msg
    for kind in (la.LA_KIND_FIXED_SPLIT, la.LA_KIND_PER_HEAD, la.LA_KIND_PULL,
                 la.LA_KIND_CHUNKS):
        st, msg = call(kind=kind)
        assert st == 1 and "lean" in msg, kind
    st, msg = call(B=1025)
    assert st == 2 and "1024" in msg
    st, msg = call(host_tables=1)
    assert st == 1 and "host_tables" in msg
    st, msg = call(tile_owner=fake)
    assert st == 1 and "tile_owner" in msg
    st, msg = call(q_tokens=65 - 1, kv_stride=8)
    assert st == 1 and "q_tokens" in msg
    st, msg = call(ctx_lens_device=fake + 2)
    assert st == 1 and "aligned" in msg
    st, msg = call(kv_stride=(1 << 24) + 1)
    assert st == 2 and "4 GiB" in msg
    q = torch.zeros(2, 4, 64, dtype=torch.float16)
    out = torch.zeros(2, 4, 64)
    kv = torch.zeros(2, 4, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="int32"):
        la.la_decode_ex(q, kv, kv, None, 2, 4, 64, 0.125, out, kv_stride=64,
                        ctx_lens_device=torch.zeros(2, dtype=torch.int64))


def test_length_marshalling():
    """Host lengths reach the library as int32 values, whatever the Python
    container, and values outside int32 are refused rather than wrapped; the
    binding's size check sums them without wrapping."""
    import array
    b = la.binding
    for src in ([5, 7, 2**31 - 1], (5, 7, 2**31 - 1), array.array("i", [5, 7, 2**31 - 1]),
                np.array([5, 7, 2**31 - 1], dtype=np.int64)):
        owner, p = b._lens(src)
        assert [int(x) for x in owner] == [5, 7, 2**31 - 1]
        assert [p[i] for i in range(3)] == [5, 7, 2**31 - 1], type(src)
    for bad in ([2**31], [-2**31 - 1], np.array([2**40])):
        with pytest.raises(ValueError, match="int32"):
            b._lens(bad)
    import torch
    q = torch.zeros(2, 1, 64, dtype=torch.float16)
    out = torch.zeros(2, 1, 64)
    kv = torch.zeros(64, 64, dtype=torch.float16)
    owner, _ = b._lens(np.array([2**30, 2**30], dtype=np.int64))   # total 2^31: past int32
    with pytest.raises(ValueError, match="k_cache"):
        b._check_sizes(q, kv, kv, out, owner, 2, 1, 64)


def test_opts_struct_matches_the_header(tmp_path):
    """The binding's ctypes mirror of la_opts has the header's fields, in its
    order, at the offsets a C compiler gives them, and the same size."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [name for name, _ in la.binding.LaOpts._fields_]
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct la_opts \{(.*?)\} la_opts;", text, flags=re.S).group(1)
    assert re.findall(r"(\w+)\s*;", body) == fields
    src = tmp_path / "opts.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"la_decode.h\"\n"
                   "int main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(la_opts, {f}));\n' for f in fields)
                   + '  printf("%zu\\n", sizeof(la_opts));\n  return 0;\n}\n')
    exe = tmp_path / "opts"
    subprocess.run([cc, "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    S = la.binding.LaOpts
    assert got == [getattr(S, f).offset for f in fields] + [ctypes.sizeof(S)]
