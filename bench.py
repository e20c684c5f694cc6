"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 512k]

One step is one decode-attention call over the whole workload: the host
computes the per-request prefix sums of tiles and tokens, they travel in the
kernel arguments, and the lean kernel derives its stream-K segments from them
and runs (above 256 requests the host builds the schedule tables and copies
them to the device instead). Inputs are seeded synthetic caches already
resident in HBM.
Prints one JSON line on stdout (the last line); progress goes to stderr.

`value` is microseconds per step (host-observed, whole call, a loop of plain
calls; the kernel times come from a second loop with HIP events). The `roofline`
object prices the lean kernel alone: algorithmic bytes per launch (K and V
once, q once, the fp32 output once) over the kernel's average duration,
measured with HIP events recorded on the call's stream right around the
launch. `cpu_baseline` times the fp64 oracle on a bounded sample of heads of
the same workload and scales it to a whole step. `comparators` times the
in-house fixed-split and per-head kernels on the same inputs.

With the default workload (512k) the line also carries a `ragged` object: the
same measurements on the ragged batch (B=16, H=32, d=128, lengths log-uniform
in [1024, 262144]), the metric's second headline workload.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import gc
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_phase_attention_amd", "csrc", f)
                  for f in ("kernels.hip", "kernels_gqa.hip", "kernels.h", "device_common.h",
                            "seg_walk.h")]
METRIC = "decode-attention µs/step + achieved HBM TB/s vs 8 TB/s peak (512k, ragged)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


@contextlib.contextmanager
def gc_paused():
    """Python's garbage collector paused over a timed region, as timeit does:
    a full collection in this process takes ~25 ms and would otherwise land
    inside a timed loop now and then (measured: one 1.2-ms-per-step loop of
    32 calls stretched by 25 ms)."""
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def time_kind(la, torch, evs, inp, kind, steps, warmup, **opts):
    """Host-observed µs/step over `steps` plain calls (synchronised on both
    sides), then kernel µs from HIP events around the kernels over another
    `steps` calls (the events add their own gaps, so they stay out of the
    first loop)."""
    B, H, d = inp.B, inp.H, inp.d
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device=inp.q.device)

    def call(ev0=None, ev1=None):
        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, B, H, d, inp.scale, out, kind=kind,
                        ev_start=ev0, ev_stop=ev1, kv_heads=inp.Hk, q_tokens=inp.Nq, **opts)

    for _ in range(warmup):
        call()
    la.la_sync_check()
    pairs = evs.create(2 * steps)
    with gc_paused():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        la.la_sync_check()
        for i in range(steps):
            call(pairs[2 * i], pairs[2 * i + 1])
        torch.cuda.synchronize()
    la.la_sync_check()
    kern = [evs.elapsed_ms(pairs[2 * i], pairs[2 * i + 1]) * 1e3 for i in range(steps)]
    evs.destroy(pairs)
    kern.sort()
    return {
        "us_per_step": (t1 - t0) * 1e6 / steps,
        "kernel_us_mean": sum(kern) / len(kern),
        "kernel_us_p10": kern[len(kern) // 10],
        "kernel_us_p50": kern[len(kern) // 2],
        "kernel_us_p90": kern[(9 * len(kern)) // 10],
    }


def host_cost(la, torch, inp, batches=8, per_batch=3, grid=0):
    """Host µs of one lean call through the Python binding while the GPU is
    still busy with the previous ones (the call only enqueues): median over
    `batches` bursts of `per_batch` calls, synchronised between bursts, with
    the context lengths changing on every call (as in decoding) and fixed;
    for the schedule derived in the launch (default) and for host tables.
    Bursts stay below the four pinned staging slots of the table path, whose
    reuse waits for the copy four calls back (that wait throttles the host to
    the GPU's pace in table mode, not the in-launch mode)."""
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device=inp.q.device)
    res = {}
    for mode, ht in (("in_launch", False), ("host_tables", True)):
        res[mode] = {}
        for vary in (True, False):
            per_call = []
            with gc_paused():
                for bt in range(batches):
                    lens = [[max(n - ((bt * per_batch + i + 1) if vary else 0), inp.Nq)
                             for n in inp.ctx_lens] for i in range(per_batch)]
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    for i in range(per_batch):
                        la.la_decode_ex(inp.q, inp.k, inp.v, lens[i], inp.B, inp.H, inp.d,
                                        inp.scale, out, kv_heads=inp.Hk, q_tokens=inp.Nq,
                                        host_tables=ht, grid=grid)
                    t1 = time.perf_counter()
                    per_call.append((t1 - t0) * 1e6 / per_batch)
            torch.cuda.synchronize()
            la.la_sync_check()
            per_call.sort()
            res[mode]["lengths_changing" if vary else "lengths_fixed"] = round(
                per_call[len(per_call) // 2], 1)
    return res


CEILING_MAX_BYTES = 16 << 30


def ceiling_bytes_for(alg_bytes: int) -> int:
    """Size of the streaming read set next to a workload of `alg_bytes`."""
    return max(64 << 10, min(alg_bytes, CEILING_MAX_BYTES))


def read_ceiling(la, torch, nbytes, reps=10, buf=None):
    """Achievable streaming-read bandwidth of this device in GB/s: the
    library's plain read kernel (the attention kernels' loads, K-like and
    V-like halves side by side, no arithmetic) over `nbytes` bytes, best of
    `reps` launches timed with events on the launch stream (torch's current
    one). Short reads pay the same launch ramp and tail as a short attention
    kernel, and a long one amortises them as a long kernel does, so the read
    is the workload's own size: one workgroup per CU, or fewer when the
    buffer holds less than the read kernel's 64 KiB per workgroup. `buf`, a
    uint8 device buffer of at least `nbytes` allocated beforehand, keeps the
    allocation out of the timed phase."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    unit = 64 << 10
    nbytes = max(nbytes, unit)
    grid = max(1, min(cus, nbytes // unit))
    if buf is None:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    else:
        buf = buf[:nbytes]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        la.la_stream_read(buf, sink, grid=grid)
    best = float("inf")
    n = 0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        n = la.la_stream_read(buf, sink, grid=grid)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    la.la_sync_check()
    # freed to torch's cache only: returning it to the driver and allocating
    # again slows every kernel for about a second afterwards
    del buf
    return n / (best * 1e-3) / 1e9, n, grid


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per lean launch from the committed counter summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"lean_kernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (FETCH_SIZE should read nbytes, WRITE_SIZE nbytes)."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes")


def occupancy(la, torch, inp, kind, blocks, **opts):
    """Per-CU busy time of one launch, from the per-workgroup timestamps: for
    every CU the union of its workgroups' [entry, exit] intervals, as a
    fraction of the kernel's span (first entry to last exit)."""
    import numpy as np
    ts = torch.zeros(blocks * 4, dtype=torch.int64, device=inp.q.device)
    out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device=inp.q.device)
    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d, inp.scale, out,
                    kind=kind, cta_timestamps=ts, kv_heads=inp.Hk, q_tokens=inp.Nq, **opts)
    la.la_sync_check()
    a = ts.view(blocks, 4).cpu().numpy().astype(np.int64)
    start, end, ids = a[:, 0], a[:, 1], a[:, 2]
    t0, t1 = int(start.min()), int(end.max())
    span = max(1, t1 - t0)
    # XCC_ID, then HW_ID bits 8..15 (CU, SH and SE ids): one key per CU
    keys = ((ids >> 32) & 0xFF) * 256 + ((ids >> 8) & 0xFF)
    busy = {}
    for k in np.unique(keys):
        sel = np.argsort(start[keys == k])
        s_, e_ = start[keys == k][sel], end[keys == k][sel]
        tot, cs, ce = 0, int(s_[0]), int(e_[0])
        for x, y in zip(s_[1:], e_[1:]):
            if x > ce:
                tot += ce - cs
                cs, ce = int(x), int(y)
            else:
                ce = max(ce, int(y))
        busy[int(k)] = tot + ce - cs
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    fr = np.array(list(busy.values())) / span
    return {
        "workgroups": blocks,
        "cus_used": len(busy),
        "cus": n_cus,
        "busy_frac_mean_all_cus": round(float(fr.sum() / n_cus), 4),
        "busy_frac_min_used": round(float(fr.min()), 4),
        "span_us": round(span / 100.0, 1),     # realtime clock: 100 MHz
    }


def host_cpu():
    """CPU model name and the number of cores this process may run on."""
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cpu, len(os.sched_getaffinity(0))


# Worker threads of the CPU baseline: a one-GPU host share here is 16 CPUs,
# whatever the affinity mask shows, so pools are sized to that share (and the
# visible count is reported beside it).
CPU_SHARE = 16


def cpu_baseline(inp, budget_s=12.0):
    """fp64 oracle on whole query rows of the workload until ~budget_s of wall
    time, scaled by (all head-tokens / head-tokens done) to microseconds per
    step. A query row is (request, head), or (request, new token, head) with
    several new tokens; it attends over its visible prefix of the cache."""
    import numpy as np

    import oracle
    import workloads as W

    cpu, visible = host_cpu()
    workers = max(1, min(CPU_SHARE, visible))
    B, H, Hk, Nq = inp.B, inp.H, inp.Hk, inp.Nq
    g = H // Hk
    starts = np.concatenate([[0], np.cumsum(inp.ctx_lens)]) * Hk
    qb = W.to_bits(inp.q).reshape(B, Nq, H, inp.d)
    heads = [(b, t, h) for b in range(B) for t in range(Nq) for h in range(H)]
    done = 0
    tokens_done = 0
    spent = 0.0
    i = 0
    while i < len(heads) and spent < budget_s:
        batch = heads[i:i + workers]
        # host copies of just these rows, made outside the timed region
        ks, vs, lens, qs = [], [], [], []
        for (b, t, h) in batch:
            n = inp.ctx_lens[b]
            vis = n - Nq + 1 + t
            r0 = int(starts[b]) + (h // g) * n
            ks.append(W.to_bits(inp.k[r0:r0 + vis]))
            vs.append(W.to_bits(inp.v[r0:r0 + vis]))
            lens.append(vis)
            qs.append(qb[b, t, h])
        kcat, vcat = np.concatenate(ks), np.concatenate(vs)
        qcat = np.stack(qs)[:, None, :]
        t0 = time.perf_counter()
        oracle.attend_fp64(qcat, kcat, vcat, lens, inp.scale, inp.dtype, workers=workers)
        spent += time.perf_counter() - t0
        done += len(batch)
        tokens_done += sum(lens)
        i += len(batch)
        del ks, vs, kcat, vcat
    total_tokens = H * sum(Nq * n - Nq * (Nq - 1) // 2 for n in inp.ctx_lens)
    value = spent * 1e6 * total_tokens / tokens_done
    kv_bytes = 2 * tokens_done * inp.d * 2        # the 16-bit K and V rows the oracle read
    return {
        "value": round(value, 1),
        "unit": "us/step",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} query rows ({tokens_done} of {total_tokens} "
                  f"head-tokens), fp64 two-pass numpy oracle, {spent:.1f} s wall, scaled by "
                  f"head-tokens; {workers} worker threads (the box's CPU share) of "
                  f"{visible} cores visible; host {cpu}",
        "wall_s": round(spent, 2),
        "kv_GBps": round(kv_bytes / spent / 1e9, 3) if spent > 0 else None,
        "host_cores_visible": visible,
        "cpu_model": cpu,
    }


def selector_shapes():
    """Decode shapes for measuring kind="auto" against every kernel: one long
    head to thousands of short ones, uniform and log-uniform lengths, d = 64
    and 128, grouped K/V heads and several new tokens."""
    import numpy as np

    def loguni(B, lo, hi, seed):
        u = np.random.default_rng(seed).random(B)
        return [int(math.exp(math.log(lo) + x * math.log(hi / lo))) for x in u]

    S = [dict(lens=[n], H=32, d=128, dt="bf16") for n in (4096, 65536)]
    S += [dict(lens=[131072], H=8, d=128, dt="bf16"),
          dict(lens=[16384] * 4, H=32, d=128, dt="bf16"),
          dict(lens=[4096] * 16, H=32, d=128, dt="bf16"),
          dict(lens=[4096] * 64, H=32, d=128, dt="bf16"),
          dict(lens=[512] * 256, H=32, d=128, dt="bf16"),
          dict(lens=[256] * 512, H=8, d=128, dt="bf16"),
          dict(lens=[16384] * 8, H=128, d=64, dt="f16"),
          dict(lens=[65536] * 2, H=16, d=64, dt="f16"),
          dict(lens=loguni(4, 1024, 262144, 1), H=32, d=128, dt="bf16"),
          dict(lens=loguni(16, 1024, 262144, 2), H=32, d=128, dt="bf16"),
          dict(lens=loguni(128, 128, 8192, 4), H=32, d=128, dt="bf16"),
          dict(lens=loguni(32, 256, 32768, 5), H=16, d=64, dt="f16"),
          dict(lens=[131072], H=32, Hk=8, d=128, dt="bf16"),
          dict(lens=[4096] * 32, H=32, Hk=8, d=128, dt="bf16"),
          dict(lens=[2048] * 64, H=64, Hk=8, d=128, dt="bf16"),
          dict(lens=[32768] * 8, H=16, Hk=1, d=64, dt="f16"),
          dict(lens=loguni(16, 1024, 262144, 6), H=32, Hk=4, d=128, dt="bf16"),
          dict(lens=loguni(16, 1024, 65536, 7), H=32, Hk=8, Nq=4, d=128, dt="bf16"),
          dict(lens=[8192] * 32, H=32, Nq=4, d=128, dt="bf16"),
          # latency-bound launches: a few short units, all at once
          dict(lens=[1024], H=4, d=64, dt="f16"),
          dict(lens=[512], H=8, d=128, dt="bf16"),
          dict(lens=[256] * 2, H=32, d=128, dt="bf16"),
          dict(lens=[512] * 8, H=32, d=128, dt="bf16"),
          dict(lens=[1024] * 4, H=8, d=64, dt="f16"),
          dict(lens=[512] * 8, H=32, Hk=8, d=128, dt="bf16"),
          dict(lens=[1024], H=32, d=128, dt="bf16"),
          dict(lens=[4096], H=1, d=128, dt="bf16")]
    return S


def selector_sweep(steps=10, warmup=2, rounds=3):
    """kind="auto" against lean (one and two workgroups per CU), per-head and
    fixed-split (heuristic K and K = 2..32) on every selector shape; prints one
    JSON line with each shape's kernel times and auto's regret (its kernel
    time over the fastest)."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for i, s in enumerate(selector_shapes()):
        Hk, Nq = s.get("Hk", s["H"]), s.get("Nq", 1)
        log(f"[selector {i}] B={len(s['lens'])} H={s['H']} Hk={Hk} Nq={Nq} d={s['d']} "
            f"N={sum(s['lens'])}")
        inp = W.make_custom(s["lens"], s["H"], s["d"], s["dt"], seed=0, device="cuda",
                            kv_heads=Hk, q_tokens=Nq)
        dt = la.LA_BF16 if s["dt"] == "bf16" else la.LA_F16
        pick, grid = la.la_select(inp.ctx_lens, inp.H, inp.d, dt, kv_heads=Hk, q_tokens=Nq)
        kinds = [("auto", "auto", {}), ("lean_1cu", "lean", {"grid": cus}),
                 ("lean_2cu", "lean", {"grid": 2 * cus}), ("pull", "pull", {}),
                 ("per_head", "per_head", {}), ("fixed_split_heuristic", "fixed_split", {})]
        kinds += [(f"fixed_split_{K}", "fixed_split", {"num_splits": K}) for K in (2, 4, 8, 16, 32)]
        # rounds over all kinds, each round starting at another kind, so that
        # no kind is always timed first; a kind's time is its best round's median
        t = {}
        for r in range(rounds):
            for j in range(len(kinds)):
                tag, kind, o = kinds[(j + r * 3) % len(kinds)]
                try:
                    us = time_kind(la, torch, evs, inp, kind, steps, warmup, **o)["kernel_us_p50"]
                except la.LaError:
                    continue                   # grid above the kernel's co-resident capacity
                t[tag] = round(min(us, t.get(tag, float("inf"))), 2)
        best = min((v, k) for k, v in t.items() if k != "auto")
        # auto runs the same kernel and grid as one explicit kind: both are
        # samples of that configuration
        same = "per_head" if pick == "per_head" else ("lean_1cu" if grid == cus else "lean_2cu")
        auto_us = min(t["auto"], t.get(same, t["auto"]))
        rows.append({"B": inp.B, "H": inp.H, "kv_heads": Hk, "q_tokens": Nq, "d": inp.d,
                     "dtype": s["dt"], "sum_n": sum(inp.ctx_lens),
                     "uniform": len(set(inp.ctx_lens)) == 1, "auto_pick": pick, "auto_grid": grid,
                     "kernel_us_p50": t, "best": best[1],
                     "auto_regret": round(auto_us / best[0], 4),
                     "lean_1cu_regret": round(t["lean_1cu"] / best[0], 4)})
        log(f"   auto={pick}@{grid} {t['auto']} us, best {best[1]} {best[0]} us, "
            f"regret {rows[-1]['auto_regret']}")
        del inp
        torch.cuda.empty_cache()
    reg = [r["auto_regret"] for r in rows]
    reg1 = [r["lean_1cu_regret"] for r in rows]
    print(json.dumps({"metric": "kind=auto kernel time over the fastest kind, per shape",
                      "shapes": len(rows), "auto_regret_max": max(reg),
                      "auto_regret_mean": round(sum(reg) / len(reg), 4),
                      "lean_1cu_regret_max": max(reg1),
                      "lean_1cu_regret_mean": round(sum(reg1) / len(reg1), 4),
                      "device": torch.cuda.get_device_name(0), "cus": cus, "rows": rows}),
          flush=True)


def masked_stream(hip, torch, n_cus, total):
    """A stream whose kernels may use only the first n_cus CUs of the device
    (hipExtStreamCreateWithCUMask; default priority)."""
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    words = (total + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for i in range(n_cus):
        mask[i // 32] |= 1 << (i % 32)
    s = ctypes.c_void_p()
    if hip.hipExtStreamCreateWithCUMask(ctypes.byref(s), words, mask) != 0:
        raise RuntimeError("hipExtStreamCreateWithCUMask failed")
    return torch.cuda.ExternalStream(s.value)


def contention(workloads, steps=10, warmup=3):
    """Each kind on streams that may use only part of the CUs (a CU mask), as
    when other kernels of a serving step hold the rest. Lean takes its
    default grid on that stream (one workgroup per CU the stream may use;
    single heads on under 70% of the CUs one per CU of the device) and, as
    lean_device_grid, one per CU of the whole device; auto is what kind auto
    picks on that stream; the pull kinds rebalance. Prints one JSON line with
    kernel p50 (us) per kind and available-CU count."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    total = torch.cuda.get_device_properties(0).multi_processor_count
    fracs = (8, 7, 6, 5, 4)                      # eighths of the CUs available
    table = {}
    for name in workloads:
        log(f"[contention] {name}")
        inp = W.make_inputs(name, seed=0, device="cuda")
        out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
        L = la.la_default_tile(inp.d)
        cols = inp.H // inp.Hk * inp.Nq
        units = inp.Hk * ((cols + 15) // 16) if cols > 1 else inp.H
        I = units * sum((n + L - 1) // L for n in inp.ctx_lens)
        G = la.la_default_grid(inp.d, la.LA_BF16 if inp.dtype == "bf16" else la.LA_F16)
        kinds = [("lean", "lean", {}), ("lean_device_grid", "lean", {"grid": G}),
                 ("auto", "auto", {}), ("pull", "pull", {}),
                 ("chunks", "chunks", {"chunk_tiles": -(-I // G)}),
                 ("fixed_split_8", "fixed_split", {"num_splits": 8}),
                 ("fixed_split_16", "fixed_split", {"num_splits": 16})]
        rows = {}
        # a second of untimed launches first: right after a large allocation
        # every kernel runs slower for about a second
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            time_kind(la, torch, evs, inp, "lean", 5, 1)
        for f in fracs:
            n = total * f // 8
            st = masked_stream(evs.hip, torch, n, total)
            # a new stream's first launches run slower: a fifth of a second of
            # untimed ones first
            with torch.cuda.stream(st):
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < 0.2:
                    la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d,
                                    inp.scale, out, kind="lean", kv_heads=inp.Hk, q_tokens=inp.Nq)
                    st.synchronize()
            row = {}
            for tag, kind, o in kinds:
                with torch.cuda.stream(st):
                    for _ in range(warmup):
                        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d,
                                        inp.scale, out, kind=kind, kv_heads=inp.Hk,
                                        q_tokens=inp.Nq, **o)
                    pairs = evs.create(2 * steps)
                    for i in range(steps):
                        la.la_decode_ex(inp.q, inp.k, inp.v, inp.ctx_lens, inp.B, inp.H, inp.d,
                                        inp.scale, out, kind=kind, ev_start=pairs[2 * i],
                                        ev_stop=pairs[2 * i + 1], kv_heads=inp.Hk,
                                        q_tokens=inp.Nq, **o)
                    st.synchronize()
                    la.la_sync_check()
                ks = sorted(evs.elapsed_ms(pairs[2 * i], pairs[2 * i + 1]) * 1e3
                            for i in range(steps))
                evs.destroy(pairs)
                row[tag] = round(ks[steps // 2], 1)
            rows[str(n)] = row
            log(f"   {n} CUs: {row}")
        table[name] = rows
        del inp, out
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode kernel p50 us when only part of the CUs is available",
                      "device": torch.cuda.get_device_name(0), "cus": total,
                      "grid": "lean its default grid (one workgroup per CU of the stream; "
                              "single heads on under 70% of the CUs one per CU of the device), "
                              "lean_device_grid and pull one per CU of the device; chunks "
                              "ceil(I / that grid) tiles each; fixed split K pieces per head",
                      "table": table}), flush=True)


def tile_sweep(workloads, steps=20, warmup=3, rounds=3):
    """The lean kernel at LeanTile sizes 32..2048 tokens on each workload (the
    pages pick the tile per head dim and hardware); prints one JSON line with
    the best of `rounds` rounds per size. Every workload's inputs are drawn
    first and kept, and the sizes are timed in rounds interleaved over all of
    them, after a second of untimed launches: timing them one after another
    right after an allocation put the first sizes inside the slow second that
    follows a large allocation."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    sizes = (32, 64, 128, 256, 512, 1024, 2048)
    inputs = {}
    for name in workloads:
        log(f"[tiles] generating {name}")
        inputs[name] = W.make_inputs(name, seed=0, device="cuda")
    torch.cuda.synchronize()
    table = {}
    for name, inp in inputs.items():
        log(f"[tiles] {name}")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            time_kind(la, torch, evs, inp, "lean", 5, 1)
        best = {L: float("inf") for L in sizes}
        for r in range(rounds):
            for L in (sizes if r % 2 == 0 else sizes[::-1]):
                t = time_kind(la, torch, evs, inp, "lean", steps, warmup, tile_tokens=L)
                best[L] = min(best[L], t["kernel_us_p50"])
        row = {str(L): round(best[L], 1) for L in sizes}
        row["default"] = la.la_default_tile(inp.d)
        table[name] = row
        log(f"   {row}")
    print(json.dumps({"metric": "lean kernel p50 us by LeanTile size (tokens)",
                      "device": torch.cuda.get_device_name(0), "table": table}), flush=True)


def pages_sweep_shapes():
    """The single-GPU sweeps of the LeanAttention evaluation (xllm-io paper
    review, §5.2 and §5.4), at the shapes the pages state, with uniform
    contexts and one query token per head:
    - context sweep at 56 heads, batch 1: 1k, 8k, 32k, 64k and 512k tokens;
    - head sweep at 64k tokens, batch 1: 16 to 192 heads;
    - batch sweep at 56 heads (the context sweep's) and 64k tokens (the head
      sweep's; the pages give no context for it): batch 1 to 16;
    - the extremes the pages quote: 16 and 24 heads at 512k, 24 heads at 1k;
    - head dimension 128 at 1k and 512k (56 heads, batch 1);
    - few heads at long contexts, where the stream-K schedule departs most
      from the per-head and fixed-split ones (review §4.3): 1, 2 and 4 heads
      of 512k tokens, one of 128k, four of 32k (d = 128).
    The pages state no precision: d = 64 runs in fp16, d = 128 in bf16, as the
    many-heads and 512k workloads do."""
    S = []
    for n in (1024, 8192, 32768, 65536, 524288):
        S.append(dict(sweep="context", B=1, H=56, d=64, n=n))
    for H in (16, 24, 32, 64, 128, 192):
        S.append(dict(sweep="heads", B=1, H=H, d=64, n=65536))
    for B in (2, 4, 8, 16):
        S.append(dict(sweep="batch", B=B, H=56, d=64, n=65536))
    for H, n in ((16, 524288), (24, 524288), (24, 1024)):
        S.append(dict(sweep="extremes", B=1, H=H, d=64, n=n))
    for n in (1024, 524288):
        S.append(dict(sweep="head_dim_128", B=1, H=56, d=128, n=n))
    for H, n in ((1, 524288), (2, 524288), (4, 524288), (1, 131072), (4, 32768)):
        S.append(dict(sweep="few_heads", B=1, H=H, d=128, n=n))
    return S


def pages_sweep(steps=20, warmup=3, rounds=3):
    """Lean against the per-head kernel (one workgroup per head over its whole
    context: the FlashAttention-2 decode schedule) and the fixed split
    (FlashDecoding's: K splits per head chosen to fill the GPU, plus the best K
    of 2..64, or up to one workgroup per CU for every head) on the pages'
    sweep shapes; prints one JSON line. Each shape's
    inputs are drawn, a second of untimed launches follows the allocation, and
    the kinds are timed in interleaved rounds (best round's median)."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    kinds = [("lean", "lean", {}), ("auto", "auto", {}), ("pull", "pull", {}),
             ("per_head", "per_head", {}), ("fixed_split_heuristic", "fixed_split", {})]
    rows = []
    for i, s in enumerate(pages_sweep_shapes()):
        # split counts up to one workgroup per CU for every head
        Ks = [K for K in (2, 4, 8, 16, 32, 64, 128, 256) if K <= 64 or K * s["B"] * s["H"] <= cus]
        kinds_s = kinds + [(f"fixed_split_{K}", "fixed_split", {"num_splits": K}) for K in Ks]
        dt = "f16" if s["d"] == 64 else "bf16"
        log(f"[pages {i}] {s['sweep']}: B={s['B']} H={s['H']} d={s['d']} n={s['n']} {dt}")
        inp = W.make_custom([s["n"]] * s["B"], s["H"], s["d"], dt, seed=i, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            time_kind(la, torch, evs, inp, "lean", 5, 1)
        t = {}
        for r in range(rounds):
            for j in range(len(kinds_s)):
                tag, kind, o = kinds_s[(j + r * 4) % len(kinds_s)]
                us = time_kind(la, torch, evs, inp, kind, steps, warmup, **o)["kernel_us_p50"]
                t[tag] = round(min(us, t.get(tag, float("inf"))), 2)
        fs = {k: v for k, v in t.items() if k.startswith("fixed_split_") and k[12:].isdigit()}
        fs_best = min(fs.items(), key=lambda kv: kv[1])
        alg = W.algorithmic_bytes(inp.ctx_lens, inp.H, inp.d)
        lean = t["lean"]
        row = {**s, "dtype": dt, "units": s["B"] * s["H"], "cus": cus,
               "lean_grid": la.la_default_grid(s["d"], la.LA_F16 if dt == "f16" else la.LA_BF16),
               "auto_pick": "%s@%d" % la.la_select(inp.ctx_lens, inp.H, inp.d,
                                                    la.LA_F16 if dt == "f16" else la.LA_BF16),
               "bytes": alg, "kernel_us_p50": t,
               "fixed_split_best": fs_best[0],
               "lean_TBps": round(alg / lean / 1e6, 3),
               "lean_frac_of_8TBps": round(alg / lean / 1e6 / 8.0, 4),
               "speedup_vs_per_head": round(t["per_head"] / lean, 3),
               "speedup_vs_fixed_split_heuristic": round(t["fixed_split_heuristic"] / lean, 3),
               "speedup_vs_fixed_split_best": round(fs_best[1] / lean, 3),
               "auto_speedup_vs_per_head": round(t["per_head"] / t["auto"], 3),
               "auto_speedup_vs_fixed_split_heuristic": round(t["fixed_split_heuristic"] / t["auto"], 3)}
        rows.append(row)
        log(f"   lean {lean} us ({row['lean_TBps']} TB/s), per-head {t['per_head']}, "
            f"fixed split {t['fixed_split_heuristic']} (best {fs_best[0]} {fs_best[1]}), "
            f"x{row['speedup_vs_per_head']} / x{row['speedup_vs_fixed_split_heuristic']}")
        del inp
        torch.cuda.empty_cache()

    def stats(key, sel):
        v = [r[key] for r in rows if sel(r)]
        return {"mean": round(sum(v) / len(v), 3),
                "geomean": round(math.exp(sum(math.log(x) for x in v) / len(v)), 3),
                "max": max(v), "min": min(v)}

    keys = ("speedup_vs_per_head", "speedup_vs_fixed_split_heuristic",
            "speedup_vs_fixed_split_best", "auto_speedup_vs_per_head",
            "auto_speedup_vs_fixed_split_heuristic")
    pages = lambda r: r["sweep"] != "few_heads"   # noqa: E731
    print(json.dumps({"metric": "lean kernel speedup over per-head and fixed-split kernels on "
                                "the pages' sweep shapes (kernel p50)",
                      "device": torch.cuda.get_device_name(0), "cus": cus, "shapes": len(rows),
                      "summary": {k: stats(k, pages) for k in keys},
                      "summary_few_heads": {k: stats(k, lambda r: not pages(r)) for k in keys},
                      "rows": rows}), flush=True)


def ragged_draws(workloads, seeds, steps=20, warmup=3, rounds=2):
    """Lean against the fixed split at every split count of 1..64 (and its
    fill-the-GPU heuristic), the dynamic pull and the per-head kernel on
    several seeded draws of each ragged workload's log-uniform lengths (the
    talk summary's ragged batches; xllm-io paper review §5.2): one JSON line
    with each draw's kernel p50s and, per workload, how lean compares with the
    best fixed split picked after the fact for each draw. Each draw's inputs
    are allocated on their own, followed by a second of untimed launches, and
    the kinds are timed in interleaved rounds (best round's median)."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Ks = (1, 2, 4, 8, 16, 32, 64)
    rows = []
    for name in workloads:
        for seed in seeds:
            log(f"[ragged draws] {name} seed {seed}")
            inp = W.make_inputs(name, seed=seed, device="cuda")
            w = inp.meta["workload"]
            dt = la.LA_BF16 if w.dtype == "bf16" else la.LA_F16
            _, G = la.la_select(inp.ctx_lens, inp.H, inp.d, dt, kv_heads=inp.Hk, q_tokens=inp.Nq)
            kinds = [("lean", "lean", {"grid": G}), ("pull", "pull", {}),
                     ("per_head", "per_head", {}), ("fixed_split_heuristic", "fixed_split", {})]
            kinds += [(f"fixed_split_{K}", "fixed_split", {"num_splits": K}) for K in Ks]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 1.0:
                time_kind(la, torch, evs, inp, "lean", 5, 1, grid=G)
            t = {}
            for r in range(rounds):
                for j in range(len(kinds)):
                    tag, kind, o = kinds[(j + r * 5) % len(kinds)]
                    us = time_kind(la, torch, evs, inp, kind, steps, warmup, **o)["kernel_us_p50"]
                    t[tag] = round(min(us, t.get(tag, float("inf"))), 2)
            fs = {K: t[f"fixed_split_{K}"] for K in Ks}
            K_best = min(fs, key=fs.get)
            alg = W.algorithmic_bytes(inp.ctx_lens, inp.H, inp.d, kv_heads=inp.Hk,
                                      q_tokens=inp.Nq)
            lens = sorted(inp.ctx_lens)
            row = {"workload": name, "seed": seed, "B": inp.B, "H": inp.H, "kv_heads": inp.Hk,
                   "q_tokens": inp.Nq, "d": inp.d, "lens_min": lens[0],
                   "lens_median": lens[len(lens) // 2], "lens_max": lens[-1],
                   "sum_n": sum(lens), "bytes": alg, "lean_grid": G, "kernel_us_p50": t,
                   "lean_TBps": round(alg / t["lean"] / 1e6, 3),
                   "fixed_split_best_K": K_best, "fixed_split_best_us": fs[K_best],
                   "lean_over_fixed_split_best": round(t["lean"] / fs[K_best], 4),
                   "lean_over_fixed_split_heuristic": round(t["lean"] / t["fixed_split_heuristic"], 4),
                   "lean_over_pull": round(t["lean"] / t["pull"], 4)}
            rows.append(row)
            log(f"   lean {t['lean']} us ({row['lean_TBps']} TB/s), best fixed split "
                f"{fs[K_best]} (K={K_best}), pull {t['pull']}, x{row['lean_over_fixed_split_best']}")
            del inp
            torch.cuda.empty_cache()

    def summary(name):
        rs = [r for r in rows if r["workload"] == name]
        out = {"draws": len(rs)}
        for k in ("lean_over_fixed_split_best", "lean_over_fixed_split_heuristic", "lean_over_pull"):
            v = [r[k] for r in rs]
            out[k] = {"geomean": round(math.exp(sum(math.log(x) for x in v) / len(v)), 4),
                      "max": max(v), "min": min(v)}
        out["draws_lean_faster_than_fixed_split_best"] = sum(
            r["lean_over_fixed_split_best"] < 1.0 for r in rs)
        return out

    print(json.dumps({"metric": "lean kernel time over the best fixed split and the dynamic pull "
                                "on seeded draws of the ragged workloads (kernel p50)",
                      "device": torch.cuda.get_device_name(0), "cus": cus,
                      "summary": {name: summary(name) for name in workloads},
                      "rows": rows}), flush=True)


def decode_loop(workloads, steps=64, warmup=4):
    """Decode steps on a [B, Hk, S, d] cache (kv_stride = S) whose contexts
    grow by one token per request every step (the rows are already in the
    cache: appending them belongs to the model's K/V projection, not to
    attention): µs per step over `steps` steps queued back to back, for the
    schedule derived in the launch from host lengths, for host tables, for
    lengths kept on the device (each step adds one to them with a small
    device kernel, then calls the library), for that step captured once into
    a HIP graph and replayed, and for 16 such steps captured into one graph;
    next to the in-launch calls at fixed lengths. Prints one JSON line."""
    import torch

    import decode_phase_attention_amd as la
    import workloads as W

    torch.cuda.set_device(0)
    la.lib()
    table = {}
    for name in workloads:
        log(f"[decode loop] {name}")
        inp = W.make_inputs(name, seed=0, device="cuda")
        B, H, Hk, d, Nq = inp.B, inp.H, inp.Hk, inp.d, inp.Nq
        base = [n - steps - warmup for n in inp.ctx_lens]
        S = max(inp.ctx_lens)
        kc = torch.empty((B, Hk, S, d), dtype=inp.k.dtype, device="cuda")
        vc = torch.empty_like(kc)
        row = 0
        for b, n in enumerate(inp.ctx_lens):
            kc[b, :, :n] = inp.k[row:row + Hk * n].view(Hk, n, d)
            vc[b, :, :n] = inp.v[row:row + Hk * n].view(Hk, n, d)
            row += Hk * n
        out = torch.empty(tuple(inp.q.shape), dtype=torch.float32, device="cuda")
        lens_of = [[n + i + 1 for n in base] for i in range(warmup + steps)]
        # a second of untimed launches after the allocations, as elsewhere in
        # this file: kernels run slower for about a second after large ones
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            la.la_decode_ex(inp.q, kc, vc, base, B, H, d, inp.scale, out, kv_heads=Hk,
                            q_tokens=Nq, kv_stride=S)
            torch.cuda.synchronize()
        row_out = {}
        for label, ht, grow in (("in_launch_lengths_growing", False, True),
                                ("host_tables_lengths_growing", True, True),
                                ("in_launch_lengths_fixed", False, False)):
            def step(i):
                la.la_decode_ex(inp.q, kc, vc, lens_of[i] if grow else base, B, H, d, inp.scale,
                                out, kv_heads=Hk, q_tokens=Nq, kv_stride=S, host_tables=ht)
            for i in range(warmup):
                step(i)
            with gc_paused():
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i in range(steps):
                    step(warmup + i)
                torch.cuda.synchronize()
                t1 = time.perf_counter()
            la.la_sync_check()
            row_out[label] = round((t1 - t0) * 1e6 / steps, 1)
        base_t = torch.tensor(base, dtype=torch.int32, device="cuda")
        dl = base_t.clone()
        s = torch.cuda.Stream()

        def dstep():
            dl.add_(1)
            la.la_decode_ex(inp.q, kc, vc, None, B, H, d, inp.scale, out, kv_heads=Hk,
                            q_tokens=Nq, kv_stride=S, ctx_lens_device=dl)
        with torch.cuda.stream(s):
            for i in range(warmup):
                dstep()
            with gc_paused():
                s.synchronize()
                t0 = time.perf_counter()
                for i in range(steps):
                    dstep()
                s.synchronize()
                t1 = time.perf_counter()
        la.la_sync_check(s.cuda_stream)
        row_out["device_lengths_growing"] = round((t1 - t0) * 1e6 / steps, 1)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dstep()
        with torch.cuda.stream(s):
            dl.copy_(base_t)
            for i in range(warmup):
                g.replay()
            with gc_paused():
                s.synchronize()
                t0 = time.perf_counter()
                for i in range(steps):
                    g.replay()
                s.synchronize()
                t1 = time.perf_counter()
        la.la_sync_check(s.cuda_stream)
        assert dl.cpu().tolist() == lens_of[-1]
        row_out["graph_device_lengths_growing"] = round((t1 - t0) * 1e6 / steps, 1)
        del g
        # several steps in one graph: the graph launch's own cost shared by them
        chain = 16
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(chain):
                dstep()
        with torch.cuda.stream(s):
            dl.copy_(base_t)
            g.replay()
            dl.copy_(base_t)
            with gc_paused():
                s.synchronize()
                t0 = time.perf_counter()
                for i in range(steps // chain):
                    g.replay()
                s.synchronize()
                t1 = time.perf_counter()
        la.la_sync_check(s.cuda_stream)
        assert dl.cpu().tolist() == lens_of[steps // chain * chain - 1]
        row_out[f"graph_{chain}_steps_device_lengths_growing"] = round(
            (t1 - t0) * 1e6 / (steps // chain * chain), 1)
        del g
        table[name] = row_out
        log(f"   {row_out}")
        del kc, vc, inp, out
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode steps us/step, contexts growing by one token per "
                                "request per step", "steps": steps,
                      "device": torch.cuda.get_device_name(0), "table": table}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="512k",
                    choices=["tiny", "65k", "512k", "ragged", "many-heads", "gqa-512k",
                             "gqa8-ragged", "mqa-32k", "spec4-ragged", "spec8-64k", "512k-h4"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--no-ragged", action="store_true",
                    help="with the default 512k workload, skip the ragged workload that the "
                         "line otherwise also carries")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only the lean kernel on the workload (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (scales the HBM counters)")
    ap.add_argument("--selector-sweep", action="store_true",
                    help="instead of the workload: measure kind=auto against every kind "
                         "on a sweep of shapes")
    ap.add_argument("--jsonl", default=None,
                    help="also append one JSON record per measured kernel kind to this file")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead of the headline line: the lean kernel at tile sizes 32..2048")
    ap.add_argument("--pages-sweep", action="store_true",
                    help="instead of the headline line: lean against per-head and fixed split "
                         "on the pages' context, head, batch and head-dim sweeps")
    ap.add_argument("--decode-loop", action="store_true",
                    help="instead of the headline line: decode steps on a [B, Hk, S, d] cache "
                         "whose contexts grow by one token per step")
    ap.add_argument("--ragged-draws", type=int, default=0, metavar="N",
                    help="instead of the headline line: lean against every fixed-split count and "
                         "the pull on N seeded draws of each ragged workload (or --workload)")
    ap.add_argument("--contention", action="store_true",
                    help="instead of the headline line: every kind on streams confined to "
                         "part of the CUs (512k and ragged, or --workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the stream-K decode path here is single-GPU)", file=sys.stderr)
        sys.exit(2)
    if args.selector_sweep:
        selector_sweep()
        return
    if args.tile_sweep:
        tile_sweep(["512k", "ragged", "65k", "many-heads", "gqa-512k", "gqa8-ragged"])
        return
    if args.pages_sweep:
        pages_sweep()
        return
    if args.decode_loop:
        decode_loop(["512k", "ragged", "gqa8-ragged", "mqa-32k", "spec4-ragged"]
                    if args.workload == "512k" else [args.workload])
        return
    if args.ragged_draws:
        ragged_draws(["ragged", "gqa8-ragged", "spec4-ragged"] if args.workload == "512k"
                     else [args.workload], range(args.ragged_draws))
        return
    if args.contention:
        contention(["512k", "ragged"] if args.workload == "512k" else [args.workload])
        return

    import torch

    import decode_phase_attention_amd as la

    torch.cuda.set_device(0)
    la.lib()
    evs = HipEvents()
    import workloads as W

    # Every workload's inputs are drawn first and stay resident until the end:
    # after a large buffer is freed and another allocated, every kernel runs
    # several percent slower for about a second (measured on ragged right after
    # freeing 512k's caches: 2130 against 2037 us for lean, 2166 against 2094
    # for the best fixed split), so nothing is freed between measurements.
    names = [args.workload]
    if args.workload == "512k" and not args.kernel_only and not args.no_ragged:
        names.append("ragged")      # the metric's second headline workload, in the same line
    inputs = {}
    for n in names:
        log(f"[bench] generating {n} (seed {args.seed})")
        inputs[n] = W.make_inputs(n, seed=args.seed, device="cuda")
    # the streaming-read ceiling's buffer too, sized for the largest workload
    read_buf = None
    if not args.kernel_only:
        need = max(ceiling_bytes_for(W.algorithmic_bytes(inp.ctx_lens, inp.H, inp.d,
                                                         kv_heads=inp.Hk, q_tokens=inp.Nq))
                   for inp in inputs.values())
        read_buf = torch.zeros(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    # a second of untimed launches: right after large allocations every
    # kernel runs slower for about a second (a short workload's whole timing
    # would fall inside it)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        time_kind(la, torch, evs, inputs[args.workload], "lean", 5, 1)
    head = measure(la, torch, evs, args.workload, inputs[args.workload], args,
                   cpu=not args.no_cpu_baseline, read_buf=read_buf)
    extra = {}
    for n in names[1:]:
        extra[n] = measure(la, torch, evs, n, inputs[n], args, cpu=not args.no_cpu_baseline,
                           read_buf=read_buf)
    lean = head.pop("_lean")
    rec = {
        "metric": METRIC,
        "value": round(lean["us_per_step"], 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(lean["us_per_step"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["config"]["inputs"],
        "data": "synthetic",
        "config": head.pop("config"),
        "achieved_tbs": head.pop("achieved_tbs"),
        "kernel_us": head.pop("kernel_us"),
        "roofline": head.pop("roofline"),
        "cpu_baseline": head.pop("cpu_baseline"),
    }
    rec.update(head)
    for name, m in extra.items():
        m.pop("_lean")
        rec[name] = m
    props = torch.cuda.get_device_properties(0)
    rec["env"] = {"torch": torch.__version__, "python": platform.python_version(),
                  "device": torch.cuda.get_device_name(0),
                  "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
                  "hbm_GiB": round(props.total_memory / 2**30, 1)}
    if args.jsonl:
        write_jsonl(args.jsonl, rec, lean, rec.get("comparators"), rec.get("occupancy"),
                    rec.get("lean_splits_per_head"), rec["roofline"]["bytes_per_launch"],
                    rec["cpu_baseline"])
    print(json.dumps(rec), flush=True)


WORKLOAD_DESC = {
    "tiny": "tiny: B=1, H=4, d=64, n=1024, fp16",
    "65k": "65k: B=1, H=32, d=128, n=65536, bf16",
    "512k": "512k: B=1, H=32, d=128, n=524288, bf16",
    "ragged": "ragged: B=16, H=32, d=128, n_b log-uniform in [1024, 262144], bf16",
    "many-heads": "many-heads: B=8, H=128, d=64, n=16384, fp16",
    "gqa-512k": "gqa-512k: B=1, H=32 over 8 K/V heads, d=128, n=524288, bf16",
    "gqa8-ragged": "gqa8-ragged: B=16, H=64 over 8 K/V heads, d=128, n_b log-uniform "
                   "in [1024, 262144], bf16",
    "mqa-32k": "mqa-32k: B=8, H=16 over 1 K/V head, d=64, n=32768, fp16",
    "spec4-ragged": "spec4-ragged: B=16, 4 new tokens each, H=32 over 8 K/V heads, d=128, "
                    "n_b log-uniform in [1024, 262144], causal among the new tokens, bf16",
    "spec8-64k": "spec8-64k: B=4, 8 new tokens each, H=32, d=128, n=65536, causal among "
                 "the new tokens, bf16",
    "512k-h4": "512k-h4: B=1, H=4, d=128, n=524288, bf16 (one GPU's share of 512k under "
               "8-way head sharding)",
}


def method_overhead(la, inp, units, L, G, d, cols, alg_bytes):
    """Bytes the lean launch moves beyond the algorithmic ones: one partial
    record (Obar[d], m, l padded to d + 4 floats) per live query column of
    every peer segment, written by the peer and read by the host, plus the
    flags. From the schedule tables of the launch."""
    import numpy as np
    sch = la.la_schedule(inp.ctx_lens, units, L, G)
    seg = sch["seg"]
    peers = seg[seg[:, 4] == 0]
    if cols > 1:
        QB = (cols + 15) // 16
        qb = (peers[:, 1] % units) % QB
        live = np.minimum(16, cols - 16 * qb)
    else:
        live = np.ones(len(peers), np.int64)
    records = int(live.sum())
    rec_bytes = (d + 4) * 4
    part = 2 * records * rec_bytes
    flags = 2 * 4 * len(peers)
    per_head = np.bincount(seg[:, 1], minlength=inp.B * units)
    return {
        "splits_per_unit": {"max": int(per_head.max()), "mean": round(float(per_head.mean()), 3)},
        "peer_segments": int(len(peers)),
        "partial_records": records,
        "partial_record_bytes": rec_bytes,
        "partial_bytes_written_and_read": part,
        "flag_bytes": flags,
        "overhead_over_algorithmic": round((part + flags) / alg_bytes, 6),
    }


def measure(la, torch, evs, name, inp, args, cpu=True, read_buf=None):
    """Every measurement of one workload: the lean kernel (host-observed µs per
    step and kernel µs from events), its roofline against 8 TB/s and against
    the device's streaming-read rate at the same size, the committed HBM
    traffic, the in-house comparators (per head, pull, fixed split with the
    fill-one-wave K and every K in 1..64), per-CU busy balance, the method's
    own overhead, the host's cost per call and the fp64 oracle on the host."""
    import workloads as W

    w = inp.meta["workload"]
    dt_code = la.LA_BF16 if w.dtype == "bf16" else la.LA_F16
    Hk, Nq = inp.Hk, inp.Nq
    # the lean kernel on the grid the library's shape rule picks (one or two
    # workgroups per CU), whichever kind that rule would run
    _, G = la.la_select(inp.ctx_lens, inp.H, w.d, dt_code, kv_heads=Hk, q_tokens=Nq)
    L = la.la_default_tile(w.d)
    cols = inp.H // Hk * Nq                                # query columns per K/V head
    grouped = cols > 1
    units = Hk * ((cols + 15) // 16) if grouped else inp.H  # schedule units per request
    I, Gu, _ = la.la_schedule_dims(inp.ctx_lens, units, L, G)
    alg_bytes = W.algorithmic_bytes(inp.ctx_lens, inp.H, w.d, kv_heads=Hk, q_tokens=Nq)
    log(f"[bench] {name}: lens={inp.ctx_lens} I={I} G={Gu} L={L} bytes={alg_bytes}")

    log(f"[bench] {name}: timing lean")
    lean = time_kind(la, torch, evs, inp, "lean", args.steps, args.warmup, grid=Gu)
    achieved = alg_bytes / (lean["kernel_us_mean"] * 1e-6) / 1e9
    log(f"[bench] {name}: lean: {lean}")

    if args.copy_calibration:
        copy_calibration(torch)

    ceiling = ceiling_bytes = ceiling_grid = None
    if not args.kernel_only:
        ceiling, ceiling_bytes, ceiling_grid = read_ceiling(la, torch, ceiling_bytes_for(alg_bytes),
                                                            buf=read_buf)
        log(f"[bench] {name}: streaming-read ceiling over {ceiling_bytes} bytes "
            f"({ceiling_grid} workgroups): {ceiling:.1f} GB/s")

    comparators = None
    if not args.no_comparators and not args.kernel_only:
        comparators = {}
        comparators["per_head"] = time_kind(la, torch, evs, inp, "per_head", 10, 2)
        comparators["fixed_split_heuristic"] = time_kind(la, torch, evs, inp, "fixed_split", 10, 2)
        comparators["pull"] = time_kind(la, torch, evs, inp, "pull", 10, 2)
        sweep = {}
        for K in (1, 2, 4, 8, 16, 32, 64):
            sweep[K] = time_kind(la, torch, evs, inp, "fixed_split", 10, 2, num_splits=K)
        bestK = min(sweep, key=lambda k: sweep[k]["kernel_us_mean"])
        comparators["fixed_split_best"] = dict(sweep[bestK], num_splits=bestK)
        comparators["fixed_split_sweep_kernel_us"] = {str(k): round(v["kernel_us_mean"], 2)
                                                      for k, v in sweep.items()}
        log(f"[bench] {name}: fixed_split best K={bestK}: {comparators['fixed_split_best']}")
        for v in comparators.values():
            if isinstance(v, dict) and "kernel_us_mean" in v:
                v["tbs"] = round(alg_bytes / (v["kernel_us_mean"] * 1e-6) / 1e12, 3)
        best = comparators["fixed_split_best"]["kernel_us_mean"]
        comparators["lean_over_fixed_split_best"] = round(lean["kernel_us_mean"] / best, 4)
        comparators["lean_over_fixed_split_heuristic"] = round(
            lean["kernel_us_mean"] / comparators["fixed_split_heuristic"]["kernel_us_mean"], 4)

    occ = overhead = None
    if not args.kernel_only:
        overhead = method_overhead(la, inp, units, L, G, w.d, cols, alg_bytes)
        occ = {"lean": occupancy(la, torch, inp, "lean", Gu, grid=Gu),
               "per_head": occupancy(la, torch, inp, "per_head", inp.B * units)}
        if comparators is not None:
            K = comparators["fixed_split_best"]["num_splits"]
            occ["fixed_split_best"] = occupancy(la, torch, inp, "fixed_split", inp.B * units * K,
                                                num_splits=K)
        log(f"[bench] {name}: occupancy: {occ}")

    host = None
    if not args.kernel_only:
        host = host_cost(la, torch, inp, grid=Gu)
        log(f"[bench] {name}: host us per call: {host}")

    cpu_res = None
    if cpu and not args.kernel_only:
        log(f"[bench] {name}: cpu baseline (oracle)")
        cpu_res = cpu_baseline(inp)
        log(f"[bench] {name}: cpu: {cpu_res}")

    res = {
        "_lean": lean,
        "config": {
            "workload": WORKLOAD_DESC[name],
            "B": inp.B, "H": inp.H, "kv_heads": Hk, "q_tokens": Nq, "d": w.d,
            "ctx_lens": inp.ctx_lens,
            "seed": args.seed,
            "inputs": w.dtype, "accumulate": "fp32", "output": "fp32",
            "kind": "lean", "grid": Gu, "tile_tokens": L, "iterations": I,
            "parallelism": "single GPU",
        },
        "us_per_step": round(lean["us_per_step"], 2),
        "achieved_tbs": round(achieved / 1e3, 3),
        "kernel_us": {k: round(v, 2) for k, v in lean.items() if k.startswith("kernel")},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "read_ceiling_GBps": round(ceiling, 1) if ceiling else None,
            "read_ceiling_bytes": ceiling_bytes,
            "read_ceiling_workgroups": ceiling_grid,
            "frac_of_read_ceiling": round(achieved / ceiling, 4) if ceiling else None,
            "traffic": committed_traffic(name),
            "kernel": "lean_gqa_kernel" if grouped else "lean_kernel",
            "bytes_per_launch": alg_bytes,
            "kernel_source_sha256_16": kernel_source_hash(),
        },
        "cpu_baseline": cpu_res,
        "comparators": comparators,
        "occupancy": occ,
        "lean_splits_per_head": overhead["splits_per_unit"] if overhead else None,
        "method_overhead": overhead,
        "host_us_per_call": host,
    }
    return res


def write_jsonl(path, rec, lean, comparators, occ, splits, alg_bytes, cpu):
    """Append one record per (workload, kernel kind) measured in this run."""
    kinds = {"lean": lean}
    for k, v in (comparators or {}).items():
        if isinstance(v, dict) and "kernel_us_mean" in v:
            kinds[k] = v
    with open(path, "a") as f:
        for k, v in kinds.items():
            us = v["kernel_us_p50"]
            r = {"workload": rec["config"]["workload"], "kernel": k,
                 "kernel_us_p10": round(v["kernel_us_p10"], 2), "kernel_us_p50": round(us, 2),
                 "kernel_us_p90": round(v["kernel_us_p90"], 2),
                 "us_per_step": round(v["us_per_step"], 2),
                 "tbs": round(alg_bytes / (us * 1e-6) / 1e12, 3),
                 "frac_of_8tbs": round(alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                 "num_splits": v.get("num_splits"),
                 "busy_frac": ((occ or {}).get(k) or {}).get("busy_frac_mean_all_cus"),
                 "grid": rec["config"]["grid"] if k == "lean" else None,
                 "tile_tokens": rec["config"]["tile_tokens"],
                 "lean_splits_per_head": splits if k == "lean" else None,
                 "fetch_bytes": rec["roofline"]["traffic"] if k == "lean" else None,
                 "seed": rec["config"]["seed"], "ctx_lens": rec["config"]["ctx_lens"],
                 "oracle_us_per_step": (cpu or {}).get("value"),
                 "oracle_cores": (cpu or {}).get("cores"), "env": rec["env"]}
            f.write(json.dumps(r) + "\n")


if __name__ == "__main__":
    main()
