"""Timeline of one pa_decode launch, from the diagnostic library libpa_trace.so (built by
``build.build(trace=True)``: the same kernels, the decode kernel recording per-workgroup
timestamps of its plan and of every item; see decode.hip, PA_DECODE_TRACE).

    python3 -m paged_kv_cache_344_amd.trace_decode [batch] [--seed S] [--reps R]

Runs the seeded batch (as bench.py: inputs resident in HBM, several rotated copies so
that no call finds its K/V in the caches), traces the last of R calls and prints: the
plan's duration, the first item's duration on the first and the second workgroup of
each compute unit (workgroups b and b + grid / 2 share one), durations by item size,
the K/V bytes streamed per 2-microsecond slice (each item's bytes spread evenly over
its duration) and the number of busy workgroups, and when workgroups finish.  Diagnostic
only: nothing in the library or its tests depends on it."""
from __future__ import annotations

import argparse
import ctypes
import math
import os
import sys

import numpy as np
import torch

from . import binding
from .build import TRACE_LIB_PATH
from . import inputs

TICKS_PER_US = 100.0  # s_memrealtime runs at 100 MHz
SLOTS = 256           # trace words per workgroup
MAX_ITEMS = 60        # items recorded per workgroup
MAX_WG = 2048


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("batch", nargs="?", default="gqa_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--reps", type=int, default=12)
    ap.add_argument("--dump", default=None,
                    help="also save the raw per-workgroup words (.npy) for offline reading")
    args = ap.parse_args(argv)
    if not os.path.exists(TRACE_LIB_PATH):
        raise SystemExit(f"{TRACE_LIB_PATH} is not built: build.build(trace=True) first")
    L = ctypes.CDLL(TRACE_LIB_PATH)
    L.pa_decode.argtypes = binding.lib().pa_decode.argtypes
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.pa_decode_trace_read.restype = ctypes.c_int

    b = inputs.make_batch(args.batch, args.seed)
    dev = "cuda:0"
    t = lambda a: inputs.as_torch(a, b.dtype, dev)  # noqa: E731
    q, kc, vc = t(b.q), t(b.k_cache), t(b.v_cache)
    bt = torch.from_numpy(b.block_tables).to(dev)
    sl = torch.from_numpy(b.seq_lens).to(dev)
    pool = kc.numel() * kc.element_size() * 2
    ncopies = max(2, math.ceil(1.2e9 / pool))
    calls = []
    for ci in range(ncopies):
        qq, kk, vv = (q, kc, vc) if ci == 0 else (q.clone(), kc.clone(), vc.clone())
        d = binding.PreparedDecode(qq, kk, vv, bt, sl, b.block_size, b.num_kv_heads, b.scale,
                                   torch.empty_like(qq), partition_size=b.partition_size,
                                   shared_blocks=b.shared_blocks > 0)
        d._fn = L.pa_decode
        calls.append(d)
    buf = np.zeros(MAX_WG * SLOTS, dtype=np.uint64)
    ev_us = 0.0
    for rep in range(args.reps):
        for w in range(3):  # evict the traced copy's K/V from the caches
            calls[(rep + w + 1) % ncopies]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        calls[rep % ncopies]()
        e1.record()
        torch.cuda.synchronize()
        ev_us = e0.elapsed_time(e1) * 1e3
        if L.pa_decode_trace_read(buf.ctypes.data, buf.nbytes) != 0:
            raise SystemExit("pa_decode_trace_read failed")
    if args.dump:
        np.save(args.dump, buf.reshape(MAX_WG, SLOTS))
    summarise(b, buf.reshape(MAX_WG, SLOTS).astype(np.int64), ev_us)


def summarise(b, tr, ev_us):
    grid = int((tr[:, 0] > 0).sum())
    tr = tr[:grid]
    t0 = tr[:, 0].min()
    us = lambda x: (x - t0) / TICKS_PER_US  # noqa: E731
    row = b.num_kv_heads * b.head_dim * (4 if b.dtype == "f32" else 2) * 2 // b.num_kv_heads
    print(f"== {b.name} seed {b.seed}: one call {ev_us:.1f} us (events), {grid} workgroups, "
          f"sum L {b.total_tokens()}, partition length {int(tr[0, 250])}")
    print(f"plan: lengths read {np.median((tr[:, 248] - tr[:, 0]) / TICKS_PER_US):.2f} us after "
          f"entry, plan done {np.median((tr[:, 1] - tr[:, 0]) / TICKS_PER_US):.2f} us (median)")
    items = []
    for g in range(grid):
        for k in range(min(int(tr[g, 254]), MAX_ITEMS)):
            s, ll, e, info = tr[g, 2 + 4 * k:6 + 4 * k]
            items.append((g, k, us(s), us(ll) if ll else np.nan, us(e), int(info) & 0xFFFFFFFF,
                          (int(info) >> 32) & 1, int(info) >> 34))
    it = np.array(items, dtype=float)
    dur = it[:, 4] - it[:, 2]
    first = it[:, 1] == 0
    half = grid // 2
    fast, slow = first & (it[:, 0] < half), first & (it[:, 0] >= half)
    print(f"first item: {np.median(dur[fast]):.1f} us median on workgroups b < {half}, "
          f"{np.median(dur[slow]):.1f} us on b >= {half} (same compute unit, later waves); "
          f"tokens {np.median(it[fast, 7]):.0f} / {np.median(it[slow, 7]):.0f}")
    print("items by tokens (one KV head tile each; one-chunk groups: four sequences, one per wave):")
    bins = [(1, 32), (33, 128), (129, 256), (257, 512), (513, 1024), (1025, 1 << 30)]
    regular = it[:, 6] == 0
    for lo, hi in bins:
        m = regular & (it[:, 7] >= lo) & (it[:, 7] <= hi)
        if m.sum():
            print(f"  {lo:6d}-{min(hi, 10 ** 6):7d}: n {int(m.sum()):5d}, start p50 "
                  f"{np.median(it[m, 2]):5.1f} us, duration p50 {np.median(dur[m]):5.1f} us, "
                  f"loop {np.nanmedian(it[m, 3] - it[m, 2]):5.1f}, epilogue "
                  f"{np.nanmedian(it[m, 4] - it[m, 3]):4.1f}, {it[m, 7].sum() * row / 1e6:6.1f} MB")
    m = it[:, 6] == 1
    if m.sum():
        print(f"  one-chunk groups: n {int(m.sum())}, start p50 {np.median(it[m, 2]):.1f} us, "
              f"duration p50 {np.median(dur[m]):.1f} us")
    end = np.nanmax(it[:, 4])
    grid_t = np.arange(0.0, end + 2.0, 2.0)
    rate = []
    busy = []
    for x in grid_t:
        live = (it[:, 2] <= x) & (it[:, 4] > x)
        busy.append(int(live.sum()))
        rate.append(float((it[live & regular, 7] * row / np.maximum(dur[live & regular], 1e-3)).sum()
                          / 1e3))  # bytes per us / 1e3 = GB/s
    print("K/V GB/s per 2 us:  " + " ".join(f"{r:.0f}" for r in rate))
    print("busy workgroups:    " + " ".join(str(v) for v in busy))
    ends = (tr[:, 255] - t0) / TICKS_PER_US
    print(f"workgroups finish at (min, p10, p50, p90, max) {np.percentile(ends, [0, 10, 50, 90, 100]).round(1)} us")


if __name__ == "__main__":
    sys.exit(main())
