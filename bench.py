#!/usr/bin/env python3
"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode step of a batch: the batch's new tokens (one per sequence) stored
in their slots and every sequence decoded, as one ``pa_cache_write_decode`` launch (the
cache write fused before the attention; the same step as two calls, ``pa_cache_write``
then ``pa_decode``, is reported beside it).  The headline batch
is the bf16 GQA-8 batch (128 sequences, 64 query / 8 KV heads, head dim 128, block
size 16, log-uniform lengths in [1, 4096], seed 0).  Inputs are resident in HBM before
timing starts; several copies of the batch are rotated so that no step finds its K/V
in L2 or the 256 MB Infinity Cache (each copy is 385 MB, four copies 1.5 GB).

Reported (one JSON line on stdout):
  value      attended KV tokens per second over the whole timed region (K steps,
             host clock, synchronised on both sides)
  roofline   the step's launch timed with HIP events on the stream it runs on, inside
             the same timed region: algorithmic bytes per call (the decode's and the
             new tokens' stores) / mean call duration, against 8 TB/s
  cpu_baseline  the fp64 oracle on the host cores, on the same batch (and one decode of
             it on one thread, for context)
  two_call_step the same step as pa_cache_write + pa_decode, with pa_decode's own roofline
  cache_write   the headline step's pa_cache_write alone (128 tokens), event-timed
  tiny_fp32     the tiny fp32 batch: cache write, decode, and the two as a pair
  copy_blocks   pa_copy_blocks bursts of 128 and 2048 block pairs (copy-on-write), against
             8 TB/s, each copy checked bit for bit
  block_manager host time of the block manager per serving step of the headline batch
  waste      KV slots held paged vs contiguously for the headline length mix, and admission
  parity     GPU output of the last timed step against the oracle
  also       the same decode-only measurement for the long-context batches, and the
             chunked-prefill and draft-verification batches through pa_multi_token
             (against the roof each meets first: MFMA flops or HBM bytes); each warms
             up W steps and then until the device has been busy SECONDARY_WARM_MS
  read_probe what a read-only kernel (pa_read_probe) gets from HBM over 2 GiB in 4 KiB
             tiles, front to back and in a random order; copy_reference a torch copy

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attended KV tokens/s and achieved HBM GB/s (% of peak), decode, 1 MI355X"
PEAK_GBPS = 8000.0  # MI355X HBM3E peak
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA (f32: vector peak)
MALL_BYTES = 256 << 20
# secondary batches: after W warmup steps, keep the device busy this long before timing
SECONDARY_WARM_MS = 50.0
CALIBRATION_BYTES = 256 << 20
HEADLINE = "gqa_bf16"
WORKLOAD_TEXT = {
    "gqa_bf16": "bf16 GQA decode step: 128 seqs, 64 q heads / 8 KV heads, head_dim 128, "
                "block_size 16, log-uniform lengths in [1, 4096], shuffled pool (+10% free); "
                "the 128 new tokens stored and every sequence decoded (one "
                "pa_cache_write_decode launch; two_call_step: the same step as two calls)",
    "long_bf16_bs16": "bf16 long-context split-K decode: 8 seqs, lengths uniform in "
                      "[32768, 131072], 32 q / 8 KV heads, head_dim 128, block_size 16, "
                      "512-token partitions",
    "long_bf16_bs32": "bf16 long-context split-K decode: 8 seqs, lengths uniform in "
                      "[32768, 131072], 32 q / 8 KV heads, head_dim 128, block_size 32, "
                      "512-token partitions",
    "long_bf16_bs16_default": "bf16 long-context split-K decode, default partitioning (sized "
                              "on the device from the lengths; the length used is reported): 8 "
                              "seqs, lengths uniform in [32768, 131072], 32 q / 8 KV heads, "
                              "head_dim 128, block_size 16",
    "long_bf16_bs32_default": "bf16 long-context split-K decode, default partitioning (sized on "
                              "the device from the lengths; the length used is reported): 8 seqs, "
                              "lengths uniform in [32768, 131072], 32 q / 8 KV heads, head_dim "
                              "128, block_size 32",
    "long_bf16_bs16_nosplit": "bf16 long-context decode without a split (one work item per "
                              "sequence and KV head): 8 seqs, lengths uniform in [32768, "
                              "131072], 32 q / 8 KV heads, head_dim 128, block_size 16",
    "mha_fp16": "fp16 MHA decode: 32 seqs, 32 heads, head_dim 128, block_size 16, "
                "lengths uniform in [128, 2048]",
    "prefix_bf16": "bf16 prefix-sharing decode: 64 seqs sharing a 1024-token prefix, "
                   "0-512 private tokens, 32 q / 8 KV heads, head_dim 128, block_size 16",
    "prefill_bf16": "bf16 chunked prefill (pa_multi_token): 8 seqs, a 512-token chunk each on "
                    "1024-8192 cached tokens, causal, 64 q / 8 KV heads, head_dim 128, "
                    "block_size 16",
    "verify_bf16": "bf16 draft-token verification (pa_multi_token, context split): 8 seqs, "
                   "5 new tokens each on 8192-32768 cached tokens, causal, 64 q / 8 KV heads, "
                   "head_dim 128, block_size 16",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def elem_bytes(dtype):
    return 4 if dtype == "f32" else 2


def decode_bytes(b, unique_shared=True):
    """Algorithmic bytes of one pa_decode call: every attended (token, KV head) K and V
    row read once (a block shared by several tables counted once when unique_shared),
    Q read and the output written once, the used table entries and lengths read."""
    import numpy as np
    e = elem_bytes(b.dtype)
    row = b.num_kv_heads * b.head_dim * e * 2
    tokens = b.total_tokens()
    if unique_shared and b.shared_blocks:
        shared_tok = b.shared_blocks * b.block_size
        tokens = shared_tok + int((b.seq_lens.astype(np.int64) - shared_tok).sum())
    nb = int(((b.seq_lens.astype(np.int64) + b.block_size - 1) // b.block_size).sum())
    return tokens * row + 2 * b.num_seqs * b.num_q_heads * b.head_dim * e + 4 * nb + 4 * b.num_seqs


def multi_token_flops(b):
    """Algorithmic flops of one pa_multi_token call: for every (new token, query head)
    pair and every position it sees, a D-long dot product and a D-long weighted sum
    (4D flops)."""
    import numpy as np
    qs = b.query_start.astype(np.int64)
    n = np.diff(qs)
    ctx = b.seq_lens.astype(np.int64) - n
    seen = int((n * ctx + n * (n + 1) // 2).sum())  # sum over j < n of (ctx + j + 1)
    return seen * b.num_q_heads * 4 * b.head_dim


def multi_token_bytes(b):
    """Algorithmic HBM bytes of one pa_multi_token call: each sequence's K and V read
    once, queries read and outputs written once, tables and lengths read."""
    import numpy as np
    e = elem_bytes(b.dtype)
    T = int(b.query_start[-1])
    nb = int(((b.seq_lens.astype(np.int64) + b.block_size - 1) // b.block_size).sum())
    return (b.total_tokens() * b.num_kv_heads * b.head_dim * e * 2 + 2 * T * b.num_q_heads *
            b.head_dim * e + 4 * nb + 8 * b.num_seqs + 4)


def read_probe(nbytes=2 << 30, reps=20):
    """What a kernel that does nothing but read gets from HBM (pa_read_probe): 2 GiB in
    4 KiB tiles, front to back and in a random order (the granule and the placement of a
    shuffled block pool), one 16-byte non-temporal load per thread and tile.  After 50 ms
    of untimed launches, the median of ``reps`` launches timed with an event pair each;
    bytes are the tiles' (the random order also reads 2 MiB of tile ids)."""
    import torch
    import paged_kv_cache_344_amd as pa
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    n = nbytes // 4096
    perm = torch.randperm(n, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(pa.binding.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device="cuda:0")

    def launch(tiles):
        pa.pa_read_probe(x, n, sink, tiles=tiles)
    out = {"bytes_read": nbytes,
           "what": "pa_read_probe: 2 GiB read once in 4 KiB tiles, 16-byte non-temporal loads"}
    for name, tiles in (("stream", None), ("random_4k_tiles", perm)):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.05:
            launch(tiles)
            torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch(tiles)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(ts)[len(ts) // 2]
        out[name] = {"gbps": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / PEAK_GBPS, "seconds": t}
    del x, perm, sink
    torch.cuda.empty_cache()
    return out


def cache_write_bytes(b):
    if b.slot_mapping is None:
        return 0
    T = b.slot_mapping.shape[0]
    return 2 * (2 * T * b.num_kv_heads * b.head_dim * elem_bytes(b.dtype)) + 8 * T


class Copy:
    """One GPU-resident copy of a batch with its calls prepared."""

    def __init__(self, b, partition_size):
        import torch
        import paged_kv_cache_344_amd as pa
        from paged_kv_cache_344_amd.inputs import as_torch
        dev = "cuda:0"
        t = lambda a: as_torch(a, b.dtype, dev)  # noqa: E731
        self.q, self.kc, self.vc = t(b.q), t(b.k_cache), t(b.v_cache)
        self.bt = torch.from_numpy(b.block_tables).to(dev)
        self.sl = torch.from_numpy(b.seq_lens).to(dev)
        self.out = torch.empty_like(self.q)
        self.write = None
        if b.query_start is not None:  # a multi-token batch: pa_multi_token in place of decode
            self.qs = torch.from_numpy(b.query_start).to(dev)
            self.decode = pa.PreparedMultiToken(
                self.q, self.kc, self.vc, self.bt, self.sl, self.qs, b.block_size,
                b.num_kv_heads, b.scale, self.out,
                max_query_len=int((b.query_start[1:] - b.query_start[:-1]).max()),
                max_seq_len=int(b.seq_lens.max()))  # a serving step knows its longest sequence
            return
        self.decode = pa.PreparedDecode(self.q, self.kc, self.vc, self.bt, self.sl, b.block_size,
                                        b.num_kv_heads, b.scale, self.out,
                                        partition_size=partition_size,
                                        shared_blocks=b.shared_blocks > 0)
        if b.slot_mapping is not None:
            self.kn, self.vn = t(b.k_new), t(b.v_new)
            self.sm = torch.from_numpy(b.slot_mapping).to(dev)
            self.write = pa.PreparedCacheWrite(self.kn, self.vn, self.sm, self.kc, self.vc)
            # the same step in one launch: new tokens stored, then decode
            self.step = pa.PreparedDecode(self.q, self.kc, self.vc, self.bt, self.sl,
                                          b.block_size, b.num_kv_heads, b.scale, self.out,
                                          partition_size=partition_size,
                                          shared_blocks=b.shared_blocks > 0,
                                          new_tokens=(self.kn, self.vn, self.sm))


def time_steps(copies, steps, warmup, with_write, fused=False, min_warm_ms=0.0):
    """Run warmup + timed steps rotating over copies; returns (elapsed_s, region_ms,
    [call_ms]).  With min_warm_ms, the warmup goes on (in groups of four steps, each
    group synchronised) until the device has been kept busy for that long: after the
    seconds of host work that build a batch, the first few milliseconds of GPU work
    run measurably slower (draft verification 141 us a call against 114 once warm).
    A step is the decode call, preceded by the batch's cache write when with_write; with
    fused, write and decode are the one pa_cache_write_decode call.  The timed steps run
    twice: first with nothing else in the stream (elapsed_s, bracketed by device
    synchronisation; region_ms: an event pair around them, divided by the steps), then
    with an event pair around each decode call (the fused call when fused) for the
    per-call spread, so that per-call event records are not part of the throughput."""
    import torch
    n = len(copies)

    def run(c, ev=None):
        if fused and with_write and c.write:
            if ev:
                ev[0].record()
            c.step()
        else:
            if with_write and c.write:
                c.write()
            if ev:
                ev[0].record()
            c.decode()
        if ev:
            ev[1].record()
    for k in range(warmup):
        run(copies[k % n])
    torch.cuda.synchronize()
    t_warm, k = time.perf_counter(), warmup
    while (time.perf_counter() - t_warm) * 1e3 < min_warm_ms:
        for _ in range(4):
            run(copies[k % n])
            k += 1
        torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for k in range(steps):
        run(copies[k % n])
    r1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_ms = r0.elapsed_time(r1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for k in range(steps):
        run(copies[k % n], ev[k])
    torch.cuda.synchronize()
    return elapsed, region_ms, [a.elapsed_time(z) for a, z in ev]


def oracle_reference(b):
    """Oracle output for the batch after its cache write, and the host pools."""
    import oracle
    kc, vc = b.k_cache.copy(), b.v_cache.copy()
    if b.slot_mapping is not None:
        oracle.cache_write(b.k_new, b.v_new, b.slot_mapping, kc, vc, b.block_size, b.dtype)
    return kc, vc


def cpu_baseline(b, kc, vc, budget_s):
    """The oracle (unchanged) decoding the whole batch on the host cores, repeated
    until about budget_s seconds have passed (at least once)."""
    import oracle
    threads = oracle.set_threads(0)
    runs, t0, ref = 0, time.perf_counter(), None
    while True:
        ref = oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.block_size,
                            b.num_kv_heads, b.scale, b.dtype)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / runs * (runs + 1) > 3 * budget_s:
            break
    # one thread, for context: one decode of the same batch
    oracle.set_threads(1)
    t1 = time.perf_counter()
    oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.block_size, b.num_kv_heads,
                  b.scale, b.dtype)
    el1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    return ref, dict(value=runs * b.total_tokens() / el, unit="tokens/s", cores=threads,
                     kind="oracle", cpu_model=cpu_model(),
                     sample=f"the whole {b.name} batch (seed {b.seed}, {b.num_seqs} seqs, "
                            f"sum L = {b.total_tokens()}), after its cache write, decoded "
                            f"{runs} time(s) in {el:.1f} s by the fp64 C oracle with "
                            f"{threads} OpenMP threads",
                     single_thread={"value": b.total_tokens() / el1, "unit": "tokens/s",
                                    "sample": f"one decode of the same batch on 1 thread "
                                              f"({el1:.2f} s)"})


def time_calls(calls, n):
    """Event-timed calls (each a zero-argument callable), run in turn n times; returns
    the sorted durations in microseconds."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for k in range(n):
        ev[k][0].record()
        calls[k % len(calls)]()
        ev[k][1].record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(z) * 1e3 for a, z in ev)


def summary_us(ts):
    return {"mean_us": sum(ts) / len(ts), "p10_us": ts[len(ts) // 10],
            "p90_us": ts[(9 * len(ts)) // 10]}


def tiny_pair(seed, n):
    """The tiny fp32 correctness batch (4 sequences, one new token each): cache write
    alone, decode alone, and the write + decode pair, event-timed (launch-bound)."""
    import torch
    from paged_kv_cache_344_amd import inputs
    b = inputs.make_batch("tiny_fp32", seed=seed)
    c = Copy(b, 0)
    for _ in range(5):
        c.write()
        c.decode()
    torch.cuda.synchronize()

    def pair():
        c.write()
        c.decode()
    return dict(workload="fp32 tiny batch: 4 seqs, lengths {5, 10, 17, 33}, block_size 4, "
                         "2 heads (MHA), head_dim 64; one new token per sequence",
                cache_write=summary_us(time_calls([c.write], n)),
                decode=summary_us(time_calls([c.decode], n)),
                write_then_decode=summary_us(time_calls([pair], n)))


def copy_blocks_bytes(pairs, num_kv_heads, block_size, head_dim, elem):
    """Algorithmic bytes of a pa_copy_blocks call: each pair reads and writes one block
    (num_kv_heads * block_size * head_dim elements) of each of the two caches."""
    return pairs * 2 * (num_kv_heads * block_size * head_dim * elem) * 2


def copy_blocks_leg(seed, reps=60):
    """pa_copy_blocks (the device half of copy-on-write) on the GQA pool shape: 8 KV heads,
    block size 16, head size 128, bf16, 32 KiB a block and cache, 16384 blocks a cache.
    Two bursts: 128 pairs (one launch: the copies a 128-sequence fork of partly filled
    last blocks makes) and 2048 pairs (16 launches of 128), each from distinct random
    source blocks to distinct random destinations, several disjoint sets rotated so that
    no call finds its blocks in the caches.  After timing, every copied block is checked
    bit for bit against its source."""
    import numpy as np
    import torch
    from paged_kv_cache_344_amd import binding
    Hkv, bs, D, N = 8, 16, 128, 16384
    torch.manual_seed(seed)
    kc = torch.empty((N, Hkv, bs, D), dtype=torch.bfloat16, device="cuda:0").normal_()
    vc = torch.empty((N, Hkv, D, bs), dtype=torch.bfloat16, device="cuda:0").normal_()
    block_bytes = Hkv * bs * D * 2
    rng = np.random.default_rng(seed)
    out = {"workload": "pa_copy_blocks on the GQA pool shape (8 KV heads, block_size 16, "
                       "head_dim 128, bf16; 32 KiB a block and cache, 16384 blocks a cache): "
                       "random distinct source and destination blocks",
           "block_bytes_per_cache": block_bytes}
    for pairs in (128, 2048):
        perm = rng.permutation(N)
        nsets = min(8, N // (2 * pairs))
        sets = [(perm[2 * k * pairs:(2 * k + 1) * pairs], perm[(2 * k + 1) * pairs:(2 * k + 2) * pairs])
                for k in range(nsets)]
        calls = [binding.PreparedCopyBlocks(kc, vc, s, d) for s, d in sets]
        for c in calls:
            c()
        torch.cuda.synchronize()
        ts = time_calls(calls, reps)
        nbytes = copy_blocks_bytes(pairs, Hkv, bs, D, 2)
        r = summary_us(ts)
        gbps = nbytes / (r["mean_us"] * 1e-6) / 1e9
        exact = all(torch.equal(kc[torch.as_tensor(d)].view(torch.int16),
                                kc[torch.as_tensor(s)].view(torch.int16)) and
                    torch.equal(vc[torch.as_tensor(d)].view(torch.int16),
                                vc[torch.as_tensor(s)].view(torch.int16)) for s, d in sets)
        r.update(pairs=pairs, launches=(pairs + 127) // 128, algorithmic_bytes=nbytes,
                 roofline={"bound": "hbm", "achieved": gbps, "peak": PEAK_GBPS, "unit": "GB/s",
                           "frac": gbps / PEAK_GBPS},
                 bit_exact=bool(exact))
        out[f"pairs_{pairs}"] = r
        log(f"copy_blocks {pairs} pairs: {r['mean_us']:.1f} us, {gbps:.0f} GB/s = "
            f"{gbps / PEAK_GBPS:.1%} of 8 TB/s, bit-exact {exact}")
    del kc, vc
    torch.cuda.empty_cache()
    return out


def block_manager_leg(seed, steps=200):
    """The host block manager (C++, include/pa_block_manager.h) serving the headline
    batch's 128 sequences: each brought to its length, then timed steps of one token
    appended to every sequence (slot ids out) plus an export of the block tables and
    lengths the kernels read, through the C-ABI with marshalled arrays (what a C caller
    pays) and through the Python binding; then a 16-way fork (beam search) and one append
    of parents and children, which makes the copy-on-write copies of shared, partly
    filled last blocks.  Host time only: nothing here touches the GPU."""
    import ctypes
    import time
    import torch
    from paged_kv_cache_344_amd import binding, inputs
    b = inputs.make_batch(HEADLINE, seed)
    S, bs = b.num_seqs, b.block_size
    maxb = (int(b.seq_lens.max()) + 2 * steps + 2 * bs) // bs + 1  # room for every append
    bm = binding.BlockManager(16384, bs, maxb)
    seqs = [bm.add_sequence() for _ in range(S)]
    left = [int(x) for x in b.seq_lens]
    while any(left):
        act = [s for s, n in zip(seqs, left) if n > 0]
        bm.append(act)
        left = [max(0, n - 1) for n in left]
    L, h = binding.lib(), bm.handle
    ids = (ctypes.c_int32 * S)(*seqs)
    slots = (ctypes.c_int64 * S)()
    cs, cd = (ctypes.c_int32 * S)(), (ctypes.c_int32 * S)()
    nc = ctypes.c_int32()
    bt = torch.empty((S, maxb), dtype=torch.int32)
    sl = torch.empty((S,), dtype=torch.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        if L.pa_bm_append(h, ids, S, slots, cs, cd, ctypes.byref(nc)) != 0:
            raise RuntimeError("pa_bm_append failed")
        if L.pa_bm_export(h, ids, S, bt.data_ptr(), sl.data_ptr()) != 0:
            raise RuntimeError("pa_bm_export failed")
    c_us = (time.perf_counter() - t0) / steps * 1e6
    t0 = time.perf_counter()
    for _ in range(steps // 4):
        bm.append(seqs)
        bm.export(seqs)
    py_us = (time.perf_counter() - t0) / (steps // 4) * 1e6
    parents = seqs[:16]
    t0 = time.perf_counter()
    children = [bm.fork(p) for p in parents]
    _, copies = bm.append(parents + children)
    fork_us = (time.perf_counter() - t0) * 1e6
    ok = bool((sl.numpy() == b.seq_lens + steps).all())
    bm.close()
    log(f"block manager: {c_us:.1f} us a step through the C-ABI, {py_us:.1f} us through the "
        f"binding (128 appends + table export); 16-way fork + append {fork_us:.0f} us, "
        f"{len(copies)} copy-on-write copies")
    return {"workload": "host block manager serving the headline batch's 128 sequences "
                        "(block_size 16, 16384 blocks): per step one token appended to every "
                        "sequence plus the export of block tables and lengths",
            "step_us_c_abi": c_us, "step_us_python_binding": py_us,
            "fork16_and_append_us": fork_us, "cow_copies": len(copies),
            "lengths_after_steps_ok": ok}


def waste_leg(seed, pool_slots=65536):
    """KV memory of the headline batch's length mix (log-uniform in [1, 4096], block size
    16) held by contiguous reservations of the longest length against the blocks the
    block manager hands out (measured by growing every request through it), and how many
    of the requests, in order, fit at once in a pool of ``pool_slots`` slots either way."""
    from paged_kv_cache_344_amd import inputs, waste
    b = inputs.make_batch(HEADLINE, seed)
    lengths = [int(x) for x in b.seq_lens]
    reserved = b.max_blocks_per_seq * b.block_size
    r = waste.account(lengths, b.block_size, reserved)
    cont, paged = waste.admitted(lengths, b.block_size, reserved, pool_slots)
    log(f"waste: paged {r.paged_waste_frac:.2%} of its slots, contiguous "
        f"{r.contiguous_waste_frac:.2%}; a {pool_slots}-slot pool admits {cont} requests "
        f"contiguously, {paged} paged")
    return {"workload": f"the headline batch's {len(lengths)} request lengths, block_size "
                        f"{b.block_size}, contiguous reservation {reserved} slots a request",
            "tokens": r.tokens, "paged_slots": r.paged_slots,
            "contiguous_slots": r.contiguous_slots,
            "paged_waste_frac": r.paged_waste_frac,
            "contiguous_waste_frac": r.contiguous_waste_frac,
            "pool_slots": pool_slots, "admitted_contiguous": cont, "admitted_paged": paged}


def copy_reference(nbytes=2 << 30, reps=5):
    """A plain 2 GiB device-to-device copy (torch copy_), for context: bytes read plus
    bytes written per second, median of ``reps`` timed copies."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[len(ts) // 2]
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": 2 * nbytes / t / 1e9, "bytes_moved": 2 * nbytes, "seconds": t,
            "what": "torch device-to-device copy of 2 GiB, read + write counted"}


def cpu_model():
    """The host CPU's model name as lscpu reports it, with its family / model / stepping
    numbers (a virtual machine may name only the product line), or /proc/cpuinfo's."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {}
        for line in out.splitlines():
            k, _, v = line.partition(":")
            f.setdefault(k.strip(), v.strip())
        if f.get("Model name"):
            ids = ", ".join(f"{k.lower()} {f[k]}" for k in ("CPU family", "Model", "Stepping")
                            if f.get(k))
            return f"{f['Model name']} ({ids})" if ids else f["Model name"]
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parity(out, ref, dtype):
    """Same rules as the parity tests: fp32 |d| <= 1e-5 + 1e-5 |ref|; fp16/bf16 |d| <= 1e-2
    (one output ulp where half an ulp at |ref| already exceeds 1e-2) and, element by
    element, |d| <= one output ulp at max(|got|, |ref|) + 2^-10 of the row's rms."""
    import numpy as np
    got = out.double().cpu().numpy()
    d = np.abs(got - ref)
    res = {}
    if dtype == "f32":
        tol = 1e-5 + 1e-5 * np.abs(ref)
        ok = (d <= tol).all()
    else:
        mant, emin = (10, -14) if dtype == "f16" else (7, -126)

        def ulp(x):
            return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin))) - mant)
        tol = np.where(0.5 * ulp(ref) > 1e-2, ulp(ref), 1e-2)
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        bound = ulp(np.maximum(np.abs(got), np.abs(ref))) + 2.0 ** -10 * rms
        res["max_over_ulp_rms_bound"] = float((d / bound).max())
        ok = (d <= tol).all() and (d <= bound).all()
    finite = bool(np.isfinite(got).all())
    res.update(max_abs=float(d.max()),
               rule="fp16/bf16: 1e-2 abs (1 ulp above 4 in bf16) and 1 ulp + 2^-10 rms(row)"
               if dtype != "f32" else "fp32: 1e-5 abs + 1e-5 rel",
               finite=finite, ok=bool(finite and ok))
    return res


def _product_code(text):
    """The source as the product library compiles it: without the diagnostic
    PA_DECODE_TRACE sections (not nested, each closed by the first #endif) and without
    whole-line comments, so that editing either leaves the digest alone."""
    out, skip = [], False
    for line in text.splitlines():
        s = line.strip()
        if s.startswith("#ifdef PA_DECODE_TRACE"):
            skip = True
        elif skip:
            skip = not s.startswith("#endif")
        elif s and not s.startswith("//"):
            out.append(line)
    return "\n".join(out)


def source_digest():
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_common.h", "cache_write.hip", "kernels.h"):
        path = os.path.join(ROOT, "paged_kv_cache_344_amd", "csrc", f)
        h.update(_product_code(open(path).read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, launches_bytes):
    """HBM bytes per decode call from the committed rocprofv3 counter summary, or None
    if there is none for the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_call")


def measure(name, seed, steps, warmup, copies_min, with_write, fused=False, min_warm_ms=0.0):
    import torch
    from paged_kv_cache_344_amd import inputs
    t = time.perf_counter()
    b = inputs.make_batch(name, seed=seed)
    pool = b.k_cache.nbytes + b.v_cache.nbytes
    n_copies = max(copies_min, math.ceil(4 * MALL_BYTES / pool)) if pool < 4 * MALL_BYTES else 1
    log(f"{name}: generated in {time.perf_counter() - t:.1f}s, sum L {b.total_tokens()}, "
        f"pool {pool / 1e6:.0f} MB, {n_copies} GPU copies")
    part = b.partition_size
    copies = [Copy(b, part) for _ in range(n_copies)]
    torch.cuda.synchronize()
    elapsed, region_ms, dms = time_steps(copies, steps, warmup, with_write, fused, min_warm_ms)
    dec_bytes = decode_bytes(b)
    if fused and b.slot_mapping is not None:  # the timed call also stores the new tokens
        dec_bytes += cache_write_bytes(b)
    # a step that is the one launch measured: its mean duration is the timed region's
    # (an event pair around all the steps, divided by their number), which includes any
    # gap between launches but no per-call event records; otherwise the per-call events'
    one_launch = fused or not with_write or b.slot_mapping is None
    mean_ms = region_ms if one_launch else sum(dms) / len(dms)
    srt = sorted(dms)
    if b.query_start is not None:
        dec_bytes = multi_token_bytes(b)
    res = dict(batch=b, copies=copies, elapsed=elapsed, decode_ms=mean_ms,
               decode_ms_event_pairs=sum(dms) / len(dms),
               call_timing=("mean: an event pair around the timed steps, divided by their "
                            "number; p10 / p90: an event pair around each call in a second "
                            "run of the steps (each pair adds its own ~1-2 us)"
                            if one_launch else "an event pair around each call"),
               decode_ms_p10=srt[len(srt) // 10], decode_ms_p90=srt[(9 * len(srt)) // 10],
               decode_bytes=dec_bytes, write_bytes=cache_write_bytes(b) if with_write else 0,
               gbps=dec_bytes / (mean_ms * 1e-3) / 1e9, n_copies=n_copies)
    log(f"{name}: {steps} steps in {elapsed * 1e3:.2f} ms; decode call {mean_ms * 1e3:.1f} us "
        f"(p10 {res['decode_ms_p10'] * 1e3:.1f}, p90 {res['decode_ms_p90'] * 1e3:.1f}); "
        f"{res['gbps']:.0f} GB/s = {res['gbps'] / PEAK_GBPS:.1%} of peak")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=4, help="minimum rotated copies of a batch")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="long_bf16_bs16,long_bf16_bs32,long_bf16_bs16_default,"
                    "long_bf16_bs32_default,long_bf16_bs16_nosplit,"
                    "mha_fp16,prefix_bf16,prefill_bf16,verify_bf16",
                    help="comma-separated secondary batches measured decode-only ('' for none)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 256 MiB device-to-device copy, a dispatch of known size "
                         "against which rocprofv3's FETCH_SIZE / WRITE_SIZE counters are scaled")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this library "
              "runs its hot path on a single MI355X)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    from paged_kv_cache_344_amd.binding import lib
    lib()
    if args.calibrate_copy:
        src = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {CALIBRATION_BYTES} bytes read and {CALIBRATION_BYTES} written")
        del src, dst
        torch.cuda.empty_cache()

    head = measure(HEADLINE, args.seed, args.steps, args.warmup, args.copies, with_write=True,
                   fused=True)
    head_part = head["copies"][0].step.partition_used()
    log(f"{HEADLINE}: partition length used {head_part}")
    b = head["batch"]
    tokens = b.total_tokens()
    value = args.steps * tokens / head["elapsed"]
    last = head["copies"][(args.steps - 1) % head["n_copies"]]
    head_out = last.out.clone()  # the last timed step's output, for the parity check

    # the same step as two calls, pa_cache_write then pa_decode (same copies), for context
    el2, _, dms2 = time_steps(head["copies"], args.steps, args.warmup, with_write=True,
                              fused=False)
    dec_bytes = decode_bytes(b)
    dec_ms = sum(dms2) / len(dms2)
    two_call = {"value": args.steps * tokens / el2, "unit": "tokens/s",
                "ms_per_step": el2 / args.steps * 1e3,
                "decode_call_us": dec_ms * 1e3,
                "decode_roofline": {"bound": "hbm", "achieved": dec_bytes / (dec_ms * 1e-3) / 1e9,
                                    "peak": PEAK_GBPS, "unit": "GB/s",
                                    "frac": dec_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_GBPS,
                                    "traffic": measured_traffic(f"{HEADLINE}/pa_decode", dec_bytes),
                                    "algorithmic_bytes_per_call": dec_bytes},
                "what": "pa_cache_write (128 tokens) then pa_decode: two launches"}
    log(f"{HEADLINE} as two calls: {two_call['ms_per_step'] * 1e3:.1f} us per step, decode call "
        f"{two_call['decode_call_us']:.1f} us "
        f"({two_call['decode_roofline']['frac']:.1%} of 8 TB/s)")

    # the cache write of the headline step alone (same copies, same slots each time)
    cw = summary_us(time_calls([c.write for c in head["copies"]], max(50, args.steps // 2)))
    cw_bytes = cache_write_bytes(b)
    cw.update(tokens=int(b.slot_mapping.shape[0]), bytes=cw_bytes,
              gbps=cw_bytes / (cw["mean_us"] * 1e-6) / 1e9)
    log(f"cache write alone: {cw['mean_us']:.1f} us for {cw['tokens']} tokens")

    kc, vc = oracle_reference(b)
    if args.no_cpu_baseline:
        import oracle
        ref = oracle.decode(b.q, kc, vc, b.block_tables, b.seq_lens, b.block_size,
                            b.num_kv_heads, b.scale, b.dtype)
        cpu = None
    else:
        ref, cpu = cpu_baseline(b, kc, vc, args.cpu_seconds)
        log(f"cpu baseline: {cpu['value']:.3g} tokens/s on {cpu['cores']} threads")
    par = parity(head_out, ref, b.dtype)
    log(f"parity: {par}")

    also = {}
    for name in [x for x in args.also.split(",") if x]:
        r = measure(name, args.seed, max(20, args.steps // 4), args.warmup, 1, with_write=False,
                    min_warm_ms=SECONDARY_WARM_MS)
        rb = r["batch"]
        if rb.query_start is not None:
            fl = multi_token_flops(rb)
            tf = fl / (r["decode_ms"] * 1e-3) / 1e12
            # the bound is the roof the call meets first: matrix cores when its flops per
            # algorithmic byte exceed the machine's balance point, HBM otherwise
            if fl / r["decode_bytes"] > PEAK_TFLOPS[rb.dtype] * 1e12 / (PEAK_GBPS * 1e9):
                roof = {"bound": "mfma", "achieved": tf, "peak": PEAK_TFLOPS[rb.dtype],
                        "unit": "TFLOP/s", "frac": tf / PEAK_TFLOPS[rb.dtype]}
            else:
                roof = {"bound": "hbm", "achieved": r["gbps"], "peak": PEAK_GBPS,
                        "unit": "GB/s", "frac": r["gbps"] / PEAK_GBPS}
            also[name] = dict(workload=WORKLOAD_TEXT.get(name, name),
                              new_tokens=int(rb.query_start[-1]), sum_L=rb.total_tokens(),
                              call_us=r["decode_ms"] * 1e3, call_us_p10=r["decode_ms_p10"] * 1e3,
                              call_us_event_pairs=r["decode_ms_event_pairs"] * 1e3,
                              call_us_p90=r["decode_ms_p90"] * 1e3, algorithmic_flops=fl,
                              roofline=roof, algorithmic_bytes=r["decode_bytes"],
                              achieved_gbps=r["gbps"],
                              split_workspace_bytes=r["copies"][0].decode.workspace_bytes)
            log(f"{name}: {tf:.0f} TFLOP/s = {tf / PEAK_TFLOPS[rb.dtype]:.1%} of dense MFMA peak; "
                f"{r['gbps']:.0f} GB/s = {r['gbps'] / PEAK_GBPS:.1%} of HBM peak "
                f"(bound: {roof['bound']})")
            del r
            torch.cuda.empty_cache()
            continue
        used = r["copies"][0].decode.partition_used()
        also[name] = dict(workload=WORKLOAD_TEXT.get(name, name), sum_L=rb.total_tokens(),
                          partition_size=rb.partition_size or "default",
                          partition_used=used,
                          tokens_per_s=rb.total_tokens() / (r["decode_ms"] * 1e-3),
                          decode_us=r["decode_ms"] * 1e3, decode_us_p10=r["decode_ms_p10"] * 1e3,
                          decode_us_event_pairs=r["decode_ms_event_pairs"] * 1e3,
                          decode_us_p90=r["decode_ms_p90"] * 1e3,
                          algorithmic_bytes=r["decode_bytes"], achieved_gbps=r["gbps"],
                          frac_of_peak=r["gbps"] / PEAK_GBPS)
        if rb.shared_blocks:  # prefix sharing: also the bytes as if nothing were shared
            lb = decode_bytes(rb, unique_shared=False)
            also[name].update(logical_bytes=lb,
                              logical_gbps=lb / (r["decode_ms"] * 1e-3) / 1e9)
        del r
        torch.cuda.empty_cache()

    tiny = tiny_pair(args.seed, 100)
    cow = copy_blocks_leg(args.seed)
    bmgr = block_manager_leg(args.seed)
    wst = waste_leg(args.seed)
    log(f"tiny batch: write + decode {tiny['write_then_decode']['mean_us']:.1f} us")
    copy = copy_reference()
    rd = read_probe()
    log(f"read probe, 2 GiB: front to back {rd['stream']['gbps']:.0f} GB/s = "
        f"{rd['stream']['frac']:.1%} of 8 TB/s; random 4 KiB tiles "
        f"{rd['random_4k_tiles']['gbps']:.0f} GB/s = {rd['random_4k_tiles']['frac']:.1%}")
    log(f"torch copy of 2 GiB: {copy['gbps']:.0f} GB/s = {copy['gbps'] / PEAK_GBPS:.1%} of 8 TB/s")
    # the headline step's rate against what a read-only kernel gets from shuffled tiles
    rd["headline_over_random_4k_tiles"] = head["gbps"] / rd["random_4k_tiles"]["gbps"]
    log(f"headline step: {rd['headline_over_random_4k_tiles']:.1%} of the read probe's "
        f"random-tile rate")
    traffic = measured_traffic(f"{HEADLINE}/pa_cache_write_decode", head["decode_bytes"])
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["elapsed"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[HEADLINE], "batch": HEADLINE, "seed": args.seed,
                   "num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": b.block_size, "sum_L": tokens,
                   "partition_size": b.partition_size or "default (chosen on the device)",
                   "partition_used": head_part,
                   "rotated_copies": head["n_copies"], "parallelism": "1 GPU"},
        "roofline": {"bound": "hbm", "achieved": head["gbps"], "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": head["gbps"] / PEAK_GBPS, "traffic": traffic,
                     "kernel": "decode_kernel<bf16, D=128, bs=16> (fused instance): one launch "
                               "per pa_cache_write_decode call (the new tokens' stores, the "
                               "partitions and the split-K merge in the same launch)",
                     "algorithmic_bytes_per_call": head["decode_bytes"],
                     "mean_call_us": head["decode_ms"] * 1e3,
                     "call_timing": head["call_timing"],
                     "event_pair_mean_call_us": head["decode_ms_event_pairs"] * 1e3,
                     "p10_call_us": head["decode_ms_p10"] * 1e3,
                     "p90_call_us": head["decode_ms_p90"] * 1e3},
        "cpu_baseline": cpu,
        "parity": par,
        "step_bytes": head["decode_bytes"],
        "two_call_step": two_call,
        "cache_write": cw,
        "tiny_fp32": tiny,
        "copy_blocks": cow,
        "block_manager": bmgr,
        "waste": wst,
        "also": also,
        "copy_reference": copy,
        "read_probe": rd,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
