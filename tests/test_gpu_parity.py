"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Cache writes and block addressing must be bit-exact; attention outputs must be
within 1e-5 (abs + rel) for fp32 and 1e-2 abs for fp16/bf16 (one output ulp where
the final rounding alone exceeds 1e-2; see tests/helpers.check_close)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_344_amd import inputs
from tests.gpu_helpers import OnGpu, oracle_after_write, oracle_decode, raw_bytes, say
from tests.helpers import check_close, nan_storage, table_array

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _parity(b, partition_size=0, what=""):
    g = OnGpu(b)  # applies the batch's cache write first, as a decode step does
    got = g.out_f64(g.decode(partition_size))
    kc, vc = oracle_after_write(b)
    ref = oracle_decode(b, kc, vc)
    rep = check_close(got, ref, b.dtype, what or b.name)
    say(f"parity {what or b.name}: {rep}")
    return g, got, ref


# ------------------------------------------------------------------ cache write

@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", {}),
    ("gqa_bf16", dict(num_seqs=40, lens=("loguniform", 1, 700), max_blocks_per_seq=44)),
    ("gqa_bf16", dict(num_seqs=24, dtype="f16", block_size=4, max_blocks_per_seq=130,
                      lens=("loguniform", 1, 500))),
    ("gqa_bf16", dict(num_seqs=16, block_size=32, head_dim=64, max_blocks_per_seq=20,
                      lens=("uniform", 1, 600))),
])
def test_cache_write_bit_exact(name, over):
    """Every byte of both pools after the write equals the oracle's pools: the new
    tokens land in exactly their slots and nothing else changes (NaN poison included)."""
    b = inputs.make_batch(name, seed=2, **over)
    g = OnGpu(b, write=False)
    g.cache_write()
    torch.cuda.synchronize()
    kc, vc = oracle_after_write(b)
    np.testing.assert_array_equal(raw_bytes(g.k_cache), kc.view(np.uint8).reshape(-1))
    np.testing.assert_array_equal(raw_bytes(g.v_cache), vc.view(np.uint8).reshape(-1))


def test_cache_write_skips_negative_and_out_of_pool_slots():
    b = inputs.make_batch("tiny_fp32", seed=4)
    g = OnGpu(b, write=False)
    slots = b.slot_mapping.copy()
    slots[1] = -1
    slots[2] = b.num_blocks * b.block_size        # one past the pool: ignored, never written
    g.slots = torch.from_numpy(slots).to("cuda:0")
    g.cache_write()
    torch.cuda.synchronize()
    keep = slots.copy()
    keep[2] = -1
    kc, vc = b.k_cache.copy(), b.v_cache.copy()
    oracle.cache_write(b.k_new, b.v_new, keep, kc, vc, b.block_size, b.dtype)
    np.testing.assert_array_equal(raw_bytes(g.k_cache), kc.view(np.uint8).reshape(-1))
    np.testing.assert_array_equal(raw_bytes(g.v_cache), vc.view(np.uint8).reshape(-1))


# ------------------------------------------------------------------ decode parity

SMALL = [
    ("tiny_fp32", {}),
    ("mha_fp16", dict(num_seqs=6, lens=("uniform", 1, 300), max_blocks_per_seq=19)),
    ("gqa_bf16", dict(num_seqs=24, lens=("loguniform", 1, 1500), max_blocks_per_seq=94)),
    ("prefix_bf16", dict(num_seqs=10, lens=("prefix", 256, 0, 200), max_blocks_per_seq=29)),
    ("long_bf16_bs16", dict(num_seqs=2, lens=("uniform", 1500, 2600), max_blocks_per_seq=163)),
    ("long_bf16_bs32", dict(num_seqs=2, lens=("uniform", 1500, 2600), max_blocks_per_seq=82)),
]


@pytest.mark.parametrize("name,over", SMALL)
@pytest.mark.parametrize("gain", [1.0, 4.0])
def test_decode_parity_small(name, over, gain):
    b = inputs.make_batch(name, seed=1, q_gain=gain, **over)
    _parity(b, what=f"{name} gain={gain}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 8, 16, 32])
def test_decode_parity_dtype_shape_grid(dtype, D, bs):
    """Every compiled (dtype, head dim, block size) instance, GQA-4 and a ragged tail,
    lengths spanning several 512-token partitions."""
    mb = (1300 + bs - 1) // bs
    b = inputs.make_batch("gqa_bf16", seed=3, dtype=dtype, head_dim=D, block_size=bs,
                          num_seqs=5, num_q_heads=8, num_kv_heads=2, max_blocks_per_seq=mb,
                          lens=("fixed", [1, 31, 33, 517, 1300]))
    _parity(b, what=f"{dtype} D={D} bs={bs}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (12, 4), (16, 1), (40, 2)])
def test_decode_parity_group_sizes(Hq, Hkv):
    """Group sizes 1, 3, 16 and 20 (two 16-head tiles, the second one partial)."""
    b = inputs.make_batch("gqa_bf16", seed=5, num_seqs=4, num_q_heads=Hq, num_kv_heads=Hkv,
                          max_blocks_per_seq=50, lens=("fixed", [3, 200, 513, 800]))
    _parity(b, what=f"Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("part", [32, 64, 96, 512, -1])
def test_forced_split_and_no_split(part):
    b = inputs.make_batch("gqa_bf16", seed=6, num_seqs=6, max_blocks_per_seq=70,
                          lens=("fixed", [1, 32, 33, 511, 512, 1100]))
    _parity(b, partition_size=part, what=f"partition={part}")


# ------------------------------------------------------------------ invariants (bit-exact)

def test_placement_independence_is_bit_exact():
    b = inputs.make_batch("gqa_bf16", seed=8, num_seqs=20, lens=("loguniform", 1, 900),
                          max_blocks_per_seq=57, cache_write=False)
    g = OnGpu(b)
    base = g.decode().clone()
    perm = np.random.default_rng(1).permutation(b.num_blocks)
    kc2 = np.empty_like(b.k_cache)
    vc2 = np.empty_like(b.v_cache)
    kc2[perm] = b.k_cache
    vc2[perm] = b.v_cache
    bt2 = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc2, "v_cache": vc2, "block_tables": bt2})
    moved = OnGpu(b2).decode().clone()
    assert torch.equal(moved.view(torch.int16), base.view(torch.int16))


def test_shared_prefix_equals_private_copies_bit_exact():
    """Tables sharing prefix blocks give the same bits as private copies of those
    blocks, with either cache policy of the K/V loads (shared_blocks on or off)."""
    b = inputs.make_batch("prefix_bf16", seed=9, num_seqs=12, lens=("prefix", 512, 0, 300),
                          max_blocks_per_seq=51)
    g = OnGpu(b)
    shared = g.decode(shared_blocks=True).clone()
    streamed = g.decode(shared_blocks=False).clone()
    assert torch.equal(streamed.view(torch.int16), shared.view(torch.int16))
    extra = b.shared_blocks * b.num_seqs
    kc = np.concatenate([b.k_cache, np.zeros((extra,) + b.k_cache.shape[1:], b.k_cache.dtype)])
    vc = np.concatenate([b.v_cache, np.zeros((extra,) + b.v_cache.shape[1:], b.v_cache.dtype)])
    bt = b.block_tables.copy()
    nxt = b.num_blocks
    for s in range(b.num_seqs):
        for j in range(b.shared_blocks):
            kc[nxt] = b.k_cache[bt[s, j]]
            vc[nxt] = b.v_cache[bt[s, j]]
            bt[s, j] = nxt
            nxt += 1
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc, "v_cache": vc, "block_tables": bt,
                         "num_blocks": nxt})
    private = OnGpu(b2).decode().clone()
    assert torch.equal(private.view(torch.int16), shared.view(torch.int16))
    check_close(OnGpu(b).out_f64(shared), oracle_decode(b), "bf16", "shared prefix")


def test_table_tail_contents_are_never_read():
    b = inputs.make_batch("gqa_bf16", seed=10, num_seqs=16, lens=("loguniform", 1, 600),
                          max_blocks_per_seq=40)
    g = OnGpu(b)
    base = g.decode().clone()
    bt = b.block_tables.copy()
    bt[bt < 0] = np.iinfo(np.int32).max
    junk = g.decode(block_tables=torch.from_numpy(bt).cuda(), out=torch.empty_like(g.out))
    assert torch.equal(junk.view(torch.int16), base.view(torch.int16))


def test_deterministic_over_repeats():
    b = inputs.make_batch("gqa_bf16", seed=11, num_seqs=32, lens=("loguniform", 1, 3000),
                          max_blocks_per_seq=188)
    g = OnGpu(b)
    first = g.decode().clone()
    for _ in range(9):
        assert torch.equal(g.decode().view(torch.int16), first.view(torch.int16))


# ------------------------------------------------------------------ needles and edges

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_needles_at_block_and_partition_edges(dtype):
    """A key aligned with the query at t = 0, bs-1, bs, 511, 512, 513 and the last token
    takes nearly all the weight, so the output is that token's value."""
    L, bs, D = 1200, 16, 128
    positions = [0, bs - 1, bs, 511, 512, 513, L - 1]
    S = len(positions)
    b = inputs.make_batch("gqa_bf16", seed=12, dtype=dtype, num_seqs=S, num_q_heads=4,
                          num_kv_heads=4, max_blocks_per_seq=L // bs + 1,
                          lens=("fixed", [L] * S), cache_write=False)
    kc = b.k_cache.copy()
    q32 = oracle.decode_elements(b.q, dtype).astype(np.float32)
    for s, j in enumerate(positions):
        blk, off = b.block_tables[s, j // bs], j % bs
        for h in range(4):
            u = q32[s, h] / np.linalg.norm(q32[s, h])
            kc[blk, h, off, :] = inputs.to_storage((20.0 * u).astype(np.float32), dtype)
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc})
    g = OnGpu(b2)
    got = g.out_f64(g.decode())
    ref = oracle_decode(b2)
    check_close(got, ref, dtype, f"needles {dtype}")
    for s, j in enumerate(positions):
        blk, off = b.block_tables[s, j // bs], j % bs
        vj = oracle.decode_elements(b.v_cache[blk, :, :, off], dtype)
        assert np.abs(ref[s] - vj).max() < 0.05       # the needle dominates
        assert np.abs(got[s] - vj).max() < 0.06


def test_worked_example_incremental_on_gpu():
    """Ten tokens appended one at a time into blocks 5, 12, 3 (block size 4), a decode
    after each append, every step against the oracle doing the same."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    p, d = g["printed"], g["derived"]
    n, bs, tab = p["tokens"], p["block_size"], p["block_table"]
    Hkv, Hq, D, N = 2, 4, 64, max(tab) + 1
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        kc = nan_storage(dtype, (N, Hkv, bs, D))
        vc = nan_storage(dtype, (N, Hkv, D, bs))
        ks = inputs.to_storage(rng.standard_normal((n, Hkv, D)).astype(np.float32), dtype)
        vs = inputs.to_storage(rng.standard_normal((n, Hkv, D)).astype(np.float32), dtype)
        q = inputs.to_storage(rng.standard_normal((1, Hq, D)).astype(np.float32), dtype)
        bt = table_array([tab], 3)
        dev = dict(kc=inputs.as_torch(kc, dtype, "cuda:0"), vc=inputs.as_torch(vc, dtype, "cuda:0"))
        qg = inputs.as_torch(q, dtype, "cuda:0")
        btg = torch.from_numpy(bt).cuda()
        out = torch.empty_like(qg)
        import paged_kv_cache_344_amd as pa
        for t in range(n):
            slot = np.array([d["token_slots"][t]], np.int64)
            oracle.cache_write(ks[t:t + 1], vs[t:t + 1], slot, kc, vc, bs, dtype)
            say(f"worked example {dtype} token {t}")
            pa.pa_cache_write(inputs.as_torch(ks[t:t + 1], dtype, "cuda:0"),
                              inputs.as_torch(vs[t:t + 1], dtype, "cuda:0"),
                              torch.from_numpy(slot).cuda(), dev["kc"], dev["vc"])
            lens = np.array([t + 1], np.int32)
            pa.pa_decode(qg, dev["kc"], dev["vc"], btg, torch.from_numpy(lens).cuda(), bs, Hkv,
                         0.125, out)
            torch.cuda.synchronize()
            ref = oracle.decode(q, kc, vc, bt, lens, bs, Hkv, 0.125, dtype)
            check_close(out.double().cpu().numpy(), ref, dtype, f"worked example t={t}")
        np.testing.assert_array_equal(raw_bytes(dev["kc"]), kc.view(np.uint8).reshape(-1))
        np.testing.assert_array_equal(raw_bytes(dev["vc"]), vc.view(np.uint8).reshape(-1))


# ------------------------------------------------------------------ contract violations

def test_empty_bad_length_and_bad_block_rows():
    """Length 0 gives zeros; a length the table cannot hold, or a used table entry
    outside the pool, gives NaN rows for that sequence only (no fault, no stray write)."""
    b = inputs.make_batch("gqa_bf16", seed=14, num_seqs=6, max_blocks_per_seq=40,
                          lens=("fixed", [100, 200, 300, 400, 500, 600]))
    g = OnGpu(b)
    lens = b.seq_lens.copy()
    lens[0] = 0
    lens[1] = b.max_blocks_per_seq * b.block_size + 1
    lens[2] = -5
    bt = b.block_tables.copy()
    bt[3, 2] = b.num_blocks          # past the pool
    bt[4, 0] = -1                    # inside the used range
    out = g.decode(block_tables=torch.from_numpy(bt).cuda(),
                   seq_lens=torch.from_numpy(lens).cuda(), out=torch.empty_like(g.out))
    o = out.double().cpu().numpy()
    assert (o[0] == 0).all()
    for s in (1, 2, 3, 4):
        assert np.isnan(o[s]).all(), s
    ref = oracle_decode(b, seqs=[5])
    check_close(o[5:6], ref, "bf16", "untouched row")
    # the same with forced split (errors must survive the merge)
    out2 = g.decode(partition_size=64, block_tables=torch.from_numpy(bt).cuda(),
                    seq_lens=torch.from_numpy(lens).cuda(), out=torch.empty_like(g.out))
    o2 = out2.double().cpu().numpy()
    assert (o2[0] == 0).all() and all(np.isnan(o2[s]).all() for s in (1, 2, 3, 4))
    check_close(o2[5:6], ref, "bf16", "untouched row (split)")


# ------------------------------------------------------------------ full-size batches

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["mha_fp16", "gqa_bf16", "prefix_bf16"])
def test_full_size_parity(name, seed):
    """The benchmark batches at full size, default partitioning, on the three seeds of
    the input recipe (seed 0 is the one measured)."""
    b = inputs.make_batch(name, seed=seed)
    _parity(b, what=f"{name} full seed {seed}")


# ------------------------------------------------------------------ workspace and launch slicing

def _counters_nonzero(ws, nctr):
    """Nonzero bytes among the queue and merge counters (the workspace's first nctr
    bytes), leaving out bytes 64..67, which record the partition length used."""
    from paged_kv_cache_344_amd.binding import PART_SLOT_BYTE
    head = ws[:nctr].clone()
    head[PART_SLOT_BYTE:PART_SLOT_BYTE + 4] = 0
    return int(torch.count_nonzero(head))


def _counter_bytes(b, partition_size):
    """Bytes at the start of a decode workspace that hold the queue and the merge
    counters: [queue, 256 B][group counters][root counters], each rounded to 256 B."""
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    mt = b.max_blocks_per_seq * b.block_size
    part = partition_size or 512
    pmax = (mt + part - 1) // part
    ht2 = b.num_kv_heads * ((b.group + 15) // 16)
    nodes = (pmax + 15) // 16
    return r(r(256 + b.num_seqs * ht2 * nodes * 4) + b.num_seqs * ht2 * 4)


def test_workspace_counters_return_to_zero_and_it_is_reusable():
    """Every call returns the queue and the group and root counters to zero, so one
    workspace serves successive calls of one shape, including the two-level merge (more
    than 16 partitions) and sequences of one partition; re-zeroed, it serves a smaller
    shape the same way."""
    import paged_kv_cache_344_amd as pa
    big = inputs.make_batch("gqa_bf16", seed=15, num_seqs=12, max_blocks_per_seq=120,
                            lens=("fixed", [1, 2, 31, 32, 33, 100, 511, 512, 513, 1024, 1800, 1920]))
    small = inputs.make_batch("gqa_bf16", seed=16, num_seqs=5, max_blocks_per_seq=60,
                              lens=("fixed", [7, 64, 300, 700, 950]))
    gb, gs = OnGpu(big), OnGpu(small)
    ws = pa.workspace_for(gb.q, gb.block_tables, big.num_blocks, big.block_size,
                          big.num_kv_heads, partition_size=32)
    need_small = pa.pa_decode_workspace_bytes(gs.q, gs.block_tables, small.num_blocks,
                                              small.block_size, small.num_kv_heads, 32)
    assert need_small <= ws.numel()
    for b, g in ((big, gb), (small, gs)):
        ws.zero_()  # a new shape starts from a zero-filled workspace
        for rep in range(3):
            say(f"workspace reuse rep {rep} {b.name} S={b.num_seqs}")
            out = torch.empty_like(g.q)
            pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                         b.num_kv_heads, b.scale, out, workspace=ws, partition_size=32)
            torch.cuda.synchronize()
            nctr = _counter_bytes(b, 32)
            assert _counters_nonzero(ws, nctr) == 0, "counters not zero after the call"
            check_close(g.out_f64(out), oracle_decode(b), "bf16", f"reuse {rep} S={b.num_seqs}")


def test_more_sequences_than_one_launch_plans():
    """1100 sequences take two launches (1024 + 76); every row matches the oracle."""
    b = inputs.make_batch("gqa_bf16", seed=17, num_seqs=1100, num_q_heads=16, num_kv_heads=4,
                          max_blocks_per_seq=40, lens=("loguniform", 1, 640))
    _parity(b, what="1100 sequences")
    _parity(b, partition_size=64, what="1100 sequences, 64-token partitions")


# ------------------------------------------------------------------ default partitioning

@pytest.mark.parametrize("lens,hq,hkv", [
    ([20000, 17000, 23456], 32, 8),          # dozens of partitions, two-level merges
    ([1, 2, 3], 8, 8),                        # fewer items than workgroups
    ([4096] + [1] * 40 + [700] * 3, 64, 8),   # one long sequence among many one-chunk ones
    ([5000, 33, 0, 64, 9000], 160, 8),        # two head tiles per KV head, an empty sequence
])
def test_default_partitioning_parity(lens, hq, hkv):
    b = inputs.make_batch("gqa_bf16", seed=21, num_seqs=len(lens), num_q_heads=hq,
                          num_kv_heads=hkv, max_blocks_per_seq=(max(lens) + 15) // 16 + 1,
                          lens=("fixed", lens), cache_write=False)
    _parity(b, partition_size=0, what=f"default partitioning lens={lens[:4]}...")


def test_default_partitioning_workspace_reuse_is_bit_stable():
    """With the default partitioning one workspace serves repeated calls of one shape
    (re-zeroed between shapes), its counters are zero after every call, and repeated
    calls give the same bits."""
    import paged_kv_cache_344_amd as pa
    big = inputs.make_batch("gqa_bf16", seed=22, num_seqs=6, max_blocks_per_seq=700,
                            lens=("fixed", [1, 11000, 512, 5000, 33, 9000]), cache_write=False)
    small = inputs.make_batch("gqa_bf16", seed=23, num_seqs=3, max_blocks_per_seq=300,
                              lens=("fixed", [4000, 70, 4700]), cache_write=False)
    gb, gs = OnGpu(big), OnGpu(small)
    ws = pa.workspace_for(gb.q, gb.block_tables, big.num_blocks, big.block_size, big.num_kv_heads)
    first = {}
    for b, g in ((big, gb), (small, gs)):
        ws.zero_()
        for rep in range(3):
            say(f"default reuse rep {rep} S={b.num_seqs}")
            out = torch.empty_like(g.q)
            pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                         b.num_kv_heads, b.scale, out, workspace=ws)
            torch.cuda.synchronize()
            nctr = _counter_bytes(b, 0)
            assert _counters_nonzero(ws, nctr) == 0, "counters not zero after the call"
            got = g.out_f64(out)
            if rep == 0:
                check_close(got, oracle_decode(b), "bf16", f"default reuse S={b.num_seqs}")
                first[b.num_seqs] = got
            else:
                np.testing.assert_array_equal(got, first[b.num_seqs])


def test_many_one_chunk_partitions_parity_and_repeats():
    """Several thousand items of one-chunk partitions (32 tokens, so three of the four
    waves of an item have no chunk), sequences with odd and even partition counts,
    merges over several groups of 16; three repeats on one workspace give the same bits
    and leave the counters at zero."""
    import paged_kv_cache_344_amd as pa
    lens = [1, 33, 64, 65, 96, 97, 500, 1000, 2000, 3000, 3333, 4097, 5000, 6001]
    b = inputs.make_batch("gqa_bf16", seed=24, num_seqs=len(lens), max_blocks_per_seq=376,
                          lens=("fixed", lens), cache_write=False)
    full = sum((L + 31) // 32 - 1 for L in lens)
    assert full * b.num_kv_heads > 6000
    g = OnGpu(b)
    ws = pa.workspace_for(g.q, g.block_tables, b.num_blocks, b.block_size, b.num_kv_heads,
                          partition_size=32)
    ref = oracle_decode(b)
    first = None
    for rep in range(3):
        say(f"one-chunk partitions rep {rep}")
        out = torch.empty_like(g.q)
        pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                     b.num_kv_heads, b.scale, out, workspace=ws, partition_size=32)
        torch.cuda.synchronize()
        assert _counters_nonzero(ws, _counter_bytes(b, 32)) == 0
        got = g.out_f64(out)
        if first is None:
            say(f"one-chunk partitions: {check_close(got, ref, 'bf16', 'one-chunk partitions')}")
            first = got
        else:
            np.testing.assert_array_equal(got, first)


def test_default_partitioning_lengthens_partitions():
    """With the default partition size the kernel sizes partitions from the lengths (here
    142,924 tokens x 8 KV heads over 2 x 256 workgroups at bf16, head dim 128: 2304-token
    partitions: 18 for the longest sequence, in two merge groups, and one for the
    sequences of 1, 513 and 1025 tokens).  That and explicit 512-token
    partitions both match the oracle, and repeated default calls give the same bits."""
    lens = [40000, 35000, 30000, 16385, 1, 513, 1025, 20000]
    b = inputs.make_batch("gqa_bf16", seed=25, num_seqs=len(lens), num_q_heads=32,
                          num_kv_heads=8, max_blocks_per_seq=2501, lens=("fixed", lens),
                          cache_write=False)
    g = OnGpu(b)
    ref = oracle_decode(b)
    auto = g.out_f64(g.decode(0))
    say(f"default partitioning, many items: {check_close(auto, ref, 'bf16', 'default, many items')}")
    np.testing.assert_array_equal(g.out_f64(g.decode(0)), auto)
    say(f"explicit 512: {check_close(g.out_f64(g.decode(512)), ref, 'bf16', 'explicit 512')}")


def _documented_partition(b, grid):
    """The default partition length as include/pa.h states it: one workgroup's even share
    of the (token, KV head tile) work, rounded up to a multiple of 256 tokens, or 3/4 of
    the share when at that length no sequence would be split but the (sequence, head
    tile) units outnumber the workgroups; at least 512."""
    max_tokens = b.max_blocks_per_seq * b.block_size
    lens = [int(n) for n in b.seq_lens if 0 < int(n) <= max_tokens]
    g = b.num_q_heads // b.num_kv_heads
    ht2 = b.num_kv_heads * -(-g // 16)
    share = sum(lens) * ht2 / grid

    def up256(x):
        return -(-int(np.ceil(min(x, max_tokens))) // 256) * 256
    pt = up256(1.0 * share)
    if pt >= max(lens) and len(lens) * ht2 > grid:
        pt = up256(0.75 * share)
    return max(512, pt)


@pytest.mark.parametrize("name,want", [("gqa_bf16", 1536), ("mha_fp16", 1792),
                                       ("prefix_bf16", 1536), ("long_bf16_bs16_default", 8448)])
def test_default_partition_rule_on_the_benchmark_batches(name, want):
    """The partition length the device chooses equals the documented rule (two workgroups
    a compute unit: these batches have more units than that), and, on MI355X's 256
    compute units, the length the measurements in the design notes were taken at."""
    import paged_kv_cache_344_amd as pa
    b = inputs.make_batch(name, seed=0)
    g = OnGpu(b)
    ws = pa.workspace_for(g.q, g.block_tables, b.num_blocks, b.block_size, b.num_kv_heads,
                          partition_size=0)
    out = torch.empty_like(g.q)
    say(f"pa_decode {name} default partitioning (rule check)")
    pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                 b.num_kv_heads, b.scale, out, workspace=ws, partition_size=0,
                 shared_blocks=b.shared_blocks > 0)
    used = pa.decode_partition_used(ws)
    grid = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    assert used == _documented_partition(b, grid), (name, used, grid)
    if grid == 512:
        assert used == want, (name, used)
