"""GPU parity of pa_multi_token (several new tokens per sequence, causal within them)
against the fp64 oracle, element by element at small sizes and on sampled rows at the
full chunked-prefill size; contract cases (bad lengths, bad table entries, query
ranges outside the output) and bit-exact invariants (placement, repeat).

Tolerances as for decode: fp32 1e-5 (abs + rel), fp16/bf16 1e-2 abs (one output ulp
where the final rounding alone exceeds 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_344_amd as pa
from paged_kv_cache_344_amd import inputs
from tests.gpu_helpers import say
from tests.helpers import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Mt:
    """A multi-token batch on cuda:0."""

    def __init__(self, b):
        self.b = b
        dt = b.dtype
        self.q = inputs.as_torch(b.q, dt, "cuda:0")
        self.k_cache = inputs.as_torch(b.k_cache, dt, "cuda:0")
        self.v_cache = inputs.as_torch(b.v_cache, dt, "cuda:0")
        self.block_tables = torch.from_numpy(b.block_tables).cuda()
        self.seq_lens = torch.from_numpy(b.seq_lens).cuda()
        self.qs = torch.from_numpy(b.query_start).cuda()
        self.max_q = int(np.diff(b.query_start).max()) if b.num_seqs else 0
        self.out = torch.empty_like(self.q)

    def run(self, seq_lens=None, block_tables=None, qs=None, max_q=None, partition_size=-1,
            workspace=None, max_seq_len=0):
        b = self.b
        say(f"pa_multi_token {b.name} seed={b.seed} {b.dtype} S={b.num_seqs} T={self.q.shape[0]} "
            f"Hq={b.num_q_heads} Hkv={b.num_kv_heads} D={b.head_dim} bs={b.block_size} "
            f"partition_size={partition_size} max_seq_len={max_seq_len}")
        call = pa.PreparedMultiToken(self.q, self.k_cache, self.v_cache,
                                     self.block_tables if block_tables is None else block_tables,
                                     self.seq_lens if seq_lens is None else seq_lens,
                                     self.qs if qs is None else qs, b.block_size, b.num_kv_heads,
                                     b.scale, self.out,
                                     max_query_len=self.max_q if max_q is None else max_q,
                                     partition_size=partition_size, max_seq_len=max_seq_len,
                                     workspace=workspace)
        self.workspace_bytes = call.workspace_bytes
        call()
        torch.cuda.synchronize()
        return self.out.double().cpu().numpy()


def _oracle(b):
    return oracle.multi_token(b.q, b.k_cache, b.v_cache, b.block_tables, b.seq_lens,
                              b.query_start, b.block_size, b.num_kv_heads, b.scale, b.dtype)


LENS = [1, 9, 33, 40, 64, 100, 130, 17]
NEW = [1, 9, 5, 40, 0, 37, 130, 16]     # one token, whole prompts, chunks, none


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,bs", [(128, 16), (64, 4), (128, 32), (64, 8)])
def test_parity_dtype_shape_grid(dtype, D, bs):
    b = inputs.make_batch("gqa_bf16", seed=3, dtype=dtype, head_dim=D, block_size=bs,
                          num_seqs=len(LENS), lens=("fixed", LENS), new_tokens=NEW,
                          max_blocks_per_seq=(max(LENS) + bs - 1) // bs + 2, cache_write=False)
    got = Mt(b).run()
    check_close(got, _oracle(b), dtype, f"multi_token {dtype} D={D} bs={bs}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (16, 1), (40, 2), (64, 2)])
def test_parity_group_sizes(Hq, Hkv):
    """G = 1, 4, 16, 20 and 32: row tiles cut through tokens at different places."""
    b = inputs.make_batch("gqa_bf16", seed=4, num_q_heads=Hq, num_kv_heads=Hkv,
                          num_seqs=len(LENS), lens=("fixed", LENS), new_tokens=NEW,
                          max_blocks_per_seq=12, cache_write=False)
    check_close(Mt(b).run(), _oracle(b), "bf16", f"multi_token Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("gain", [1.0, 4.0])
def test_parity_long_chunks(gain):
    """Chunks of 300 new tokens on 0-1200 cached ones (many row tiles and chunks),
    also with a peaked softmax."""
    lens = [300, 700, 1500, 333]
    new = [300, 300, 300, 33]
    b = inputs.make_batch("gqa_bf16", seed=5, num_seqs=4, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=100, cache_write=False, q_gain=gain)
    check_close(Mt(b).run(), _oracle(b), "bf16", f"multi_token long chunks gain={gain}")


def test_full_size_prefill_sampled():
    """The chunked-prefill batch the benchmark times, at full size (8 sequences, 512 new
    tokens on 1024-8192 cached, GQA-8): every output of the sequences with the longest
    and the shortest context against the oracle, and sampled rows of every sequence,
    each computed as the decode of the sequence cut just after that token (the causal
    definition)."""
    b = inputs.make_batch("prefill_bf16", seed=0)
    got = Mt(b).run()
    assert np.isfinite(got).all()
    qs = b.query_start
    ctxs = b.seq_lens - np.diff(qs)
    for s in sorted({int(np.argmax(ctxs)), int(np.argmin(ctxs))}):
        sub_qs = np.array([0, qs[s + 1] - qs[s]], np.int32)
        want = oracle.multi_token(b.q[qs[s]:qs[s + 1]], b.k_cache, b.v_cache,
                                  b.block_tables[s:s + 1], b.seq_lens[s:s + 1], sub_qs,
                                  b.block_size, b.num_kv_heads, b.scale, b.dtype)
        rep = check_close(got[qs[s]:qs[s + 1]], want, "bf16", f"prefill every output of s={s}")
        say(f"prefill s={s} (context {int(ctxs[s])}) every output: {rep}")
    rng = np.random.default_rng(0)
    for s in range(b.num_seqs):
        n = int(qs[s + 1] - qs[s])
        ctx = int(b.seq_lens[s]) - n
        for j in sorted(set([0, 1, 31, 32, 127, 128, n - 1] + rng.integers(0, n, 5).tolist())):
            lens = np.array([ctx + j + 1], np.int32)
            want = oracle.decode(b.q[qs[s] + j:qs[s] + j + 1], b.k_cache, b.v_cache,
                                 b.block_tables[s:s + 1], lens, b.block_size, b.num_kv_heads,
                                 b.scale, b.dtype)
            check_close(got[qs[s] + j:qs[s] + j + 1], want, "bf16", f"prefill s={s} j={j}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_size_verify_every_output(seed):
    """The draft-verification batch the benchmark times (8 sequences, 5 draft tokens each
    on 8-32 thousand cached tokens, GQA-8; seed 0 is the measured one), with the automatic
    context split the benchmark uses: every output row against the oracle."""
    b = inputs.make_batch("verify_bf16", seed=seed)
    g = Mt(b)
    got = g.run(partition_size=0)
    assert g.workspace_bytes > 0  # the call splits
    rep = check_close(got, _oracle(b), "bf16", f"verify full size seed {seed}")
    say(f"verify full size seed {seed}: {rep}")


def test_placement_independence_and_repeat_are_bit_exact():
    lens, new = [70, 200, 45], [70, 64, 20]
    b = inputs.make_batch("gqa_bf16", seed=6, num_seqs=3, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=16, cache_write=False)
    g = Mt(b)
    first = g.run().copy()
    np.testing.assert_array_equal(g.run(), first)
    # move every physical block elsewhere and relabel the tables
    N = b.num_blocks
    perm = np.random.default_rng(1).permutation(N)
    kc, vc = np.empty_like(b.k_cache), np.empty_like(b.v_cache)
    kc[perm] = b.k_cache
    vc[perm] = b.v_cache
    bt = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc, "v_cache": vc, "block_tables": bt})
    moved = Mt(b2).run()
    np.testing.assert_array_equal(moved, first)


def test_contract_violations():
    """n > L or L past the table: NaN rows; a bad table entry: NaN rows for that
    sequence; query ranges outside [0, T]: nothing written; the rest still right."""
    lens, new = [40, 50, 60, 30], [8, 8, 8, 6]
    b = inputs.make_batch("gqa_bf16", seed=7, num_seqs=4, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=5, cache_write=False)
    ref = _oracle(b)
    g = Mt(b)
    sl = b.seq_lens.copy()
    sl[0] = 5                       # fewer cached tokens than new ones
    sl[1] = 5 * 16 + 1              # more than the table can hold
    bt = b.block_tables.copy()
    bt[2, 1] = b.num_blocks + 7     # a used entry outside the pool
    g.out.fill_(7.0)
    got = g.run(seq_lens=torch.from_numpy(sl).cuda(), block_tables=torch.from_numpy(bt).cuda())
    qs = b.query_start
    for s in (0, 1, 2):
        assert np.isnan(got[qs[s]:qs[s + 1]]).all(), s
    check_close(got[qs[3]:], ref[qs[3]:], "bf16", "multi_token healthy sequence")
    # query_start pointing past the output: that sequence is skipped
    bad_qs = b.query_start.copy()
    bad_qs[3] = 9999
    g.out.fill_(7.0)
    got = g.run(qs=torch.from_numpy(bad_qs).cuda())
    assert (got[qs[2]:] == 7.0).all()
    check_close(got[:qs[2]], ref[:qs[2]], "bf16", "multi_token before the skipped ones")


# Logit profiles along the context, in log2 units (position t): the kernel moves a row's
# exponent base only when a logit passes it by more than 8, so these make the base move
# at every jump (steps of 12), every few chunks (a slow ramp), never after the first
# chunk (jumps of 7.5 that come and go), or at every chunk over a range of hundreds
# (weights of the early positions underflow to 0, as they do in the oracle's fp64).
MOVING = {
    "steps": lambda t: 12.0 * (t // 64) - 50.0,
    "ramp": lambda t: 0.06 * t,
    "below": lambda t: 7.5 * ((t // 32) % 2) + 0.001 * t,
    "wide": lambda t: 0.5 * t - 300.0,
}


def _moving_base_batch(profile, dtype, seed):
    """Every query row is A u and every cached key of position t is c(t) u for one unit
    vector u, so that each row's logit at t is the profile's value (the values stay
    random)."""
    lens, new = [700, 1200, 333, 64], [300, 100, 33, 64]
    b = inputs.make_batch("gqa_bf16", seed=seed, dtype=dtype, num_q_heads=16, num_kv_heads=2,
                          num_seqs=4, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=80, cache_write=False)
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(b.head_dim)
    u /= np.linalg.norm(u)
    A = 4.0
    b.q = inputs.to_storage(np.broadcast_to(A * u, b.q.shape).astype(np.float32), dtype)
    for s, L in enumerate(lens):
        t = np.arange(L)
        c = MOVING[profile](t) / (b.scale * A * np.log2(np.e))
        rows = inputs.to_storage((c[:, None] * u[None, :]).astype(np.float32), dtype)
        blk = b.block_tables[s, t // b.block_size]
        for g in range(b.num_kv_heads):
            b.k_cache[blk, g, t % b.block_size, :] = rows
    return b


# fp32 runs every profile but "wide": there the logits that carry the weight lie 270-300
# log2 units from zero, and an fp32 dot product of that size is off by about
# 2^-24 |q| |k|, which moves the weights by more than the 1e-5 fp32 bound allows (8e-5
# measured); only the oracle's fp64 resolves them.
@pytest.mark.parametrize("profile,dtype", [(p, d) for d in ("bf16", "f16", "f32")
                                           for p in sorted(MOVING) if (p, d) != ("wide", "f32")])
def test_parity_moving_base(profile, dtype):
    """Logits that climb along the context, so that the exponent base moves (or just
    does not) by known amounts, whole and split into 256-position partitions."""
    b = _moving_base_batch(profile, dtype, seed=21)
    g = Mt(b)
    ref = _oracle(b)
    check_close(g.run(), ref, dtype, f"moving base {profile} {dtype}")
    check_close(g.run(partition_size=256), ref, dtype, f"moving base {profile} {dtype} split 256")


# ---- context split: partitions of the positions, merged with log-sum-exp weights

@pytest.mark.parametrize("psz", [32, 64, 96, 128])
@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f32", 64, 4), ("f16", 128, 32)])
def test_split_parity(psz, dtype, D, bs):
    """Forced partitions, including ones that start past some rows' causal limits and
    partitions with nothing to do, against the oracle and against the unsplit call."""
    b = inputs.make_batch("gqa_bf16", seed=11, dtype=dtype, head_dim=D, block_size=bs,
                          num_seqs=len(LENS), lens=("fixed", LENS), new_tokens=NEW,
                          max_blocks_per_seq=(max(LENS) + bs - 1) // bs + 2, cache_write=False)
    g = Mt(b)
    whole = g.run().copy()
    got = g.run(partition_size=psz)
    assert g.workspace_bytes > 0
    ref = _oracle(b)
    check_close(got, ref, dtype, f"split {psz} {dtype} D={D} bs={bs}")
    check_close(got, whole, dtype, f"split {psz} vs unsplit")


@pytest.mark.parametrize("psz", [64, 256])
def test_split_long_chunks(psz):
    """300-token chunks on up to 1200 cached tokens cut into partitions: row tiles whose
    rows see different numbers of partitions, partitions wholly past some rows."""
    lens = [300, 700, 1500, 333]
    new = [300, 300, 300, 33]
    b = inputs.make_batch("gqa_bf16", seed=12, num_seqs=4, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=100, cache_write=False, q_gain=4.0)
    check_close(Mt(b).run(partition_size=psz), _oracle(b), "bf16", f"split long chunks {psz}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_automatic_verify(dtype):
    """Draft-token verification: 2 sequences of 9-20 thousand cached tokens, 4 new ones
    each, GQA-8.  Too few row tiles to fill the device, so the call splits by itself."""
    b = inputs.make_batch("gqa_bf16", seed=13, dtype=dtype, num_seqs=2,
                          lens=("fixed", [20000, 9001]), new_tokens=[4, 3],
                          max_blocks_per_seq=1280, cache_write=False)
    g = Mt(b)
    got = g.run(partition_size=0)
    assert g.workspace_bytes > 0
    check_close(got, _oracle(b), dtype, f"automatic split verify {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_sized_from_max_seq_len(dtype):
    """A table 16 times wider than the sequences (as when a pool is sized for the longest
    request a server admits): with max_seq_len the automatic split is sized from the
    stated bound instead of the capacity, so it cuts these sequences into more
    partitions; both agree with the oracle, and a sequence longer than the bound gets
    NaN rows while the others stay exact."""
    lens, new = [3000, 1700, 2900, 1000], [5, 5, 4, 5]
    b = inputs.make_batch("gqa_bf16", seed=16, dtype=dtype, num_seqs=4, lens=("fixed", lens),
                          new_tokens=new, max_blocks_per_seq=3072, cache_write=False)
    ref = _oracle(b)
    g = Mt(b)
    wide = g.run(partition_size=0)
    ws_wide = g.workspace_bytes
    check_close(wide, ref, dtype, f"split sized from the capacity {dtype}")
    tight = g.run(partition_size=0, max_seq_len=max(lens))
    assert g.workspace_bytes > 0 and g.workspace_bytes != ws_wide
    check_close(tight, ref, dtype, f"split sized from max_seq_len {dtype}")
    got = g.run(partition_size=0, max_seq_len=2950)     # sequence 0 (3000) is longer
    qs = b.query_start
    assert np.isnan(got[qs[0]:qs[1]]).all()
    check_close(got[qs[1]:], ref[qs[1]:], dtype, f"sequences within max_seq_len {dtype}")


def test_split_contract_violations():
    """Under a split: bad lengths give NaN rows (written by the merge), a bad table
    entry in any partition NaN rows for that sequence, skipped sequences nothing."""
    lens, new = [40, 50, 60, 30], [8, 8, 8, 6]
    b = inputs.make_batch("gqa_bf16", seed=7, num_seqs=4, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=5, cache_write=False)
    ref = _oracle(b)
    g = Mt(b)
    sl = b.seq_lens.copy()
    sl[0] = 5
    sl[1] = 5 * 16 + 1
    bt = b.block_tables.copy()
    bt[2, 3] = b.num_blocks + 7     # in the second partition of 32 positions
    g.out.fill_(7.0)
    got = g.run(seq_lens=torch.from_numpy(sl).cuda(), block_tables=torch.from_numpy(bt).cuda(),
                partition_size=32)
    qs = b.query_start
    for s in (0, 1, 2):
        assert np.isnan(got[qs[s]:qs[s + 1]]).all(), s
    check_close(got[qs[3]:], ref[qs[3]:], "bf16", "split healthy sequence")
    bad_qs = b.query_start.copy()
    bad_qs[3] = 9999
    g.out.fill_(7.0)
    got = g.run(qs=torch.from_numpy(bad_qs).cuda(), partition_size=32)
    assert (got[qs[2]:] == 7.0).all()
    check_close(got[:qs[2]], ref[:qs[2]], "bf16", "split before the skipped ones")


def test_split_repeat_and_placement_are_bit_exact():
    lens, new = [700, 2000, 450], [7, 64, 20]
    b = inputs.make_batch("gqa_bf16", seed=14, num_seqs=3, lens=("fixed", lens), new_tokens=new,
                          max_blocks_per_seq=130, cache_write=False)
    g = Mt(b)
    ws = torch.empty(1 << 27, dtype=torch.uint8, device="cuda:0")
    first = g.run(partition_size=128, workspace=ws).copy()
    assert 0 < g.workspace_bytes <= ws.numel()
    ws.fill_(0xFF)                  # scratch: its old contents do not matter
    np.testing.assert_array_equal(g.run(partition_size=128, workspace=ws), first)
    N = b.num_blocks
    perm = np.random.default_rng(2).permutation(N)
    kc, vc = np.empty_like(b.k_cache), np.empty_like(b.v_cache)
    kc[perm] = b.k_cache
    vc[perm] = b.v_cache
    bt = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc, "v_cache": vc, "block_tables": bt})
    np.testing.assert_array_equal(Mt(b2).run(partition_size=128, workspace=ws), first)
