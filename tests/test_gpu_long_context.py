"""Long-context decode at full length: every output of the long-context batches against
the oracle, and needles placed at every position of the split-K merge tree.

Paging does not change the attention formula, so every way of cutting a sequence into
partitions and merging them must reproduce the unsplit result ([AB]
"什么是分页注意力（PagedAttention）？" 边界与常见误解).  At these lengths outputs are a few
thousandths, so the checks rely on the bound of tests/helpers.faithful_bound (one
output ulp plus 2^-10 of the row's rms), which rejects a lost or doubled partition
(tests/test_parity_power.py), besides the 1e-2 spec bound.

Needles: in each sequence and KV head one key is replaced by c * w, w the unit vector
along the sum of the group's unit query vectors; its logit then exceeds every other by
far more than log(length), so each of the group's outputs must equal that token's
value.  The spots (one per KV head) are: inside partition 0, the last token of
partition 0, the last token of merge group 0 (16 partitions), the first token of group
1, inside group 2, the first token of the last partition, the first token of the last
group, and the sequence's last token."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_344_amd as pa
from paged_kv_cache_344_amd import inputs
from tests.gpu_helpers import OnGpu, oracle_decode, say
from tests.helpers import check_close, check_faithful, ulp

pytestmark = pytest.mark.gpu

FAN = 16  # partitions per merge group


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode(g, part):
    """Decode with its own workspace; returns (output, partition length used)."""
    b = g.b
    ws = pa.workspace_for(g.q, g.block_tables, b.num_blocks, b.block_size, b.num_kv_heads,
                          partition_size=part)
    out = torch.empty_like(g.q)
    say(f"pa_decode {b.name} bs={b.block_size} S={b.num_seqs} part={part}")
    pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                 b.num_kv_heads, b.scale, out, workspace=ws, partition_size=part)
    return g.out_f64(out), pa.decode_partition_used(ws)


@pytest.mark.parametrize("name", ["long_bf16_bs16", "long_bf16_bs32", "long_bf16_bs16_default",
                                  "long_bf16_bs32_default", "long_bf16_bs16_nosplit"])
def test_full_size_long_context_every_output(name):
    """The long-context batch (seed 0, the measured one) in the launch configuration the
    benchmark times: every sequence, every head (also unsplit: one item per sequence and
    KV head, every partition as long as the table's capacity)."""
    b = inputs.make_batch(name, seed=0)
    g = OnGpu(b)
    got, used = _decode(g, b.partition_size)
    if b.partition_size > 0:
        assert used == b.partition_size
    elif b.partition_size < 0:
        assert used >= int(b.seq_lens.max()), used
    ref = oracle_decode(b)
    rep = check_close(got, ref, b.dtype, f"{name} full")
    say(f"parity {name} (partition {used}): {rep}")


@pytest.mark.parametrize("seed", [1, 2])
def test_full_size_long_context_default_other_seeds(seed):
    """The default partitioning on the input recipe's other seeds: other lengths, so the
    device picks other partition lengths (the rule of include/pa.h), every output."""
    b = inputs.make_batch("long_bf16_bs16_default", seed=seed)
    g = OnGpu(b)
    got, used = _decode(g, b.partition_size)
    assert used % 256 == 0 and used >= 512, used
    rep = check_close(got, oracle_decode(b), b.dtype, f"long default seed {seed}")
    say(f"parity long default seed {seed} (partition {used}): {rep}")


def _spots(L, P):
    n = (L + P - 1) // P
    last_group = ((n - 1) // FAN) * FAN
    s = [3, P - 1, FAN * P - 1, FAN * P, 2 * FAN * P + P // 2 + 5, (n - 1) * P, last_group * P,
         L - 1]
    assert n > 2 * FAN, (L, P, n)  # the sequence reaches merge group 2
    return [min(t, L - 1) for t in s]


def _place_needles(b, spots_by_seq, c=96.0):
    kc = b.k_cache.copy()
    q32 = oracle.decode_elements(b.q, "bf16")
    G = b.num_q_heads // b.num_kv_heads
    for s, spots in enumerate(spots_by_seq):
        for g, t in enumerate(spots):
            u = q32[s, g * G:(g + 1) * G]
            u = u / np.linalg.norm(u, axis=1, keepdims=True)
            w = u.sum(0)
            w /= np.linalg.norm(w)
            blk, off = b.block_tables[s, t // b.block_size], t % b.block_size
            kc[blk, g, off, :] = inputs.to_storage((c * w).astype(np.float32), "bf16")
    return inputs.Batch(**{**b.__dict__, "k_cache": kc})


@pytest.mark.parametrize("bs", [16, 32])
def test_long_context_needles_at_every_merge_position(bs):
    """Two sequences of 65,537 and 131,072 tokens.  Sequence 0 carries needles placed
    for 512-token partitions, sequence 1 for the default partition length (read back
    from the device: one workgroup's share, 3328 tokens here, so 40 partitions, the last
    one ragged, reaching merge group 2); both partitionings are decoded and every needle
    must be found."""
    name = "long_bf16_bs16" if bs == 16 else "long_bf16_bs32"
    lens = [65537, 131072]
    b = inputs.make_batch(name, seed=43, num_seqs=2, lens=("fixed", lens), cache_write=False)
    g0 = OnGpu(b)
    _, p_default = _decode(g0, 0)
    del g0
    torch.cuda.empty_cache()
    say(f"default partition for lengths {lens}: {p_default}")
    b2 = _place_needles(b, [_spots(lens[0], 512), _spots(lens[1], p_default)])
    g = OnGpu(b2)
    ref = oracle_decode(b2)
    G = b.num_q_heads // b.num_kv_heads
    v = oracle.decode_elements(b2.v_cache, "bf16")  # [N][Hkv][D][bs]
    for part in (512, 0):
        got, used = _decode(g, part)
        assert used == (512 if part else p_default)
        rep = check_close(got, ref, "bf16", f"needles bs={bs} part={part}")
        say(f"needles bs={bs} partition {used}: {rep}")
        for s, spots in enumerate([_spots(lens[0], 512), _spots(lens[1], p_default)]):
            for kv, t in enumerate(spots):
                blk, off = b2.block_tables[s, t // bs], t % bs
                vt = v[blk, kv, :, off]
                rows = slice(kv * G, (kv + 1) * G)
                # the oracle finds the needle (its weight is all but 1) ...
                assert np.abs(ref[s, rows] - vt).max() < 1e-6 * (1 + np.abs(vt).max()), (s, kv, t)
                # ... and so does the kernel, to within the output rounding
                lim = ulp(np.abs(vt), "bf16") + 1e-6
                assert (np.abs(got[s, rows] - vt) <= lim).all(), (part, s, kv, t)


def test_split_and_single_pass_agree_to_an_ulp():
    """512-token partitions and no split at all on the same peaked batch: each within
    the bound of the oracle, and the two within one output ulp of each other (both are
    the exact result rounded once, up to fp32 error)."""
    b = inputs.make_batch("long_bf16_bs16", seed=7, num_seqs=2, max_blocks_per_seq=300,
                          lens=("uniform", 3000, 4800), q_gain=4.0)
    g = OnGpu(b)
    split = g.out_f64(g.decode(512).clone())
    whole = g.out_f64(g.decode(-1).clone())
    ref = oracle_decode(b)
    check_close(split, ref, "bf16", "split")
    check_close(whole, ref, "bf16", "whole")
    lim = ulp(np.maximum(np.abs(split), np.abs(whole)), "bf16")
    assert (np.abs(split - whole) <= lim).all()
    check_faithful(split, whole, "bf16", "split vs whole")
