"""pa_cache_write_decode (one launch: store each sequence's new token, then decode)
against pa_cache_write followed by pa_decode on the same inputs: the same output bits and
the same bytes in both pools, for every dtype / head size / block size family, forced
and default partitions, and sequences whose new token is their only token, opens a
block or a chunk, or has no slot (slot < 0).  The slot each new token fills is NaN in
the pool until the write, so a decode that read it from the cache inside the fused
launch would show NaN; the full-size GQA-8 step is also checked against the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_344_amd as pa
from paged_kv_cache_344_amd import inputs
from tests.gpu_helpers import OnGpu, oracle_after_write, oracle_decode, raw_bytes, say
from tests.helpers import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _separate_and_fused(b, part, slots=None):
    """(separate output, pools) and (fused output, pools) from fresh copies of b."""
    res = []
    for fused in (False, True):
        g = OnGpu(b, write=False)
        if slots is not None:
            g.slots = torch.from_numpy(slots).cuda()
        out = torch.empty_like(g.q)
        say(f"{'fused' if fused else 'separate'} step {b.name} {b.dtype} D={b.head_dim} "
            f"bs={b.block_size} S={b.num_seqs} part={part}")
        if fused:
            pa.pa_cache_write_decode(g.k_new, g.v_new, g.slots, g.q, g.k_cache, g.v_cache,
                                     g.block_tables, g.seq_lens, b.block_size, b.num_kv_heads,
                                     b.scale, out, partition_size=part)
        else:
            pa.pa_cache_write(g.k_new, g.v_new, g.slots, g.k_cache, g.v_cache)
            pa.pa_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.seq_lens, b.block_size,
                         b.num_kv_heads, b.scale, out, partition_size=part)
        torch.cuda.synchronize()
        res.append((out, raw_bytes(g.k_cache), raw_bytes(g.v_cache)))
        del g
    return res


def _same(a, b, what):
    (oa, ka, va), (ob, kb, vb) = a, b
    ia = oa.view(torch.int32 if oa.dtype == torch.float32 else torch.int16)
    ib = ob.view(torch.int32 if ob.dtype == torch.float32 else torch.int16)
    assert torch.equal(ia, ib), f"{what}: outputs differ"
    np.testing.assert_array_equal(ka, kb, err_msg=f"{what}: k_cache")
    np.testing.assert_array_equal(va, vb, err_msg=f"{what}: v_cache")


LENS = [1, 2, 16, 17, 31, 32, 33, 64, 65, 511, 512, 513, 1200]


@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f16", 128, 32), ("bf16", 64, 8),
                                        ("f32", 128, 16), ("f32", 64, 4), ("f16", 64, 4)])
@pytest.mark.parametrize("part", [0, 32, 512])
def test_fused_step_equals_write_then_decode(dtype, D, bs, part):
    b = inputs.make_batch("gqa_bf16", seed=61, dtype=dtype, head_dim=D, block_size=bs,
                          num_seqs=len(LENS), num_q_heads=16, num_kv_heads=4,
                          lens=("fixed", LENS), max_blocks_per_seq=1200 // bs + 2)
    sep, fus = _separate_and_fused(b, part)
    _same(sep, fus, f"{dtype} D={D} bs={bs} part={part}")
    check_close(fus[0].double().cpu().numpy(), oracle_decode(b), dtype, "fused step")


def test_fused_step_skips_negative_slots():
    """A sequence without a new token (slot < 0): nothing is stored for it and its decode
    reads its last position from the cache, exactly as the two separate calls do."""
    b = inputs.make_batch("gqa_bf16", seed=62, num_seqs=6, lens=("fixed", [5, 40, 70, 33, 1, 600]),
                          max_blocks_per_seq=40)
    # give the skipped sequences a finite value where the new token would have gone
    kc, vc = b.k_cache.copy(), b.v_cache.copy()
    slots = b.slot_mapping.copy()
    for s in (1, 3):
        blk, off = divmod(int(slots[s]), b.block_size)
        kc[blk, :, off, :] = b.k_new[s]
        vc[blk, :, :, off] = b.v_new[s]
        slots[s] = -1
    b2 = inputs.Batch(**{**b.__dict__, "k_cache": kc, "v_cache": vc})
    sep, fus = _separate_and_fused(b2, 0, slots=slots)
    _same(sep, fus, "negative slots")


def test_fused_step_full_size_gqa():
    """The timed GQA-8 step (seed 0): fused against separate, bit for bit, and against
    the oracle."""
    b = inputs.make_batch("gqa_bf16", seed=0)
    sep, fus = _separate_and_fused(b, 0)
    _same(sep, fus, "full-size GQA step")
    kc, vc = oracle_after_write(b)
    np.testing.assert_array_equal(fus[1], kc.view(np.uint8).reshape(-1))
    np.testing.assert_array_equal(fus[2], vc.view(np.uint8).reshape(-1))
    rep = check_close(fus[0].double().cpu().numpy(), oracle_decode(b, kc, vc), "bf16",
                      "fused full-size step")
    say(f"fused full-size step: {rep}")
