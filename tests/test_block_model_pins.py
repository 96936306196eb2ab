"""Pins of the Python model of KV block bookkeeping (``oracle/block_manager.py``):
the walk-through and block table printed on [RK] "什么是 LLM 中的分页注意力(Paged
Attention)?它是如何工作的?" (news.rkmt.cn), the shared block tables printed on [CY]
"深入解析 PagedAttention：vLLM 显存优化的核心魔法" (cygnushan.xyz, 工作原理), the waste
figures of [RK] 问题所在 and 分页注意力为何如此有效, and invariants that hold for any
sequence of operations (reference counts equal table memberships; every block is
either free or referenced; every sequence reads back exactly the tokens it was
given, whatever its siblings wrote).  CPU only."""
import json
import os
import random

import pytest

from oracle import block_manager as model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rk_free_order(n):
    """A pool whose first free blocks are 5, 12, 3 (the positions [RK] 块表 prints)."""
    head = [5, 12, 3]
    return head + [b for b in range(n) if b not in head]


# ---------------------------------------------------------------------------------
def test_model_worked_example_rk():
    g = _golden("worked_example.json")
    p, d = g["printed"], g["derived"]
    bs = p["block_size"]
    m = model.BlockModel(16, bs, 8, free_order=_rk_free_order(16))
    s = m.add_sequence()
    slots, taken_before = [], []
    for t in range(p["tokens"]):
        before = m.free_blocks()
        sl, copies = m.append([s])
        assert copies == []
        if m.free_blocks() < before:
            taken_before.append(t)
        slots += sl
    rows, lens = m.export([s])
    assert taken_before == p["blocks_taken_before_token"]
    assert rows[0][:p["paged_blocks_used"]] == p["block_table"]
    assert all(x == -1 for x in rows[0][p["paged_blocks_used"]:])
    assert lens == [p["tokens"]]
    assert slots == d["token_slots"]
    counts = [sum(1 for x in slots if x // bs == blk) for blk in p["block_table"]]
    assert counts == p["paged_block_token_counts"]
    assert model.paged_waste([p["tokens"]], bs) == p["paged_wasted_slots"]
    assert model.contiguous_waste([p["tokens"]], p["contiguous_reserved_slots"]) == \
        p["contiguous_wasted_slots"]
    assert model.contiguous_waste([p["reservation_used"]], p["reservation_slots"]) == \
        p["reservation_wasted"]


def test_model_shared_prefix_tables_cy():
    """[CY] 工作原理: sequence 1 holds blocks 0, 1, 2 (tokens 1-12 at four a block);
    sequence 2 shares the first two.  Reading: sequence 2 is a fork of sequence 1
    taken when it held 8 tokens."""
    g = _golden("shared_prefix_tables.json")["printed"]
    bs = g["block_size"]
    m = model.BlockModel(8, bs, len(g["table_seq2"]))
    s1 = m.add_sequence()
    for _ in range(8):
        m.append([s1])
    s2 = m.fork(s1)
    for _ in range(4):
        _, copies = m.append([s1])
        assert copies == []           # the shared blocks are full: nothing to copy
    rows, lens = m.export([s1, s2])
    assert rows[0][:3] == g["table_seq1"]
    assert rows[1] == g["table_seq2"]
    assert lens == [12, 8]
    for blk, toks in g["physical_block_tokens_1based"].items():
        # token t (1-based) of sequence 1 sits in block (t-1) // bs of its table
        assert [rows[0][(t - 1) // bs] for t in toks] == [int(blk)] * len(toks)
    assert m.refs[0] == m.refs[1] == 2 and m.refs[2] == 1


def test_model_copy_on_write_of_a_partly_filled_shared_block():
    m = model.BlockModel(8, 4, 4)
    a = m.add_sequence()
    for _ in range(6):                # blocks 0 (full) and 1 (2 of 4)
        m.append([a])
    b = m.fork(a)
    slots, copies = m.append([b])     # b would write into shared block 1: copy it first
    assert copies == [(1, 2)]
    assert slots == [2 * 4 + 2]
    assert m.tables[a] == [0, 1] and m.tables[b] == [0, 2]
    assert m.refs[:3] == [2, 1, 1]
    slots, copies = m.append([a])     # a now holds block 1 alone: no copy
    assert copies == [] and slots == [1 * 4 + 2]


def test_model_siblings_appending_together_copy_all_but_one():
    """Holders of one shared, partly filled block appending in the same call: all but
    the last listed copy it, and the last, then alone on it, writes in place -- so the
    call needs refs - 1 free blocks, not one per holder."""
    m = model.BlockModel(3, 4, 4)
    a = m.add_sequence()
    for _ in range(6):                # blocks 0 (full) and 1 (2 of 4); block 2 free
        m.append([a])
    b = m.fork(a)
    slots, copies = m.append([a, b])  # one free block is enough
    assert copies == [(1, 2)]
    assert slots == [2 * 4 + 2, 1 * 4 + 2]
    assert m.tables[a] == [0, 2] and m.tables[b] == [0, 1]
    assert m.refs == [2, 1, 1] and m.free_blocks() == 0
    # three holders of block 1: two copies; with one free block the call fails untouched
    m = model.BlockModel(4, 4, 4)
    a = m.add_sequence()
    for _ in range(6):
        m.append([a])
    b, c = m.fork(a), m.fork(a)
    m.add_sequence()
    d = m.add_sequence()
    m.append([d])                     # takes block 2: one free block left
    with pytest.raises(model.CapacityError):
        m.append([c, a, b])
    assert m.refs[1] == 3 and m.free_blocks() == 1 and m.lengths[a] == 6
    m.free_sequence(d)                # two free blocks
    slots, copies = m.append([c, a, b])
    assert [s for s, _ in copies] == [1, 1] and m.refs[1] == 1
    assert m.tables[b] == [0, 1] and slots[2] == 1 * 4 + 2


def test_model_frees_at_zero_and_fifo_reuse():
    m = model.BlockModel(4, 2, 4)
    a = m.add_sequence()
    for _ in range(3):
        m.append([a])                 # blocks 0, 1
    b = m.fork(a)
    m.free_sequence(a)
    assert m.free_blocks() == 2       # b still holds 0 and 1
    m.free_sequence(b)
    assert list(m.free) == [2, 3, 1, 0] or list(m.free) == [2, 3, 0, 1]
    c = m.add_sequence()
    assert m.append([c])[0] == [2 * 2]   # oldest free block first


def test_model_capacity_errors_change_nothing():
    m = model.BlockModel(2, 2, 1)
    a = m.add_sequence()
    m.append([a])
    m.append([a])
    with pytest.raises(model.CapacityError):
        m.append([a])                 # table full at one block
    b, c = m.add_sequence(), m.add_sequence()
    m.append([b])
    with pytest.raises(model.CapacityError):
        m.append([c, a])
    assert m.lengths == {a: 2, b: 1, c: 0} and m.free_blocks() == 0


@pytest.mark.parametrize("seed", range(6))
def test_model_invariants_and_readback(seed):
    """Brute force: a shadow pool (slot -> token value) is updated exactly as the
    device would be -- block copies first, then the new tokens -- and after every
    step every sequence must read back its own history through its table, the
    reference counts must equal table memberships, and the free blocks must be
    exactly those no table holds."""
    rng = random.Random(seed)
    bs = rng.choice([1, 2, 4, 16])
    N = rng.choice([8, 24, 64])
    m = model.BlockModel(N, bs, 64, free_order=rng.sample(range(N), N))
    pool, history, value = {}, {}, 0
    for _ in range(300):
        live = list(m.tables)
        r = rng.random()
        if r < 0.08 or not live:
            history[m.add_sequence()] = []
        elif r < 0.16:
            p = rng.choice(live)
            history[m.fork(p)] = list(history[p])
        elif r < 0.22 and len(live) > 1:
            s = rng.choice(live)
            m.free_sequence(s)
            del history[s]
        else:
            seqs = rng.sample(live, rng.randint(1, len(live)))
            try:
                slots, copies = m.append(seqs)
            except model.CapacityError:
                slots, copies = [], []
            for src, dst in copies:
                for o in range(bs):
                    if src * bs + o in pool:
                        pool[dst * bs + o] = pool[src * bs + o]
            for s, slot in zip(seqs, slots):
                value += 1
                pool[slot] = value
                history[s].append(value)
        member = [0] * N
        for t in m.tables.values():
            for blk in t:
                member[blk] += 1
        assert member == m.refs
        assert sorted(m.free) == [blk for blk in range(N) if m.refs[blk] == 0]
        for s, t in m.tables.items():
            assert len(t) == -(-m.lengths[s] // bs) and m.lengths[s] == len(history[s])
            assert [pool[t[i // bs] * bs + i % bs] for i in range(m.lengths[s])] == history[s]


def test_readback_catches_a_dropped_copy(monkeypatch):
    """The read-back check above fails if the model forgets to copy a shared block."""
    m = model.BlockModel(8, 4, 4)
    a = m.add_sequence()
    for _ in range(2):
        m.append([a])
    b = m.fork(a)
    orig = m.append

    def no_copy(seqs):
        slots, copies = orig(seqs)
        return slots, []
    monkeypatch.setattr(m, "append", no_copy)
    pool = {0: 1, 1: 2}
    slots, copies = m.append([b])
    for src, dst in copies:
        for o in range(4):
            if src * 4 + o in pool:
                pool[dst * 4 + o] = pool[src * 4 + o]
    pool[slots[0]] = 3
    t = m.tables[b]
    assert [pool.get(t[i // 4] * 4 + i % 4) for i in range(3)] != [1, 2, 3]


def test_model_waste_and_admission_closed_forms():
    for bs in (1, 4, 16):
        for n in range(0, 70):
            assert model.paged_waste([n], bs) == (-n) % bs
    assert model.admitted([10] * 5, 4, 16, 48) == (3, 4)
    assert model.admitted([50] * 40, 16, 2048, 4096) == (2, 40)


