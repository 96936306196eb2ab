"""Plain Python model of KV-cache block bookkeeping, and of the memory it wastes.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the library's C++ block manager; the tests run both on the same operations and
compare every observable (slots, tables, lengths, copies, free counts, references).

Pages cited (title, site):
  [AB]  "什么是分页注意力（PagedAttention）？" aiboss88.com, section 工作机制
  [CY]  "深入解析 PagedAttention：vLLM 显存优化的核心魔法" cygnushan.xyz, sections
        PagedAttention 的核心思想 (工作原理) and 多序列共享 (引用计数机制)
  [ASP] "PagedAttention" awesome-system-papers, sections 核心思想 and 实现要点
  [RK]  "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?" news.rkmt.cn,
        sections 问题所在, 分页注意力是如何工作的, 块表, 分页注意力为何如此有效

The model keeps its state as plain lists and dicts and recomputes nothing cleverly:
  - a pool of physical blocks, each with room for ``block_size`` tokens; the free
    ones wait in a queue and are handed out oldest first ([ASP] 核心思想: any free
    block can serve any sequence);
  - per sequence, a block table (logical block j -> physical block, [RK] 块表) and
    a token count;
  - a new block is taken only when a token arrives and the sequence's last block is
    full or missing ([RK] 分页注意力是如何工作的: one block of four after every
    fourth token; [AB] 工作机制);
  - per block, the number of tables holding it; a fork copies the parent's table
    and counts each block once more; freeing a sequence counts each of its blocks
    once less, and a block at zero goes back to the free queue ([CY] 引用计数机制;
    [ASP] 实现要点);
  - copy-on-write: a token bound for a last block that other tables also hold and
    that still has empty slots is written into a fresh copy of that block instead,
    which replaces it in this sequence's table ([CY] 引用计数机制; [ASP] 实现要点).
    A full shared block is never written, so it is never copied.  (The pages name
    copy-on-write without fixing when the copy happens; this is the reading in which
    no sequence ever writes into a block another sequence reads.)
"""
from __future__ import annotations

from collections import deque


class CapacityError(RuntimeError):
    """No free block, or a block table would grow past its row length."""


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 free_order=None):
        if free_order is None:
            free_order = list(range(num_blocks))
        assert sorted(free_order) == list(range(num_blocks)), "free_order must be a permutation"
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        self.free = deque(free_order)
        self.refs = [0] * num_blocks
        self.tables = {}   # sequence id -> list of physical blocks
        self.lengths = {}  # sequence id -> tokens
        self.next_id = 0

    # -- sequences ---------------------------------------------------------------
    def add_sequence(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        child = self.add_sequence()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refs[b] += 1
        return child

    def free_sequence(self, sid: int) -> None:
        for b in self.tables.pop(sid):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)
        del self.lengths[sid]

    # -- one new token for each listed sequence ----------------------------------
    def append(self, seqs):
        """Returns (slot ids, [(source, destination) block copies]); raises
        CapacityError and changes nothing if the pool or a table would overflow.

        Blocks needed: one for every sequence whose last block is full (or that has
        none), and for every shared, partly filled last block X listed by k of its
        holders, min(k, refs(X) - 1) copies: the holders are served in the order given,
        each copy drops X's count by one, and once the last remaining holder is alone
        on X it writes into X itself."""
        assert len(set(seqs)) == len(seqs), "each sequence at most once per step"
        need = 0
        holders = {}                      # shared, partly filled last block -> listed holders
        for sid in seqs:
            if self.lengths[sid] % self.block_size == 0:
                if len(self.tables[sid]) + 1 > self.max_blocks:
                    raise CapacityError(f"sequence {sid} would need more than {self.max_blocks} blocks")
                need += 1
            elif self.refs[self.tables[sid][-1]] > 1:
                x = self.tables[sid][-1]
                holders[x] = holders.get(x, 0) + 1
        for x, k in holders.items():
            need += min(k, self.refs[x] - 1)
        if need > len(self.free):
            raise CapacityError(f"{need} free blocks needed, {len(self.free)} free")
        slots, copies = [], []
        for sid in seqs:
            table = self.tables[sid]
            offset = self.lengths[sid] % self.block_size
            if offset == 0:
                b = self.free.popleft()
                self.refs[b] = 1
                table.append(b)
            elif self.refs[table[-1]] > 1:
                old = table[-1]
                b = self.free.popleft()
                self.refs[b] = 1
                self.refs[old] -= 1
                table[-1] = b
                copies.append((old, b))
            slots.append(table[-1] * self.block_size + offset)
            self.lengths[sid] += 1
        return slots, copies

    # -- what the kernels read ---------------------------------------------------
    def export(self, seqs):
        rows = [self.tables[s] + [-1] * (self.max_blocks - len(self.tables[s])) for s in seqs]
        return rows, [self.lengths[s] for s in seqs]

    def free_blocks(self) -> int:
        return len(self.free)


# -- memory waste ([RK] 问题所在 and 分页注意力为何如此有效) --------------------------
def contiguous_waste(lengths, reserved: int) -> int:
    """Slots reserved up front for each request and never filled: each request holds
    ``reserved`` contiguous slots whatever its length."""
    return sum(reserved - n for n in lengths)


def paged_waste(lengths, block_size: int) -> int:
    """Empty slots when each request holds just enough whole blocks for its tokens:
    only the last block of a request can have empty slots."""
    total = 0
    for n in lengths:
        blocks = -(-n // block_size)
        total += blocks * block_size - n
    return total


def admitted(lengths, block_size: int, reserved: int, pool_slots: int):
    """Requests, taken in order, that fit at once in ``pool_slots`` slots:
    (contiguous: whole reservations of ``reserved`` slots; paged: whole blocks
    covering each request's tokens, in a pool of pool_slots // block_size blocks)."""
    contiguous = min(len(lengths), pool_slots // reserved)
    blocks_left = pool_slots // block_size
    paged = 0
    for n in lengths:
        need = -(-n // block_size)
        if need > blocks_left:
            break
        blocks_left -= need
        paged += 1
    return contiguous, paged
