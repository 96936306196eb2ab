"""KV-cache memory accounting: slots a contiguous per-request reservation holds
against slots the block manager actually hands out, for a list of request lengths.

Pages cited: [RK] "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?"
news.rkmt.cn, sections 问题所在 (a request reserves its maximum length up front and
wastes what it never fills), 分页注意力是如何工作的 and 分页注意力为何如此有效 (blocks
are taken on demand, so only the last block of a request has empty slots); [CY]
"深入解析 PagedAttention：vLLM 显存优化的核心魔法" cygnushan.xyz, section 显存对比实验
(the pages' own contiguous-vs-paged comparison, which needs a model; this is its
model-free counterpart).

The paged side is measured, not computed: every request is added to a real
``BlockManager`` (the library's C++ bookkeeping) and grown one token at a time,
and the slots held are read back from the manager's free count.  The contiguous
side is the reservation itself: ``reserved`` slots per request.
"""
from __future__ import annotations

import dataclasses

from .binding import BlockManager, PaError, PA_ERR_CAPACITY


@dataclasses.dataclass
class WasteReport:
    requests: int
    tokens: int               # KV entries the requests store
    block_size: int
    reserved: int             # contiguous slots per request
    paged_slots: int          # slots in the blocks the manager handed out
    contiguous_slots: int     # requests * reserved

    @property
    def paged_waste(self) -> int:
        return self.paged_slots - self.tokens

    @property
    def contiguous_waste(self) -> int:
        return self.contiguous_slots - self.tokens

    @property
    def paged_waste_frac(self) -> float:
        return self.paged_waste / self.paged_slots if self.paged_slots else 0.0

    @property
    def contiguous_waste_frac(self) -> float:
        return self.contiguous_waste / self.contiguous_slots if self.contiguous_slots else 0.0


def _grow(bm: BlockManager, lengths) -> list:
    """Add one sequence per length and append tokens until each reaches its length;
    returns the sequence ids.  Appends all still-growing sequences per step."""
    ids = [bm.add_sequence() for _ in lengths]
    pending = [(s, n) for s, n in zip(ids, lengths) if n > 0]
    step = 0
    while pending:
        bm.append([s for s, _ in pending])
        step += 1
        pending = [(s, n) for s, n in pending if n > step]
    return ids


def account(lengths, block_size: int, reserved: int) -> WasteReport:
    """Slots held by contiguous reservations of ``reserved`` slots against the paged
    pool for requests of the given lengths (each at most ``reserved``)."""
    lengths = [int(n) for n in lengths]
    if any(n < 0 or n > reserved for n in lengths):
        raise ValueError("every length must lie in [0, reserved]")
    max_blocks = max(1, -(-reserved // block_size))
    num_blocks = max(1, len(lengths) * max_blocks)
    bm = BlockManager(num_blocks, block_size, max_blocks)
    try:
        _grow(bm, lengths)
        held = num_blocks - bm.free_blocks()
    finally:
        bm.close()
    return WasteReport(requests=len(lengths), tokens=sum(lengths), block_size=block_size,
                       reserved=reserved, paged_slots=held * block_size,
                       contiguous_slots=len(lengths) * reserved)


def admitted(lengths, block_size: int, reserved: int, pool_slots: int) -> tuple:
    """How many of the requests, taken in order, fit at once in a pool of
    ``pool_slots`` slots: (contiguous, paged).  Contiguously each request takes
    ``reserved`` slots; paged, requests are admitted one by one and grown to their
    length until the manager reports the pool exhausted."""
    lengths = [int(n) for n in lengths]
    contiguous = min(len(lengths), pool_slots // reserved)
    num_blocks = pool_slots // block_size
    if num_blocks < 1:
        return contiguous, 0
    max_blocks = max(1, -(-reserved // block_size))
    bm = BlockManager(num_blocks, block_size, max_blocks)
    paged = 0
    try:
        for n in lengths:
            s = bm.add_sequence()
            try:
                for _ in range(n):
                    bm.append([s])
            except PaError as e:
                if e.status != PA_ERR_CAPACITY:
                    raise
                bm.free_sequence(s)
                break
            paged += 1
    finally:
        bm.close()
    return contiguous, paged
