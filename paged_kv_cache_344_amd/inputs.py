"""Seeded synthetic decode batches.

This module is the one piece shared by the GPU path's tests/benchmark and the CPU
oracle: it draws inputs and holds none of the attention arithmetic.  It plays the
part of the block manager that sits in front of the hot path: it picks sequence
lengths, hands out physical blocks from a shuffled pool (any free block will do:
[ASP] "PagedAttention" 核心思想, no external fragmentation), writes the block
tables and, for batches that append a token, names the slot each new token goes
to.  Values are N(0, 1) drawn in float32 and rounded to the storage dtype with
round-to-nearest-even.

Storage convention of the cache (the library's definition; the pages fix none):
``k_cache[N][Hkv][bs][D]`` and ``v_cache[N][Hkv][D][bs]``.  Arrays are returned as
raw numpy storage: float32, float16, or uint16 bit patterns for bf16.

Draw order for one batch: lengths, block permutation, Q and the new tokens' K and V
come from ``default_rng(seed)`` in that order; the K and V pools are filled chunk by
chunk from child generators of ``SeedSequence(seed)`` (spawn keys 1 and 2), so large
pools can be drawn on several threads with the same result.  Unused table entries
are -1 ([CY] "深入解析 PagedAttention" 核心思想, Block Table example).  Every slot no sequence owns (free blocks, the unfilled tail
of a sequence's last block, and the slot a pending new token will fill) holds NaN,
so a kernel that touches one shows it.

Pages: [ASP] "PagedAttention" (awesome-system-papers); [CY] "深入解析
PagedAttention：vLLM 显存优化的核心魔法" (cygnushan.xyz); [RK] "什么是 LLM 中的分页注意力
(Paged Attention)?它是如何工作的?" (news.rkmt.cn).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

# name -> recipe.  Sizes follow the five decode batches the library is measured on.
CONFIGS = {
    # tiny correctness batch: lengths fixed, 64-block pool, one appended token per sequence
    "tiny_fp32": dict(dtype="f32", num_seqs=4, num_q_heads=2, num_kv_heads=2, head_dim=64,
                      block_size=4, max_blocks_per_seq=9, lens=("fixed", [5, 10, 17, 33]),
                      pool=("fixed", 64), cache_write=True),
    # Llama-7B-like MHA layer
    "mha_fp16": dict(dtype="f16", num_seqs=32, num_q_heads=32, num_kv_heads=32, head_dim=128,
                     block_size=16, max_blocks_per_seq=128, lens=("uniform", 128, 2048),
                     pool=("slack", 0.10), cache_write=False),
    # GQA-8 batch with skewed lengths; one appended token per sequence written first
    "gqa_bf16": dict(dtype="bf16", num_seqs=128, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     block_size=16, max_blocks_per_seq=256, lens=("loguniform", 1, 4096),
                     pool=("slack", 0.10), cache_write=True),
    # 64 sequences sharing a 1024-token prefix, 0-512 private tokens each
    "prefix_bf16": dict(dtype="bf16", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        block_size=16, max_blocks_per_seq=96, lens=("prefix", 1024, 0, 512),
                        pool=("slack", 0.10), cache_write=False),
    # long context, split into 512-token partitions
    "long_bf16_bs16": dict(dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, max_blocks_per_seq=8192,
                           lens=("uniform", 32768, 131072), pool=("slack", 0.10),
                           cache_write=False, partition_size=512),
    "long_bf16_bs32": dict(dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=32, max_blocks_per_seq=4096,
                           lens=("uniform", 32768, 131072), pool=("slack", 0.10),
                           cache_write=False, partition_size=512),
    # the same long-context batches with the default partition size, which the kernel
    # chooses on the device from the lengths (8448 tokens for seed 0)
    "long_bf16_bs16_default": dict(dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
                                   head_dim=128, block_size=16, max_blocks_per_seq=8192,
                                   lens=("uniform", 32768, 131072), pool=("slack", 0.10),
                                   cache_write=False, partition_size=0),
    "long_bf16_bs32_default": dict(dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
                                   head_dim=128, block_size=32, max_blocks_per_seq=4096,
                                   lens=("uniform", 32768, 131072), pool=("slack", 0.10),
                                   cache_write=False, partition_size=0),
    # the same long-context batch decoded without a split: one work item per (sequence,
    # KV head), the comparison point for the 512-token partitions
    "long_bf16_bs16_nosplit": dict(dtype="bf16", num_seqs=8, num_q_heads=32, num_kv_heads=8,
                                   head_dim=128, block_size=16, max_blocks_per_seq=8192,
                                   lens=("uniform", 32768, 131072), pool=("slack", 0.10),
                                   cache_write=False, partition_size=-1),
    # chunked prefill: a 512-token prompt chunk per sequence on top of 1024-8192 cached
    # tokens, GQA-8; every new token attends causally (pa_multi_token)
    "prefill_bf16": dict(dtype="bf16", num_seqs=8, num_q_heads=64, num_kv_heads=8,
                         head_dim=128, block_size=16, max_blocks_per_seq=544,
                         lens=("chunk", 1024, 8192, 512), pool=("slack", 0.10),
                         cache_write=False),
    # draft-token verification (speculative decoding over the paged cache): 5 new tokens
    # per sequence on 8192-32768 cached ones, GQA-8; too few row tiles to fill the
    # device, so pa_multi_token splits the context
    "verify_bf16": dict(dtype="bf16", num_seqs=8, num_q_heads=64, num_kv_heads=8,
                        head_dim=128, block_size=16, max_blocks_per_seq=2049,
                        lens=("chunk", 8192, 32768, 5), pool=("slack", 0.10),
                        cache_write=False),
}


@dataclasses.dataclass
class Batch:
    name: str
    seed: int
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks_per_seq: int
    num_blocks: int
    scale: float
    seq_lens: np.ndarray        # int32 [S]; counts every attended token, the new one included
    block_tables: np.ndarray    # int32 [S, max_blocks_per_seq], -1 past the used blocks
    q: np.ndarray               # [S, Hq, D] ([T, Hq, D] for multi-token batches)
    k_cache: np.ndarray         # [N, Hkv, bs, D]
    v_cache: np.ndarray         # [N, Hkv, D, bs]
    query_start: Optional[np.ndarray] = None  # int32 [S+1] for multi-token batches: q rows
                                              # of sequence s are qs[s] .. qs[s+1]-1
    k_new: Optional[np.ndarray] = None      # [T, Hkv, D]
    v_new: Optional[np.ndarray] = None      # [T, Hkv, D]
    slot_mapping: Optional[np.ndarray] = None  # int64 [T]
    partition_size: int = 0
    shared_blocks: int = 0      # prefix blocks every table starts with (prefix batches)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (round to nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    import torch  # bf16 rounding: torch's CPU cast rounds to nearest even
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _nan(dtype: str):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]


_CHUNK_VALUES = 1 << 22


def _fill_pool(block_shape, N, seed, key, dtype, owned) -> np.ndarray:
    """[N, *block_shape] storage: N(0, 1) in owned blocks, NaN elsewhere.  Drawn in
    chunks of whole blocks, chunk i from child i of SeedSequence(seed, spawn_key=(key,)),
    so the values do not depend on how many threads fill it."""
    per_block = int(np.prod(block_shape))
    chunk = max(1, _CHUNK_VALUES // per_block)
    n_chunks = (N + chunk - 1) // chunk
    children = np.random.SeedSequence(entropy=seed, spawn_key=(key,)).spawn(n_chunks)
    out = np.empty((N,) + tuple(block_shape), dtype=STORAGE[dtype])
    nan = _nan(dtype)

    def work(i):
        a, b = i * chunk, min(N, (i + 1) * chunk)
        x = np.random.default_rng(children[i]).standard_normal((b - a,) + tuple(block_shape),
                                                              dtype=np.float32)
        out[a:b] = to_storage(x, dtype)
        out[a:b][~owned[a:b]] = nan

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    if n_chunks == 1 or threads == 1:
        for i in range(n_chunks):
            work(i)
    else:
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def _draw_lengths(rng, spec, S):
    kind = spec[0]
    if kind == "fixed":
        lens = np.asarray(spec[1], dtype=np.int64)
        if lens.shape != (S,):
            raise ValueError("fixed lengths must give one length per sequence")
        return lens, None
    if kind == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=S), None
    if kind == "loguniform":
        lo, hi = spec[1], spec[2]
        u = rng.uniform(math.log(lo), math.log(hi + 1), size=S)
        return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi), None
    if kind == "chunk":  # cached context uniform in [lo, hi], then n new tokens
        lo, hi, n = spec[1], spec[2], spec[3]
        return rng.integers(lo, hi + 1, size=S) + n, None
    if kind == "prefix":
        prefix, lo, hi = spec[1], spec[2], spec[3]
        private = rng.integers(lo, hi + 1, size=S)
        return prefix + private, prefix
    raise ValueError(f"unknown length spec {spec}")


def make_batch(name: str, seed: int = 0, **over) -> Batch:
    """Build one seeded batch.  ``over`` replaces recipe fields (e.g. ``num_seqs``,
    ``lens``, ``dtype``, ``q_gain`` to multiply Q for a peaked softmax, ``new_tokens``
    to give each sequence that many query tokens, its last ones, for pa_multi_token)."""
    cfg = dict(CONFIGS[name])
    q_gain = over.pop("q_gain", 1.0)
    cfg.update(over)
    dtype = cfg["dtype"]
    S, Hq, Hkv, D = cfg["num_seqs"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    bs, MB = cfg["block_size"], cfg["max_blocks_per_seq"]
    rng = np.random.default_rng(seed)

    lens, prefix = _draw_lengths(rng, cfg["lens"], S)
    if (lens > MB * bs).any():
        raise ValueError("a drawn length exceeds max_blocks_per_seq * block_size")
    nblk = (lens + bs - 1) // bs
    shared = 0
    if prefix is not None:
        if prefix % bs:
            raise ValueError("the shared prefix must fill whole blocks")
        shared = prefix // bs
        demand = shared + int((nblk - shared).sum())
    else:
        demand = int(nblk.sum())
    pool = cfg["pool"]
    N = pool[1] if pool[0] == "fixed" else int(math.ceil((1.0 + pool[1]) * demand))
    if N < demand:
        raise ValueError("pool smaller than demand")

    perm = rng.permutation(N).astype(np.int64)
    bt = np.full((S, MB), -1, dtype=np.int32)
    nxt = 0
    if shared:
        shared_ids = perm[:shared]
        nxt = shared
    for s in range(S):
        n_own = int(nblk[s]) - shared
        row = []
        if shared:
            row.extend(shared_ids.tolist())
        row.extend(perm[nxt:nxt + n_own].tolist())
        nxt += n_own
        bt[s, :len(row)] = row

    qs = None
    if cfg["lens"][0] == "chunk" or "new_tokens" in cfg:
        # the last n_s cached tokens of each sequence are new and each has a query
        if "new_tokens" in cfg:
            new = np.minimum(np.asarray(cfg["new_tokens"], dtype=np.int64), lens)
        else:
            new = np.full(S, cfg["lens"][3], dtype=np.int64)
        qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        q32 = rng.standard_normal((int(qs[-1]), Hq, D), dtype=np.float32)
    else:
        q32 = rng.standard_normal((S, Hq, D), dtype=np.float32)
    if q_gain != 1.0:
        q32 *= np.float32(q_gain)

    # pools: N(0, 1) in every owned block, NaN in every free block
    owned = np.zeros(N, dtype=bool)
    for s in range(S):
        owned[bt[s, :nblk[s]]] = True
    k_cache = _fill_pool((Hkv, bs, D), N, seed, 1, dtype, owned)
    v_cache = _fill_pool((Hkv, D, bs), N, seed, 2, dtype, owned)
    nan = _nan(dtype)
    for s in range(S):  # the unfilled tail of each sequence's last block
        L = int(lens[s])
        if L % bs:
            last = bt[s, L // bs]
            k_cache[last, :, L % bs:, :] = nan
            v_cache[last, :, :, L % bs:] = nan

    k_new = v_new = slots = None
    if cfg.get("cache_write"):
        # the last attended position of each sequence is the token being appended
        pos = lens - 1
        if (pos < 0).any():
            raise ValueError("a batch that appends a token needs every length >= 1")
        blk = bt[np.arange(S), pos // bs].astype(np.int64)
        off = pos % bs
        slots = blk * bs + off
        k_cache[blk, :, off, :] = nan
        v_cache[blk, :, :, off] = nan
        kn32 = rng.standard_normal((S, Hkv, D), dtype=np.float32)
        vn32 = rng.standard_normal((S, Hkv, D), dtype=np.float32)
        k_new, v_new = to_storage(kn32, dtype), to_storage(vn32, dtype)

    scale = float(np.float32(1.0 / math.sqrt(D)))
    return Batch(name=name, seed=seed, dtype=dtype, num_seqs=S, num_q_heads=Hq,
                 num_kv_heads=Hkv, head_dim=D, block_size=bs, max_blocks_per_seq=MB,
                 num_blocks=N, scale=scale, seq_lens=lens.astype(np.int32), block_tables=bt,
                 q=to_storage(q32, dtype), k_cache=k_cache, v_cache=v_cache, query_start=qs,
                 k_new=k_new, v_new=v_new,
                 slot_mapping=None if slots is None else slots.astype(np.int64),
                 partition_size=int(cfg.get("partition_size", 0)), shared_blocks=shared)


def as_torch(arr: np.ndarray, dtype: str, device="cpu"):
    """View numpy storage as a torch tensor of the matching dtype (no rounding)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """Inverse of ``as_torch``: raw numpy storage of a (CPU or GPU) tensor."""
    import torch
    t = t.detach().contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()
