"""ctypes binding for libpa.so: the C entry points under the same names, taking torch
tensors.  Argument marshalling only -- shapes, dtypes and device placement are checked
here, pointers and the current HIP stream are handed to the library, and every step
of the computation runs in the library's kernels.  There is no fallback: if the
library is missing or a call fails, an exception says so."""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

from .build import LIB_PATH, INCLUDE

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_CAPACITY = range(6)
PA_F32, PA_F16, PA_BF16 = range(3)
ABI_VERSION = 4  # PA_ABI_VERSION of the header these structures mirror
TORCH_DTYPE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}


class PaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class DecodeExt(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("partition_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
                ("shared_blocks", ctypes.c_int32)]


class CacheWriteExt(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("stream", ctypes.c_void_p)]


class MultiTokenExt(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("max_query_len", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("partition_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
                ("max_seq_len", ctypes.c_int32)]


class CopyBlocksExt(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("stream", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libpa.so (built in-tree by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run paged_kv_cache_344_amd/build.py "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.pa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp,
                                ctypes.POINTER(DecodeExt)]
        L.pa_decode.restype = ctypes.c_int
        L.pa_cache_write_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                            ctypes.c_float, vp, ctypes.POINTER(DecodeExt)]
        L.pa_cache_write_decode.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = L.pa_decode.argtypes
        L.pa_decode_noalloc.restype = ctypes.c_int
        L.pa_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeExt), i32, i32,
                                                ctypes.POINTER(ctypes.c_size_t)]
        L.pa_decode_workspace_bytes.restype = ctypes.c_int
        L.pa_cache_write.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(CacheWriteExt)]
        L.pa_cache_write.restype = ctypes.c_int
        L.pa_multi_token.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp,
                                     ctypes.POINTER(MultiTokenExt)]
        L.pa_multi_token.restype = ctypes.c_int
        L.pa_multi_token_workspace_bytes.argtypes = [ctypes.POINTER(MultiTokenExt), i32, i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
        L.pa_multi_token_workspace_bytes.restype = ctypes.c_int
        L.pa_copy_blocks.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(CopyBlocksExt)]
        L.pa_copy_blocks.restype = ctypes.c_int
        L.pa_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int64, vp, ctypes.c_size_t, vp]
        L.pa_read_probe.restype = ctypes.c_int
        P32, P64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        L.pa_bm_create.argtypes = [ctypes.c_int64, i32, i32, vp, ctypes.POINTER(vp)]
        L.pa_bm_destroy.argtypes = [vp]
        L.pa_bm_destroy.restype = None
        L.pa_bm_add_sequence.argtypes = [vp, P32]
        L.pa_bm_fork.argtypes = [vp, i32, P32]
        L.pa_bm_free_sequence.argtypes = [vp, i32]
        L.pa_bm_append.argtypes = [vp, vp, i32, vp, vp, vp, P32]
        L.pa_bm_length.argtypes = [vp, i32, P32]
        L.pa_bm_export.argtypes = [vp, vp, i32, vp, vp]
        L.pa_bm_free_blocks.argtypes = [vp]
        L.pa_bm_free_blocks.restype = ctypes.c_int64
        L.pa_bm_ref_count.argtypes = [vp, i32, P32]
        for f in ("pa_bm_create", "pa_bm_add_sequence", "pa_bm_fork", "pa_bm_free_sequence",
                  "pa_bm_append", "pa_bm_length", "pa_bm_export", "pa_bm_ref_count"):
            getattr(L, f).restype = ctypes.c_int
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_last_error.argtypes = []
        L.pa_last_error.restype = ctypes.c_char_p
        L.pa_abi_version.argtypes = []
        L.pa_abi_version.restype = ctypes.c_int32
        if L.pa_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.pa_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


HEADERS = ("pa.h", "pa_block_manager.h", "pa_probe.h")


def header_functions() -> list:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        text = open(os.path.join(INCLUDE, h)).read()
        names |= set(re.findall(
            r"^\s*(?:pa_status|const char\s*\*|int32_t|int64_t|size_t|void)\s+(pa_\w+)\s*\(",
            text, re.M))
    return sorted(names)


def _check(status: int, where: str):
    if status != PA_OK:
        L = lib()
        raise PaError(status, where, L.pa_last_error().decode() or L.pa_status_string(status).decode())


def _torch_stream(device: torch.device, stream):
    """The stream a call runs on, as a torch stream object: the current one when None, a
    torch stream as given, or a raw hipStream_t (int) wrapped as an external stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream_ptr(device: torch.device, stream) -> Optional[int]:
    return _torch_stream(device, stream).cuda_stream


def _scratch_on(stream_obj, nbytes: int, zero: bool) -> torch.Tensor:
    """A byte tensor allocated (and zero-filled when asked) on the stream the call runs on,
    so that torch's caching allocator orders any later reuse of its memory after the
    call's kernels, even when the tensor is dropped right after the call returns."""
    with torch.cuda.stream(stream_obj):
        if zero:
            return torch.zeros(nbytes, dtype=torch.uint8, device=stream_obj.device)
        return torch.empty(nbytes, dtype=torch.uint8, device=stream_obj.device)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def workspace_for(q: torch.Tensor, block_tables: torch.Tensor, num_blocks: int,
                  block_size: int, num_kv_heads: int, partition_size: int = 0) -> torch.Tensor:
    """A zero-filled decode workspace for calls of this shape (reusable across calls
    that are ordered on one stream)."""
    n = pa_decode_workspace_bytes(q, block_tables, num_blocks, block_size, num_kv_heads,
                                  partition_size)
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def decode_ext(q: torch.Tensor, block_tables: torch.Tensor, num_blocks: int,
               partition_size: int = 0) -> DecodeExt:
    S, Hq, D = q.shape
    return DecodeExt(num_seqs=S, num_q_heads=Hq, head_dim=D,
                     max_blocks_per_seq=block_tables.shape[1], num_blocks=num_blocks,
                     partition_size=partition_size, dtype=TORCH_DTYPE[q.dtype],
                     workspace=None, workspace_bytes=0, stream=None)


def pa_decode_workspace_bytes(q: torch.Tensor, block_tables: torch.Tensor, num_blocks: int,
                              block_size: int, num_kv_heads: int,
                              partition_size: int = 0) -> int:
    ext = decode_ext(q, block_tables, num_blocks, partition_size)
    n = ctypes.c_size_t(0)
    _check(lib().pa_decode_workspace_bytes(ctypes.byref(ext), block_size, num_kv_heads,
                                           ctypes.byref(n)), "pa_decode_workspace_bytes")
    return int(n.value)


class PreparedDecode:
    """A pa_decode call with all marshalling done once; calling the object issues the
    single C call (no Python-side checks or allocation), e.g. inside a timed loop or
    HIP graph capture.  Keeps references to every tensor it points at."""

    def __init__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                 num_kv_heads: int, scale: float, out: torch.Tensor, *,
                 workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                 shared_blocks: bool = False, stream=None, noalloc: bool = False,
                 new_tokens=None):
        dev = q.device
        _need(dev.type == "cuda", "tensors must be on a GPU")
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                        ("block_tables", block_tables), ("seq_lens", seq_lens), ("out", out)):
            _need(t.device == dev, f"{name} is on {t.device}, q on {dev}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(q.dtype in TORCH_DTYPE, f"unsupported dtype {q.dtype}")
        _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype and out.dtype == q.dtype,
              "q, k_cache, v_cache and out must share one dtype")
        _need(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32,
              "block_tables and seq_lens must be int32")
        S, Hq, D = q.shape
        N = k_cache.shape[0]
        _need(k_cache.shape == (N, num_kv_heads, block_size, D),
              f"k_cache shape {tuple(k_cache.shape)}")
        _need(v_cache.shape == (N, num_kv_heads, D, block_size),
              f"v_cache shape {tuple(v_cache.shape)}")
        _need(block_tables.dim() == 2 and block_tables.shape[0] == S, "block_tables shape")
        _need(seq_lens.shape == (S,), "seq_lens shape")
        _need(out.shape == q.shape, "out shape")
        ext = decode_ext(q, block_tables, N, partition_size)
        need = ctypes.c_size_t(0)
        _check(lib().pa_decode_workspace_bytes(ctypes.byref(ext), block_size, num_kv_heads,
                                               ctypes.byref(need)), "pa_decode")
        ts = _torch_stream(dev, stream)
        if noalloc:
            _need(workspace is None, "a no-allocation call takes no workspace")
        else:
            if workspace is None:
                # zero-filled, as the library requires before a workspace's first use
                # (every call returns its counters to zero); allocated and cleared on the
                # launch stream, so its memory is not handed out again before the kernel
                # is done
                workspace = _scratch_on(ts, need.value, zero=True)
            _need(workspace.device == dev and workspace.is_contiguous(), "workspace placement")
            ext.workspace = workspace.data_ptr()
            ext.workspace_bytes = workspace.numel() * workspace.element_size()
        ext.stream = ts.cuda_stream
        ext.shared_blocks = 1 if shared_blocks else 0
        self.ext = ext
        self.tensors = (q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
        self.out = out
        self._where = "pa_decode_noalloc" if noalloc else "pa_decode"
        self._fn = lib().pa_decode_noalloc if noalloc else lib().pa_decode
        self._args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                      block_tables.data_ptr(), seq_lens.data_ptr(), block_size, num_kv_heads,
                      ctypes.c_float(scale), out.data_ptr(), ctypes.byref(ext))
        if new_tokens is not None:
            # one launch: each sequence's new token is stored, then decoded over
            _need(not noalloc, "the fused write + decode takes a workspace")
            k, v, slot_mapping = new_tokens
            for name, t in (("k", k), ("v", v), ("slot_mapping", slot_mapping)):
                _need(t.device == dev and t.is_contiguous(), f"{name} placement")
            _need(k.dtype == q.dtype and v.dtype == q.dtype, "k and v must have q's dtype")
            _need(k.shape == (S, num_kv_heads, D) and v.shape == k.shape, "k / v shape")
            _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (S,),
                  "slot_mapping must be int64 [S]")
            self._where = "pa_cache_write_decode"
            self._fn = lib().pa_cache_write_decode
            self._args = (k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr()) + (
                q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                seq_lens.data_ptr(), block_size, num_kv_heads, ctypes.c_float(scale),
                out.data_ptr(), ctypes.byref(ext))
            self.new_tokens = (k, v, slot_mapping)

    def __call__(self) -> torch.Tensor:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, self._where)
        return self.out

    def partition_used(self) -> int:
        """Tokens per split-K partition that the last call used (waits for it)."""
        _need(self.tensors[-1] is not None, "a no-allocation call keeps no workspace to read")
        return decode_partition_used(self.tensors[-1])


PART_SLOT_BYTE = 64  # workspace bytes 64..67: the partition length the last call used


def decode_partition_used(workspace: torch.Tensor) -> int:
    """The partition length (tokens) recorded in a decode workspace by the last call that
    used it; synchronises the device."""
    torch.cuda.synchronize(workspace.device)
    return int(workspace[PART_SLOT_BYTE:PART_SLOT_BYTE + 4].cpu().view(torch.int32).item())


def pa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
              num_kv_heads: int, scale: float, out: torch.Tensor, *,
              workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
              shared_blocks: bool = False, stream=None) -> torch.Tensor:
    """Decode attention over the paged cache (see include/pa.h for the contract).

    q, out [S, Hq, D]; k_cache [N, Hkv, bs, D]; v_cache [N, Hkv, D, bs];
    block_tables int32 [S, max_blocks]; seq_lens int32 [S].  All on one GPU.
    ``workspace`` is a byte tensor of at least ``pa_decode_workspace_bytes`` bytes,
    zero-filled before its first use (every call returns its counters to zero, so
    it can be reused); when omitted, a zero-filled one is allocated for this call.
    ``shared_blocks``: the tables may share physical blocks (common prefixes, parallel
    sampling, beam search), so K/V loads keep the default cache policy; the result is
    the same either way."""
    return PreparedDecode(q, k_cache, v_cache, block_tables, seq_lens, block_size,
                          num_kv_heads, scale, out, workspace=workspace,
                          partition_size=partition_size, shared_blocks=shared_blocks,
                          stream=stream)()


def pa_cache_write_decode(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                          q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                          num_kv_heads: int, scale: float, out: torch.Tensor, *,
                          workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                          shared_blocks: bool = False, stream=None) -> torch.Tensor:
    """One decode step in one launch (see include/pa.h): each sequence's new token (row s
    of k, v [S, Hkv, D]) is stored in slot_mapping[s] (int64 [S]), then every sequence is
    decoded; the same bits as pa_cache_write followed by pa_decode."""
    return PreparedDecode(q, k_cache, v_cache, block_tables, seq_lens, block_size,
                          num_kv_heads, scale, out, workspace=workspace,
                          partition_size=partition_size, shared_blocks=shared_blocks,
                          stream=stream, new_tokens=(k, v, slot_mapping))()


def pa_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                      num_kv_heads: int, scale: float, out: torch.Tensor, *,
                      partition_size: int = 0, shared_blocks: bool = False,
                      stream=None) -> torch.Tensor:
    """pa_decode without a workspace: the library's per-GPU static scratch serves the call
    (see include/pa.h, pa_decode_noalloc); nothing is allocated here either."""
    call = PreparedDecode(q, k_cache, v_cache, block_tables, seq_lens, block_size,
                          num_kv_heads, scale, out, partition_size=partition_size,
                          shared_blocks=shared_blocks, stream=stream, noalloc=True)
    return call()


class PreparedCacheWrite:
    """A pa_cache_write call with all marshalling done once (see PreparedDecode)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor, *, stream=None):
        dev = k.device
        _need(dev.type == "cuda", "tensors must be on a GPU")
        for name, t in (("k", k), ("v", v), ("slot_mapping", slot_mapping),
                        ("k_cache", k_cache), ("v_cache", v_cache)):
            _need(t.device == dev, f"{name} is on {t.device}, k on {dev}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(k.dtype in TORCH_DTYPE, f"unsupported dtype {k.dtype}")
        _need(v.dtype == k.dtype and k_cache.dtype == k.dtype and v_cache.dtype == k.dtype,
              "k, v and the caches must share one dtype")
        _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
        T, Hkv, D = k.shape
        N, _, bs, _ = k_cache.shape
        _need(v.shape == k.shape and slot_mapping.shape == (T,), "k / v / slot_mapping shapes")
        _need(k_cache.shape == (N, Hkv, bs, D) and v_cache.shape == (N, Hkv, D, bs),
              "cache shapes")
        self.ext = CacheWriteExt(num_tokens=T, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                                 num_blocks=N, dtype=TORCH_DTYPE[k.dtype],
                                 stream=_stream_ptr(dev, stream))
        self.tensors = (k, v, slot_mapping, k_cache, v_cache)
        self._fn = lib().pa_cache_write
        self._args = (k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
                      v_cache.data_ptr(), ctypes.byref(self.ext))

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, "pa_cache_write")


def pa_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, *, stream=None) -> None:
    """Store new tokens' K/V in their slots (see include/pa.h).  k, v [T, Hkv, D];
    slot_mapping int64 [T]; caches as for pa_decode."""
    PreparedCacheWrite(k, v, slot_mapping, k_cache, v_cache, stream=stream)()


class PreparedMultiToken:
    """A pa_multi_token call with all marshalling done once (see PreparedDecode)."""

    def __init__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start: torch.Tensor,
                 block_size: int, num_kv_heads: int, scale: float, out: torch.Tensor, *,
                 max_query_len: int, partition_size: int = 0, max_seq_len: int = 0,
                 workspace: Optional[torch.Tensor] = None, stream=None):
        dev = q.device
        _need(dev.type == "cuda", "tensors must be on a GPU")
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                        ("block_tables", block_tables), ("seq_lens", seq_lens),
                        ("query_start", query_start), ("out", out)):
            _need(t.device == dev, f"{name} is on {t.device}, q on {dev}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        _need(q.dtype in TORCH_DTYPE, f"unsupported dtype {q.dtype}")
        _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype and out.dtype == q.dtype,
              "q, k_cache, v_cache and out must share one dtype")
        _need(block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32 and
              query_start.dtype == torch.int32, "block_tables, seq_lens, query_start must be int32")
        T, Hq, D = q.shape
        S = seq_lens.shape[0]
        N = k_cache.shape[0]
        _need(k_cache.shape == (N, num_kv_heads, block_size, D),
              f"k_cache shape {tuple(k_cache.shape)}")
        _need(v_cache.shape == (N, num_kv_heads, D, block_size),
              f"v_cache shape {tuple(v_cache.shape)}")
        _need(block_tables.dim() == 2 and block_tables.shape[0] == S, "block_tables shape")
        _need(query_start.shape == (S + 1,), "query_start shape")
        _need(out.shape == q.shape, "out shape")
        ext = MultiTokenExt(num_seqs=S, num_tokens=T, max_query_len=max_query_len,
                            num_q_heads=Hq, head_dim=D, max_blocks_per_seq=block_tables.shape[1],
                            num_blocks=N, partition_size=partition_size,
                            dtype=TORCH_DTYPE[q.dtype], max_seq_len=max_seq_len)
        need = ctypes.c_size_t(0)
        _check(lib().pa_multi_token_workspace_bytes(ctypes.byref(ext), block_size, num_kv_heads,
                                                    ctypes.byref(need)), "pa_multi_token")
        self.workspace_bytes = need.value
        ts = _torch_stream(dev, stream)
        if workspace is None and need.value:
            workspace = _scratch_on(ts, need.value, zero=False)  # scratch, on the launch stream
        if workspace is not None:
            _need(workspace.device == dev and workspace.is_contiguous(), "workspace placement")
            ext.workspace = workspace.data_ptr()
            ext.workspace_bytes = workspace.numel() * workspace.element_size()
        ext.stream = ts.cuda_stream
        self.ext = ext
        self.tensors = (q, k_cache, v_cache, block_tables, seq_lens, query_start, out, workspace)
        self.out = out
        self._fn = lib().pa_multi_token
        self._args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                      block_tables.data_ptr(), seq_lens.data_ptr(), query_start.data_ptr(),
                      block_size, num_kv_heads, ctypes.c_float(scale), out.data_ptr(),
                      ctypes.byref(self.ext))

    def __call__(self) -> torch.Tensor:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, "pa_multi_token")
        return self.out


def pa_multi_token(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start: torch.Tensor,
                   block_size: int, num_kv_heads: int, scale: float, out: torch.Tensor, *,
                   max_query_len: int, partition_size: int = 0, max_seq_len: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention for several new tokens per sequence (see include/pa.h): q, out
    [T, Hq, D]; query_start int32 [S+1] on the GPU; ``max_query_len`` >= every
    sequence's number of new tokens (a host value: it sizes the launch).
    ``partition_size``: 0 splits the context automatically when the launch would be
    small, < 0 never, > 0 into partitions of that many tokens.  ``max_seq_len`` (a host
    value, 0 = the table's capacity) bounds every length: the automatic split is sized
    for it, and a longer sequence gets NaN rows.  A split call needs a
    byte tensor of ``pa_multi_token_workspace_bytes`` bytes (scratch, no zero-fill);
    when omitted, one is allocated for this call."""
    return PreparedMultiToken(q, k_cache, v_cache, block_tables, seq_lens, query_start,
                              block_size, num_kv_heads, scale, out,
                              max_query_len=max_query_len, partition_size=partition_size,
                              max_seq_len=max_seq_len, workspace=workspace, stream=stream)()


class PreparedCopyBlocks:
    """A pa_copy_blocks call with all marshalling done once (see PreparedDecode).
    ``src`` and ``dst`` are host sequences of block ids; the ids travel to the GPU
    inside the kernel arguments, so the call needs no device memory of its own."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, src, dst, *,
                 stream=None):
        dev = k_cache.device
        _need(dev.type == "cuda", "caches must be on a GPU")
        _need(v_cache.device == dev, f"v_cache is on {v_cache.device}, k_cache on {dev}")
        _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
        _need(k_cache.dtype in TORCH_DTYPE and v_cache.dtype == k_cache.dtype,
              "k_cache and v_cache must share one supported dtype")
        N, Hkv, bs, D = k_cache.shape
        _need(v_cache.shape == (N, Hkv, D, bs), f"v_cache shape {tuple(v_cache.shape)}")
        src, dst = [int(x) for x in src], [int(x) for x in dst]
        _need(len(src) == len(dst), "src and dst differ in length")
        n = len(src)
        self.src = (ctypes.c_int32 * max(n, 1))(*src)
        self.dst = (ctypes.c_int32 * max(n, 1))(*dst)
        self.ext = CopyBlocksExt(num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=N,
                                 dtype=TORCH_DTYPE[k_cache.dtype],
                                 stream=_stream_ptr(dev, stream))
        self.tensors = (k_cache, v_cache)
        self._fn = lib().pa_copy_blocks
        self._args = (k_cache.data_ptr(), v_cache.data_ptr(), self.src, self.dst, n,
                      ctypes.byref(self.ext))

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st, "pa_copy_blocks")


def pa_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src, dst, *,
                   stream=None) -> None:
    """Copy whole physical blocks of both caches, block src[i] onto block dst[i]
    (see include/pa.h): the device half of copy-on-write."""
    PreparedCopyBlocks(k_cache, v_cache, src, dst, stream=stream)()


READ_PROBE_SINK_BYTES = 2048 * 4 * 4  # PA_READ_PROBE_SINK_BYTES of include/pa_probe.h


def pa_read_probe(src: torch.Tensor, n_tiles: int, sink: torch.Tensor,
                  tiles: Optional[torch.Tensor] = None, stream=None) -> None:
    """Read n_tiles 4 KiB tiles of src once each (include/pa_probe.h): tiles 0 ..
    n_tiles-1 in order, or the int32 ids in ``tiles``; sink (at least
    READ_PROBE_SINK_BYTES bytes) receives an XOR fold of what was read.  A measurement
    aid: what a read-only kernel gets from HBM."""
    dev = src.device
    _need(src.is_cuda and src.is_contiguous(), "src must be a contiguous device tensor")
    _need(sink.device == dev and sink.is_contiguous(), "sink placement")
    if tiles is not None:
        _need(tiles.device == dev and tiles.dtype == torch.int32 and tiles.is_contiguous()
              and tiles.numel() >= n_tiles, "tiles must be int32 on src's device, n_tiles long")
    _check(lib().pa_read_probe(src.data_ptr(), src.numel() * src.element_size(),
                               None if tiles is None else tiles.data_ptr(), int(n_tiles),
                               sink.data_ptr(), sink.numel() * sink.element_size(),
                               _stream_ptr(dev, stream)), "pa_read_probe")


class BlockManager:
    """The host block manager of include/pa_block_manager.h: one C object per
    instance, freed with the instance (or by ``close()``)."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 free_order=None):
        L = lib()
        self._L = L
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        order = None
        if free_order is not None:
            free_order = [int(x) for x in free_order]
            _need(len(free_order) == num_blocks, "free_order must list every block once")
            order = (ctypes.c_int32 * num_blocks)(*free_order)
        h = ctypes.c_void_p()
        _check(L.pa_bm_create(num_blocks, block_size, max_blocks_per_seq, order,
                              ctypes.byref(h)), "pa_bm_create")
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        """The pa_block_manager* of include/pa_block_manager.h, for callers that drive the
        C functions (``lib().pa_bm_*``) with arrays of their own."""
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._L.pa_bm_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def add_sequence(self) -> int:
        out = ctypes.c_int32()
        _check(self._L.pa_bm_add_sequence(self._h, ctypes.byref(out)), "pa_bm_add_sequence")
        return out.value

    def fork(self, parent: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pa_bm_fork(self._h, parent, ctypes.byref(out)), "pa_bm_fork")
        return out.value

    def free_sequence(self, seq: int) -> None:
        _check(self._L.pa_bm_free_sequence(self._h, seq), "pa_bm_free_sequence")

    def append(self, seqs):
        """One token for each of ``seqs``: returns (slot ids, [(src, dst) copies])."""
        seqs = [int(x) for x in seqs]
        n = len(seqs)
        m = max(n, 1)
        ids = (ctypes.c_int32 * m)(*seqs)
        slots = (ctypes.c_int64 * m)()
        cs, cd = (ctypes.c_int32 * m)(), (ctypes.c_int32 * m)()
        nc = ctypes.c_int32()
        _check(self._L.pa_bm_append(self._h, ids, n, slots, cs, cd, ctypes.byref(nc)),
               "pa_bm_append")
        return list(slots[:n]), [(cs[i], cd[i]) for i in range(nc.value)]

    def length(self, seq: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pa_bm_length(self._h, seq, ctypes.byref(out)), "pa_bm_length")
        return out.value

    def export(self, seqs):
        """(block tables [n][max_blocks] padded with -1, lengths [n]) as int32 CPU tensors."""
        seqs = [int(x) for x in seqs]
        n = len(seqs)
        ids = (ctypes.c_int32 * max(n, 1))(*seqs)
        bt = torch.empty((n, self.max_blocks), dtype=torch.int32)
        sl = torch.empty((n,), dtype=torch.int32)
        _check(self._L.pa_bm_export(self._h, ids, n, bt.data_ptr() if n else None,
                                    sl.data_ptr() if n else None), "pa_bm_export")
        return bt, sl

    def free_blocks(self) -> int:
        return int(self._L.pa_bm_free_blocks(self._h))

    def ref_count(self, block: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pa_bm_ref_count(self._h, block, ctypes.byref(out)), "pa_bm_ref_count")
        return out.value
