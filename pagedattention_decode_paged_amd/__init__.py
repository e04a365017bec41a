"""Paged decode attention for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libpagedkv.so`` (the C ABI in
``include/pagedkv.h``).  It only marshals arguments: every step of the path
runs in the library's HIP kernels.  PyTorch is used to hold device memory and
to name the current stream.  There is no fallback: if the library is missing
or fails to load, importing the binding raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDKV_LIBRARY names another build of the same library (the host-sanitizer
# build of sanitize_check.py); the default is the in-tree libpagedkv.so.
LIB_PATH = os.environ.get("PAGEDKV_LIBRARY") or os.path.join(_HERE, "libpagedkv.so")

KVP_OK, KVP_ERR_INVALID_ARG, KVP_ERR_OUT_OF_MEMORY, KVP_ERR_UNSUPPORTED, KVP_ERR_HIP = 0, -1, -2, -3, -4
KVP_F32, KVP_BF16, KVP_INT8, KVP_INT4 = 0, 1, 2, 3

# the pool dtype of an INT4 cache (torch has no 4-bit type: its codes are
# viewed as uint8, two per byte)
INT4 = "int4"

_TORCH_TO_KVP = {torch.float32: KVP_F32, torch.bfloat16: KVP_BF16, torch.int8: KVP_INT8}
_KVP_TO_TORCH = {v: k for k, v in _TORCH_TO_KVP.items()}


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class _PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("latent", ctypes.c_int32)]


class _PoolView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("total_bytes", ctypes.c_size_t),
                ("desc", _PoolDesc)]


class _DecodeDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_h", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
                ("split_tokens", ctypes.c_int32), ("total_context_len", ctypes.c_int64),
                ("workgroups", ctypes.c_int32), ("shared_prefix_tokens", ctypes.c_int32),
                ("window", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python pagedattention_decode_paged_amd/build.py`"
            " (or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "kvp_last_error": (ctypes.c_char_p, []),
        "kvp_version": (ctypes.c_char_p, []),
        "kv_pool_required_bytes": (SZ, [ctypes.POINTER(_PoolDesc)]),
        "kv_pool_create": (ctypes.c_int, [ctypes.POINTER(_PoolDesc), P, SZ, ctypes.POINTER(P)]),
        "kv_pool_destroy": (None, [P]),
        "kv_pool_view_get": (ctypes.c_int, [P, ctypes.POINTER(_PoolView)]),
        "paged_slot_mapping": (ctypes.c_int, [P, I32, I32, P, P, I64, P, P]),
        "reshape_and_cache": (ctypes.c_int, [P, P, P, ctypes.c_int, P, I64, P]),
        "paged_decode_workspace_size": (SZ, [ctypes.POINTER(_DecodeDesc)]),
        "paged_decode_split_tokens": (I32, [ctypes.POINTER(_DecodeDesc)]),
        "paged_decode_mla_workgroups": (I32, [ctypes.POINTER(_DecodeDesc)]),
        "paged_decode_attention": (ctypes.c_int, [P, P, P, P, P, F, P, ctypes.POINTER(_DecodeDesc), P, SZ, P]),
        "paged_decode_attention_int8": (ctypes.c_int, [P, P, P, P, P, P, P, F, P,
                                                       ctypes.POINTER(_DecodeDesc), P, SZ, P]),
        "paged_decode_attention_mla": (ctypes.c_int, [P, P, P, P, F, P, ctypes.POINTER(_DecodeDesc), P, SZ, P]),
        "paged_decode_attention_int4": (ctypes.c_int, [P, P, P, P, P, P, P, I32, P, P, F, P,
                                                       ctypes.POINTER(_DecodeDesc), P, SZ, P]),
        "paged_decode_attention_append": (ctypes.c_int, [P, P, P, P, P, P, F, P, ctypes.POINTER(_DecodeDesc),
                                                         P, SZ, P]),
        "paged_decode_attention_append_noalloc": (ctypes.c_int, [P, P, P, P, P, P, F, P,
                                                                 ctypes.POINTER(_DecodeDesc), P]),
        "paged_gather": (ctypes.c_int, [P, I32, I32, I32, I32, P, I32, P, I32, I32, P, P]),
        "kvp_stream_read": (ctypes.c_int, [P, SZ, P, I32, P]),
        "kvp_mfma_peak": (ctypes.c_int, [P, I32, I32, P]),
        "paged_prefill_attention": (ctypes.c_int, [P, P, P, P, P, P, F, P, ctypes.POINTER(_DecodeDesc), I32, P]),
        "kvp_allocator_create": (ctypes.c_int, [I64, I32, P, ctypes.POINTER(P)]),
        "kvp_allocator_destroy": (None, [P]),
        "kvp_block_hash": (ctypes.c_uint64, [ctypes.c_uint64, P, I32]),
        "kvp_allocate_prompt": (ctypes.c_int, [P, P, I64, P, I32, ctypes.POINTER(I32), ctypes.POINTER(I64)]),
        "kvp_append_slot": (ctypes.c_int, [P, P, ctypes.POINTER(I32), I32, ctypes.POINTER(I64),
                                           ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "kvp_fork_sequence": (ctypes.c_int, [P, P, I32]),
        "kvp_free_sequence": (ctypes.c_int, [P, P, I32]),
        "kvp_allocator_block_state": (ctypes.c_int, [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                                     ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_uint64)]),
        "kvp_allocator_evictable": (I64, [P, P, I64]),
        "kv_pool_block_bytes": (SZ, [P]),
        "copy_blocks": (ctypes.c_int, [P, P, I64, P]),
        "swap_out_blocks": (ctypes.c_int, [P, P, I64, P, P, P]),
        "swap_in_blocks": (ctypes.c_int, [P, P, I64, P, P, P]),
        "paged_decode_validate": (ctypes.c_int, [P, P, ctypes.POINTER(_DecodeDesc), I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED_SYMBOLS = (
    "kvp_last_error", "kvp_version", "kv_pool_required_bytes", "kv_pool_create", "kv_pool_destroy",
    "kv_pool_view_get", "paged_slot_mapping", "reshape_and_cache", "paged_decode_workspace_size",
    "paged_decode_split_tokens", "paged_decode_mla_workgroups", "paged_decode_attention",
    "paged_decode_attention_int8",
    "paged_decode_attention_mla", "paged_decode_attention_append", "paged_decode_attention_append_noalloc",
    "paged_gather", "paged_decode_validate", "paged_decode_attention_int4",
    "kvp_allocator_create", "kvp_allocator_destroy", "kvp_block_hash", "kvp_allocate_prompt", "kvp_append_slot",
    "kvp_fork_sequence", "kvp_free_sequence", "kvp_allocator_block_state", "kvp_allocator_evictable",
    "kv_pool_block_bytes", "copy_blocks", "swap_out_blocks", "swap_in_blocks", "paged_prefill_attention",
    "kvp_stream_read", "kvp_mfma_peak",
)


def lib() -> ctypes.CDLL:
    return _lib


def version() -> str:
    return _lib.kvp_version().decode()


def _check(status: int) -> None:
    if status != KVP_OK:
        raise PagedKVError(status, _lib.kvp_last_error().decode())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts: torch.Tensor) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        dev = t.device if dev is None else dev
    return dev


# --------------------------------------------------------------------- pool

@dataclass
class KVPool:
    """A pool created by ``kv_pool_create``; its memory is a torch uint8
    tensor owned by this object, and ``k``/``v``/``k_scale``/``v_scale`` are
    views of it in the pool layout ``[num_blocks, block_size, n_kv, d]``."""
    handle: ctypes.c_void_p
    storage: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    k_scale: torch.Tensor | None
    v_scale: torch.Tensor | None
    num_blocks: int
    block_size: int
    n_kv: int
    d_k: int
    d_v: int
    dtype: torch.dtype
    latent: bool

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:   # (None at interpreter exit)
            _lib.kv_pool_destroy(h)
            self.handle = ctypes.c_void_p(None)


def _kvp_dtype(dtype) -> int:
    return KVP_INT4 if dtype == INT4 else _TORCH_TO_KVP[dtype]


def kv_pool_required_bytes(num_blocks, block_size, n_kv, d_k, d_v, dtype, latent=False) -> int:
    d = _PoolDesc(num_blocks, block_size, n_kv, d_k, d_v, _kvp_dtype(dtype), int(latent))
    return int(_lib.kv_pool_required_bytes(ctypes.byref(d)))


def kv_pool_create(num_blocks: int, block_size: int, n_kv: int, d_k: int, d_v: int,
                   dtype: torch.dtype, latent: bool = False, device="cuda") -> KVPool:
    if dtype != INT4 and dtype not in _TORCH_TO_KVP:
        raise ValueError(f"unsupported pool dtype {dtype}")
    d = _PoolDesc(num_blocks, block_size, n_kv, d_k, d_v, _kvp_dtype(dtype), int(latent))
    nbytes = int(_lib.kv_pool_required_bytes(ctypes.byref(d)))
    if nbytes == 0:
        # let the library name the problem
        h = ctypes.c_void_p()
        _check(_lib.kv_pool_create(ctypes.byref(d), None, 0, ctypes.byref(h)))
    storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
    h = ctypes.c_void_p()
    _check(_lib.kv_pool_create(ctypes.byref(d), _ptr(storage), nbytes, ctypes.byref(h)))
    view = _PoolView()
    _check(_lib.kv_pool_view_get(h, ctypes.byref(view)))
    base = storage.data_ptr()

    def sub(addr, count, dt, shape):
        if addr is None:
            return None
        off = addr - base
        nb = count * torch.empty((), dtype=dt).element_size()
        return storage[off:off + nb].view(dt).view(shape)

    slots = num_blocks * block_size
    if dtype == INT4:      # codes as uint8, two per byte
        k = sub(view.k, slots * n_kv * d_k // 2, torch.uint8, (num_blocks, block_size, n_kv, d_k // 2))
        v = sub(view.v, slots * n_kv * d_v // 2, torch.uint8, (num_blocks, block_size, n_kv, d_v // 2))
    else:
        k = sub(view.k, slots * n_kv * d_k, dtype, (num_blocks, block_size, n_kv, d_k))
        v = k if latent else sub(view.v, slots * n_kv * d_v, dtype, (num_blocks, block_size, n_kv, d_v))
    ks = sub(view.k_scale, slots * n_kv, torch.float32, (num_blocks, n_kv, block_size))
    vs = sub(view.v_scale, slots * n_kv, torch.float32, (num_blocks, n_kv, block_size))
    return KVPool(h, storage, k, v, ks, vs, num_blocks, block_size, n_kv, d_k, d_v, dtype, latent)


# --------------------------------------------------------------------- cache ops

def paged_slot_mapping(block_table: torch.Tensor, seq_ids: torch.Tensor, positions: torch.Tensor,
                       block_size: int, out: torch.Tensor | None = None) -> torch.Tensor:
    dev = _need_cuda(block_table, seq_ids, positions)
    if block_table.dtype != torch.int32 or seq_ids.dtype != torch.int32 or positions.dtype != torch.int32:
        raise TypeError("block_table, seq_ids and positions must be int32")
    n = seq_ids.numel()
    if positions.numel() != n:
        raise ValueError("seq_ids and positions differ in length")
    if out is None:
        out = torch.empty(n, dtype=torch.int64, device=dev)
    _check(_lib.paged_slot_mapping(_ptr(block_table), block_table.shape[1], block_size,
                                   _ptr(seq_ids), _ptr(positions), n, _ptr(out), _stream(dev)))
    return out


def reshape_and_cache(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor | None,
                      slot_mapping: torch.Tensor) -> None:
    dev = _need_cuda(k_new, v_new, slot_mapping)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    n = slot_mapping.numel()
    if k_new.shape != (n, pool.n_kv, pool.d_k):
        raise ValueError(f"k_new must be [{n}, {pool.n_kv}, {pool.d_k}]")
    if not pool.latent and (v_new is None or v_new.shape != (n, pool.n_kv, pool.d_v)):
        raise ValueError(f"v_new must be [{n}, {pool.n_kv}, {pool.d_v}]")
    if v_new is not None and v_new.dtype != k_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    _check(_lib.reshape_and_cache(pool.handle, _ptr(k_new), _ptr(v_new), _TORCH_TO_KVP[k_new.dtype],
                                  _ptr(slot_mapping), n, _stream(dev)))


def paged_gather(pool: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                 max_context_len: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows 0..ctx-1 of each sequence in logical order, bit for bit:
    ``[B, max_context_len, n_kv, d]``; rows past a sequence's length keep
    ``out``'s previous contents (zeros when ``out`` is None)."""
    dev = _need_cuda(pool, block_table, context_lens)
    nb, bs, n_kv, d = pool.shape
    B = context_lens.numel()
    if out is None:
        out = torch.zeros((B, max_context_len, n_kv, d), dtype=pool.dtype, device=dev)
    _check(_lib.paged_gather(_ptr(pool), pool.element_size(), bs, n_kv, d, _ptr(block_table),
                             block_table.shape[1], _ptr(context_lens), B, max_context_len, _ptr(out),
                             _stream(dev)))
    return out


# --------------------------------------------------------------------- decode

def _desc(q, block_table, context_lens, n_kv, d_k, d_v, block_size, kv_dtype, max_context_len,
          split_tokens, total_context_len, workgroups=0, shared_prefix_tokens=0, window=0) -> _DecodeDesc:
    B, n_h, _ = q.shape
    return _DecodeDesc(B, n_h, n_kv, d_k, d_v, block_size, block_table.shape[1], int(max_context_len),
                       _TORCH_TO_KVP[q.dtype], kv_dtype, int(split_tokens), int(total_context_len),
                       int(workgroups), int(shared_prefix_tokens), int(window))


def decode_workspace_size(desc: _DecodeDesc) -> int:
    return int(_lib.paged_decode_workspace_size(ctypes.byref(desc)))


def decode_split_tokens(desc: _DecodeDesc) -> int:
    return int(_lib.paged_decode_split_tokens(ctypes.byref(desc)))


def decode_mla_workgroups(desc: _DecodeDesc) -> int:
    return int(_lib.paged_decode_mla_workgroups(ctypes.byref(desc)))


def alloc_workspace(desc: _DecodeDesc, device="cuda") -> torch.Tensor | None:
    """A workspace for calls of this description (reusable by later calls
    on the same stream that need no more bytes)."""
    need = decode_workspace_size(desc)
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def _workspace(desc, workspace, dev):
    need = decode_workspace_size(desc)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, needs {need}")
    return workspace, workspace.numel()


def paged_decode_attention(q, k_pool, v_pool, block_table, context_lens, scale, out=None, *,
                           max_context_len, split_tokens=0, total_context_len=0, workspace=None,
                           shared_prefix_tokens=0, window=0):
    """``out[b, h] = softmax(scale * q[b, h] . K) V`` over each sequence's
    paged K/V (pools ``[num_blocks, block_size, n_kv, d]``).
    ``shared_prefix_tokens``: a hint that the sequences' first tokens share
    physical blocks (read once for all of them; checked on the device).
    ``window``: attend to each sequence's last ``window`` tokens only."""
    dev = _need_cuda(q, k_pool, v_pool, block_table, context_lens)
    _, bs, n_kv, d_k = k_pool.shape
    d_v = v_pool.shape[3]
    desc = _desc(q, block_table, context_lens, n_kv, d_k, d_v, bs, _TORCH_TO_KVP[k_pool.dtype],
                 max_context_len, split_tokens, total_context_len, 0, shared_prefix_tokens, window)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], d_v), dtype=q.dtype, device=dev)
    ws, wsb = _workspace(desc, workspace, dev)
    _check(_lib.paged_decode_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                       _ptr(context_lens), float(scale), _ptr(out), ctypes.byref(desc),
                                       _ptr(ws), wsb, _stream(dev)))
    return out


def paged_decode_attention_int8(q, k_codes, k_scale, v_codes, v_scale, block_table, context_lens,
                                scale, out=None, *, max_context_len, split_tokens=0,
                                total_context_len=0, workspace=None, window=0):
    dev = _need_cuda(q, k_codes, k_scale, v_codes, v_scale, block_table, context_lens)
    _, bs, n_kv, d_k = k_codes.shape
    d_v = v_codes.shape[3]
    desc = _desc(q, block_table, context_lens, n_kv, d_k, d_v, bs, KVP_INT8, max_context_len,
                 split_tokens, total_context_len, 0, 0, window)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], d_v), dtype=q.dtype, device=dev)
    ws, wsb = _workspace(desc, workspace, dev)
    _check(_lib.paged_decode_attention_int8(_ptr(q), _ptr(k_codes), _ptr(k_scale), _ptr(v_codes),
                                            _ptr(v_scale), _ptr(block_table), _ptr(context_lens),
                                            float(scale), _ptr(out), ctypes.byref(desc), _ptr(ws), wsb,
                                            _stream(dev)))
    return out


def paged_decode_attention_int4(q, k_codes, k_scale, v_codes, v_scale, sink_k, sink_v, block_table, context_lens,
                                scale, out=None, *, max_context_len, split_tokens=0, total_context_len=0,
                                workspace=None):
    """INT4 cache (codes ``uint8 [NB, bs, n_kv, d / 2]``, two per byte) with
    the first ``sink_k.shape[1]`` positions of every sequence taken
    unquantized from ``sink_k`` / ``sink_v`` (``bf16 [B, n_sink, n_kv, d]``;
    None for no sink)."""
    dev = _need_cuda(q, k_codes, k_scale, v_codes, v_scale, block_table, context_lens, sink_k, sink_v)
    _, bs, n_kv, half = k_codes.shape
    d = 2 * half
    desc = _desc(q, block_table, context_lens, n_kv, d, d, bs, KVP_INT4, max_context_len, split_tokens,
                 total_context_len)
    n_sink = 0 if sink_k is None else int(sink_k.shape[1])
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], d), dtype=q.dtype, device=dev)
    ws, wsb = _workspace(desc, workspace, dev)
    _check(_lib.paged_decode_attention_int4(_ptr(q), _ptr(k_codes), _ptr(k_scale), _ptr(v_codes), _ptr(v_scale),
                                            _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(block_table),
                                            _ptr(context_lens), float(scale), _ptr(out), ctypes.byref(desc),
                                            _ptr(ws), wsb, _stream(dev)))
    return out


def paged_decode_attention_mla(q, latent_pool, block_table, context_lens, scale, d_v, out=None, *,
                               max_context_len, total_context_len=0, workgroups=0, workspace=None):
    """Absorbed MLA: ``out[b, h] = softmax(scale * q[b, h] . C) C[:, :d_v]``
    over each sequence's paged latent rows (pool ``[num_blocks, block_size,
    1, d_k]``).  ``workgroups`` = persistent workgroups (0 = one per CU)."""
    dev = _need_cuda(q, latent_pool, block_table, context_lens)
    _, bs, n_kv, d_k = latent_pool.shape
    desc = _desc(q, block_table, context_lens, n_kv, d_k, d_v, bs, _TORCH_TO_KVP[latent_pool.dtype],
                 max_context_len, 0, total_context_len, workgroups)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], d_v), dtype=q.dtype, device=dev)
    ws, wsb = _workspace(desc, workspace, dev)
    _check(_lib.paged_decode_attention_mla(_ptr(q), _ptr(latent_pool), _ptr(block_table),
                                           _ptr(context_lens), float(scale), _ptr(out),
                                           ctypes.byref(desc), _ptr(ws), wsb, _stream(dev)))
    return out


def _append_desc(pool: KVPool, q, block_table, context_lens, max_context_len, split_tokens,
                 total_context_len, workgroups, window=0) -> _DecodeDesc:
    kv = KVP_INT8 if pool.dtype == torch.int8 else _kvp_dtype(pool.dtype)
    return _desc(q, block_table, context_lens, pool.n_kv, pool.d_k, pool.d_v, pool.block_size, kv,
                 max_context_len, split_tokens, total_context_len, workgroups, 0, window)


def paged_decode_attention_append(pool: KVPool, q, k_new, v_new, block_table, context_lens, scale,
                                  out=None, *, max_context_len, split_tokens=0, total_context_len=0,
                                  workgroups=0, workspace=None, window=0):
    """One decode step: write each sequence's new K/V row (``k_new``/``v_new``
    ``[B, n_kv, d]`` in q's dtype; ``v_new`` None for a latent pool) at position
    ``context_lens[b] - 1``, then attend (the decode call of the pool's kind)."""
    dev = _need_cuda(q, k_new, block_table, context_lens)
    desc = _append_desc(pool, q, block_table, context_lens, max_context_len, split_tokens,
                        total_context_len, workgroups, window)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], pool.d_v), dtype=q.dtype, device=dev)
    ws, wsb = _workspace(desc, workspace, dev)
    _check(_lib.paged_decode_attention_append(pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                              _ptr(block_table), _ptr(context_lens), float(scale),
                                              _ptr(out), ctypes.byref(desc), _ptr(ws), wsb, _stream(dev)))
    return out


def paged_decode_attention_append_noalloc(pool: KVPool, q, k_new, v_new, block_table, context_lens,
                                          scale, out, *, max_context_len, split_tokens=0,
                                          total_context_len=0, workgroups=0):
    """``paged_decode_attention_append`` with the library's static scratch
    instead of a workspace: allocates nothing (``out`` is the caller's)."""
    dev = _need_cuda(q, k_new, block_table, context_lens, out)
    desc = _append_desc(pool, q, block_table, context_lens, max_context_len, split_tokens,
                        total_context_len, workgroups)
    _check(_lib.paged_decode_attention_append_noalloc(pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                                      _ptr(block_table), _ptr(context_lens), float(scale),
                                                      _ptr(out), ctypes.byref(desc), _stream(dev)))
    return out


def make_desc(*, B, n_h, n_kv, d_k, d_v, block_size, max_blocks_per_seq, max_context_len,
              q_dtype, kv_dtype, split_tokens=0, total_context_len=0, workgroups=0,
              shared_prefix_tokens=0, window=0) -> _DecodeDesc:
    """A decode description from plain values (dtype codes KVP_F32/BF16/INT8)."""
    return _DecodeDesc(B, n_h, n_kv, d_k, d_v, block_size, max_blocks_per_seq, max_context_len,
                       q_dtype, kv_dtype, split_tokens, total_context_len, workgroups, shared_prefix_tokens,
                       window)


def paged_decode_validate(block_table, context_lens, desc: _DecodeDesc, num_blocks: int) -> None:
    dev = _need_cuda(block_table, context_lens)
    _check(_lib.paged_decode_validate(_ptr(block_table), _ptr(context_lens), ctypes.byref(desc),
                                      int(num_blocks), _stream(dev)))


def paged_prefill_attention(q, k_pool, v_pool, block_table, start_pos, chunk_lens, scale, out=None, *,
                            max_context_len):
    """Causal attention of each sequence's chunk of new tokens (``q [B, C,
    n_h, 128]`` bf16, positions ``start_pos[b] + i`` for ``i <
    chunk_lens[b]``) over its paged cache, the chunk's own K/V included."""
    dev = _need_cuda(q, k_pool, v_pool, block_table, start_pos, chunk_lens)
    B, C, n_h, d = q.shape
    _, bs, n_kv, d_k = k_pool.shape
    desc = _DecodeDesc(B, n_h, n_kv, d_k, v_pool.shape[3], bs, block_table.shape[1], int(max_context_len),
                       _TORCH_TO_KVP[q.dtype], _TORCH_TO_KVP[k_pool.dtype], 0, 0, 0, 0, 0)
    if out is None:
        out = torch.zeros((B, C, n_h, v_pool.shape[3]), dtype=q.dtype, device=dev)
    _check(_lib.paged_prefill_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(start_pos),
                                        _ptr(chunk_lens), float(scale), _ptr(out), ctypes.byref(desc), C,
                                        _stream(dev)))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0) -> None:
    """The read-ceiling probe: a plain streaming read of ``buf``."""
    dev = _need_cuda(buf, sink)
    _check(_lib.kvp_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), workgroups, _stream(dev)))


def mfma_peak(sink: torch.Tensor, workgroups: int = 0, iterations: int = 4096) -> int:
    """The matrix-core probe; returns the FLOPs the call performs."""
    dev = _need_cuda(sink)
    _check(_lib.kvp_mfma_peak(_ptr(sink), workgroups, iterations, _stream(dev)))
    wg = workgroups if workgroups > 0 else 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    return wg * 4 * iterations * 8 * 16384


# --------------------------------------------------------------------- block allocator

def _i32_array(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*[int(v) for v in values])
    return arr


def block_hash(parent: int, token_ids) -> int:
    """One step of the allocator's chained block hash (BLAKE2b-64)."""
    arr = _i32_array(token_ids)
    return int(_lib.kvp_block_hash(ctypes.c_uint64(parent), arr, len(token_ids)))


class BlockAllocator:
    """The library's host block allocator (``kvp_allocator_*``): reference
    counts, chained-hash prefix reuse, an LRU list of evictable blocks and
    copy-on-write.  Block tables are Python lists of block ids."""

    def __init__(self, num_blocks: int, block_size: int, order=None, max_blocks_per_seq: int = 1 << 16):
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        h = ctypes.c_void_p()
        arr = None if order is None else _i32_array(order)
        _check(_lib.kvp_allocator_create(num_blocks, block_size, arr, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.kvp_allocator_destroy(h)
            self._h = ctypes.c_void_p(None)

    def allocate_prompt(self, token_ids) -> tuple[list[int], int]:
        toks = _i32_array(token_ids)
        out = (ctypes.c_int32 * self.max_blocks)()
        nb, cached = ctypes.c_int32(), ctypes.c_int64()
        _check(_lib.kvp_allocate_prompt(self._h, toks, len(token_ids), out, self.max_blocks, ctypes.byref(nb),
                                        ctypes.byref(cached)))
        return list(out[:nb.value]), int(cached.value)

    def allocate_batch(self, prompts):
        """Tables of a batch of new prompts, allocated in order (a prompt
        that repeats an earlier one's leading full blocks shares them):
        ``(block_table int32 [B, max blocks] padded with -1, context_lens
        int32 [B], tokens found cached per prompt)``."""
        tables, cached = [], []
        for p in prompts:
            t, c = self.allocate_prompt(p)
            tables.append(t)
            cached.append(c)
        width = max([len(t) for t in tables] + [1])
        bt = np.full((len(tables), width), -1, dtype=np.int32)
        for b, t in enumerate(tables):
            bt[b, :len(t)] = t
        ctx = np.array([len(p) for p in prompts], dtype=np.int32)
        return bt, ctx, cached

    def append_slot(self, table: list[int]):
        """Slot of one appended token; ``table`` is updated in place.
        Returns ``(slot, (src, dst) or None)``."""
        arr = (ctypes.c_int32 * self.max_blocks)(*table)
        nb = ctypes.c_int32(len(table))
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.kvp_append_slot(self._h, arr, ctypes.byref(nb), self.max_blocks, ctypes.byref(slot),
                                    ctypes.byref(src), ctypes.byref(dst)))
        table[:] = list(arr[:nb.value])
        return int(slot.value), (None if src.value < 0 else (int(src.value), int(dst.value)))

    def fork(self, table: list[int]) -> list[int]:
        _check(_lib.kvp_fork_sequence(self._h, _i32_array(table), len(table)))
        return list(table)

    def free_sequence(self, table) -> None:
        _check(_lib.kvp_free_sequence(self._h, _i32_array(table), len(table)))

    def block_state(self, block: int):
        """``(ref_count, fill, hashed, hash)`` of one block."""
        r, f, hd, hv = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
        _check(_lib.kvp_allocator_block_state(self._h, block, ctypes.byref(r), ctypes.byref(f), ctypes.byref(hd),
                                              ctypes.byref(hv)))
        return int(r.value), int(f.value), bool(hd.value), int(hv.value)

    def evictable(self) -> list[int]:
        n = int(_lib.kvp_allocator_evictable(self._h, None, 0))
        out = (ctypes.c_int32 * max(1, n))()
        _lib.kvp_allocator_evictable(self._h, out, n)
        return list(out[:n])


# --------------------------------------------------------------------- block copies and swaps

def kv_pool_block_bytes(pool: KVPool) -> int:
    return int(_lib.kv_pool_block_bytes(pool.handle))


def copy_blocks(pool: KVPool, pairs: torch.Tensor) -> None:
    """Copy block src onto block dst for each row (src, dst) of ``pairs``
    (device int32 ``[n, 2]``), in every region of the pool."""
    dev = _need_cuda(pairs)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n, 2] tensor")
    _check(_lib.copy_blocks(pool.handle, _ptr(pairs), pairs.shape[0], _stream(dev)))


def _swap_args(pool: KVPool, blocks: torch.Tensor, staging: torch.Tensor, host: torch.Tensor):
    dev = _need_cuda(blocks, staging)
    if blocks.dtype != torch.int32 or blocks.dim() != 1 or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous int32 [n] tensor")
    if host.is_cuda or not host.is_contiguous():
        raise ValueError("host must be a contiguous host tensor")
    need = blocks.numel() * kv_pool_block_bytes(pool)
    for name, t in (("staging", staging), ("host", host)):
        if not t.is_contiguous() or t.numel() * t.element_size() < need:
            raise ValueError(f"{name} must be contiguous with at least {need} bytes")
    return dev


def swap_out_blocks(pool: KVPool, blocks: torch.Tensor, staging: torch.Tensor, host: torch.Tensor) -> None:
    """Blocks (device int32 ``[n]``) -> ``host`` (pinned uint8, ``n *
    kv_pool_block_bytes`` bytes) through the device ``staging`` buffer."""
    dev = _swap_args(pool, blocks, staging, host)
    _check(_lib.swap_out_blocks(pool.handle, _ptr(blocks), blocks.numel(), _ptr(staging), _ptr(host), _stream(dev)))


def swap_in_blocks(pool: KVPool, blocks: torch.Tensor, staging: torch.Tensor, host: torch.Tensor) -> None:
    """The inverse of :func:`swap_out_blocks`: ``host`` -> staging -> blocks."""
    dev = _swap_args(pool, blocks, staging, host)
    _check(_lib.swap_in_blocks(pool.handle, _ptr(blocks), blocks.numel(), _ptr(staging), _ptr(host), _stream(dev)))


# --------------------------------------------------------------------- prepared calls

class PreparedCall:
    """A library call with its arguments marshalled once (for tight loops:
    decode steps over many layers).  Calling it enqueues the same work on
    the current stream of the tensors' device."""

    def __init__(self, fn, args, device, keep):
        self._fn = fn
        self._args = list(args)
        self._device = device
        self._keep = keep          # tensors that must stay alive

    def __call__(self) -> None:
        self._args[-1] = _stream(self._device)
        _check(self._fn(*self._args))


def prepare_decode(q, k_pool, v_pool, block_table, context_lens, scale, out, *, max_context_len,
                   split_tokens=0, total_context_len=0, workspace=None,
                   shared_prefix_tokens=0) -> PreparedCall:
    dev = _need_cuda(q, k_pool, v_pool, block_table, context_lens, out)
    _, bs, n_kv, d_k = k_pool.shape
    desc = _desc(q, block_table, context_lens, n_kv, d_k, v_pool.shape[3], bs,
                 _TORCH_TO_KVP[k_pool.dtype], max_context_len, split_tokens, total_context_len, 0,
                 shared_prefix_tokens)
    ws, wsb = _workspace(desc, workspace, dev)
    args = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(context_lens),
            ctypes.c_float(scale), _ptr(out), ctypes.byref(desc), _ptr(ws), wsb, None)
    return PreparedCall(_lib.paged_decode_attention, args, dev,
                        (q, k_pool, v_pool, block_table, context_lens, out, ws, desc))


def prepare_reshape_and_cache(pool: KVPool, k_new, v_new, slot_mapping) -> PreparedCall:
    dev = _need_cuda(k_new, v_new, slot_mapping)
    n = slot_mapping.numel()
    args = (pool.handle, _ptr(k_new), _ptr(v_new), _TORCH_TO_KVP[k_new.dtype], _ptr(slot_mapping), n, None)
    return PreparedCall(_lib.reshape_and_cache, args, dev, (pool, k_new, v_new, slot_mapping))


def prepare_decode_append(pool: KVPool, q, k_new, v_new, block_table, context_lens, scale, out, *,
                          max_context_len, split_tokens=0, total_context_len=0,
                          workspace=None) -> PreparedCall:
    dev = _need_cuda(q, k_new, block_table, context_lens, out)
    desc = _append_desc(pool, q, block_table, context_lens, max_context_len, split_tokens,
                        total_context_len, 0)
    ws, wsb = _workspace(desc, workspace, dev)
    args = (pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(context_lens),
            ctypes.c_float(scale), _ptr(out), ctypes.byref(desc), _ptr(ws), wsb, None)
    return PreparedCall(_lib.paged_decode_attention_append, args, dev,
                        (pool, q, k_new, v_new, block_table, context_lens, out, ws, desc))
