"""The debug checks of the boundary on the GPU: paged_decode_validate, the
PAGEDKV_VALIDATE=1 mode of the decode entry points, and the out-of-memory
status of kv_pool_create.

Every table that breaks a precondition is first shown to be rejected by
paged_decode_validate itself before a decode entry point sees it, and the
debug mode is shown to be active (a context beyond max_context_len over a
table that still maps it, which no kernel would read out of bounds) before
any table with a block id outside the pool is passed: no kernel ever runs on
such a table.
"""

import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import device_normal_
from synth.workloads import custom_structure

from parity_support import TOL_BF16, host, max_err, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _desc(B, max_blocks, max_ctx, n_h=16, n_kv=2, d=128, bs=16, kv=None):
    return pk.make_desc(B=B, n_h=n_h, n_kv=n_kv, d_k=d, d_v=d, block_size=bs, max_blocks_per_seq=max_blocks,
                        max_context_len=max_ctx, q_dtype=pk.KVP_BF16,
                        kv_dtype=pk.KVP_BF16 if kv is None else kv)


def _validate_status(bt, ctx, desc, num_blocks):
    lib = pk.lib()
    rc = lib.paged_decode_validate(ctypes.c_void_p(bt.data_ptr()), ctypes.c_void_p(ctx.data_ptr()),
                                   ctypes.byref(desc), int(num_blocks),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, lib.kvp_last_error().decode()


CTXS = [37, 50, 0, 16]


def _case():
    s = custom_structure(CTXS, 16, num_blocks=20, seed=3, pad_blocks=2)
    return s, *tables_to_device(s)


def test_validate_accepts_valid_tables():
    s, bt, ctx = _case()
    # entries past each sequence's blocks are -1 (never read), and pass
    assert (s.block_table < 0).any()
    rc, msg = _validate_status(bt, ctx, _desc(len(CTXS), s.max_blocks_per_seq, 50), s.num_blocks)
    assert rc == pk.KVP_OK, msg


@pytest.mark.parametrize("case", ["block_too_large", "block_negative", "ctx_too_long", "ctx_negative"])
def test_validate_names_the_violation(case):
    s, bt, ctx = _case()
    bt_h, ctx_h = s.block_table.copy(), s.context_lens.copy()
    max_ctx = 50
    if case == "block_too_large":
        bt_h[1, 2] = s.num_blocks                  # logical block 2 of sequence 1 (tokens 32..47 < 50)
        want = f"block_table[1][2] = {s.num_blocks} outside [0, {s.num_blocks})"
    elif case == "block_negative":
        bt_h[0, 2] = -1                            # token 36 of sequence 0 lives in logical block 2
        want = "block_table[0][2] = -1"
    elif case == "ctx_too_long":
        ctx_h[3] = 51
        want = "context_lens[3] = 51 outside [0, 50]"
    else:
        ctx_h[2] = -1
        want = "context_lens[2] = -1 outside [0, 50]"
    rc, msg = _validate_status(torch.from_numpy(bt_h).cuda(), torch.from_numpy(ctx_h).cuda(),
                               _desc(len(CTXS), s.max_blocks_per_seq, max_ctx), s.num_blocks)
    assert rc == pk.KVP_ERR_INVALID_ARG
    assert want in msg, msg


def test_validate_checks_only_the_blocks_a_sequence_uses():
    s, bt, ctx = _case()
    bt_h = s.block_table.copy()
    bt_h[3, 1] = 10 ** 6                           # sequence 3 has 16 tokens: one block
    rc, msg = _validate_status(torch.from_numpy(bt_h).cuda(), ctx, _desc(len(CTXS), s.max_blocks_per_seq, 50),
                               s.num_blocks)
    assert rc == pk.KVP_OK, msg


@pytest.fixture
def validate_env():
    old = os.environ.get("PAGEDKV_VALIDATE")
    os.environ["PAGEDKV_VALIDATE"] = "1"
    yield
    if old is None:
        os.environ.pop("PAGEDKV_VALIDATE", None)
    else:
        os.environ["PAGEDKV_VALIDATE"] = old


def _pool_case(seed):
    s, bt, ctx = _case()
    pool = pk.kv_pool_create(s.num_blocks, 16, 2, 128, 128, torch.bfloat16)
    device_normal_(pool.storage.view(torch.bfloat16), seed)
    q = device_normal_(torch.empty((len(CTXS), 16, 128), dtype=torch.bfloat16, device="cuda"), seed + 1)
    return s, bt, ctx, pool, q


def test_validate_mode_rejects_before_any_launch(validate_env):
    s, bt, ctx, pool, q = _pool_case(10)
    scale = 1.0 / math.sqrt(128.0)
    # Sentinel: a context beyond max_context_len whose positions the table
    # still maps (in bounds for any kernel).  The debug mode rejects it, which
    # shows the mode is on before any out-of-pool table is passed.
    ctx_h = s.context_lens.copy()
    ctx_h[3] = 17                                   # sequence 3 owns two blocks (pad_blocks gives room)
    bt_h = s.block_table.copy()
    bt_h[3, 1] = bt_h[1, 0]
    with pytest.raises(pk.PagedKVError) as ei:
        pk.paged_decode_attention(q, pool.k, pool.v, torch.from_numpy(bt_h).cuda(), torch.from_numpy(ctx_h).cuda(),
                                  scale, max_context_len=16)
    assert ei.value.status == pk.KVP_ERR_INVALID_ARG and "context_lens[0] = 37 outside [0, 16]" in str(ei.value)
    # a block id past the pool, through the pool registry (plain and append)
    bt_h = s.block_table.copy()
    bt_h[1, 3] = s.num_blocks + 3
    bad = torch.from_numpy(bt_h).cuda()
    rc, _ = _validate_status(bad, ctx, _desc(len(CTXS), s.max_blocks_per_seq, 50), s.num_blocks)
    assert rc == pk.KVP_ERR_INVALID_ARG
    with pytest.raises(pk.PagedKVError) as ei:
        pk.paged_decode_attention(q, pool.k, pool.v, bad, ctx, scale, max_context_len=50)
    assert f"block_table[1][3] = {s.num_blocks + 3} outside [0, {s.num_blocks})" in str(ei.value)
    kv_new = device_normal_(torch.empty((2, len(CTXS), 2, 128), dtype=torch.bfloat16, device="cuda"), 12)
    before = pool.storage.clone()
    with pytest.raises(pk.PagedKVError):
        pk.paged_decode_attention_append(pool, q, kv_new[0], kv_new[1], bad, ctx, scale, max_context_len=50)
    torch.cuda.synchronize()
    assert torch.equal(before, pool.storage)        # nothing was written
    # a negative block id inside a context, on pools that are plain tensors
    bt_h = s.block_table.copy()
    bt_h[0, 1] = -7
    neg = torch.from_numpy(bt_h).cuda()
    rc, _ = _validate_status(neg, ctx, _desc(len(CTXS), s.max_blocks_per_seq, 50), s.num_blocks)
    assert rc == pk.KVP_ERR_INVALID_ARG
    k2, v2 = pool.k.clone(), pool.v.clone()
    with pytest.raises(pk.PagedKVError) as ei:
        pk.paged_decode_attention(q, k2, v2, neg, ctx, scale, max_context_len=50)
    assert "block_table[0][1] = -7" in str(ei.value)


def test_validate_mode_passes_valid_calls_unchanged(validate_env):
    """With valid tables the debug mode returns the same bits as the fast
    path, for pools from kv_pool_create and for plain device tensors."""
    s, bt, ctx, pool, q = _pool_case(20)
    scale = 1.0 / math.sqrt(128.0)
    a = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=50)
    b = pk.paged_decode_attention(q, pool.k.clone(), pool.v.clone(), bt, ctx, scale, max_context_len=50)
    del os.environ["PAGEDKV_VALIDATE"]
    c = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=50)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(b.view(torch.int16), c.view(torch.int16))
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale)
    assert max_err(c, ref) <= TOL_BF16


def test_pool_create_reports_out_of_memory():
    """A pool the device cannot hold (2 PB): kv_pool_create with storage NULL
    returns KVP_ERR_OUT_OF_MEMORY and a message, and the device stays usable."""
    lib = pk.lib()
    pd = pk._PoolDesc(1 << 30, 256, 8, 128, 128, pk.KVP_F32, 0)
    assert lib.kv_pool_required_bytes(ctypes.byref(pd)) == 2 * (1 << 30) * 256 * 8 * 128 * 4
    h = ctypes.c_void_p()
    rc = lib.kv_pool_create(ctypes.byref(pd), None, 0, ctypes.byref(h))
    assert rc == pk.KVP_ERR_OUT_OF_MEMORY
    assert b"out of device memory" in lib.kvp_last_error()
    assert not h.value
    # a pool the library allocates itself, then frees
    pd_ok = pk._PoolDesc(64, 16, 2, 128, 128, pk.KVP_BF16, 0)
    assert lib.kv_pool_create(ctypes.byref(pd_ok), None, 0, ctypes.byref(h)) == pk.KVP_OK
    lib.kv_pool_destroy(h)
    x = torch.ones(1024, device="cuda")
    assert float(x.sum()) == 1024.0


def test_stream_read_probe():
    """The read-ceiling probe (kvp_stream_read): reads the buffer, leaves the
    sink alone (a buffer of ones never folds to the key), and refuses a
    misaligned buffer or a size that is not a multiple of 16 bytes."""
    buf = torch.ones(1 << 22, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for wg in (0, 1, 7, 4096):
        pk.stream_read(buf, sink, wg)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(pk.PagedKVError):
        pk.stream_read(buf[1:17], sink)
    with pytest.raises(pk.PagedKVError):
        pk.stream_read(buf[:24], sink)


def test_mfma_peak_probe():
    """The matrix-core probe (kvp_mfma_peak): runs, never writes the sink,
    reports the FLOPs of the call, and refuses a bad sink or iteration count."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = pk.mfma_peak(sink, 8, 16)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 16 * 8 * 16384 and float(sink.item()) == 0.0
    with pytest.raises(pk.PagedKVError):
        pk.mfma_peak(sink, 8, 0)
    with pytest.raises(pk.PagedKVError):
        pk.mfma_peak(torch.zeros(2, dtype=torch.uint8, device="cuda")[1:], 8, 16)
