"""GPU parity of chunked-prefill attention over the paged cache against the
fp64 oracle (faulkner's chunked prefill: each chunk attends causally to the
cache before it and to itself).  The chunk's K/V rows are written through
reshape_and_cache first; every slot no position up to the chunk's end owns
holds NaN.  Tolerance 2e-2 (bf16), every output row of every chunk (sampled
rows at the 70B-shaped size)."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import device_normal_
from synth.workloads import custom_structure

from parity_support import TOL_BF16, host, max_err, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _case(starts, chunks, g, n_kv, bs, seed, C=None):
    ends = [s + c for s, c in zip(starts, chunks)]
    st = custom_structure(ends, bs, seed=seed, pad_blocks=1)
    pool = pk.kv_pool_create(st.num_blocks, bs, n_kv, 128, 128, torch.bfloat16)
    device_normal_(pool.storage.view(torch.bfloat16), seed)
    owned = owned_slots(st.block_table, st.context_lens, bs)
    poison_unowned_(pool.k, owned)
    poison_unowned_(pool.v, owned)
    B = len(starts)
    C = C or max(max(chunks), 1)
    q = device_normal_(torch.empty((B, C, g * n_kv, 128), dtype=torch.bfloat16, device="cuda"), seed + 1)
    bt, _ = tables_to_device(st)
    sp = torch.tensor(starts, dtype=torch.int32, device="cuda")
    cl = torch.tensor(chunks, dtype=torch.int32, device="cuda")
    return st, pool, q, bt, sp, cl, max(ends)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("bs", [1, 16, 64])
def test_prefill_ragged_chunks(g, bs):
    starts, chunks = [0, 37, 100, 5, 640], [20, 50, 1, 0, 129]
    n_kv = 2
    st, pool, q, bt, sp, cl, mx = _case(starts, chunks, g, n_kv, bs, 10 + g + bs)
    scale = 1.0 / math.sqrt(128.0)
    out = torch.full_like(q, float("nan"))
    pk.paged_prefill_attention(q, pool.k, pool.v, bt, sp, cl, scale, out, max_context_len=mx)
    torch.cuda.synchronize()
    ref = oracle.paged_prefill_attention(host(q), host(pool.k), host(pool.v), st.block_table, starts, chunks, scale)
    for b, n in enumerate(chunks):
        if n:
            assert max_err(out[b, :n], ref[b, :n]) <= TOL_BF16, b
        assert bool(torch.isnan(out[b, n:].float()).all())        # rows past the chunk are not written


def test_prefill_in_chunks_equals_causal_prefill_of_the_prompt():
    """A 1000-token prompt taken 256 tokens per step, each step writing the
    chunk's K/V then attending, equals causal attention over the whole
    prompt (oracle), row for row."""
    n_kv, g, bs, T = 8, 8, 16, 1000
    st = custom_structure([T], bs, seed=3)
    pool = pk.kv_pool_create(st.num_blocks, bs, n_kv, 128, 128, torch.bfloat16)
    pool.storage.fill_(0xFF)
    kv = device_normal_(torch.empty((2, T, n_kv, 128), dtype=torch.bfloat16, device="cuda"), 4)
    qa = device_normal_(torch.empty((1, T, g * n_kv, 128), dtype=torch.bfloat16, device="cuda"), 5)
    bt, _ = tables_to_device(st)
    seq = torch.zeros(T, dtype=torch.int32, device="cuda")
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    slots = pk.paged_slot_mapping(bt, seq, pos, bs)
    scale = 1.0 / math.sqrt(128.0)
    got = torch.empty_like(qa)
    for p0 in range(0, T, 256):
        n = min(256, T - p0)
        pk.reshape_and_cache(pool, kv[0, p0:p0 + n].contiguous(), kv[1, p0:p0 + n].contiguous(),
                             slots[p0:p0 + n].contiguous())
        qc = torch.zeros((1, 256, g * n_kv, 128), dtype=torch.bfloat16, device="cuda")
        qc[0, :n] = qa[0, p0:p0 + n]
        o = pk.paged_prefill_attention(qc, pool.k, pool.v, bt, torch.tensor([p0], dtype=torch.int32, device="cuda"),
                                       torch.tensor([n], dtype=torch.int32, device="cuda"), scale, max_context_len=T)
        got[0, p0:p0 + n] = o[0, :n]
    torch.cuda.synchronize()
    ref = oracle.paged_prefill_attention(host(qa), host(pool.k), host(pool.v), st.block_table, [0], [T], scale)
    assert max_err(got, ref) <= TOL_BF16


@pytest.mark.parametrize("bs", [16, 1])
def test_prefill_long_context_in_table_chunks(bs):
    """A chunk at position 9000: with block 16 the table holds 563 blocks,
    with block 1 9064, so the kernel walks the context in several staged
    table chunks; sampled rows against decode attention over the same
    positions (the oracle's chunk-end identity)."""
    starts, chunks = [9000, 0], [64, 64]
    st, pool, q, bt, sp, cl, mx = _case(starts, chunks, 8, 8, bs, 21)
    scale = 1.0 / math.sqrt(128.0)
    out = pk.paged_prefill_attention(q, pool.k, pool.v, bt, sp, cl, scale, max_context_len=mx)
    torch.cuda.synchronize()
    kh, vh, qh = host(pool.k), host(pool.v), host(q)
    for b in range(2):
        for i in (0, 1, 17, 63):
            ref = oracle.paged_decode_attention(qh[b, i][None], kh, vh, st.block_table[b:b + 1],
                                                [starts[b] + i + 1], scale)
            assert max_err(out[b, i:i + 1], ref) <= TOL_BF16, (b, i)


def test_prefill_70b_shaped_chunks_sampled():
    """The chunked-prefill workload: four 512-token chunks of 70B-shaped
    heads (n_h 64, n_kv 8) at positions 0, 1024, 4096 and 7680; fifteen rows
    of every chunk (every 37th, which crosses each 64-token stage at a
    different offset, and the last) against decode attention over the same
    positions."""
    starts, chunks = [0, 1024, 4096, 7680], [512] * 4
    st, pool, q, bt, sp, cl, mx = _case(starts, chunks, 8, 8, 16, 31)
    scale = 1.0 / math.sqrt(128.0)
    out = pk.paged_prefill_attention(q, pool.k, pool.v, bt, sp, cl, scale, max_context_len=mx)
    torch.cuda.synchronize()
    kh, vh, qh = host(pool.k), host(pool.v), host(q)
    for b in range(4):
        for i in list(range(0, 512, 37)) + [511]:
            ref = oracle.paged_decode_attention(qh[b, i][None], kh, vh, st.block_table[b:b + 1],
                                                [starts[b] + i + 1], scale)
            assert max_err(out[b, i:i + 1], ref) <= TOL_BF16, (b, i)


def test_prefill_skips_sequences_outside_the_contract():
    """A chunk longer than the q rows, a negative start and a chunk running
    past its block table are skipped (their rows keep the fill); the other
    sequences are still computed against the oracle."""
    starts, chunks = [0, 40, 0, 30], [20, 30, 10, 16]
    st, pool, q, bt, sp, cl, mx = _case(starts, chunks, 8, 2, 16, 44, C=32)
    scale = 1.0 / math.sqrt(128)
    bad_cl = cl.clone()
    bad_cl[1] = 33                                  # longer than the 32 q rows
    bad_sp = sp.clone()
    bad_sp[2] = -5                                  # negative start
    bad_sp[3] = st.max_blocks_per_seq * 16 - 8      # 16 tokens from 8 before the table's end
    out = torch.full_like(q, float("nan"))
    pk.paged_prefill_attention(q, pool.k, pool.v, bt, bad_sp, bad_cl, scale, out, max_context_len=mx)
    torch.cuda.synchronize()
    ref = oracle.paged_prefill_attention(host(q), host(pool.k), host(pool.v), st.block_table, starts, chunks, scale)
    assert max_err(out[0, :20], ref[0, :20]) <= TOL_BF16
    for b in (1, 2, 3):
        assert bool(torch.isnan(out[b].float()).all()), b
