"""GPU: paged_decode_attention_append (one decode step in one call: each
sequence's new K/V row is written at position context_lens[b] - 1, then the
attention runs) against the same step done in separate calls:
paged_slot_mapping + reshape_and_cache + the decode call of the pool's kind.

The output and the pool afterwards must match bit for bit: the appended
rows are the same copies (or the same quantization), and the attention is
the same kernel over the same bytes.  The cases cover the fused path (bf16,
g in {4, 8}: the attention kernel writes the rows itself), block sizes 1, 16
and 64, forced context splits (the last split is one of several), contexts
of 0 and 1 tokens and at block and stage boundaries, and the other kernels
(bf16 g = 2, fp32, INT8, MLA), where the cache kernel writes the rows first.
One case is also checked against the fp64 oracle, so that the appended row
is seen to enter the attention.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import device_normal_
from synth.workloads import custom_structure, prefill_tokens

from parity_support import TOL_BF16, host, max_err, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")

TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def _bits(t: torch.Tensor) -> torch.Tensor:
    """The tensor's bytes as integers (NaN-safe bit equality)."""
    return t.contiguous().view(torch.uint8)


def _history(pool, s, rows_dtype, n_kv, d_k, d_v, latent, seed):
    """Every position but the last of each sequence, written through
    reshape_and_cache (the cache before the decode step)."""
    hist = np.maximum(s.context_lens - 1, 0)
    seq, pos = prefill_tokens(hist)
    if len(seq) == 0:
        return
    bt, _ = tables_to_device(s)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                                  pool.block_size)
    k = device_normal_(torch.empty((len(seq), n_kv, d_k), dtype=rows_dtype, device="cuda"), seed)
    v = None if latent else device_normal_(torch.empty((len(seq), n_kv, d_v), dtype=rows_dtype,
                                                       device="cuda"), seed + 1)
    pk.reshape_and_cache(pool, k, v, slots)


def _two_pools(kind, s, bs, n_kv, d_k, d_v, latent, seed):
    pool_dtype = torch.int8 if kind == "int8" else TORCH[kind]
    rows_dtype = torch.bfloat16 if kind == "int8" else TORCH[kind]
    a = pk.kv_pool_create(s.num_blocks, bs, n_kv, d_k, d_v, pool_dtype, latent=latent)
    a.storage.zero_()
    _history(a, s, rows_dtype, n_kv, d_k, d_v, latent, seed)
    b = pk.kv_pool_create(s.num_blocks, bs, n_kv, d_k, d_v, pool_dtype, latent=latent)
    b.storage.copy_(a.storage)
    return a, b, rows_dtype


def _separate_calls(pool, kind, q, k_new, v_new, bt, ctx, s, scale, split, latent, d_v):
    """The decode step as separate calls: slots of position ctx - 1 (none
    for an empty sequence), reshape_and_cache, then the decode."""
    B = len(s.context_lens)
    seq = torch.arange(B, dtype=torch.int32, device="cuda")
    pos = (ctx - 1).to(torch.int32)
    slots = pk.paged_slot_mapping(bt, seq, pos, pool.block_size)
    pk.reshape_and_cache(pool, k_new, v_new, slots)
    mc = int(s.context_lens.max(initial=0))
    if latent:
        return pk.paged_decode_attention_mla(q, pool.k, bt, ctx, scale, d_v, max_context_len=mc)
    if kind == "int8":
        return pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx,
                                              scale, max_context_len=mc, split_tokens=split)
    return pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=mc,
                                     split_tokens=split)


CASES = [
    # name, kind, n_h, n_kv, d, block, contexts, split_tokens (0 = automatic)
    ("bf16_g8_d128", "bf16", 16, 2, 128, 16, [1, 17, 64, 65, 300, 0, 2049], 0),
    ("bf16_g8_split256", "bf16", 16, 2, 128, 16, [1, 700, 1024, 1025, 3000], 256),
    ("bf16_g4_d64", "bf16", 8, 2, 64, 16, [5, 129, 64, 1000], 0),
    ("bf16_g8_block1", "bf16", 8, 1, 128, 1, [1, 3, 70], 0),
    ("bf16_g8_block64", "bf16", 8, 1, 128, 64, [1, 63, 64, 65, 200], 256),
    ("bf16_g2_generic", "bf16", 4, 2, 128, 16, [1, 40, 300], 0),
    ("f32_g1_generic", "f32", 4, 4, 64, 16, [1, 40, 300, 0], 0),
    ("int8_g8", "int8", 16, 2, 128, 16, [1, 40, 300, 0], 0),
    ("bf16_g16_d128", "bf16", 32, 2, 128, 16, [1, 17, 64, 65, 300, 0, 2049], 0),
    ("int8_g16", "int8", 32, 2, 128, 16, [1, 40, 300, 0], 0),
]


@pytest.mark.parametrize("name,kind,n_h,n_kv,d,bs,ctxs,split", CASES, ids=[c[0] for c in CASES])
def test_append_equals_separate_calls(name, kind, n_h, n_kv, d, bs, ctxs, split):
    s = custom_structure(ctxs, bs, seed=len(ctxs) + bs, pad_blocks=1)
    seed = 31 + n_h + bs
    pa, pb, rows_dtype = _two_pools(kind, s, bs, n_kv, d, d, False, seed)
    B = len(ctxs)
    q = device_normal_(torch.empty((B, n_h, d), dtype=rows_dtype, device="cuda"), seed + 2)
    k_new = device_normal_(torch.empty((B, n_kv, d), dtype=rows_dtype, device="cuda"), seed + 3)
    v_new = device_normal_(torch.empty((B, n_kv, d), dtype=rows_dtype, device="cuda"), seed + 4)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(d)
    out_a = _separate_calls(pa, kind, q, k_new, v_new, bt, ctx, s, scale, split, False, d)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, v_new, bt, ctx, scale,
                                             max_context_len=int(max(ctxs)), split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)


def test_append_mla_equals_separate_calls():
    ctxs = [1, 33, 300, 64]
    s = custom_structure(ctxs, 64, seed=3, pad_blocks=1)
    pa, pb, rows_dtype = _two_pools("bf16", s, 64, 1, 576, 512, True, 41)
    q = device_normal_(torch.empty((len(ctxs), 16, 576), dtype=torch.bfloat16, device="cuda"), 42)
    k_new = device_normal_(torch.empty((len(ctxs), 1, 576), dtype=torch.bfloat16, device="cuda"), 43)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(192.0)
    out_a = _separate_calls(pa, "bf16", q, k_new, None, bt, ctx, s, scale, 0, True, 512)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, None, bt, ctx, scale,
                                             max_context_len=max(ctxs))
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)


def test_append_row_enters_the_attention():
    """Against the oracle on the pool after the call: the new row sits at
    position ctx - 1 and the output attends over it (a one-token sequence's
    output is exactly its new V row)."""
    ctxs = [1, 100, 513]
    s = custom_structure(ctxs, 16, seed=9, pad_blocks=1)
    pa, pb, _ = _two_pools("bf16", s, 16, 2, 128, 128, False, 51)
    q = device_normal_(torch.empty((3, 16, 128), dtype=torch.bfloat16, device="cuda"), 52)
    k_new = device_normal_(torch.empty((3, 2, 128), dtype=torch.bfloat16, device="cuda"), 53)
    v_new = device_normal_(torch.empty((3, 2, 128), dtype=torch.bfloat16, device="cuda"), 54)
    bt, ctx = tables_to_device(s)
    out = pk.paged_decode_attention_append(pb, q, k_new, v_new, bt, ctx, 0.0884,
                                           max_context_len=513)
    torch.cuda.synchronize()
    kh, vh = host(pb.k), host(pb.v)
    for b, c in enumerate(ctxs):
        blk, off = s.block_table[b, (c - 1) // 16], (c - 1) % 16
        assert np.array_equal(kh[blk, off], host(k_new)[b]) and np.array_equal(vh[blk, off], host(v_new)[b])
    ref = oracle.paged_decode_attention(host(q), kh, vh, s.block_table, s.context_lens, 0.0884)
    assert max_err(out, ref) <= TOL_BF16
    o = host(out)
    assert np.array_equal(o[0].reshape(2, 8, 128), np.broadcast_to(host(v_new)[0][:, None, :], (2, 8, 128)))


def test_append_on_the_stream_grid():
    """Ragged batch with a total-context hint (the stream grid): the
    workgroup holding a sequence's last token writes the new rows, even when
    the sequence is cut across workgroups.  Bit for bit against the same
    step in separate calls with the same hint."""
    ctxs = [1, 700, 4000, 0, 65, 2500, 33]
    s = custom_structure(ctxs, 16, seed=12, pad_blocks=1)
    pa, pb, _ = _two_pools("bf16", s, 16, 2, 128, 128, False, 61)
    B = len(ctxs)
    q = device_normal_(torch.empty((B, 16, 128), dtype=torch.bfloat16, device="cuda"), 62)
    k_new = device_normal_(torch.empty((B, 2, 128), dtype=torch.bfloat16, device="cuda"), 63)
    v_new = device_normal_(torch.empty((B, 2, 128), dtype=torch.bfloat16, device="cuda"), 64)
    bt, ctx = tables_to_device(s)
    hint = int(sum(ctxs))
    seq = torch.arange(B, dtype=torch.int32, device="cuda")
    slots = pk.paged_slot_mapping(bt, seq, (ctx - 1).to(torch.int32), 16)
    pk.reshape_and_cache(pa, k_new, v_new, slots)
    out_a = pk.paged_decode_attention(q, pa.k, pa.v, bt, ctx, 0.0884, max_context_len=4000,
                                      total_context_len=hint)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, v_new, bt, ctx, 0.0884, max_context_len=4000,
                                             total_context_len=hint)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)
    ref = oracle.paged_decode_attention(host(q), host(pb.k), host(pb.v), s.block_table, s.context_lens, 0.0884)
    assert max_err(out_b, ref) <= TOL_BF16


@pytest.mark.parametrize("ctxs,split", [([1, 17, 32, 33, 64, 65, 300, 2049], 0), ([31, 33, 700, 1024, 1025, 3000], 256)])
def test_append_slot_poisoned_before_the_call(ctxs, split):
    """The fused bf16 append with every appended slot holding NaN before the
    call: the attention must see the new rows, whether the sequence's last
    token falls in the first stage its workgroup reads (the store completes
    before that stage's DMA) or in a later one (the stage loop's own waits
    order the store before that DMA).  Equal bit for bit to the separate
    calls on an identically poisoned pool, and finite."""
    s = custom_structure(ctxs, 16, seed=71 + split, pad_blocks=1)
    pa, pb, _ = _two_pools("bf16", s, 16, 2, 128, 128, False, 72)
    for pool in (pa, pb):
        for b, c in enumerate(ctxs):
            blk, off = int(s.block_table[b, (c - 1) // 16]), (c - 1) % 16
            pool.k[blk, off] = float("nan")
            pool.v[blk, off] = float("nan")
    B = len(ctxs)
    q = device_normal_(torch.empty((B, 16, 128), dtype=torch.bfloat16, device="cuda"), 73)
    k_new = device_normal_(torch.empty((B, 2, 128), dtype=torch.bfloat16, device="cuda"), 74)
    v_new = device_normal_(torch.empty((B, 2, 128), dtype=torch.bfloat16, device="cuda"), 75)
    bt, ctx = tables_to_device(s)
    out_a = _separate_calls(pa, "bf16", q, k_new, v_new, bt, ctx, s, 0.0884, split, False, 128)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, v_new, bt, ctx, 0.0884,
                                             max_context_len=max(ctxs), split_tokens=split)
    torch.cuda.synchronize()
    assert torch.isfinite(out_b.float()).all()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)


@pytest.mark.parametrize("n_kv,d,hint", [(4, 128, True), (3, 128, False), (2, 64, True), (4, 128, False)])
def test_append_int8_fused_with_poisoned_scales(n_kv, d, hint):
    """INT8 pools, where the attention kernel quantizes and writes the new
    rows itself (two KV heads per workgroup at n_kv = 4, one at n_kv = 3 or
    d = 64; the compact grid with a total-context hint, the split grid
    without), with the scales of every appended slot NaN before the call:
    the output equals the separate calls bit for bit and is finite, and the
    pool (codes and scales) equals theirs."""
    ctxs = [1, 31, 33, 300, 2049, 64, 5000]
    g = 8
    s = custom_structure(ctxs, 16, seed=81 + n_kv + d, pad_blocks=1)
    pa, pb, _ = _two_pools("int8", s, 16, n_kv, d, d, False, 82)
    for pool in (pa, pb):
        for b, c in enumerate(ctxs):
            blk, off = int(s.block_table[b, (c - 1) // 16]), (c - 1) % 16
            pool.k_scale[blk, :, off] = float("nan")
            pool.v_scale[blk, :, off] = float("nan")
    B = len(ctxs)
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), 83)
    k_new = device_normal_(torch.empty((B, n_kv, d), dtype=torch.bfloat16, device="cuda"), 84)
    v_new = device_normal_(torch.empty((B, n_kv, d), dtype=torch.bfloat16, device="cuda"), 85)
    bt, ctx = tables_to_device(s)
    kw = {"total_context_len": int(sum(ctxs))} if hint else {}
    seq = torch.arange(B, dtype=torch.int32, device="cuda")
    slots = pk.paged_slot_mapping(bt, seq, (ctx - 1).to(torch.int32), 16)
    pk.reshape_and_cache(pa, k_new, v_new, slots)
    out_a = pk.paged_decode_attention_int8(q, pa.k, pa.k_scale, pa.v, pa.v_scale, bt, ctx, 0.0884,
                                           max_context_len=max(ctxs), **kw)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, v_new, bt, ctx, 0.0884, max_context_len=max(ctxs), **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(out_b.float()).all()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)


@pytest.mark.parametrize("n_h,workgroups", [(128, 0), (160, 3), (16, 1), (128, 7)])
def test_append_mla_fused_with_poisoned_slots(n_h, workgroups):
    """Latent pools, where the MLA kernel writes the new rows itself (the
    workgroup holding a sequence's last tile; two head groups at n_h = 160
    both write the same row), with every appended slot NaN before the call:
    bit for bit the separate calls on an identically poisoned pool, finite."""
    ctxs = [1, 33, 300, 64, 0, 2049, 95]
    s = custom_structure(ctxs, 64, seed=91 + n_h + workgroups, pad_blocks=1)
    pa, pb, _ = _two_pools("bf16", s, 64, 1, 576, 512, True, 92)
    for pool in (pa, pb):
        for b, c in enumerate(ctxs):
            if c > 0:
                pool.k[int(s.block_table[b, (c - 1) // 64]), (c - 1) % 64] = float("nan")
    B = len(ctxs)
    q = device_normal_(torch.empty((B, n_h, 576), dtype=torch.bfloat16, device="cuda"), 93)
    k_new = device_normal_(torch.empty((B, 1, 576), dtype=torch.bfloat16, device="cuda"), 94)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(192.0)
    seq = torch.arange(B, dtype=torch.int32, device="cuda")
    slots = pk.paged_slot_mapping(bt, seq, (ctx - 1).to(torch.int32), 64)
    pk.reshape_and_cache(pa, k_new, None, slots)
    out_a = pk.paged_decode_attention_mla(q, pa.k, bt, ctx, scale, 512, max_context_len=max(ctxs),
                                          workgroups=workgroups)
    out_b = pk.paged_decode_attention_append(pb, q, k_new, None, bt, ctx, scale, max_context_len=max(ctxs),
                                             workgroups=workgroups)
    torch.cuda.synchronize()
    assert torch.isfinite(out_b.float()).all()
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(pa.storage, pb.storage)
