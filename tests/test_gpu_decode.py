"""GPU parity of paged decode attention (float pools) against the fp64 oracle.

Every case runs the HIP path through the C ABI on seeded inputs and compares
every output element (or, at the 70B shape, every output of sampled
sequences) with the oracle: max |gpu - oracle| <= 1e-5 for fp32 inputs and
<= 2e-2 for bf16 inputs.  Unused pool slots hold NaN, so any read past a
context length shows up as NaN in the output.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import custom_structure, prefill_tokens, decode_positions

from parity_support import (TOL_BF16, TOL_F32, device_from_host, host, host_normal, max_err,
                            owned_slots, poison_unowned_, tables_to_device)

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _prefilled_case(cfg, s, seed, kind):
    """Pools written token by token through reshape_and_cache from contiguous
    logical-order K/V (the tiny workloads' recipe)."""
    rng = np.random.default_rng(seed)
    dtype = torch.float32 if kind == "f32" else torch.bfloat16
    pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, dtype)
    pool.storage.fill_(0xFF)
    seq, pos = prefill_tokens(s.context_lens)
    k_new = host_normal(rng, (len(seq), cfg.n_kv, cfg.d_k), kind)
    v_new = host_normal(rng, (len(seq), cfg.n_kv, cfg.d_v), kind)
    q = host_normal(rng, (len(s.context_lens), cfg.n_h, cfg.d_k), kind)
    bt, ctx = tables_to_device(s)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                                  cfg.block_size)
    pk.reshape_and_cache(pool, device_from_host(k_new), device_from_host(v_new), slots)
    return pool, bt, ctx, device_from_host(q), (k_new, v_new, q, seq)


def _run(pool, q, bt, ctx, s, scale, **kw):
    return pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale,
                                     max_context_len=int(s.context_lens.max(initial=0)), **kw)


@pytest.mark.parametrize("name", ["tiny", "tiny_mha"])
def test_tiny_fp32_against_oracle_and_contiguous(name):
    cfg = CONFIGS[name]
    s = structure(cfg)
    pool, bt, ctx, q, (k_new, v_new, qh, seq) = _prefilled_case(cfg, s, cfg.seed, "f32")
    out = _run(pool, q, bt, ctx, s, cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(qh, host(pool.k), host(pool.v), s.block_table,
                                        s.context_lens, cfg.scale)
    assert max_err(out, ref) <= TOL_F32
    # the same against contiguous (unpaged) attention on the logical rows
    t = 0
    for b, c in enumerate(s.context_lens):
        cref = oracle.decode_attention_contiguous(qh[b], k_new[t:t + c], v_new[t:t + c], cfg.scale)
        assert np.max(np.abs(host(out)[b].astype(np.float64) - cref)) <= TOL_F32
        t += c


@pytest.mark.parametrize("kind,d,g", [("f32", 64, 2), ("f32", 32, 4), ("bf16", 128, 8),
                                      ("bf16", 64, 1), ("bf16", 128, 2), ("bf16", 64, 4),
                                      ("bf16", 128, 16), ("bf16", 64, 16)])
@pytest.mark.parametrize("bs", [1, 16, 64])
def test_ragged_contexts(kind, d, g, bs):
    ctxs = [1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700]
    n_kv = 2
    n_h = n_kv * g
    cfg = type("C", (), dict(block_size=bs, n_kv=n_kv, d_k=d, d_v=d, n_h=n_h))
    s = custom_structure(ctxs, bs, seed=bs * 7 + d, pad_blocks=2)
    pool, bt, ctx, q, (_, _, qh, _) = _prefilled_case(cfg, s, 17 + g, kind)
    scale = 1.0 / math.sqrt(d)
    out = _run(pool, q, bt, ctx, s, scale)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(qh, host(pool.k), host(pool.v), s.block_table,
                                        s.context_lens, scale)
    tol = TOL_F32 if kind == "f32" else TOL_BF16
    assert max_err(out, ref) <= tol


@pytest.mark.parametrize("n_kv,g", [(1, 8), (2, 8), (3, 8), (4, 4), (6, 4), (8, 8), (1, 16), (3, 16), (4, 16)])
def test_kv_head_groups_bf16(n_kv, g):
    """bf16 with d = 128 runs two adjacent KV heads per workgroup when n_kv
    is even and one otherwise; both against the oracle on the plain grid,
    with several context splits and on the stream grid."""
    ctxs = [1, 17, 40, 300, 1025, 0, 64]
    d, bs = 128, 16
    cfg = type("C", (), dict(block_size=bs, n_kv=n_kv, d_k=d, d_v=d, n_h=n_kv * g))
    s = custom_structure(ctxs, bs, seed=n_kv * 10 + g, pad_blocks=1)
    pool, bt, ctx, q, (_, _, qh, _) = _prefilled_case(cfg, s, 300 + n_kv + g, "bf16")
    scale = 1.0 / math.sqrt(d)
    ref = oracle.paged_decode_attention(qh, host(pool.k), host(pool.v), s.block_table, s.context_lens, scale)
    for kw in (dict(), dict(split_tokens=256), dict(total_context_len=int(s.context_lens.sum()))):
        out = _run(pool, q, bt, ctx, s, scale, **kw)
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL_BF16, kw


def test_single_token_context_returns_v_exactly_and_empty_context_gives_zero():
    cfg = CONFIGS["tiny"]
    s = custom_structure([1, 0, 1], 16, seed=2)
    pool, bt, ctx, q, (k_new, v_new, qh, seq) = _prefilled_case(
        type("C", (), dict(block_size=16, n_kv=2, d_k=64, d_v=64, n_h=4)), s, 3, "f32")
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, cfg.scale, max_context_len=1)
    torch.cuda.synchronize()
    o = host(out)
    assert np.array_equal(o[0, 0], v_new[0, 0]) and np.array_equal(o[0, 3], v_new[0, 1])
    assert np.array_equal(o[2, 1], v_new[1, 0])
    assert np.all(o[1] == 0)


def test_block_size_and_permutation_invariance():
    """The same logical K/V through block size 1 and 16 and through two
    different physical permutations give the oracle's answer."""
    rng = np.random.default_rng(21)
    ctxs = [300, 77, 513]
    n_kv, g, d = 2, 4, 128
    K = [host_normal(rng, (c, n_kv, d), "bf16") for c in ctxs]
    V = [host_normal(rng, (c, n_kv, d), "bf16") for c in ctxs]
    qh = host_normal(rng, (3, n_kv * g, d), "bf16")
    ref = np.stack([oracle.decode_attention_contiguous(qh[b], K[b], V[b], 0.088) for b in range(3)])
    outs = []
    for bs, seed in [(1, 1), (16, 2), (16, 3)]:
        s = custom_structure(ctxs, bs, seed=seed, pad_blocks=1)
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
        pool.storage.fill_(0xFF)
        seq, pos = prefill_tokens(s.context_lens)
        bt, ctx = tables_to_device(s)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        pk.reshape_and_cache(pool, device_from_host(np.concatenate(K)), device_from_host(np.concatenate(V)), slots)
        out = pk.paged_decode_attention(device_from_host(qh), pool.k, pool.v, bt, ctx, 0.088,
                                        max_context_len=513)
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL_BF16
        outs.append(host(out))
    # identical inputs in a different physical arrangement: same bits
    assert np.array_equal(outs[1], outs[2])


def _big_case(cfg, s, seed, poison=True):
    """Pools filled directly with N(0,1) draws on the device (every slot is a
    fresh token), unowned slots NaN, plus the decode step's new K/V written
    at position ctx-1 through the slot mapping."""
    dtype = torch.bfloat16
    k = torch.empty((s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k), dtype=dtype, device="cuda")
    v = torch.empty((s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_v), dtype=dtype, device="cuda")
    device_normal_(k, seed)
    device_normal_(v, seed + 1)
    if poison:
        owned = owned_slots(s.block_table, s.context_lens, cfg.block_size)
        poison_unowned_(k, owned)
        poison_unowned_(v, owned)
    q = device_normal_(torch.empty((cfg.B, cfg.n_h, cfg.d_k), dtype=dtype, device="cuda"), seed + 2)
    return k, v, q


@pytest.mark.parametrize("split", [0, 256, 2048])
def test_llama8b_shared_prefix_full_size(split):
    cfg = CONFIGS["llama8b"]
    s = structure(cfg)
    k, v, q = _big_case(cfg, s, cfg.seed)
    bt, ctx = tables_to_device(s)
    # decode step: new K/V of the last position, written where the position
    # is private to its sequence (a write into the shared prefix would be a
    # copy-on-write case, which this path leaves to the allocator).
    seq, pos = decode_positions(s.context_lens)
    private = (pos // cfg.block_size) >= s.shared_blocks
    pos_w = np.where(private, pos, -1).astype(np.int32)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos_w).cuda(),
                                  cfg.block_size)
    pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16)
    pool.k.copy_(k)
    pool.v.copy_(v)
    rng = np.random.default_rng(cfg.seed)
    k_new = host_normal(rng, (cfg.B, cfg.n_kv, cfg.d_k), "bf16")
    v_new = host_normal(rng, (cfg.B, cfg.n_kv, cfg.d_v), "bf16")
    k0, v0 = host(pool.k), host(pool.v)
    pk.reshape_and_cache(pool, device_from_host(k_new), device_from_host(v_new), slots)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, cfg.scale,
                                    max_context_len=s.max_context_len, split_tokens=split,
                                    total_context_len=int(s.context_lens.sum()))
    torch.cuda.synchronize()
    ref_slots = np.array([oracle.slot_of(s.block_table[b], int(pos[b]), cfg.block_size) if private[b] else -1
                          for b in range(cfg.B)], dtype=np.int64)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    k1 = oracle.reshape_and_cache(k0, k_new, ref_slots)
    v1 = oracle.reshape_and_cache(v0, v_new, ref_slots)
    assert np.array_equal(host(pool.k), k1) and np.array_equal(host(pool.v), v1)
    ref = oracle.paged_decode_attention(host(q), k1, v1, s.block_table, s.context_lens, cfg.scale)
    assert max_err(out, ref) <= TOL_BF16


def test_llama70b_layers_full_shape_append_every_sequence():
    """The 70B-shaped layer at full size (B=16, ctx 8192, 8192 permuted
    blocks) through paged_decode_attention_append in the launch
    configuration the bench times (automatic split; the attention kernel
    writes the new K/V rows at position 8191 itself); two layers, every
    output element of all 16 sequences against the oracle over the pool as
    the call left it, and the pool bit-exact against the oracle's write."""
    cfg = CONFIGS["llama70b"]
    for layer in (0, 79):
        s = structure(cfg, layer=layer)
        k, v, q = _big_case(cfg, s, cfg.seed * 100 + layer, poison=False)
        bt, ctx = tables_to_device(s)
        pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16)
        pool.k.copy_(k)
        pool.v.copy_(v)
        del k, v
        kv_new = device_normal_(torch.empty((2, cfg.B, cfg.n_kv, cfg.d_k), dtype=torch.bfloat16,
                                            device="cuda"), cfg.seed * 100 + layer + 7)
        k0, v0 = host(pool.k), host(pool.v)
        out = pk.paged_decode_attention_append(pool, q, kv_new[0], kv_new[1], bt, ctx, cfg.scale,
                                               max_context_len=8192)
        torch.cuda.synchronize()
        seq, pos = decode_positions(s.context_lens)
        slots = oracle.slot_mapping(s.block_table, seq, pos, cfg.block_size)
        k1 = oracle.reshape_and_cache(k0, host(kv_new[0]), slots)
        v1 = oracle.reshape_and_cache(v0, host(kv_new[1]), slots)
        del k0, v0
        kh, vh = host(pool.k), host(pool.v)
        assert np.array_equal(kh, k1) and np.array_equal(vh, v1), layer
        del k1, v1
        ref = oracle.paged_decode_attention(host(q), kh, vh, s.block_table, s.context_lens, cfg.scale)
        assert ref.shape == (cfg.B, cfg.n_h, cfg.d_v)
        assert max_err(out, ref) <= TOL_BF16, layer
        del pool, kh, vh


def test_g16_on_the_70b_shaped_pool_full_shape_append():
    """128 query heads on the 70B-shaped layer's 8 KV heads (g = 16; B = 16,
    ctx 8192, 8192 permuted blocks) through paged_decode_attention_append
    with the automatic split, as the 70B-shaped layer runs: every output
    element against the oracle over the pool as the call left it, and the
    appended rows bit-exact."""
    cfg = dataclasses.replace(CONFIGS["llama70b"], n_h=128)
    s = structure(cfg, layer=3)
    k, v, q = _big_case(cfg, s, cfg.seed * 100 + 3, poison=False)
    bt, ctx = tables_to_device(s)
    pool = pk.kv_pool_create(s.num_blocks, cfg.block_size, cfg.n_kv, cfg.d_k, cfg.d_v, torch.bfloat16)
    pool.k.copy_(k)
    pool.v.copy_(v)
    del k, v
    kv_new = device_normal_(torch.empty((2, cfg.B, cfg.n_kv, cfg.d_k), dtype=torch.bfloat16, device="cuda"),
                            cfg.seed * 100 + 10)
    k0, v0 = host(pool.k), host(pool.v)
    out = pk.paged_decode_attention_append(pool, q, kv_new[0], kv_new[1], bt, ctx, cfg.scale, max_context_len=8192)
    torch.cuda.synchronize()
    seq, pos = decode_positions(s.context_lens)
    slots = oracle.slot_mapping(s.block_table, seq, pos, cfg.block_size)
    k1 = oracle.reshape_and_cache(k0, host(kv_new[0]), slots)
    v1 = oracle.reshape_and_cache(v0, host(kv_new[1]), slots)
    del k0, v0
    kh, vh = host(pool.k), host(pool.v)
    assert np.array_equal(kh, k1) and np.array_equal(vh, v1)
    del k1, v1
    ref = oracle.paged_decode_attention(host(q), kh, vh, s.block_table, s.context_lens, cfg.scale)
    assert ref.shape == (cfg.B, 128, cfg.d_v)
    assert max_err(out, ref) <= TOL_BF16


def test_split_count_invariance():
    cfg = CONFIGS["llama8b"]
    s = structure(cfg)
    k, v, q = _big_case(cfg, s, 77)
    bt, ctx = tables_to_device(s)
    outs = [pk.paged_decode_attention(q, k, v, bt, ctx, cfg.scale, max_context_len=s.max_context_len,
                                      split_tokens=sp).float()
            for sp in (256, 512, 1024, 2048)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) <= TOL_BF16
    # repeated runs are bit-stable
    again = pk.paged_decode_attention(q, k, v, bt, ctx, cfg.scale, max_context_len=s.max_context_len,
                                      split_tokens=256).float()
    assert torch.equal(again, outs[0])



def test_one_workspace_serves_calls_of_different_shapes():
    """One workspace, sized for the largest call, serves calls of different
    split sizes and batch shapes in a row; every result matches the oracle."""
    cfg = CONFIGS["llama8b"]
    s = structure(cfg)
    k, v, q = _big_case(cfg, s, 91)
    bt, ctx = tables_to_device(s)
    ref = oracle.paged_decode_attention(host(q), host(k), host(v), s.block_table, s.context_lens,
                                        cfg.scale)
    big = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=cfg.n_kv, d_k=128, d_v=128, block_size=16,
                       max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=s.max_context_len,
                       q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, split_tokens=256)
    ws = pk.alloc_workspace(big)
    for split, rows in [(256, slice(None)), (1024, slice(None)), (512, slice(3, 11)),
                        (256, slice(0, 5)), (2048, slice(None))]:
        qq, bb, cc = q[rows].contiguous(), bt[rows].contiguous(), ctx[rows].contiguous()
        out = pk.paged_decode_attention(qq, k, v, bb, cc, cfg.scale, max_context_len=s.max_context_len,
                                        split_tokens=split, workspace=ws)
        torch.cuda.synchronize()
        assert max_err(out, ref[rows]) <= TOL_BF16, split


@pytest.mark.parametrize("kind", ["bf16", "int8"])
@pytest.mark.parametrize("g,d,bs", [(8, 128, 16), (4, 64, 16), (8, 128, 1), (4, 128, 64), (16, 128, 16),
                                    (16, 64, 16)])
def test_ragged_grids_with_total_hint(kind, g, d, bs):
    """Ragged batch with a total-context hint and no split forced.  bf16: the
    LDS-ring kernel's stream grid (the batch's tokens cut into equal ranges,
    one per workgroup; a sequence cut across workgroups is merged from its
    pieces), against the oracle with the true total, with a hint of 1 (one
    workgroup per KV-head group takes the whole batch, so the long sequences
    run in several block-table chunks) and with a hint 50 times too large
    (which makes the batch look uniform: the plain split grid).  INT8: the compact grid
    (only the splits that exist), whose grid size the hint sets (a hint of 1
    leaves each workgroup looping over many splits).  Empty sequences are
    zeroed."""
    ctxs = [50, 3000, 0, 700, 9000, 64, 1, 2049, 128, 4500, 0]
    n_kv = 2
    s = custom_structure(ctxs, bs, seed=g + d + bs, pad_blocks=1)
    bt, ctx = tables_to_device(s)
    B = len(ctxs)
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), 90 + g)
    total = int(sum(ctxs))
    scale = 1.0 / math.sqrt(d)
    if kind == "bf16":
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
        device_normal_(pool.storage.view(torch.bfloat16), 91 + g)
        call = lambda hint: pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=9000,
                                                      total_context_len=hint)
        ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table,
                                            s.context_lens, scale)
    else:
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
        seq, pos = prefill_tokens(s.context_lens)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        rows = device_normal_(torch.empty((2, len(seq), n_kv, d), dtype=torch.bfloat16, device="cuda"), 92)
        pk.reshape_and_cache(pool, rows[0], rows[1], slots)
        call = lambda hint: pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt,
                                                           ctx, scale, max_context_len=9000,
                                                           total_context_len=hint)
        ref = oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                                 host(pool.v_scale), s.block_table, s.context_lens, scale)
    for hint in (total, 1, 50 * total):
        out = call(hint)
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL_BF16, hint
        assert torch.count_nonzero(out[2]) == 0 and torch.count_nonzero(out[10]) == 0


@pytest.mark.parametrize("kind", ["bf16", "int8"])
@pytest.mark.parametrize("factor", [1.3, 10.0])
def test_ragged_grids_with_an_oversized_hint(kind, factor):
    """A hint too large but still ragged (max_context_len well above every
    context): more workgroups are launched than the real tokens fill.
    bf16: the stream grid (asserted through its workspace size), whose
    trailing workgroups get empty ranges; INT8: the compact grid (asserted
    through its split size), whose extra workgroups find no unit.  Against
    the oracle; empty sequences are zeroed."""
    ctxs = [5, 90, 0, 33, 200, 16, 1, 47, 0, 128, 64]
    n_kv, g, d, bs = 2, 8, 128, 16
    max_ctx = 2048
    s = custom_structure(ctxs, bs, seed=31, pad_blocks=max_ctx // bs)
    bt, ctx = tables_to_device(s)
    B = len(ctxs)
    total = int(sum(ctxs))
    hint = int(factor * total)
    assert 4 * hint < 3 * B * max_ctx                      # still ragged by the hint
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), 32)
    scale = 1.0 / math.sqrt(d)
    desc = pk.make_desc(B=B, n_h=g * n_kv, n_kv=n_kv, d_k=d, d_v=d, block_size=bs,
                        max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=max_ctx,
                        q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16 if kind == "bf16" else pk.KVP_INT8,
                        total_context_len=hint)
    if kind == "bf16":
        w = min(2 * 256 // (n_kv // 2), -(-hint // 256))      # stream workgroups per KV-head pair
        r = lambda n: -(-n // 256) * 256
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert pk.decode_workspace_size(desc) == (r((w + B) * g * n_kv * d * 4) + r((w + B) * g * n_kv * 8)
                                                      + r(B * 8))
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
        device_normal_(pool.storage.view(torch.bfloat16), 33)
        out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=max_ctx,
                                        total_context_len=hint)
        ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table,
                                            s.context_lens, scale)
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        avail = 2 * cus - ((B + 1) // 2) * (n_kv // 2)
        split = -(-(hint * (n_kv // 2)) // avail)
        split = max(256, -(-split // 256) * 256)
        assert pk.decode_split_tokens(desc) == split           # the compact grid's rule
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
        seq, pos = prefill_tokens(s.context_lens)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        rows = device_normal_(torch.empty((2, len(seq), n_kv, d), dtype=torch.bfloat16, device="cuda"), 34)
        pk.reshape_and_cache(pool, rows[0], rows[1], slots)
        out = pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, scale,
                                             max_context_len=max_ctx, total_context_len=hint)
        ref = oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                                 host(pool.v_scale), s.block_table, s.context_lens, scale)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL_BF16
    assert torch.count_nonzero(out[2]) == 0 and torch.count_nonzero(out[8]) == 0


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_ragged_grids_at_the_batch_limit(kind):
    """B = 512, the most sequences the ragged grids take (wave 0 forms the
    per-sequence prefix 8 sequences per lane): contexts 0 .. 300 with a
    total hint, bf16 on the stream grid and INT8 on the compact grid,
    against the oracle."""
    rng = np.random.default_rng(77)
    ctxs = [int(c) for c in rng.integers(0, 301, size=512)]
    ctxs[0], ctxs[511] = 0, 300
    n_kv, g, d, bs = 2, 8, 128, 16
    s = custom_structure(ctxs, bs, seed=78, pad_blocks=1)
    bt, ctx = tables_to_device(s)
    B = len(ctxs)
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), 79)
    scale = 1.0 / math.sqrt(d)
    hint = int(sum(ctxs))
    if kind == "bf16":
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
        device_normal_(pool.storage.view(torch.bfloat16), 80)
        out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=300,
                                        total_context_len=hint)
        ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table,
                                            s.context_lens, scale)
    else:
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
        seq, pos = prefill_tokens(s.context_lens)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        rows = device_normal_(torch.empty((2, len(seq), n_kv, d), dtype=torch.bfloat16, device="cuda"), 81)
        pk.reshape_and_cache(pool, rows[0], rows[1], slots)
        out = pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, scale,
                                             max_context_len=300, total_context_len=hint)
        ref = oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                                 host(pool.v_scale), s.block_table, s.context_lens, scale)
    torch.cuda.synchronize()
    assert max_err(out, ref) <= TOL_BF16
    assert torch.count_nonzero(out[0]) == 0
