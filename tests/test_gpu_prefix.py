"""GPU parity of the shared-prefix path of paged_decode_attention (the
shared_prefix_tokens hint): the prefix's K/V rows are read once for every
sequence whose block table over them is the longest sequence's, and every
other sequence reads its own blocks.  The hint only plans the work, so
every case compares with the fp64 oracle (max |gpu - oracle| <= 2e-2, bf16)
on every output element, whatever the hint: true, too long, too short, or
on tables that share only part of the prefix.  Slots no token owns hold
NaN.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import Structure, shared_prefix_prompts, shared_prefix_structure

from parity_support import TOL_BF16, host, max_err, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _case(s, n_h, n_kv, bs, seed):
    B = len(s.context_lens)
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, 128, 128, torch.bfloat16)
    device_normal_(pool.storage.view(torch.bfloat16), seed)
    owned = owned_slots(s.block_table, s.context_lens, bs)
    poison_unowned_(pool.k, owned)
    poison_unowned_(pool.v, owned)
    q = device_normal_(torch.empty((B, n_h, 128), dtype=torch.bfloat16, device="cuda"), seed + 1)
    return pool, q


def _prefix_ws(B, n_h, n_kv, hint, max_ctx, total, bs=16, cus=256, chunk=192):
    """Workspace of the prefix plan: 192-token chunks, stream workgroups
    filling one round of two per compute unit after the prefix ones, pieces
    (stream + B + chunks * B)."""
    g = n_h // n_kv
    S = min(hint, max_ctx) // 64 * 64
    nc = -(-S // chunk)
    spg = 4 * (32 // g)
    wgs = 2 * nc * (-(-B // spg))
    w = max(1, min(2 * cus // (n_kv // 2) - wgs, -(-total // 256)))
    rows = (w + B + nc * B) * n_h
    r = lambda n: -(-n // 256) * 256
    return r(rows * 128 * 4) + r(rows * 8) + r(B * 8)


@pytest.mark.parametrize("hint", [2048, 4096, 1000, 64, 0])
def test_llama8b_shared_prefix_hint_full_size(hint):
    """The 8B-shaped layer (B=32, g=4, contexts U[512, 4096], the first 128
    blocks shared by all) at full size with the true prefix length, one too
    long (the stretch past 2048 differs per sequence: those chunks run on
    each sequence's own blocks), shorter ones, and none."""
    cfg = CONFIGS["llama8b"]
    s = structure(cfg)
    pool, q = _case(s, cfg.n_h, cfg.n_kv, cfg.block_size, cfg.seed + hint)
    bt, ctx = tables_to_device(s)
    total = int(s.context_lens.sum())
    if hint == 2048 and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        desc = pk.make_desc(B=cfg.B, n_h=cfg.n_h, n_kv=cfg.n_kv, d_k=128, d_v=128, block_size=16,
                            max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=s.max_context_len,
                            q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, total_context_len=total,
                            shared_prefix_tokens=hint)
        assert pk.decode_workspace_size(desc) == _prefix_ws(cfg.B, cfg.n_h, cfg.n_kv, hint,
                                                            s.max_context_len, total)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, cfg.scale, max_context_len=s.max_context_len,
                                    total_context_len=total, shared_prefix_tokens=hint)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens,
                                        cfg.scale)
    assert max_err(out, ref) <= TOL_BF16


@pytest.mark.parametrize("hint", [2048, 0])
def test_llama8b_allocator_tables_full_size(hint):
    """The 8B-shaped batch with its tables built by the library's block
    allocator from the prompts' token ids: the shared 2K system prompt's
    full blocks are found by prefix caching and shared by every sequence (a
    prompt shorter than 2K keeps its partly filled last block to itself).
    Full size, every output element, with the hint and without."""
    cfg = CONFIGS["llama8b"]
    prompts, nb, order = shared_prefix_prompts(cfg)
    bt_np, ctx_np, cached = pk.BlockAllocator(nb, cfg.block_size, order=order).allocate_batch(prompts)
    full = np.minimum(ctx_np, 2048) // 16
    for b in range(1, cfg.B):                   # every full prefix block is shared with sequence 0's
        n = min(full[b], full[0])
        assert np.array_equal(bt_np[b, :n], bt_np[0, :n])
    assert cached[0] == 0 and sum(cached) > 0
    s = Structure(ctx_np, bt_np, nb)
    pool, q = _case(s, cfg.n_h, cfg.n_kv, cfg.block_size, 77 + hint)
    bt, ctx = tables_to_device(s)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, cfg.scale, max_context_len=s.max_context_len,
                                    total_context_len=int(ctx_np.sum()), shared_prefix_tokens=hint)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), bt_np, ctx_np, cfg.scale)
    assert max_err(out, ref) <= TOL_BF16


CTXS = [0, 1, 63, 64, 65, 300, 511, 512, 513, 700, 1100, 1, 900, 2000, 64, 129, 1500, 0, 777, 1024,
        256, 255, 257, 33, 1800, 640, 960, 12, 450, 1301, 2, 999, 1536, 1537, 16, 17, 3000, 70, 5, 880]


@pytest.mark.parametrize("g", [4, 8, 16])
@pytest.mark.parametrize("bs", [16, 64, 1])
@pytest.mark.parametrize("hint", [1024, 1536, 3000])
def test_prefix_partly_shared_ragged(g, bs, hint):
    """40 ragged sequences (two or three sequence groups), contexts 0 ..
    3000, the first 1536 tokens' blocks shared, except where some sequences
    have their own block (inside the first chunk, mid-prefix, at the last
    shared block) and one sequence shares nothing; hints below, at and past
    the shared length."""
    n_kv = 2
    shared_tok = 1536
    sb = shared_tok // bs
    div = [(3, 0), (9, sb // 2), (13, sb - 1), (20, 1 % sb), (36, sb // 3)]
    div += [(25, j) for j in range(sb)]               # sequence 25 shares nothing
    s = shared_prefix_structure(CTXS, bs, sb, seed=g + bs, diverge=div, pad_blocks=1)
    pool, q = _case(s, g * n_kv, n_kv, bs, 100 + g + bs + hint)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(128.0)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=3000,
                                    total_context_len=int(sum(CTXS)), shared_prefix_tokens=hint)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale)
    assert max_err(out, ref) <= TOL_BF16
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[17]) == 0


@pytest.mark.parametrize("case", ["pieces", "equal_ranges"])
def test_prefix_stream_parts_both_cuts(case):
    """The stream parts after a shared prefix are cut per sequence (each
    workgroup one piece of one sequence) while fewer sequences have a part
    than there are stream workgroups, and into equal ranges of their
    concatenation otherwise.  "pieces": 64 sequences of one KV-head pair,
    most parts a few tokens or blocks long, some thousands; "equal_ranges":
    512 sequences over four KV-head pairs, each with a part past a 64-token
    hint (more parts than the 96 stream workgroups of a pair)."""
    rng = np.random.default_rng(7 if case == "pieces" else 8)
    if case == "pieces":
        n_kv, g, shared, hint = 2, 8, 64, 1024
        ctxs = [int(x) for x in rng.choice([1025, 1030, 1040, 1100, 1300, 2000, 4500], size=64)]
        ctxs[5], ctxs[9] = 1024, 700                   # no part past the prefix, shorter than it
    else:
        n_kv, g, shared, hint = 8, 4, 4, 64
        ctxs = [int(x) for x in rng.integers(65, 400, size=512)]
    s = shared_prefix_structure(ctxs, 16, shared, seed=len(ctxs), pad_blocks=1)
    pool, q = _case(s, g * n_kv, n_kv, 16, 300 + len(ctxs))
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(128.0)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=max(ctxs),
                                    total_context_len=int(sum(ctxs)), shared_prefix_tokens=hint)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale)
    assert max_err(out, ref) <= TOL_BF16


def test_prefix_with_more_kv_heads_and_one_sequence():
    """n_kv = 8 (four KV-head pairs) with g = 4, a batch of one sequence
    (the reference itself), and a batch where every context ends inside the
    prefix (no stream work at all)."""
    scale = 1.0 / math.sqrt(128.0)
    for ctxs, hint in (([2500], 2048), ([100, 300, 640, 64, 1], 1024)):
        s = shared_prefix_structure(ctxs, 16, 64, seed=len(ctxs))
        pool, q = _case(s, 32, 8, 16, 7 + len(ctxs))
        bt, ctx = tables_to_device(s)
        out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=max(ctxs),
                                        total_context_len=int(sum(ctxs)), shared_prefix_tokens=hint)
        torch.cuda.synchronize()
        ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table,
                                            s.context_lens, scale)
        assert max_err(out, ref) <= TOL_BF16, ctxs


def test_prefix_hint_is_ignored_by_append_and_repeatable():
    """The append entry point runs without the prefix path (bit for bit the
    same as without the hint), and a repeated prefix call gives the same
    bits."""
    ctxs = [700, 1200, 1500, 690, 1000]               # every last token past the 640 shared ones
    s = shared_prefix_structure(ctxs, 16, 40, seed=3, pad_blocks=1)
    pool, q = _case(s, 32, 8, 16, 55)
    pool2 = pk.kv_pool_create(s.num_blocks, 16, 8, 128, 128, torch.bfloat16)
    pool2.storage.copy_(pool.storage)
    bt, ctx = tables_to_device(s)
    kv = device_normal_(torch.empty((2, len(ctxs), 8, 128), dtype=torch.bfloat16, device="cuda"), 56)
    scale = 1.0 / math.sqrt(128.0)
    mc = int(s.context_lens.max())
    a = pk.paged_decode_attention_append(pool, q, kv[0], kv[1], bt, ctx, scale, max_context_len=mc)
    desc = pk.make_desc(B=len(ctxs), n_h=32, n_kv=8, d_k=128, d_v=128, block_size=16,
                        max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=mc, q_dtype=pk.KVP_BF16,
                        kv_dtype=pk.KVP_BF16, shared_prefix_tokens=640)
    ws = pk.alloc_workspace(desc)
    out = torch.empty_like(a)
    pk._check(pk.lib().paged_decode_attention_append(
        pool2.handle, pk._ptr(q), pk._ptr(kv[0]), pk._ptr(kv[1]), pk._ptr(bt), pk._ptr(ctx),
        pk.ctypes.c_float(scale), pk._ptr(out), pk.ctypes.byref(desc), pk._ptr(ws), ws.numel(),
        pk._stream(q.device)))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))
    assert torch.equal(pool.storage, pool2.storage)
    r1 = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=mc, shared_prefix_tokens=640)
    r2 = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=mc, shared_prefix_tokens=640)
    torch.cuda.synchronize()
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale)
    assert max_err(r1, ref) <= TOL_BF16
