"""The device side of the block allocator on the GPU: copy_blocks (the
copy-on-write copy) and block swaps to pinned host memory and back,
bit-exact against the oracle on every pool kind; and decode over tables
the library's allocator built: the 8B-shaped batch (32 prompts sharing a
2048-token system prompt, hx 4.2) decoded with the shared-prefix hint, and
a copy-on-write step of forked sequences, against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_

from parity_support import TOL_BF16, host, max_err

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")

KINDS = [("bf16", 16, 8, 128, 128, False), ("f32", 4, 2, 64, 64, False), ("int8", 16, 8, 128, 128, False),
         ("bf16", 64, 1, 576, 512, True)]


def _pool(kind, nb, bs, n_kv, d_k, d_v, latent, seed):
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "int8": torch.int8}[kind]
    pool = pk.kv_pool_create(nb, bs, n_kv, d_k, d_v, dt, latent=latent)
    g = torch.Generator(device="cuda").manual_seed(seed)
    pool.storage.copy_(torch.randint(0, 256, pool.storage.shape, dtype=torch.uint8, device="cuda", generator=g))
    return pool


def _arrays(pool):
    out = [host(pool.k)] if pool.dtype != torch.int8 else [pool.k.cpu().numpy()]
    if not pool.latent:
        out.append(host(pool.v) if pool.dtype != torch.int8 else pool.v.cpu().numpy())
    if pool.k_scale is not None:
        out.append(pool.k_scale.cpu().numpy())
        if pool.v_scale is not None:
            out.append(pool.v_scale.cpu().numpy())
    return [np.ascontiguousarray(a).view(np.uint8).reshape(a.shape[0], -1) for a in out]


@pytest.mark.parametrize("kind,bs,n_kv,d_k,d_v,latent", KINDS)
def test_copy_blocks_bit_exact(kind, bs, n_kv, d_k, d_v, latent):
    nb = 40
    pool = _pool(kind, nb, bs, n_kv, d_k, d_v, latent, 1)
    before = _arrays(pool)
    pairs = np.array([[3, 17], [0, 39], [25, 5], [8, 8], [-1, 2], [41, 3], [12, 30]], dtype=np.int32)
    pk.copy_blocks(pool, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    valid = [(s, d) for s, d in pairs.tolist() if 0 <= s < nb and 0 <= d < nb]   # out-of-range pairs are skipped
    for got, arr in zip(_arrays(pool), before):
        assert np.array_equal(got, oracle.copy_blocks(arr, valid))


@pytest.mark.parametrize("kind,bs,n_kv,d_k,d_v,latent", KINDS)
def test_swap_out_and_in_round_trip(kind, bs, n_kv, d_k, d_v, latent):
    nb = 40
    pool = _pool(kind, nb, bs, n_kv, d_k, d_v, latent, 2)
    before = _arrays(pool)
    blocks = [7, 0, 39, 22, 13]
    bb = pk.kv_pool_block_bytes(pool)
    assert bb == sum(a.shape[1] for a in before)
    staging = torch.empty(len(blocks) * bb, dtype=torch.uint8, device="cuda")
    hbuf = torch.empty(len(blocks) * bb, dtype=torch.uint8, pin_memory=True)
    bl = torch.tensor(blocks, dtype=torch.int32, device="cuda")
    pk.swap_out_blocks(pool, bl, staging, hbuf)
    torch.cuda.synchronize()
    hb = hbuf.numpy().reshape(len(blocks), bb)
    off = 0
    for arr in before:
        w = arr.shape[1]
        assert np.array_equal(hb[:, off:off + w], oracle.swap_out(arr, blocks)), off
        off += w
    # wipe the swapped blocks, swap back in: the pool is whole again
    for arr_t in [pool.k] + ([] if latent else [pool.v]):
        arr_t.view(torch.uint8)[bl.long()] = 0xFF
    staging.zero_()
    pk.swap_in_blocks(pool, bl, staging, hbuf)
    torch.cuda.synchronize()
    for got, arr in zip(_arrays(pool), before):
        assert np.array_equal(got, arr)


def test_block_moves_at_the_bench_size():
    """The bench's block-move workload: a 70B-shaped layer pool (8192 blocks
    of 64 KiB), copy_blocks of 2048 (src, dst) pairs of distinct random
    blocks, then a swap out and back in of 1024 random blocks: every byte
    of the pool against the oracle's copy, the host rows against its swap."""
    nb = 8192
    pool = _pool("bf16", nb, 16, 8, 128, 128, False, 5)
    before = _arrays(pool)
    perm = np.random.default_rng(5).permutation(nb).astype(np.int32)
    pairs = perm[:4096].reshape(2, 2048).T.copy()
    pk.copy_blocks(pool, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    after = _arrays(pool)
    for got, arr in zip(after, before):
        assert np.array_equal(got, oracle.copy_blocks(arr, pairs.tolist()))
    blocks = perm[:1024]
    bb = pk.kv_pool_block_bytes(pool)
    staging = torch.empty(len(blocks) * bb, dtype=torch.uint8, device="cuda")
    hbuf = torch.empty(len(blocks) * bb, dtype=torch.uint8, pin_memory=True)
    bl = torch.from_numpy(blocks.copy()).cuda()
    pk.swap_out_blocks(pool, bl, staging, hbuf)
    torch.cuda.synchronize()
    hb = hbuf.numpy().reshape(len(blocks), bb)
    off = 0
    for arr in after:
        w = arr.shape[1]
        assert np.array_equal(hb[:, off:off + w], oracle.swap_out(arr, blocks.tolist()))
        off += w
    for arr_t in (pool.k, pool.v):
        arr_t.view(torch.uint8)[bl.long()] = 0xFF
    pk.swap_in_blocks(pool, bl, staging.zero_(), hbuf)
    torch.cuda.synchronize()
    for got, arr in zip(_arrays(pool), after):
        assert np.array_equal(got, arr)


def _write_tokens(pool, tables, lens, seed):
    """K/V rows for every token of every sequence, written through
    reshape_and_cache at the slots the tables give."""
    seq = np.concatenate([[b] * n for b, n in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    mb = max(len(t) for t in tables)
    bt = np.full((len(tables), mb), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        bt[b, :len(t)] = t
    slots = oracle.slot_mapping(bt, seq, pos, pool.block_size)
    rows = device_normal_(torch.empty((2, len(seq), pool.n_kv, pool.d_k), dtype=torch.bfloat16, device="cuda"), seed)
    pk.reshape_and_cache(pool, rows[0], rows[1], torch.from_numpy(slots).cuda())
    return bt


def test_llama8b_batch_from_the_allocator_with_prefix_hint():
    """Tables of the 8B-shaped batch made by the library allocator: a pool
    sized to the batch, handed out in a seeded random order, 32 prompts of
    the workload's context lengths sharing a 2048-token system prompt.
    Every sequence after the first reuses the prompt's full blocks (cached
    tokens = its full shared blocks); every sequence's rows are written
    through its own table, so a shared slot is written by several sequences
    (one write stands; the oracle reads the pool as the writes left it);
    decoded with the prefix hint against the oracle on every element."""
    cfg = CONFIGS["llama8b"]
    s = structure(cfg)
    lens = [int(c) for c in s.context_lens]
    rng = np.random.default_rng(cfg.seed)
    system = [int(t) for t in rng.integers(0, 50000, size=2048)]
    need = 128 + sum(-(-max(0, n - 2048) // 16) + (1 if n < 2048 and n % 16 else 0) for n in lens)
    alloc = pk.BlockAllocator(need, 16, order=rng.permutation(need), max_blocks_per_seq=256)
    tables = []
    for b, n in enumerate(lens):
        toks = system[:n] + [int(t) for t in rng.integers(0, 50000, size=max(0, n - 2048))]
        t, cached = alloc.allocate_prompt(toks)
        tables.append(t)
        if b > 0:
            full_shared = min(n, 2048) // 16
            prev_full = max(min(lens[j], 2048) // 16 for j in range(b))
            assert cached == 16 * min(full_shared, prev_full), b
    assert alloc.evictable() == []
    pool = pk.kv_pool_create(need, 16, 8, 128, 128, torch.bfloat16)
    bt = _write_tokens(pool, tables, lens, 5)
    q = device_normal_(torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda"), 6)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = pk.paged_decode_attention(q, pool.k, pool.v, torch.from_numpy(bt).cuda(), ctx, cfg.scale,
                                    max_context_len=max(lens), total_context_len=sum(lens), shared_prefix_tokens=2048)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), bt, np.array(lens), cfg.scale)
    assert max_err(out, ref) <= TOL_BF16


def test_copy_on_write_decode_step():
    """Parallel sampling: a prompt with a partly filled tail is forked three
    times; each branch appends its own token.  The allocator reports a
    copy-on-write for all but the last branch to append; copy_blocks copies
    the tail's rows, the new tokens' rows are written at the returned slots,
    and decode over the branches' tables matches the oracle (the branches
    share every full block and differ in their tails)."""
    bs, n_kv, d = 16, 2, 128
    alloc = pk.BlockAllocator(64, bs, order=np.random.default_rng(1).permutation(64))
    prompt = list(range(1000, 1000 + 70))                   # 4 full blocks + 6 slots
    t0, _ = alloc.allocate_prompt(prompt)
    branches = [t0] + [alloc.fork(t0) for _ in range(3)]
    pool = pk.kv_pool_create(64, bs, n_kv, d, d, torch.bfloat16)
    _write_tokens(pool, [t0], [70], 7)
    slots, cows = [], []
    for t in branches:
        slot, cow = alloc.append_slot(t)
        slots.append(slot)
        cows.append(cow)
    assert all(c is not None for c in cows[:3]) and cows[3] is None
    pk.copy_blocks(pool, torch.tensor([list(c) for c in cows[:3]], dtype=torch.int32, device="cuda"))
    rows = device_normal_(torch.empty((2, 4, n_kv, d), dtype=torch.bfloat16, device="cuda"), 8)
    pk.reshape_and_cache(pool, rows[0], rows[1], torch.tensor(slots, dtype=torch.int64, device="cuda"))
    bt = np.array(branches, dtype=np.int32)
    assert len({tuple(t[:4]) for t in branches}) == 1 and len({t[4] for t in branches}) == 4
    q = device_normal_(torch.empty((4, 16, d), dtype=torch.bfloat16, device="cuda"), 9)
    ctx = torch.full((4,), 71, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = pk.paged_decode_attention(q, pool.k, pool.v, torch.from_numpy(bt).cuda(), ctx, scale, max_context_len=71)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), bt, np.full(4, 71), scale)
    assert max_err(out, ref) <= TOL_BF16
    # the copied tails hold the prompt's six tail rows
    kh = host(pool.k)
    for c in cows[:3]:
        assert np.array_equal(kh[c[1], :6], kh[c[0], :6])
