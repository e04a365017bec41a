"""The library's host block allocator (C++, no device work) against the
oracle's model, on the CPU: seeded random streams of prompts that share
prefixes, decode appends (with forks, so copy-on-write happens), frees and
exhaustion, comparing every returned table, cached count, slot and
copy-on-write pair, and the full allocator state (reference counts, fills,
hashes, the evictable order) after every step.  The chained hash is
checked against the oracle's (BLAKE2b-64 from hashlib)."""

import numpy as np
import pytest

import oracle

pk = pytest.importorskip("pagedattention_decode_paged_amd",
                         reason="libpagedkv.so not built (run __graft_entry__.build())")


def _state_equal(lib_a, ref_a, nb):
    assert lib_a.evictable() == list(ref_a.evictable)
    for b in range(nb):
        r, f, hashed, h = lib_a.block_state(b)
        assert r == ref_a.ref[b], b
        assert f == len(ref_a.tokens[b]), b
        assert hashed == (ref_a.hash[b] is not None), b
        if hashed:
            assert h == ref_a.hash[b], b


def test_block_hash_matches_the_oracle():
    rng = np.random.default_rng(0)
    for n in (0, 1, 16, 31, 33, 64):                      # crosses BLAKE2b's 128-byte buffer
        toks = [int(t) for t in rng.integers(0, 2 ** 31, size=n)]
        parent = int(rng.integers(0, 2 ** 63))
        assert pk.block_hash(parent, toks) == oracle.block_hash(parent, toks)


@pytest.mark.parametrize("seed", range(6))
def test_random_streams_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    nb, bs = int(rng.choice([24, 64, 200])), int(rng.choice([1, 2, 4, 16]))
    order = rng.permutation(nb) if seed % 2 else None
    lib_a = pk.BlockAllocator(nb, bs, order=order)
    ref_a = oracle.BlockAllocator(nb, bs, order=order)
    prefixes = [list(rng.integers(0, 1000, size=int(rng.integers(0, 5 * bs + 3)))) for _ in range(3)]
    live = []                                               # (lib table, ref table)
    for step in range(300):
        op = rng.random()
        if op < 0.35 or not live:
            p = prefixes[int(rng.integers(0, 3))]
            toks = p + list(rng.integers(0, 1000, size=int(rng.integers(0, 3 * bs + 2))))
            if not toks:
                continue
            try:
                want = ref_a.allocate_prompt(toks)
            except MemoryError:
                with pytest.raises(pk.PagedKVError) as ei:
                    lib_a.allocate_prompt(toks)
                assert ei.value.status == pk.KVP_ERR_OUT_OF_MEMORY
            else:
                got = lib_a.allocate_prompt(toks)
                assert got == want, step
                live.append((got[0], list(want[0])))
        elif op < 0.65:
            i = int(rng.integers(0, len(live)))
            lt, rt = live[i]
            try:
                cow = ref_a.append_token(rt, int(rng.integers(0, 1000)))
            except MemoryError:
                with pytest.raises(pk.PagedKVError) as ei:
                    lib_a.append_slot(lt)
                assert ei.value.status == pk.KVP_ERR_OUT_OF_MEMORY
            else:
                slot, lcow = lib_a.append_slot(lt)
                assert lt == rt and lcow == cow, step
                assert slot == rt[-1] * bs + len(ref_a.tokens[rt[-1]]) - 1
        elif op < 0.75:
            i = int(rng.integers(0, len(live)))
            lt, rt = live[i]
            live.append((lib_a.fork(lt), ref_a.fork(rt)))
        else:
            i = int(rng.integers(0, len(live)))
            lt, rt = live.pop(i)
            ref_a.free_sequence(rt)
            lib_a.free_sequence(lt)
        _state_equal(lib_a, ref_a, nb)


def test_errors_leave_the_allocator_unchanged():
    a = pk.BlockAllocator(4, 4, max_blocks_per_seq=8)
    t, _ = a.allocate_prompt(list(range(6)))
    before = ([a.block_state(b) for b in range(4)], a.evictable())
    with pytest.raises(pk.PagedKVError) as ei:
        a.allocate_prompt(list(range(100, 109)))
    assert ei.value.status == pk.KVP_ERR_OUT_OF_MEMORY and "out of KV cache blocks" in str(ei.value)
    with pytest.raises(pk.PagedKVError):
        a.free_sequence(t + t)                              # freed more often than held
    with pytest.raises(pk.PagedKVError):
        a.fork([3])                                         # a block nobody holds
    assert ([a.block_state(b) for b in range(4)], a.evictable()) == before
    with pytest.raises(pk.PagedKVError):
        pk.BlockAllocator(4, 4, order=[0, 1, 1, 3])


def test_shared_prefix_batch_tables_match_the_oracle():
    """The 8B-shaped batch's tables as the bench and the GPU tests build
    them (the library's allocator over the prompts' token ids): identical to
    the oracle allocator's from the same free order, and every full block
    of the shared 2K system prompt is one physical block for all."""
    from synth import CONFIGS
    from synth.workloads import shared_prefix_prompts
    cfg = CONFIGS["llama8b"]
    prompts, nb, order = shared_prefix_prompts(cfg)
    bt, ctx, cached = pk.BlockAllocator(nb, cfg.block_size, order=order).allocate_batch(prompts)
    ref = oracle.BlockAllocator(nb, cfg.block_size, order=order)
    for b, p in enumerate(prompts):
        table, c = ref.allocate_prompt(p)
        assert list(bt[b, :len(table)]) == table and np.all(bt[b, len(table):] == -1)
        assert cached[b] == c
    assert list(ctx) == [len(p) for p in prompts]
    full = np.minimum(ctx, 2048) // cfg.block_size
    longest = int(np.argmax(full))
    for b in range(cfg.B):
        assert np.array_equal(bt[b, :full[b]], bt[longest, :full[b]])
