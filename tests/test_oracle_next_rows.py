"""Pins of the oracle's next-row functions: sliding-window decode, the INT4
cache with an attention sink, chunked-prefill attention, and the block
allocator (chained hashes, reference counts, LRU reuse, copy-on-write) with
block copies and swaps.  Every pin is something the pages or the
mathematics fix independently of the function under test."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth.workloads import custom_structure


# ---------------------------------------------------------------- sliding window

def _paged_case(ctxs, n_kv=2, g=2, d=16, bs=4, seed=0):
    rng = np.random.default_rng(seed)
    s = custom_structure(ctxs, bs, seed=seed + 1, pad_blocks=1)
    k = rng.standard_normal((s.num_blocks, bs, n_kv, d))
    v = rng.standard_normal((s.num_blocks, bs, n_kv, d))
    q = rng.standard_normal((len(ctxs), n_kv * g, d))
    return s, k, v, q


def test_window_covering_the_context_is_full_attention():
    s, k, v, q = _paged_case([1, 7, 13, 20])
    full = oracle.paged_decode_attention(q, k, v, s.block_table, s.context_lens, 0.3)
    for w in (20, 21, 1000):
        assert np.array_equal(oracle.paged_decode_attention(q, k, v, s.block_table, s.context_lens, 0.3, w), full)


def test_window_of_one_returns_the_last_value():
    """One token in the window: its weight is 1, the output its V row."""
    s, k, v, q = _paged_case([1, 5, 9, 16], g=3)
    out = oracle.paged_decode_attention(q, k, v, s.block_table, s.context_lens, 0.3, 1)
    for b, L in enumerate(s.context_lens):
        phys, off = oracle.logical_position(s.block_table[b], int(L) - 1, 4)
        for h in range(6):
            assert np.array_equal(out[b, h], v[phys, off, h // 3])


def test_window_matches_a_rolling_cache():
    """guijiagi section 5.1's cache: append every token, keep the last w,
    then attend over what is kept; built here as a contiguous rolling
    buffer, token by token, against the windowed paged oracle."""
    rng = np.random.default_rng(3)
    ctxs = [1, 6, 11, 17, 30]
    s, k, v, q = _paged_case(ctxs, seed=4)
    for w in (1, 3, 8, 16):
        out = oracle.paged_decode_attention(q, k, v, s.block_table, s.context_lens, 0.25, w)
        for b, L in enumerate(ctxs):
            keep_k, keep_v = [], []
            for j in range(L):
                phys, off = oracle.logical_position(s.block_table[b], j, 4)
                keep_k.append(k[phys, off])
                keep_v.append(v[phys, off])
                if len(keep_k) > w:
                    keep_k.pop(0)
                    keep_v.pop(0)
            ref = oracle.decode_attention_contiguous(q[b], np.stack(keep_k), np.stack(keep_v), 0.25)
            assert np.allclose(out[b], ref, rtol=0, atol=1e-14), (w, b)
    assert oracle.window_start(10, 4) == 6 and oracle.window_start(3, 4) == 0 and oracle.window_start(9, 0) == 0
    with pytest.raises(ValueError):
        oracle.window_start(5, -1)


def test_window_int8_equals_window_over_the_dequantized_cache():
    rng = np.random.default_rng(5)
    s = custom_structure([3, 40, 17], 16, seed=6, pad_blocks=1)
    x = rng.standard_normal((2, s.num_blocks, 16, 2, 32)).astype(np.float32)
    kc, ks = oracle.quantize_int8_rows(x[0])
    vc, vs = oracle.quantize_int8_rows(x[1])
    q = rng.standard_normal((3, 4, 32))
    got = oracle.paged_decode_attention_int8(q, kc, np.swapaxes(ks, 1, 2), vc, np.swapaxes(vs, 1, 2),
                                             s.block_table, s.context_lens, 0.2, 9)
    ref = oracle.paged_decode_attention(q, kc.astype(np.float64) * ks[..., None], vc.astype(np.float64) * vs[..., None],
                                        s.block_table, s.context_lens, 0.2, 9)
    assert np.allclose(got, ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- INT4 + sink

def test_int4_hand_rows(golden_dir):
    """Rows worked by hand from guijiagi 4.2's 4-bit branch (absmax / 7,
    round half to even, clamp [-8, 7]) in binary32."""
    import json, os
    cases = json.load(open(os.path.join(golden_dir, "int4_hand.json")))["rows"]
    for c in cases:
        codes, scale = oracle.quantize_int4_rows(np.asarray(c["x"], dtype=np.float32))
        assert codes.tolist() == c["codes"], c
        assert float(scale) == float(np.float32(c["scale"])), c


def test_int4_codes_properties():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((500, 64)) * rng.uniform(0.01, 50, (500, 1))).astype(np.float32)
    x[3] = 0.0
    codes, scale = oracle.quantize_int4_rows(x)
    assert codes.dtype == np.int8 and codes.min() >= -8 and codes.max() <= 7
    nz = scale > 0
    # the absolute maximum maps to +-7; the reconstruction error is at most
    # half a step (plus the rounding of the fp32 quotient)
    assert np.all(np.abs(codes[nz]).max(axis=1) == 7)
    err = np.abs(x.astype(np.float64) - codes * scale[:, None].astype(np.float64))
    assert np.all(err[nz] <= scale[nz, None] * (0.5 + 2.0 ** -20))
    assert np.all(codes[3] == 0) and scale[3] == 0.0


def test_int4_packing_round_trip_and_layout():
    rng = np.random.default_rng(8)
    codes = rng.integers(-8, 8, size=(5, 3, 64)).astype(np.int8)
    packed = oracle.pack_int4(codes)
    assert packed.shape == (5, 3, 32) and packed.dtype == np.uint8
    assert np.array_equal(oracle.unpack_int4(packed), codes)
    # byte 0 of [-8, 7, ...] is 0x78 (low nibble 8 = -8, high nibble 7)
    one = np.zeros(4, dtype=np.int8); one[0], one[1], one[2], one[3] = -8, 7, -1, 0
    assert oracle.pack_int4(one).tolist() == [0x78, 0x0F]


def test_int4_attention_with_and_without_sink():
    """The sink positions come from the unquantized rows, every other one
    from the dequantized INT4 pool; with no sink it is attention over the
    dequantized pool, and positions past n_sink ignore the sink arrays."""
    rng = np.random.default_rng(9)
    bs, n_kv, d = 16, 2, 32
    s = custom_structure([1, 3, 4, 5, 40], bs, seed=10, pad_blocks=1)
    B = len(s.context_lens)
    x = rng.standard_normal((2, s.num_blocks, bs, n_kv, d)).astype(np.float32)
    kc, ks = oracle.quantize_int4_rows(x[0])
    vc, vs = oracle.quantize_int4_rows(x[1])
    kp, vp = oracle.pack_int4(kc), oracle.pack_int4(vc)
    ksT, vsT = np.swapaxes(ks, 1, 2), np.swapaxes(vs, 1, 2)
    q = rng.standard_normal((B, 4, d))
    sink_k = rng.standard_normal((B, 4, n_kv, d)).astype(np.float32)
    sink_v = rng.standard_normal((B, 4, n_kv, d)).astype(np.float32)
    got = oracle.paged_decode_attention_int4(q, kp, ksT, vp, vsT, sink_k, sink_v, s.block_table, s.context_lens, 0.3)
    kd = kc.astype(np.float64) * ks[..., None]
    vd = vc.astype(np.float64) * vs[..., None]
    for b, L in enumerate(s.context_lens):
        K = oracle.gather_sequence(kd, s.block_table[b], int(L)).copy()
        V = oracle.gather_sequence(vd, s.block_table[b], int(L)).copy()
        n = min(int(L), 4)
        K[:n], V[:n] = sink_k[b, :n], sink_v[b, :n]
        ref = oracle.decode_attention_contiguous(q[b], K, V, 0.3)
        assert np.allclose(got[b], ref, rtol=0, atol=1e-14)
    none = oracle.paged_decode_attention_int4(q, kp, ksT, vp, vsT, sink_k[:, :0], sink_v[:, :0], s.block_table,
                                              s.context_lens, 0.3)
    assert np.allclose(none, oracle.paged_decode_attention(q, kd, vd, s.block_table, s.context_lens, 0.3), atol=1e-14)


def test_attention_sink_lowers_the_error_when_early_keys_draw_attention():
    """guijiagi 4.3's point, on a case built to show it: the first tokens'
    keys are large and aligned with the query (they draw most of the
    attention); keeping those four unquantized gives a smaller error than
    quantizing them, measured against the exact fp64 attention."""
    rng = np.random.default_rng(11)
    bs, d, L = 16, 64, 200
    s = custom_structure([L], bs, seed=12)
    k = rng.standard_normal((s.num_blocks, bs, 1, d)).astype(np.float32)
    v = rng.standard_normal((s.num_blocks, bs, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d))
    for j in range(4):
        phys, off = oracle.logical_position(s.block_table[0], j, bs)
        k[phys, off, 0] = (3.0 * q[0, 0] / np.linalg.norm(q[0, 0]) + 0.3 * rng.standard_normal(d)).astype(np.float32)
        v[phys, off, 0] *= 8.0
    exact = oracle.paged_decode_attention(q, k, v, s.block_table, s.context_lens, 0.5)
    kc, ks = oracle.quantize_int4_rows(k)
    vc, vs = oracle.quantize_int4_rows(v)
    args = (oracle.pack_int4(kc), np.swapaxes(ks, 1, 2), oracle.pack_int4(vc), np.swapaxes(vs, 1, 2))
    sk = np.stack([k[oracle.logical_position(s.block_table[0], j, bs)] for j in range(4)])[None]
    sv = np.stack([v[oracle.logical_position(s.block_table[0], j, bs)] for j in range(4)])[None]
    with_sink = oracle.paged_decode_attention_int4(q, *args, sk, sv, s.block_table, s.context_lens, 0.5)
    no_sink = oracle.paged_decode_attention_int4(q, *args, sk[:, :0], sv[:, :0], s.block_table, s.context_lens, 0.5)
    assert np.abs(with_sink - exact).max() < 0.5 * np.abs(no_sink - exact).max()


# ---------------------------------------------------------------- chunked prefill

def test_chunked_prefill_matches_causal_attention_and_decode():
    """Chunk by chunk over one prompt equals causal attention over the whole
    prompt (torch CPU fp64 scaled_dot_product_attention with is_causal, on
    the contiguous K/V, heads expanded for GQA); a chunk's last query equals
    decode attention with the context ending there."""
    rng = np.random.default_rng(13)
    bs, n_kv, g, d, T = 4, 2, 3, 16, 37
    s = custom_structure([T], bs, seed=14)
    k = rng.standard_normal((s.num_blocks, bs, n_kv, d))
    v = rng.standard_normal((s.num_blocks, bs, n_kv, d))
    qa = rng.standard_normal((T, n_kv * g, d))
    K = oracle.gather_sequence(k, s.block_table[0], T)
    V = oracle.gather_sequence(v, s.block_table[0], T)
    tq = torch.from_numpy(qa).permute(1, 0, 2)[None]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.2)[0].permute(1, 0, 2)
    got = np.zeros((T, n_kv * g, d))
    for p0 in range(0, T, 10):
        n = min(10, T - p0)
        qc = np.zeros((1, 10, n_kv * g, d)); qc[0, :n] = qa[p0:p0 + n]
        out = oracle.paged_prefill_attention(qc, k, v, s.block_table, [p0], [n], 0.2)
        got[p0:p0 + n] = out[0, :n]
        assert np.all(out[0, n:] == 0)
        dec = oracle.paged_decode_attention(qa[p0 + n - 1][None], k, v, s.block_table, [p0 + n], 0.2)
        assert np.array_equal(out[0, n - 1], dec[0])
    assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- allocator

def _blake2b_rfc7693(data: bytes, outlen: int) -> bytes:
    """BLAKE2b written from RFC 7693 (no key), to pin the hash independently
    of hashlib."""
    M64 = (1 << 64) - 1
    IV = [0x6A09E667F3BCC908, 0xBB67AE8584CAA73B, 0x3C6EF372FE94F82B, 0xA54FF53A5F1D36F1,
          0x510E527FADE682D1, 0x9B05688C2B3E6C1F, 0x1F83D9ABFB41BD6B, 0x5BE0CD19137E2179]
    SIGMA = [[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15],
             [14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3],
             [11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4],
             [7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8],
             [9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13],
             [2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9],
             [12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11],
             [13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10],
             [6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5],
             [10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0]]
    rot = lambda x, n: ((x >> n) | (x << (64 - n))) & M64

    def compress(h, block, t, last):
        m = [int.from_bytes(block[8 * i:8 * i + 8], "little") for i in range(16)]
        v = h[:] + IV[:]
        v[12] ^= t & M64
        v[13] ^= t >> 64
        if last:
            v[14] ^= M64
        for r in range(12):
            s = SIGMA[r % 10]
            for i, (a, b, c, d) in enumerate([(0, 4, 8, 12), (1, 5, 9, 13), (2, 6, 10, 14), (3, 7, 11, 15),
                                              (0, 5, 10, 15), (1, 6, 11, 12), (2, 7, 8, 13), (3, 4, 9, 14)]):
                x, y = m[s[2 * i]], m[s[2 * i + 1]]
                v[a] = (v[a] + v[b] + x) & M64; v[d] = rot(v[d] ^ v[a], 32)
                v[c] = (v[c] + v[d]) & M64; v[b] = rot(v[b] ^ v[c], 24)
                v[a] = (v[a] + v[b] + y) & M64; v[d] = rot(v[d] ^ v[a], 16)
                v[c] = (v[c] + v[d]) & M64; v[b] = rot(v[b] ^ v[c], 63)
        return [h[i] ^ v[i] ^ v[i + 8] for i in range(8)]

    h = IV[:]
    h[0] ^= 0x01010000 ^ outlen
    blocks = [data[i:i + 128] for i in range(0, len(data), 128)] or [b""]
    t = 0
    for i, blk in enumerate(blocks):
        t += len(blk)
        h = compress(h, blk.ljust(128, b"\0"), t, i == len(blocks) - 1)
    return b"".join(x.to_bytes(8, "little") for x in h)[:outlen]


def test_blake2b_rfc_vector_and_chained_block_hash():
    # RFC 7693 appendix A: BLAKE2b-512("abc")
    assert _blake2b_rfc7693(b"abc", 64).hex().startswith("ba80a53f981c4d0d6a2797b69f12f6e94c212f14685ac4b7")
    for parent, toks in [(0, list(range(16))), (0x0123456789ABCDEF, [7] * 16), (2 ** 64 - 1, [2 ** 32 - 1, 0, 5])]:
        data = parent.to_bytes(8, "little") + b"".join(t.to_bytes(4, "little") for t in toks)
        want = int.from_bytes(_blake2b_rfc7693(data, 8), "little")
        assert oracle.block_hash(parent, toks) == want


def test_prefix_hits_share_blocks_and_count_references():
    a = oracle.BlockAllocator(16, 4)
    t1, c1 = a.allocate_prompt(list(range(10)))          # blocks 0, 1 full + partial 2
    assert t1 == [0, 1, 2] and c1 == 0
    t2, c2 = a.allocate_prompt(list(range(8)) + [99])     # same first two full blocks
    assert t2[:2] == [0, 1] and c2 == 8 and a.ref[0] == 2 and a.ref[1] == 2
    assert t2[2] == 3                                     # the partial tail is never matched
    t3, c3 = a.allocate_prompt([0, 1, 2, 3, 9, 9, 9, 9] + list(range(8, 12)))
    assert t3[0] == 0 and c3 == 4 and a.ref[0] == 3       # matching stops at the first miss
    assert t3[1] not in (1,) and a.ref[1] == 2
    # the block after a miss is registered under its own chained hash
    h0 = oracle.block_hash(0, [0, 1, 2, 3])
    h1 = oracle.block_hash(h0, [9, 9, 9, 9])
    assert a.by_hash[h1] == t3[1] and a.hash[t3[1]] == h1


def test_freed_blocks_park_in_lru_order_and_are_reused_on_a_hit():
    a = oracle.BlockAllocator(6, 2)
    ta, _ = a.allocate_prompt([1, 2, 3, 4])              # blocks 0, 1
    tb, _ = a.allocate_prompt([5, 6, 7, 8])              # blocks 2, 3
    a.free_sequence(tb)
    a.free_sequence(ta)
    assert list(a.evictable) == [4, 5, 2, 3, 0, 1]       # untouched first, then in freeing order
    # a prompt matching ta's blocks takes them back out of the pool
    tc, cached = a.allocate_prompt([1, 2, 3, 4, 10])
    assert tc[:2] == [0, 1] and cached == 4 and a.ref[0] == 1 and 0 not in a.evictable
    assert tc[2] == 4                                    # the tail takes the least recently used block
    # later blocks come from the LRU end and lose their hash
    a.allocate_prompt([11, 12])                          # takes block 5
    td, _ = a.allocate_prompt([13, 14])                  # takes block 2 (tb's first, hash dropped)
    assert td == [2] and oracle.block_hash(0, [5, 6]) not in a.by_hash


def test_copy_on_write_of_a_shared_tail_block():
    a = oracle.BlockAllocator(8, 4)
    t, _ = a.allocate_prompt([1, 2, 3, 4, 5, 6])         # blocks 0 (full), 1 (2 slots)
    u = a.fork(t)
    assert a.ref[1] == 2
    cow = a.append_token(u, 7)
    assert cow == (1, u[1]) and u[0] == 0 and u[1] != 1
    assert a.ref[1] == 1 and a.tokens[u[1]] == [5, 6, 7] and a.tokens[1] == [5, 6]
    assert a.append_token(t, 8) is None and a.tokens[1] == [5, 6, 8]   # sole owner appends in place
    a.append_token(t, 9)
    assert a.append_token(t, 10) is None and len(t) == 3              # full tail: a new block


def test_running_out_of_blocks_raises_memory_error_and_changes_nothing():
    a = oracle.BlockAllocator(4, 4)
    t, _ = a.allocate_prompt(list(range(6)))              # blocks 0, 1 (tail holds 2)
    snap = lambda: (list(a.ref), list(a.hash), [list(x) for x in a.tokens], list(a.evictable), dict(a.by_hash))
    before = snap()
    with pytest.raises(MemoryError):
        a.allocate_prompt(list(range(100, 109)))          # needs 3 fresh blocks, 2 are left
    assert snap() == before
    u = a.fork(t)
    a.allocate_prompt([7, 7, 7, 7, 7, 7, 7, 7])            # the last two blocks
    before = snap()
    with pytest.raises(MemoryError):                      # copy-on-write of the shared tail needs a block
        a.append_token(u, 9)
    assert snap() == before and a.ref[t[1]] == 2
    a.free_sequence(u)
    assert a.append_token(t, 9) is None                   # sole owner again: in place


def test_internal_waste_is_below_one_block_per_sequence():
    """faulkner (logical/physical block mapping): waste is confined to each
    sequence's last block, at most block_size - 1 slots."""
    rng = np.random.default_rng(15)
    a = oracle.BlockAllocator(4000, 16)
    lens = rng.integers(1, 500, size=60)
    used = 0
    for n in lens:
        t, _ = a.allocate_prompt(list(rng.integers(0, 50000, size=n)))
        used += len(t)
        assert len(t) * 16 - n <= 15
    assert used * 16 - lens.sum() <= 60 * 15


def test_copy_blocks_and_swap_round_trip():
    rng = np.random.default_rng(16)
    pool = rng.standard_normal((10, 4, 2, 8)).astype(np.float32)
    out = oracle.copy_blocks(pool, [(1, 7), (3, 2)])
    assert np.array_equal(out[7], pool[1]) and np.array_equal(out[2], pool[3])
    assert np.array_equal(np.delete(out, [7, 2], 0), np.delete(pool, [7, 2], 0))
    host = oracle.swap_out(pool, [4, 0, 9])
    assert host.shape == (3, 4, 2, 8) and np.array_equal(host[1], pool[0])
    wiped = pool.copy(); wiped[[4, 0, 9]] = np.nan
    back = oracle.swap_in(wiped, host, [4, 0, 9])
    assert np.array_equal(back, pool)
