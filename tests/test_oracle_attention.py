"""Pins of the oracle's attention: exact decimal brute force, closed forms,
special cases that reduce to a library routine, and structural invariants
(block size, physical permutation, GQA replication).  CPU only."""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from synth.workloads import custom_structure, prefill_tokens


def _paged_from_contiguous(Ks, Vs, ctxs, bs, seed, extra_blocks=1):
    """Build paged pools (NaN in every unowned cell) holding the given
    logical-order rows, using the oracle's own write path."""
    s = custom_structure(ctxs, bs, seed=seed, pad_blocks=1)
    nb = s.num_blocks + extra_blocks
    n_kv, dk = Ks[0].shape[1], Ks[0].shape[2]
    dv = Vs[0].shape[2]
    kp = np.full((nb, bs, n_kv, dk), np.nan)
    vp = np.full((nb, bs, n_kv, dv), np.nan)
    seq, pos = prefill_tokens(s.context_lens)
    slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    kp = oracle.reshape_and_cache(kp, np.concatenate(Ks), slots)
    vp = oracle.reshape_and_cache(vp, np.concatenate(Vs), slots)
    return kp, vp, s


def _decimal_attention(q, K, V, scale, g):
    """Brute force in 50-digit decimal arithmetic: loops only."""
    getcontext().prec = 50
    n_h, dk = len(q), len(q[0])
    L = len(K)
    out = []
    for h in range(n_h):
        kvh = h // g
        s = []
        for j in range(L):
            acc = Decimal(0)
            for d in range(dk):
                acc += Decimal(float(q[h][d])) * Decimal(float(K[j][kvh][d]))
            s.append(acc * Decimal(float(scale)))
        m = max(s)
        e = [(x - m).exp() for x in s]
        z = sum(e)
        row = []
        for d in range(len(V[0][kvh])):
            acc = Decimal(0)
            for j in range(L):
                acc += e[j] / z * Decimal(float(V[j][kvh][d]))
            row.append(acc)
        out.append(row)
    return out


@settings(max_examples=25, deadline=None)
@given(st.integers(1, 6), st.sampled_from([(4, 2), (4, 4), (4, 1), (2, 2)]),
       st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_matches_decimal_brute_force(L, heads, d, seed):
    n_h, n_kv = heads
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_h, d))
    K = rng.standard_normal((L, n_kv, d))
    V = rng.standard_normal((L, n_kv, d + 1))
    scale = 0.37
    exact = _decimal_attention(q.tolist(), K.tolist(), V.tolist(), scale, n_h // n_kv)
    got = oracle.decode_attention_contiguous(q, K, V, scale)
    assert np.max(np.abs(got - np.array([[float(x) for x in r] for r in exact]))) <= 1e-12
    # the same through a paged pool with a random permutation, block size 2
    kp, vp, s = _paged_from_contiguous([K], [V], [L], 2, seed)
    paged = oracle.paged_decode_attention(q[None], kp, vp, s.block_table, s.context_lens, scale)
    assert np.array_equal(paged[0], got)


def test_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "softmax_hand.json")) as f:
        g = json.load(f)
    scale = math.log(3.0)
    q = np.array([g["q"]])
    K = np.array(g["K"])[:, None, :]
    V = np.array(g["V"])[:, None, :]
    w = oracle.softmax_weights(q[0], K[:, 0], scale)
    assert np.allclose(w, g["expected_weights"], rtol=0, atol=1e-15)
    o = oracle.decode_attention_contiguous(q, K, V, scale)
    assert np.allclose(o[0], g["expected_out"], rtol=0, atol=1e-14)


def test_weights_sum_to_one_and_are_positive():
    rng = np.random.default_rng(3)
    for L in [1, 2, 17, 300]:
        w = oracle.softmax_weights(rng.standard_normal(64), rng.standard_normal((L, 64)) * 3, 0.125)
        assert abs(w.sum() - 1.0) < 1e-13
        assert np.all(w > 0)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    K = rng.standard_normal((1, 2, 64)).astype(np.float32)
    V = rng.standard_normal((1, 2, 64)).astype(np.float32)
    o = oracle.decode_attention_contiguous(q, K, V, 0.125)
    for h in range(4):
        assert np.array_equal(o[h], V[0, h // 2].astype(np.float64))


def test_zero_query_and_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((23, 2, 16))
    V = rng.standard_normal((23, 2, 8))
    o = oracle.decode_attention_contiguous(np.zeros((4, 16)), K, V, 0.3)
    for h in range(4):
        assert np.allclose(o[h], V[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)
    Keq = np.repeat(rng.standard_normal((1, 2, 16)), 23, axis=0)
    o2 = oracle.decode_attention_contiguous(rng.standard_normal((4, 16)), Keq, V, 0.3)
    for h in range(4):
        assert np.allclose(o2[h], V[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_empty_context_gives_zeros():
    o = oracle.decode_attention_contiguous(np.ones((4, 8)), np.zeros((0, 2, 8)),
                                           np.zeros((0, 2, 5)), 1.0)
    assert o.shape == (4, 5) and np.all(o == 0)


@pytest.mark.parametrize("n_h,n_kv", [(4, 2), (8, 1), (6, 6), (64, 8)])
def test_matches_torch_sdpa_with_repeated_kv_heads(n_h, n_kv):
    """GQA reduces to ordinary attention with each KV head repeated g times
    (torch's CPU float64 scaled_dot_product_attention as the library
    routine)."""
    rng = np.random.default_rng(n_h * 10 + n_kv)
    L, d = 41, 32
    q = rng.standard_normal((n_h, d))
    K = rng.standard_normal((L, n_kv, d))
    V = rng.standard_normal((L, n_kv, d))
    g = n_h // n_kv
    tq = torch.from_numpy(q)[:, None, :]                                  # [n_h, 1, d]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)  # [n_h, L, d]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.contiguous(), tv.contiguous(), scale=0.2)[:, 0, :].numpy()
    got = oracle.decode_attention_contiguous(q, K, V, 0.2)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_gqa_equals_mha_with_replicated_heads():
    rng = np.random.default_rng(8)
    n_h, n_kv, L, d = 8, 2, 19, 16
    q = rng.standard_normal((n_h, d))
    K = rng.standard_normal((L, n_kv, d))
    V = rng.standard_normal((L, n_kv, d))
    g = n_h // n_kv
    Kr = np.repeat(K, g, axis=1)
    Vr = np.repeat(V, g, axis=1)
    assert np.array_equal(oracle.decode_attention_contiguous(q, K, V, 0.25),
                          oracle.decode_attention_contiguous(q, Kr, Vr, 0.25))


def test_kv_head_choice_is_contiguous_groups():
    """Query heads 0..g-1 read KV head 0: make KV head 1 poisonous and check
    the first group is unaffected, the second is NaN."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((5, 2, 8))
    V = rng.standard_normal((5, 2, 8))
    V[:, 1] = np.nan
    o = oracle.decode_attention_contiguous(q, K, V, 0.5)
    assert np.all(np.isfinite(o[:2])) and np.all(np.isnan(o[2:]))


@settings(max_examples=30, deadline=None)
@given(st.lists(st.integers(1, 60), min_size=1, max_size=3), st.integers(0, 2**31 - 1))
def test_block_size_and_physical_permutation_do_not_matter(ctxs, seed):
    rng = np.random.default_rng(seed)
    n_h, n_kv, d = 4, 2, 8
    Ks = [rng.standard_normal((c, n_kv, d)) for c in ctxs]
    Vs = [rng.standard_normal((c, n_kv, d)) for c in ctxs]
    q = rng.standard_normal((len(ctxs), n_h, d))
    ref = np.stack([oracle.decode_attention_contiguous(q[b], Ks[b], Vs[b], 0.3)
                    for b in range(len(ctxs))])
    for bs in (1, 16):
        kp, vp, s = _paged_from_contiguous(Ks, Vs, ctxs, bs, seed + bs)
        out = oracle.paged_decode_attention(q, kp, vp, s.block_table, s.context_lens, 0.3)
        assert np.array_equal(out, ref)
        # relabel physical blocks by a permutation pi: pool'[pi(p)] = pool[p]
        pi = rng.permutation(kp.shape[0])
        kp2 = np.empty_like(kp)
        vp2 = np.empty_like(vp)
        kp2[pi] = kp
        vp2[pi] = vp
        bt2 = np.where(s.block_table >= 0, pi[np.maximum(s.block_table, 0)], -1)
        out2 = oracle.paged_decode_attention(q, kp2, vp2, bt2, s.context_lens, 0.3)
        assert np.array_equal(out2, ref)


def test_partial_tail_block_is_never_read():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((37, 2, 8))
    V = rng.standard_normal((37, 2, 8))
    kp, vp, s = _paged_from_contiguous([K], [V], [37], 16, 1)
    q = rng.standard_normal((1, 4, 8))
    out = oracle.paged_decode_attention(q, kp, vp, s.block_table, s.context_lens, 0.3)
    assert np.all(np.isfinite(out))     # positions 37..47 of the tail block hold NaN


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 200), st.integers(1, 7), st.integers(0, 2**31 - 1))
def test_split_merge_identity(L, nsplit, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(16)
    K = rng.standard_normal((L, 16)) * 2
    V = rng.standard_normal((L, 5))
    cuts = sorted(rng.integers(0, L + 1, size=nsplit - 1).tolist())
    bounds = list(zip([0] + cuts, cuts + [L]))
    merged = oracle.merge_partials(oracle.split_partials(q, K, V, 0.4, bounds))
    full = oracle.softmax_weights(q, K, 0.4) @ V
    assert np.max(np.abs(merged - full)) < 1e-13


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x4049, 0x0001], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 0.0
    assert np.signbit(got[3]) and got[3] == 0.0
    assert np.isinf(got[4])
    assert got[5] == 3.140625                       # 0x4049: 1.5703125 * 2
    assert got[6] == 2.0 ** -133                    # smallest bf16 subnormal
    t = torch.tensor([1.7, -2.3e-5, 3.0e30], dtype=torch.bfloat16)
    b = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.widen(b), t.to(torch.float64).numpy())
