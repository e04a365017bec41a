"""Pins of the oracle's INT8 quantizer, INT8 attention, MLA attention and
closed forms (CPU only)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from synth.workloads import custom_structure, prefill_tokens


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- INT8

def test_int8_hand_rows(golden_dir):
    g = _golden(golden_dir, "int8_hand.json")
    for row in g["rows"]:
        x = np.array(row["x"], dtype=np.float32)[None]
        codes, scale = oracle.quantize_int8_rows(x)
        assert codes[0].tolist() == row["codes"], row["why"]
        if "scale" in row:
            assert scale[0] == np.float32(row["scale"])
        else:
            assert scale[0] == np.float32(np.float32(12.7) / np.float32(127.0))


def _nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded binary32 value of an exact rational (ties to even),
    found by bracketing with nextafter; independent of numpy's division."""
    c = np.float32(float(fr))            # within one ulp of the answer
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        if best is None or err < best[0] or (err == best[0] and
                                            (int(np.float32(cand).view(np.uint32)) & 1) == 0):
            best = (err, cand)
    return np.float32(best[1])


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2**31 - 1), st.sampled_from([1.0, 1e-3, 37.0]))
def test_int8_codes_follow_the_fp32_steps(seed, mag):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 24)) * mag).astype(np.float32)
    codes, scale = oracle.quantize_int8_rows(x)
    for r in range(3):
        a = np.abs(x[r]).max()
        s = _nearest_f32(Fraction(float(a)) / 127)
        assert scale[r] == s
        for d in range(24):
            qt = _nearest_f32(Fraction(float(x[r, d])) / Fraction(float(s)))
            fl = math.floor(Fraction(float(qt)))
            frac = Fraction(float(qt)) - fl
            if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
                fl += 1
            assert codes[r, d] == max(-128, min(127, fl))


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_int8_properties(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((5, 7, 128)).astype(np.float32)
    x[0, 0] = 0.0
    codes, scale = oracle.quantize_int8_rows(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert scale[0, 0] == 0 and np.all(codes[0, 0] == 0)
    nz = scale > 0
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=-1)[nz] == 127)
    err = np.abs(x.astype(np.float64) - oracle.dequantize_int8(codes, scale))
    # rint adds at most 1/2; the binary32 quotient x / scale (|x / scale| <= 128)
    # carries at most half an ulp of 128, i.e. 2^-17, in units of the scale
    bound = scale.astype(np.float64)[..., None] * (0.5 + 2.0 ** -17)
    assert np.all(err <= bound)


def test_int8_accepts_bf16_bits():
    x = np.array([[1.0, -0.5, 0.25]], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    c1, s1 = oracle.quantize_int8_rows(x)
    c2, s2 = oracle.quantize_int8_rows(bits)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_int8_attention_is_attention_over_the_dequantized_cache():
    rng = np.random.default_rng(12)
    ctxs = [5, 33]
    bs, n_kv, d = 16, 2, 16
    s = custom_structure(ctxs, bs, seed=2)
    kx = rng.standard_normal((s.num_blocks, bs, n_kv, d)).astype(np.float32)
    vx = rng.standard_normal((s.num_blocks, bs, n_kv, d)).astype(np.float32)
    kc, ks = oracle.quantize_int8_rows(kx)
    vc, vs = oracle.quantize_int8_rows(vx)
    q = rng.standard_normal((2, 4, d))
    # the pool keeps a block's scales head by head: [NB, n_kv, bs]
    got = oracle.paged_decode_attention_int8(q, kc, ks.transpose(0, 2, 1), vc, vs.transpose(0, 2, 1),
                                             s.block_table, s.context_lens, 0.25)
    # explicit dequantization, then the contiguous definition per sequence
    for b, c in enumerate(ctxs):
        K = np.stack([kc[s.block_table[b, j // bs], j % bs].astype(np.float64)
                      * ks[s.block_table[b, j // bs], j % bs][:, None].astype(np.float64)
                      for j in range(c)])
        V = np.stack([vc[s.block_table[b, j // bs], j % bs].astype(np.float64)
                      * vs[s.block_table[b, j // bs], j % bs][:, None].astype(np.float64)
                      for j in range(c)])
        ref = oracle.decode_attention_contiguous(q[b], K, V, 0.25)
        assert np.max(np.abs(got[b] - ref)) < 1e-14


# ---------------------------------------------------------------- MLA

def test_mla_equals_general_attention_with_copied_values():
    rng = np.random.default_rng(13)
    ctxs, bs, dk, dv, n_h = [3, 70], 64, 24, 16, 8
    s = custom_structure(ctxs, bs, seed=5)
    lat = rng.standard_normal((s.num_blocks, bs, 1, dk))
    q = rng.standard_normal((2, n_h, dk))
    got = oracle.paged_decode_attention_mla(q, lat, s.block_table, s.context_lens, 0.1, dv)
    vpool = lat[..., :dv].copy()
    ref = oracle.paged_decode_attention(q, lat, vpool, s.block_table, s.context_lens, 0.1)
    assert np.array_equal(got, ref)
    # the values really are the first d_v columns: perturbing a rope column
    # changes scores only, perturbing a latent column changes both
    lat2 = lat.copy()
    lat2[..., dv:] = 0.0
    got2 = oracle.paged_decode_attention_mla(q, lat2, s.block_table, s.context_lens, 0.1, dv)
    assert not np.allclose(got2, got)


def test_mla_absorption_identity():
    """faulkner, matrix-absorption section: scoring the cached latent with a
    query that has W^UK folded in, and up-projecting the latent-space output
    with W^UV, equals attention over explicitly up-projected keys/values
    (plus the decoupled rope part shared by all heads)."""
    rng = np.random.default_rng(14)
    d_model, d_c, d_r, d_h, n_h, L = 12, 6, 3, 4, 3, 9
    h_t = rng.standard_normal(d_model)
    W_Q = rng.standard_normal((n_h, d_model, d_h))
    W_UK = rng.standard_normal((n_h, d_c, d_h))
    W_UV = rng.standard_normal((n_h, d_c, d_h))
    q_rope = rng.standard_normal((n_h, d_r))
    c = rng.standard_normal((L, d_c))
    k_rope = rng.standard_normal((L, d_r))
    scale = 1 / math.sqrt(d_h + d_r)
    explicit = np.zeros((n_h, d_h))
    absorbed_q = np.zeros((n_h, d_c + d_r))
    for i in range(n_h):
        q_i = h_t @ W_Q[i]
        k = c @ W_UK[i]
        v = c @ W_UV[i]
        s = scale * (k @ q_i + k_rope @ q_rope[i])
        w = np.exp(s - s.max())
        w /= w.sum()
        explicit[i] = w @ v
        absorbed_q[i, :d_c] = h_t @ (W_Q[i] @ W_UK[i].T)
        absorbed_q[i, d_c:] = q_rope[i]
    latent_rows = np.concatenate([c, k_rope], axis=1)[:, None, :]   # [L, 1, d_c + d_r]
    pool = latent_rows.reshape(L, 1, 1, d_c + d_r)                 # block size 1
    bt = np.arange(L, dtype=np.int32)[None]
    o_lat = oracle.paged_decode_attention_mla(absorbed_q[None], pool, bt,
                                              np.array([L]), scale, d_c)[0]
    up = np.stack([o_lat[i] @ W_UV[i] for i in range(n_h)])
    assert np.max(np.abs(up - explicit)) < 1e-12


# ---------------------------------------------------------------- closed forms

def test_kv_size_closed_form(golden_dir):
    g = _golden(golden_dir, "kv_sizes.json")
    for c in g["cases"]:
        got = oracle.kv_cache_bytes(c["L"], c["n_kv"], c["d_h"], c["S"], c["B"], c["bytes"])
        assert got == c["expected_bytes"], c["cite"]
    for c in g["rounded_cases"]:
        got = oracle.kv_cache_bytes(c["L"], c["n_kv"], c["d_h"], c["S"], c["B"], c["bytes"])
        assert round(got / c["unit"], c["digits"]) == c["printed_gb"], c["cite"]
    # 40 GiB exactly for the 70B-shaped batch
    assert oracle.kv_cache_bytes(80, 8, 128, 8192, 16, 2) == 40 * 2**30
    # INT8 halves it, INT4 quarters it (guijiagi section 2.1 byte sizes)
    assert oracle.kv_cache_bytes(80, 8, 128, 8192, 16, 1) == 20 * 2**30
    assert oracle.kv_cache_bytes(80, 8, 128, 8192, 16, 0.5) == 10 * 2**30


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_decode_intensity_tends_to_g(g):
    I = oracle.decode_attention_intensity(g, 8192, 128)
    assert I == pytest.approx(4 * g * 8192 / (4 * 8192 + 2 * g))
    assert abs(I - g) / g < 1e-3
    # and equals FLOPs/bytes counted directly: 2 flops per MAC, QK^T and PV
    flops = 2 * g * 8192 * 128 * 2
    bytes_ = 2 * 8192 * 128 * 2 + g * 128 * 2
    assert I == pytest.approx(flops / bytes_)
