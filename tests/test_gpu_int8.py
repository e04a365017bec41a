"""GPU parity of the INT8 path: quantize-on-write codes and scales bit-exact
against the oracle's fp32-step quantizer, and decode attention with the
dequantization fused into the kernel against the oracle's attention over the
dequantized cache (bf16 q and output: max abs error <= 2e-2)."""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import custom_structure, prefill_tokens

from parity_support import TOL_BF16, device_from_host, host, max_err, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _int8_case(s, n_h, n_kv, d, seed, src_dtype=torch.bfloat16):
    B = len(s.context_lens)
    bs = int(s.extra.get("bs", 16))
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
    pool.k.fill_(0x55)
    pool.v.fill_(0x55)
    pool.k_scale.fill_(float("nan"))             # a scale no token owns is NaN
    pool.v_scale.fill_(float("nan"))
    seq, pos = prefill_tokens(s.context_lens)
    T = len(seq)
    k_src = device_normal_(torch.empty((T, n_kv, d), dtype=src_dtype, device="cuda"), seed)
    v_src = device_normal_(torch.empty((T, n_kv, d), dtype=src_dtype, device="cuda"), seed + 1)
    q = device_normal_(torch.empty((B, n_h, d), dtype=torch.bfloat16, device="cuda"), seed + 2)
    bt, ctx = tables_to_device(s)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
    pk.reshape_and_cache(pool, k_src, v_src, slots)
    torch.cuda.synchronize()
    ref_slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    # codes and scales bit-exact against the oracle's quantizer
    for src, codes_t, scales_t in [(k_src, pool.k, pool.k_scale), (v_src, pool.v, pool.v_scale)]:
        c_ref, s_ref = oracle.quantize_int8_rows(host(src))
        codes = host(codes_t).reshape(-1, n_kv, d)
        scales = host(scales_t).transpose(0, 2, 1).reshape(-1, n_kv)   # [NB, n_kv, bs] -> per slot
        assert np.array_equal(codes[ref_slots], c_ref)
        assert np.array_equal(scales[ref_slots].view(np.uint32), s_ref.view(np.uint32))
    return pool, q, bt, ctx


def _check_attention(pool, q, bt, ctx, s, scale, **kw):
    out = pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, scale,
                                         max_context_len=s.max_context_len, **kw)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                             host(pool.v_scale), s.block_table, s.context_lens, scale)
    err = max_err(out, ref)
    assert err <= TOL_BF16, err
    return out


def test_int8_70b_full_size():
    cfg = CONFIGS["int8_70b"]
    s = structure(cfg)
    pool, q, bt, ctx = _int8_case(s, cfg.n_h, cfg.n_kv, cfg.d_k, cfg.seed)
    out = _check_attention(pool, q, bt, ctx, s, cfg.scale, total_context_len=int(s.context_lens.sum()))
    # split-count invariance on the skewed contexts
    out2 = pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx,
                                          cfg.scale, max_context_len=s.max_context_len, split_tokens=256)
    torch.cuda.synchronize()
    assert float((out.float() - out2.float()).abs().max()) <= TOL_BF16


@pytest.mark.parametrize("d,g,bs", [(128, 8, 16), (128, 1, 16), (64, 4, 16), (64, 2, 16),
                                    (128, 4, 16), (128, 8, 1), (128, 4, 64), (64, 8, 1), (64, 4, 64),
                                    (128, 16, 16), (128, 16, 1), (64, 16, 16)])
def test_int8_ragged(d, g, bs):
    ctxs = [1, 15, 16, 17, 64, 65, 255, 257, 600]
    s = custom_structure(ctxs, bs, seed=d + g + bs, pad_blocks=1)
    s.extra["bs"] = bs
    n_kv = 2
    pool, q, bt, ctx = _int8_case(s, n_kv * g, n_kv, d, 100 + d + g)
    _check_attention(pool, q, bt, ctx, s, 1.0 / math.sqrt(d))
    # several context splits: the partial merge over the INT8 path
    _check_attention(pool, q, bt, ctx, s, 1.0 / math.sqrt(d), split_tokens=256)


@pytest.mark.parametrize("n_kv,g", [(1, 8), (2, 8), (4, 8), (6, 4), (8, 4), (12, 8), (1, 16), (4, 16)])
def test_int8_kv_head_groups(n_kv, g):
    """INT8 with d = 128 runs four adjacent KV heads per workgroup when n_kv
    is a multiple of 4, two when it is even, else one: all against the oracle
    on the plain grid, with several context splits and on the compact grid."""
    ctxs = [1, 17, 40, 300, 1025, 0, 64]
    s = custom_structure(ctxs, 16, seed=n_kv * 10 + g, pad_blocks=1)
    pool, q, bt, ctx = _int8_case(s, n_kv * g, n_kv, 128, 300 + n_kv + g)
    scale = 1.0 / math.sqrt(128)
    _check_attention(pool, q, bt, ctx, s, scale)
    _check_attention(pool, q, bt, ctx, s, scale, split_tokens=256)
    _check_attention(pool, q, bt, ctx, s, scale, total_context_len=int(s.context_lens.sum()))


def test_int8_from_fp32_rows():
    s = custom_structure([40, 300], 16, seed=4)
    pool, q, bt, ctx = _int8_case(s, 16, 2, 128, 9, src_dtype=torch.float32)
    _check_attention(pool, q, bt, ctx, s, 0.0883)


@pytest.mark.parametrize("d,g", [(128, 8), (128, 4), (64, 8), (128, 16)])
def test_int8_query_outliers(d, g):
    """Queries with outlier channels (every 37th channel 30 times the rest)
    and one head all zero.  The matrix-core INT8 path holds each head's
    query as 8-bit parts under one scale set by its largest channel, so the
    small channels must survive that scale; the outliers also make the
    softmax steep, where a score error shows in the output.  Against the
    oracle on the plain grid and with several context splits."""
    ctxs = [300, 1025, 64, 1]
    s = custom_structure(ctxs, 16, seed=d + g + 5, pad_blocks=1)
    n_kv = 2
    pool, q, bt, ctx = _int8_case(s, n_kv * g, n_kv, d, 500 + d + g)
    qf = q.float()
    qf[:, :, ::37] *= 30.0
    qf[0, 1, :] = 0.0                            # uniform weights for this head
    q = qf.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    _check_attention(pool, q, bt, ctx, s, scale)
    _check_attention(pool, q, bt, ctx, s, scale, split_tokens=256)


@pytest.mark.parametrize("g,bs", [(8, 16), (4, 64)])
def test_int8_scales_not_16_byte_aligned(g, bs):
    """Scale arrays 4- but not 16-byte aligned (the kernel fetches one fp32
    per lane and token): the outputs are bit-identical to those from the
    aligned arrays, with every unowned scale slot NaN.  A scale array that is
    not 4-byte aligned is refused with a message."""
    ctxs = [1, 15, 17, 300, 1025, 64]
    s = custom_structure(ctxs, bs, seed=g + bs, pad_blocks=1)
    s.extra["bs"] = bs
    n_kv, d = 2, 128
    pool, q, bt, ctx = _int8_case(s, n_kv * g, n_kv, d, 900 + g + bs)
    scale = 1.0 / math.sqrt(d)
    out_a = _check_attention(pool, q, bt, ctx, s, scale, total_context_len=int(s.context_lens.sum()))
    outs = {}
    for name, shift in (("aligned", 0), ("offset4", 1)):
        ks = torch.empty(pool.k_scale.numel() + 4, dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        k_sc = ks[shift:shift + pool.k_scale.numel()].view(pool.k_scale.shape)
        v_sc = vs[shift:shift + pool.v_scale.numel()].view(pool.v_scale.shape)
        k_sc.copy_(pool.k_scale)
        v_sc.copy_(pool.v_scale)
        assert (k_sc.data_ptr() % 16 == 0) == (shift == 0)
        for split in (0, 256):
            outs[(name, split)] = pk.paged_decode_attention_int8(
                q, pool.k, k_sc, pool.v, v_sc, bt, ctx, scale, max_context_len=s.max_context_len,
                split_tokens=split, total_context_len=int(s.context_lens.sum()))
    torch.cuda.synchronize()
    assert torch.equal(outs[("aligned", 0)], out_a)
    for split in (0, 256):
        assert torch.equal(outs[("offset4", split)], outs[("aligned", split)])
    raw = torch.empty(pool.k_scale.numel() * 4 + 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(pk.PagedKVError, match="4-byte aligned"):
        pk._check(pk._lib.paged_decode_attention_int8(
            pk._ptr(q), pk._ptr(pool.k), ctypes.c_void_p(raw.data_ptr() + 2), pk._ptr(pool.v),
            pk._ptr(pool.v_scale), pk._ptr(bt), pk._ptr(ctx), ctypes.c_float(scale),
            pk._ptr(torch.empty_like(q)), ctypes.byref(pk.make_desc(
                B=len(ctxs), n_h=n_kv * g, n_kv=n_kv, d_k=d, d_v=d, block_size=bs,
                max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=s.max_context_len,
                q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_INT8)), None, 0, None))
