"""GPU parity of the INT4 cache with an attention sink (guijiagi 4.2, 4-bit
branch; 4.3, the first tokens kept unquantized): quantize-on-write codes and
scales bit-exact against the oracle's fp32 quantizer and nibble packing,
and decode against the oracle's attention over the mixed cache (sink rows
exact, the rest dequantized), within 2e-2 (bf16 q), every output element."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import custom_structure, prefill_tokens

from parity_support import TOL_BF16, host, max_err, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _int4_case(s, n_kv, bs, seed, src_dtype=torch.bfloat16):
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, 128, 128, pk.INT4)
    pool.storage.fill_(0xFF)                       # NaN scales wherever nothing is written
    seq, pos = prefill_tokens(s.context_lens)
    bt, ctx = tables_to_device(s)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
    rows = device_normal_(torch.empty((2, len(seq), n_kv, 128), dtype=src_dtype, device="cuda"), seed)
    pk.reshape_and_cache(pool, rows[0], rows[1], slots)
    return pool, rows, slots, bt, ctx


@pytest.mark.parametrize("src", [torch.bfloat16, torch.float32])
def test_int4_quantize_on_write_bit_exact(src):
    s = custom_structure([3, 17, 100, 1], 16, seed=4, pad_blocks=1)
    pool, rows, slots, _, _ = _int4_case(s, 2, 16, 5, src)
    torch.cuda.synchronize()
    x = host(rows) if src == torch.bfloat16 else rows.cpu().numpy()
    sl = slots.cpu().numpy()
    kc, kscale = oracle.quantize_int4_rows(x[0])
    vc, vscale = oracle.quantize_int4_rows(x[1])
    want_k = oracle.pack_int4(kc)
    want_v = oracle.pack_int4(vc)
    got_k, got_v = pool.k.cpu().numpy(), pool.v.cpu().numpy()
    ks, vs = pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy()
    bs = 16
    for t, slot in enumerate(sl):
        blk, off = slot // bs, slot % bs
        assert np.array_equal(got_k[blk, off], want_k[t]) and np.array_equal(got_v[blk, off], want_v[t]), t
        for h in range(2):
            assert ks[blk, h, off].view(np.uint32) == kscale[t, h].view(np.uint32)
            assert vs[blk, h, off].view(np.uint32) == vscale[t, h].view(np.uint32)
    # every byte no token owns is untouched
    owned = np.zeros(s.num_blocks * bs, dtype=bool)
    owned[sl] = True
    assert np.all(got_k.reshape(s.num_blocks * bs, -1)[~owned] == 0xFF)


def _sinks(s, rows, n_sink, n_kv, seed):
    """Sink rows: the unquantized K/V of each sequence's first n_sink tokens
    (the rows that were quantized into the pool), as bf16."""
    B = len(s.context_lens)
    sk = torch.zeros((B, n_sink, n_kv, 128), dtype=torch.bfloat16, device="cuda")
    sv = torch.zeros_like(sk)
    start = 0
    for b, c in enumerate(s.context_lens):
        n = min(int(c), n_sink)
        sk[b, :n] = rows[0, start:start + n].to(torch.bfloat16)
        sv[b, :n] = rows[1, start:start + n].to(torch.bfloat16)
        start += int(c)
    return sk, sv


CTXS = [1, 2, 3, 4, 5, 16, 17, 33, 300, 1000, 2049, 0, 7000, 64]


@pytest.mark.parametrize("g,n_kv", [(8, 2), (4, 8), (8, 8), (16, 2)])
@pytest.mark.parametrize("bs", [16, 64, 1])
@pytest.mark.parametrize("n_sink", [0, 4, 16])
@pytest.mark.parametrize("grid", ["split", "compact", "forced"])
def test_int4_decode_with_sink(g, n_kv, bs, n_sink, grid):
    s = custom_structure(CTXS, bs, seed=g + bs + n_sink, pad_blocks=1)
    pool, rows, _, bt, ctx = _int4_case(s, n_kv, bs, 60 + g + n_sink)
    sk, sv = _sinks(s, rows, n_sink, n_kv, 0) if n_sink else (None, None)
    B = len(CTXS)
    q = device_normal_(torch.empty((B, g * n_kv, 128), dtype=torch.bfloat16, device="cuda"), 61 + bs)
    scale = 1.0 / math.sqrt(128.0)
    kw = dict(max_context_len=max(CTXS))
    if grid == "compact":
        kw["total_context_len"] = int(sum(CTXS))
    if grid == "forced":
        kw["split_tokens"] = 256
    out = pk.paged_decode_attention_int4(q, pool.k, pool.k_scale, pool.v, pool.v_scale, sk, sv, bt, ctx, scale, **kw)
    torch.cuda.synchronize()
    sk_h = host(sk) if n_sink else np.zeros((B, 0, n_kv, 128), dtype=np.uint16)
    sv_h = host(sv) if n_sink else np.zeros((B, 0, n_kv, 128), dtype=np.uint16)
    ref = oracle.paged_decode_attention_int4(host(q), pool.k.cpu().numpy(), pool.k_scale.cpu().numpy(),
                                             pool.v.cpu().numpy(), pool.v_scale.cpu().numpy(), sk_h, sv_h,
                                             s.block_table, s.context_lens, scale)
    assert max_err(out, ref) <= TOL_BF16
    assert torch.count_nonzero(out[11]) == 0


def test_int4_full_size_skewed_batch():
    """The INT8 workload's shape (B=32, n_h 64, n_kv 8, contexts log-uniform
    in [50, 32768]) on an INT4 cache with a 4-token sink, on the compact
    grid the bench times: every output element against the oracle."""
    cfg = CONFIGS["int8_70b"]
    s = structure(cfg)
    pool, rows, _, bt, ctx = _int4_case(s, cfg.n_kv, cfg.block_size, 90)
    sk, sv = _sinks(s, rows, 4, cfg.n_kv, 0)
    del rows
    q = device_normal_(torch.empty((cfg.B, cfg.n_h, 128), dtype=torch.bfloat16, device="cuda"), 91)
    out = pk.paged_decode_attention_int4(q, pool.k, pool.k_scale, pool.v, pool.v_scale, sk, sv, bt, ctx, cfg.scale,
                                         max_context_len=s.max_context_len,
                                         total_context_len=int(s.context_lens.sum()))
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention_int4(host(q), pool.k.cpu().numpy(), pool.k_scale.cpu().numpy(),
                                             pool.v.cpu().numpy(), pool.v_scale.cpu().numpy(), host(sk), host(sv),
                                             s.block_table, s.context_lens, cfg.scale)
    assert max_err(out, ref) <= TOL_BF16


def test_int4_unsupported_uses_are_refused():
    s = custom_structure([10, 20], 16, seed=1)
    bt, ctx = tables_to_device(s)
    pool = pk.kv_pool_create(s.num_blocks, 16, 2, 128, 128, pk.INT4)
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((2, 2, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pk.PagedKVError) as ei:                       # append: INT4 decodes through its own call
        pk.paged_decode_attention_append(pool, q, kv[0], kv[1], bt, ctx, 0.1, max_context_len=20)
    assert ei.value.status == pk.KVP_ERR_UNSUPPORTED
    desc = pk.make_desc(B=2, n_h=16, n_kv=2, d_k=128, d_v=128, block_size=16, max_blocks_per_seq=s.max_blocks_per_seq,
                        max_context_len=20, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_INT4, window=8)
    out = torch.empty((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    rc = pk.lib().paged_decode_attention_int4(pk._ptr(q), pk._ptr(pool.k), pk._ptr(pool.k_scale), pk._ptr(pool.v),
                                              pk._ptr(pool.v_scale), None, None, 0, pk._ptr(bt), pk._ptr(ctx),
                                              pk.ctypes.c_float(0.1), pk._ptr(out), pk.ctypes.byref(desc), None, 0, None)
    assert rc == pk.KVP_ERR_UNSUPPORTED                               # no sliding window on INT4
    desc.window = 0
    rc = pk.lib().paged_decode_attention_int4(pk._ptr(q), pk._ptr(pool.k), pk._ptr(pool.k_scale), pk._ptr(pool.v),
                                              pk._ptr(pool.v_scale), None, None, 65, pk._ptr(bt), pk._ptr(ctx),
                                              pk.ctypes.c_float(0.1), pk._ptr(out), pk.ctypes.byref(desc), None, 0, None)
    assert rc == pk.KVP_ERR_INVALID_ARG                               # n_sink above 64
