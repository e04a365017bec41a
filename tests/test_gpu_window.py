"""GPU parity of sliding-window decode (guijiagi 5.1: a sequence attends to
its last `window` positions only) against the fp64 oracle, on bf16 and INT8
pools, on the split, stream and compact grids and through the append entry
point.  Every slot a sequence owns below its window start is NaN, as are the
slots no token owns, so a read of a skipped position shows up in the
output.  Tolerance 2e-2 (bf16 inputs), every output element."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import custom_structure, prefill_tokens

from parity_support import TOL_BF16, host, max_err, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")

CTXS = [0, 1, 15, 16, 17, 100, 255, 256, 257, 700, 1500, 3000, 33, 4100, 64, 999]


def _visible_slots(s, bs, window):
    """Slots of the positions each sequence attends to."""
    seq, pos = [], []
    for b, c in enumerate(s.context_lens):
        lo = oracle.window_start(int(c), window)
        seq.extend([b] * (int(c) - lo))
        pos.extend(range(lo, int(c)))
    return oracle.slot_mapping(s.block_table, np.asarray(seq, dtype=np.int32), np.asarray(pos, dtype=np.int32), bs)


@pytest.mark.parametrize("g,d,bs", [(8, 128, 16), (4, 128, 64), (4, 64, 16), (8, 128, 1), (16, 128, 16)])
@pytest.mark.parametrize("window", [1, 40, 256, 1000, 5000])
@pytest.mark.parametrize("grid", ["split", "stream", "forced"])
def test_window_bf16(g, d, bs, window, grid):
    n_kv = 2
    s = custom_structure(CTXS, bs, seed=g + d + bs, pad_blocks=1)
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
    device_normal_(pool.storage.view(torch.bfloat16), window + g)
    vis = _visible_slots(s, bs, window)
    poison_unowned_(pool.k, vis)
    poison_unowned_(pool.v, vis)
    bt, ctx = tables_to_device(s)
    B = len(CTXS)
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), window + 1)
    scale = 1.0 / math.sqrt(d)
    kw = dict(max_context_len=max(CTXS), window=window)
    if grid == "stream":
        kw["total_context_len"] = int(sum(CTXS))
    if grid == "forced":
        kw["split_tokens"] = 256
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, **kw)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale,
                                        window)
    assert max_err(out, ref) <= TOL_BF16
    assert torch.count_nonzero(out[0]) == 0


@pytest.mark.parametrize("window", [1, 100, 2048])
@pytest.mark.parametrize("hint", [True, False])
@pytest.mark.parametrize("g", [8, 16])
def test_window_int8(window, hint, g):
    n_kv, d, bs = 64 // g, 128, 16
    s = custom_structure(CTXS, bs, seed=window, pad_blocks=1)
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
    seq, pos = prefill_tokens(s.context_lens)
    bt, ctx = tables_to_device(s)
    slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
    rows = device_normal_(torch.empty((2, len(seq), n_kv, d), dtype=torch.bfloat16, device="cuda"), 70 + window)
    pk.reshape_and_cache(pool, rows[0], rows[1], slots)
    # NaN scales at every position outside the windows (never read)
    vis = torch.zeros(s.num_blocks * bs, dtype=torch.bool)
    vis[torch.from_numpy(_visible_slots(s, bs, window))] = True
    hidden = (~vis).view(s.num_blocks, 1, bs).expand(s.num_blocks, n_kv, bs).cuda()
    pool.k_scale[hidden] = float("nan")
    pool.v_scale[hidden] = float("nan")
    B = len(CTXS)
    q = device_normal_(torch.empty((B, g * n_kv, d), dtype=torch.bfloat16, device="cuda"), 71)
    scale = 1.0 / math.sqrt(d)
    out = pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, scale,
                                         max_context_len=max(CTXS), window=window,
                                         total_context_len=int(sum(CTXS)) if hint else 0)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                             host(pool.v_scale), s.block_table, s.context_lens, scale, window)
    assert max_err(out, ref) <= TOL_BF16


def test_window_append_and_full_window_equals_no_window():
    """The append entry point with a window: the new row enters the window;
    a window at least as long as every context gives the same bits as no
    window."""
    n_kv, g, d, bs = 8, 8, 128, 16
    ctxs = [1, 300, 4100, 17]
    s = custom_structure(ctxs, bs, seed=5, pad_blocks=1)
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
    device_normal_(pool.storage.view(torch.bfloat16), 6)
    bt, ctx = tables_to_device(s)
    q = device_normal_(torch.empty((4, 64, d), dtype=torch.bfloat16, device="cuda"), 7)
    kv = device_normal_(torch.empty((2, 4, n_kv, d), dtype=torch.bfloat16, device="cuda"), 8)
    scale = 1.0 / math.sqrt(d)
    out = pk.paged_decode_attention_append(pool, q, kv[0], kv[1], bt, ctx, scale, max_context_len=4100, window=200)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, scale, 200)
    assert max_err(out, ref) <= TOL_BF16
    a = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=4100, window=4100)
    b = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, max_context_len=4100)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_window_full_size_70b_layer():
    """The 70B-shaped layer at full size (B=16, ctx 8192) with a 4096-token
    window: every output element against the oracle."""
    cfg = CONFIGS["llama70b"]
    s = structure(cfg, layer=3)
    pool = pk.kv_pool_create(s.num_blocks, 16, 8, 128, 128, torch.bfloat16)
    device_normal_(pool.k, 30)
    device_normal_(pool.v, 31)
    bt, ctx = tables_to_device(s)
    q = device_normal_(torch.empty((16, 64, 128), dtype=torch.bfloat16, device="cuda"), 32)
    out = pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, cfg.scale, max_context_len=8192, window=4096)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens, cfg.scale,
                                        4096)
    assert max_err(out, ref) <= TOL_BF16


def test_window_unsupported_shapes_are_refused():
    s = custom_structure([10, 20], 16, seed=1)
    bt, ctx = tables_to_device(s)
    k = torch.zeros((s.num_blocks, 16, 2, 64), dtype=torch.float32, device="cuda")
    q = torch.zeros((2, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(pk.PagedKVError) as ei:
        pk.paged_decode_attention(q, k, k, bt, ctx, 0.1, max_context_len=20, window=5)
    assert ei.value.status == pk.KVP_ERR_UNSUPPORTED
    lat = torch.zeros((s.num_blocks, 16, 1, 576), dtype=torch.bfloat16, device="cuda")
    qm = torch.zeros((2, 16, 576), dtype=torch.bfloat16, device="cuda")
    desc = pk.make_desc(B=2, n_h=16, n_kv=1, d_k=576, d_v=512, block_size=16, max_blocks_per_seq=s.max_blocks_per_seq,
                        max_context_len=20, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, window=5)
    ws = pk.alloc_workspace(desc)
    out = torch.empty((2, 16, 512), dtype=torch.bfloat16, device="cuda")
    rc = pk.lib().paged_decode_attention_mla(pk._ptr(qm), pk._ptr(lat), pk._ptr(bt), pk._ptr(ctx), pk.ctypes.c_float(0.1),
                                             pk._ptr(out), pk.ctypes.byref(desc), pk._ptr(ws), ws.numel(), None)
    assert rc == pk.KVP_ERR_UNSUPPORTED
