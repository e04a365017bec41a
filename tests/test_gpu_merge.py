"""GPU checks of the split path (qwbw, section 8 Q2: a long context is cut
into splits whose partial softmax states are merged by log-sum-exp) under
the conditions a serving loop creates: a workspace holding anything (never
cleared), repeated calls on one workspace, and a captured graph replayed
with eager calls on the same workspace in between.  Every result must be
the oracle's (max |gpu - oracle| <= 2e-2, bf16) and the same bits every
time."""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import device_normal_
from synth.workloads import custom_structure

from parity_support import TOL_BF16, host, max_err, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")

CTXS = [0, 1, 513, 1000, 5000, 8192, 4096, 17]


def _case(g, n_kv, kind, seed):
    bs, d = 16, 128
    s = custom_structure(CTXS, bs, seed=seed, pad_blocks=1)
    bt, ctx = tables_to_device(s)
    q = device_normal_(torch.empty((len(CTXS), g * n_kv, d), dtype=torch.bfloat16, device="cuda"), seed + 1)
    if kind == "bf16":
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.bfloat16)
        device_normal_(pool.storage.view(torch.bfloat16), seed)
        owned = owned_slots(s.block_table, s.context_lens, bs)
        poison_unowned_(pool.k, owned)
        poison_unowned_(pool.v, owned)
    else:
        from synth.workloads import prefill_tokens
        pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
        pool.storage.zero_()                       # slots no token owns: codes and scales 0
        seq, pos = prefill_tokens(s.context_lens)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        rows = device_normal_(torch.empty((2, len(seq), n_kv, d), dtype=torch.bfloat16, device="cuda"), seed + 2)
        pk.reshape_and_cache(pool, rows[0], rows[1], slots)
    return s, bt, ctx, q, pool


def _call(kind, q, pool, bt, ctx, scale, out, ws, split):
    kw = dict(max_context_len=max(CTXS), split_tokens=split, workspace=ws)
    if kind == "bf16":
        return pk.paged_decode_attention(q, pool.k, pool.v, bt, ctx, scale, out, **kw)
    return pk.paged_decode_attention_int8(q, pool.k, pool.k_scale, pool.v, pool.v_scale, bt, ctx, scale, out, **kw)


def _ref(kind, s, q, pool, scale):
    if kind == "bf16":
        return oracle.paged_decode_attention(host(q), host(pool.k), host(pool.v), s.block_table, s.context_lens,
                                             scale)
    return oracle.paged_decode_attention_int8(host(q), host(pool.k), host(pool.k_scale), host(pool.v),
                                              host(pool.v_scale), s.block_table, s.context_lens, scale)


@pytest.mark.parametrize("kind,g,n_kv,split", [("bf16", 8, 8, 512), ("bf16", 4, 2, 256), ("int8", 8, 4, 1024),
                                                ("int8", 16, 2, 256)])
def test_merge_with_a_never_cleared_workspace_and_repeated_calls(kind, g, n_kv, split):
    s, bt, ctx, q, pool = _case(g, n_kv, kind, 40 + g + n_kv)
    scale = 1.0 / math.sqrt(128)
    desc = pk.make_desc(B=len(CTXS), n_h=g * n_kv, n_kv=n_kv, d_k=128, d_v=128, block_size=16,
                        max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=max(CTXS),
                        q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16 if kind == "bf16" else pk.KVP_INT8,
                        split_tokens=split)
    ws = torch.randint(0, 256, (pk.decode_workspace_size(desc),), dtype=torch.uint8, device="cuda")
    out = torch.empty((len(CTXS), g * n_kv, 128), dtype=torch.bfloat16, device="cuda")
    ref = _ref(kind, s, q, pool, scale)
    first = None
    for _ in range(3):
        out.fill_(float("nan"))
        _call(kind, q, pool, bt, ctx, scale, out, ws, split)
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL_BF16
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int16), first.view(torch.int16))


def test_merge_under_graph_replay():
    """One captured call (decode kernel and split reduce) replayed four
    times, eager calls on the same workspace in between: every replay equals
    the eager result bit for bit."""
    s, bt, ctx, q, pool = _case(8, 8, "bf16", 61)
    scale = 1.0 / math.sqrt(128)
    desc = pk.make_desc(B=len(CTXS), n_h=64, n_kv=8, d_k=128, d_v=128, block_size=16,
                        max_blocks_per_seq=s.max_blocks_per_seq, max_context_len=max(CTXS),
                        q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, split_tokens=512)
    ws = torch.zeros(pk.decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    eager = torch.empty((len(CTXS), 64, 128), dtype=torch.bfloat16, device="cuda")
    _call("bf16", q, pool, bt, ctx, scale, eager, ws, 512)
    torch.cuda.synchronize()
    assert max_err(eager, _ref("bf16", s, q, pool, scale)) <= TOL_BF16
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _call("bf16", q, pool, bt, ctx, scale, out, ws, 512)          # warm on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call("bf16", q, pool, bt, ctx, scale, out, ws, 512)
    for _ in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
        other = torch.empty_like(eager)
        _call("bf16", q, pool, bt, ctx, scale, other, ws, 512)    # an eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))
