"""paged_decode_attention_append_noalloc: the decode step with the library's
static device scratch instead of a caller workspace.

Each case runs two no-allocation calls in a row, the second on a smaller
batch (fewer sequences), and compares each with
paged_decode_attention_append given its own workspace on a twin pool: the
outputs and the pools after the call agree bit for bit (the same kernels in
the same launch shapes), and the first call's output matches the fp64
oracle within the bf16 tolerance.  A description that needs more scratch
than the buffer holds is refused on the host.
"""

import ctypes
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


def _twin_pools(s, bs, n_kv, d_k, d_v, kind, latent, seed):
    dtype = torch.int8 if kind == "int8" else torch.bfloat16
    pa = pk.kv_pool_create(s.num_blocks, bs, n_kv, d_k, d_v, dtype, latent=latent)
    if kind == "int8":
        seq, pos = prefill_tokens(s.context_lens)
        bt, _ = tables_to_device(s)
        slots = pk.paged_slot_mapping(bt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), bs)
        rows = device_normal_(torch.empty((2, len(seq), n_kv, d_k), dtype=torch.bfloat16, device="cuda"), seed)
        pk.reshape_and_cache(pa, rows[0], rows[1], slots)
    else:
        device_normal_(pa.storage.view(torch.bfloat16), seed)
    pb = pk.kv_pool_create(s.num_blocks, bs, n_kv, d_k, d_v, dtype, latent=latent)
    pb.storage.copy_(pa.storage)
    return pa, pb


def _bits(t):
    return t.view(torch.int16)


def _two_calls(kind, s, n_h, n_kv, d_k, d_v, bs, latent, scale, small, seed, hint):
    pa, pb = _twin_pools(s, bs, n_kv, d_k, d_v, kind, latent, seed)
    B = len(s.context_lens)
    bt, ctx = tables_to_device(s)
    q = device_normal_(torch.empty((B, n_h, d_k), dtype=torch.bfloat16, device="cuda"), seed + 1)
    k_new = device_normal_(torch.empty((B, n_kv, d_k), dtype=torch.bfloat16, device="cuda"), seed + 2)
    v_new = None if latent else device_normal_(torch.empty((B, n_kv, d_v), dtype=torch.bfloat16,
                                                           device="cuda"), seed + 3)
    results = []
    for rows in (slice(None), slice(0, small)):
        qq, bb, cc = q[rows].contiguous(), bt[rows].contiguous(), ctx[rows].contiguous()
        kn = k_new[rows].contiguous()
        vn = None if latent else v_new[rows].contiguous()
        c_h = s.context_lens[rows]
        mc = int(c_h.max())
        tot = int(c_h.sum()) if hint else 0
        ref = pk.paged_decode_attention_append(pa, qq, kn, vn, bb, cc, scale, max_context_len=mc,
                                               total_context_len=tot)
        out = torch.full_like(ref, float("nan"))
        pk.paged_decode_attention_append_noalloc(pb, qq, kn, vn, bb, cc, scale, out, max_context_len=mc,
                                                 total_context_len=tot)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ref), _bits(out)), (kind, rows)
        assert torch.equal(pa.storage, pb.storage), (kind, rows)
        results.append((out, qq))
    return pb, results


@pytest.mark.parametrize("kind", ["bf16_stream", "bf16_split", "int8", "mla"])
def test_noalloc_matches_the_workspace_entry_point(kind):
    if kind == "bf16_stream":
        rng = np.random.default_rng(5)
        ctxs = [int(c) for c in rng.integers(512, 4097, size=32)]
        s = custom_structure(ctxs, 16, seed=6, pad_blocks=1)
        args = dict(n_h=32, n_kv=8, d_k=128, d_v=128, bs=16, latent=False, scale=1 / math.sqrt(128),
                    small=9, hint=True)
        k = "bf16"
    elif kind == "bf16_split":
        s = custom_structure([8192] * 4, 16, seed=7)
        args = dict(n_h=64, n_kv=8, d_k=128, d_v=128, bs=16, latent=False, scale=1 / math.sqrt(128),
                    small=2, hint=False)
        k = "bf16"
    elif kind == "int8":
        rng = np.random.default_rng(8)
        ctxs = [int(c) for c in np.clip(np.round(np.exp(rng.uniform(np.log(50), np.log(32768), 16))), 50, 32768)]
        s = custom_structure(ctxs, 16, seed=9, pad_blocks=1)
        args = dict(n_h=64, n_kv=8, d_k=128, d_v=128, bs=16, latent=False, scale=1 / math.sqrt(128),
                    small=5, hint=True)
        k = "int8"
    else:
        cfg = CONFIGS["mla"]
        s = structure(cfg)
        args = dict(n_h=128, n_kv=1, d_k=576, d_v=512, bs=64, latent=True, scale=cfg.scale, small=10,
                    hint=True)
        k = "mla"
    pb, results = _two_calls(k if k != "mla" else "bf16", s, args["n_h"], args["n_kv"], args["d_k"],
                             args["d_v"], args["bs"], args["latent"], args["scale"], args["small"], 40,
                             args["hint"])
    out, q = results[0]
    if k == "mla":
        ref = oracle.paged_decode_attention_mla(host(q), host(pb.k), s.block_table, s.context_lens,
                                                args["scale"], args["d_v"])
    elif k == "int8":
        ref = oracle.paged_decode_attention_int8(host(q), host(pb.k), host(pb.k_scale), host(pb.v),
                                                 host(pb.v_scale), s.block_table, s.context_lens, args["scale"])
    else:
        ref = oracle.paged_decode_attention(host(q), host(pb.k), host(pb.v), s.block_table, s.context_lens,
                                            args["scale"])
    assert max_err(out, ref) <= TOL_BF16


def test_noalloc_refuses_what_the_buffer_cannot_hold():
    """Forced 256-token splits of 4096 sequences of 8192 tokens need 4.4 GB
    of partials: refused on the host with a message, nothing enqueued (the
    pool handle is over caller-given storage that is never touched)."""
    lib = pk.lib()
    P = ctypes.c_void_p
    pd = pk._PoolDesc(64, 16, 8, 128, 128, pk.KVP_BF16, 0)
    need = lib.kv_pool_required_bytes(ctypes.byref(pd))
    handle = P()
    assert lib.kv_pool_create(ctypes.byref(pd), P(1 << 20), need, ctypes.byref(handle)) == pk.KVP_OK
    try:
        desc = pk.make_desc(B=4096, n_h=64, n_kv=8, d_k=128, d_v=128, block_size=16, max_blocks_per_seq=512,
                            max_context_len=8192, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16, split_tokens=256)
        assert pk.decode_workspace_size(desc) > 64 << 20
        rc = lib.paged_decode_attention_append_noalloc(handle, P(4096), P(4096), P(4096), P(4096), P(4096),
                                                       ctypes.c_float(0.1), P(4096), ctypes.byref(desc), None)
        assert rc == pk.KVP_ERR_UNSUPPORTED
        assert b"static buffer holds 67108864" in lib.kvp_last_error()
    finally:
        lib.kv_pool_destroy(handle)
