"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any GPU work."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

pk = pytest.importorskip("pagedattention_decode_paged_amd",
                         reason="libpagedkv.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in skip})


def test_every_declared_function_is_exported():
    lib = pk.lib()
    declared = _declared_functions()
    assert "paged_decode_attention" in declared and "kv_pool_create" in declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in pagedkv.h but not exported"
    assert set(pk.EXPORTED_SYMBOLS) <= set(declared)


def test_version_and_empty_error():
    assert "gfx950" in pk.version()


def test_pool_sizes():
    # 16 blocks x 16 slots x 2 heads x 64 fp32, K and V, 256-byte aligned regions
    n = pk.kv_pool_required_bytes(16, 16, 2, 64, 64, pk.torch.float32)
    assert n == 2 * 16 * 16 * 2 * 64 * 4
    # INT8 adds fp32 scales per (slot, head) for K and V
    n8 = pk.kv_pool_required_bytes(10, 16, 8, 128, 128, pk.torch.int8)
    codes = 10 * 16 * 8 * 128
    scales = 10 * 16 * 8 * 4
    assert n8 == 2 * codes + 2 * ((scales + 255) // 256 * 256)
    # latent pool: one region
    nl = pk.kv_pool_required_bytes(4, 64, 1, 576, 512, pk.torch.bfloat16, latent=True)
    assert nl == 4 * 64 * 576 * 2
    # INT4: two codes per byte plus the same scales as INT8
    n4 = pk.kv_pool_required_bytes(10, 16, 8, 128, 128, pk.INT4)
    assert n4 == 2 * (codes // 2) + 2 * ((scales + 255) // 256 * 256)
    assert pk.kv_pool_required_bytes(10, 16, 8, 12, 12, pk.INT4) == 0     # d must be a multiple of 8
    # invalid descriptions size to 0
    assert pk.kv_pool_required_bytes(16, 12, 2, 64, 64, pk.torch.float32) == 0   # block not pow2
    assert pk.kv_pool_required_bytes(0, 16, 2, 64, 64, pk.torch.float32) == 0
    assert pk.kv_pool_required_bytes(4, 64, 2, 576, 512, pk.torch.bfloat16, latent=True) == 0


def _desc(**kw):
    base = dict(B=16, n_h=64, n_kv=8, d_k=128, d_v=128, block_size=16, max_blocks_per_seq=512,
                max_context_len=8192, q_dtype=pk.KVP_BF16, kv_dtype=pk.KVP_BF16)
    base.update(kw)
    return pk.make_desc(**base)


def test_split_planning_and_workspace():
    d = _desc()
    split = pk.decode_split_tokens(d)
    assert split % 256 == 0 and 256 <= split <= 2048
    ns = -(-8192 // split)
    ws = pk.decode_workspace_size(d)
    if ns > 1:
        rows = 16 * 64 * ns
        assert ws >= rows * 128 * 4 + rows * 8
    # one split, no workspace
    d1 = _desc(max_context_len=200, split_tokens=256)
    assert pk.decode_workspace_size(d1) == 0
    # explicit split respected
    d2 = _desc(split_tokens=512)
    assert pk.decode_split_tokens(d2) == 512
    assert pk.decode_workspace_size(d2) == (16 * 64 * 16 * 128 * 4) + (16 * 64 * 16 * 2 * 4)
    # MLA: 32-token tiles shared out to persistent workgroups; never more
    # workgroups than tiles, and a workspace for the per-sequence records
    # plus the partials of (workgroups + B) pieces
    dm = _desc(B=64, n_h=128, n_kv=1, d_k=576, d_v=512, block_size=64, max_blocks_per_seq=128,
               max_context_len=8192)
    assert pk.decode_split_tokens(dm) == 32
    W = pk.decode_mla_workgroups(dm)
    assert 1 <= W <= 64 * 256
    rows = (W + 64) * 128
    # fp32 (max, sum) per head and a bf16 unnormalised output per head
    assert pk.decode_workspace_size(dm) >= 64 * 2 * 4 + rows * 2 * 4 + rows * 512 * 2
    # n_h = 160 launches two groups of 128 heads: the outputs cover both
    dm160 = _desc(B=64, n_h=160, n_kv=1, d_k=576, d_v=512, block_size=64, max_blocks_per_seq=128,
                  max_context_len=8192)
    W160 = pk.decode_mla_workgroups(dm160)
    assert pk.decode_workspace_size(dm160) >= (64 * 2 * 4 + (W160 + 64) * 160 * 2 * 4
                                               + (W160 + 64) * 256 * 512 * 2)
    dm1 = _desc(B=2, n_h=128, n_kv=1, d_k=576, d_v=512, block_size=64, max_blocks_per_seq=1,
                max_context_len=20, workgroups=0)
    assert pk.decode_mla_workgroups(dm1) == 2          # two tiles in the whole batch
    dm2 = _desc(B=2, n_h=128, n_kv=1, d_k=576, d_v=512, block_size=64, max_blocks_per_seq=1,
                max_context_len=20, workgroups=1)
    assert pk.decode_mla_workgroups(dm2) == 1
    assert pk.decode_workspace_size(dm2) == 256        # records only: nothing is cut
    assert pk.decode_mla_workgroups(d) == 0            # not an MLA description


def _call_decode(desc, **ptrs):
    lib = pk.lib()
    P = ctypes.c_void_p
    args = dict(q=P(16), k=P(16), v=P(16), bt=P(16), ctx=P(16), out=P(16))
    args.update(ptrs)
    return lib.paged_decode_attention(args["q"], args["k"], args["v"], args["bt"], args["ctx"],
                                      ctypes.c_float(0.1), args["out"], ctypes.byref(desc),
                                      None, 0, None)


def test_decode_rejects_bad_arguments_on_host():
    lib = pk.lib()
    assert _call_decode(_desc(n_h=63)) == pk.KVP_ERR_INVALID_ARG
    assert b"multiple of n_kv" in lib.kvp_last_error()
    assert _call_decode(_desc(block_size=12)) == pk.KVP_ERR_INVALID_ARG
    assert _call_decode(_desc(max_context_len=512 * 16 + 1)) == pk.KVP_ERR_INVALID_ARG
    assert _call_decode(_desc(split_tokens=300, max_context_len=200)) == pk.KVP_ERR_INVALID_ARG
    assert _call_decode(_desc(max_context_len=200), q=None) == pk.KVP_ERR_INVALID_ARG
    assert _call_decode(_desc(max_context_len=200), q=ctypes.c_void_p(18)) == pk.KVP_ERR_INVALID_ARG
    assert b"aligned" in lib.kvp_last_error()
    # the default split of an 8K context needs a workspace
    assert _call_decode(_desc()) == pk.KVP_ERR_INVALID_ARG
    assert b"workspace" in lib.kvp_last_error()
    # shapes without a kernel
    assert _call_decode(_desc(d_k=96, d_v=96, max_context_len=200)) == pk.KVP_ERR_UNSUPPORTED
    assert _call_decode(_desc(q_dtype=pk.KVP_F32, max_context_len=200)) == pk.KVP_ERR_UNSUPPORTED
    assert _call_decode(_desc(n_h=256, n_kv=8, max_context_len=200)) == pk.KVP_ERR_UNSUPPORTED   # g = 32
    assert (_call_decode(_desc(n_h=128, n_kv=8, kv_dtype=pk.KVP_F32, q_dtype=pk.KVP_F32, d_k=64, d_v=64,
                               max_context_len=200)) == pk.KVP_ERR_UNSUPPORTED)             # fp32, g = 16
    # INT8 pools must go through the INT8 entry point; MLA shapes through MLA
    assert _call_decode(_desc(kv_dtype=pk.KVP_INT8, max_context_len=200)) == pk.KVP_ERR_INVALID_ARG
    assert _call_decode(_desc(n_kv=1, d_k=576, d_v=512, max_context_len=200)) == pk.KVP_ERR_INVALID_ARG
    # B == 0 is a no-op
    assert _call_decode(_desc(B=0)) == pk.KVP_OK


def test_cache_ops_reject_bad_arguments_on_host():
    lib = pk.lib()
    P = ctypes.c_void_p
    assert lib.paged_slot_mapping(P(16), 4, 12, P(16), P(16), 3, P(16), None) == pk.KVP_ERR_INVALID_ARG
    assert lib.paged_slot_mapping(None, 4, 16, P(16), P(16), 3, P(16), None) == pk.KVP_ERR_INVALID_ARG
    assert lib.paged_slot_mapping(None, 4, 16, None, None, 0, None, None) == pk.KVP_OK
    assert lib.reshape_and_cache(None, P(16), P(16), pk.KVP_F32, P(16), 1, None) == pk.KVP_ERR_INVALID_ARG
    assert lib.paged_gather(P(16), 3, 16, 2, 64, P(16), 4, P(16), 2, 50, P(16), None) == pk.KVP_ERR_INVALID_ARG
    assert lib.paged_gather(P(16), 4, 16, 2, 64, P(16), 4, P(16), 2, 65, P(16), None) == pk.KVP_ERR_INVALID_ARG
    assert lib.kv_pool_create(None, None, 0, ctypes.byref(P())) == pk.KVP_ERR_INVALID_ARG


def test_append_rejects_bad_arguments_on_host():
    """paged_decode_attention_append checks the pool against the description
    and its row pointers before any device work (a pool handle over
    caller-given storage touches no device memory)."""
    lib = pk.lib()
    P = ctypes.c_void_p
    pd = pk._PoolDesc(64, 16, 8, 128, 128, pk.KVP_BF16, 0)
    need = lib.kv_pool_required_bytes(ctypes.byref(pd))
    handle = P()
    assert lib.kv_pool_create(ctypes.byref(pd), P(1 << 20), need, ctypes.byref(handle)) == pk.KVP_OK

    def call(desc, pool=handle, k_new=P(4096), v_new=P(4096)):
        return lib.paged_decode_attention_append(pool, P(4096), k_new, v_new, P(4096), P(4096),
                                                 ctypes.c_float(0.1), P(4096), ctypes.byref(desc),
                                                 None, 0, None)
    try:
        good = _desc(max_context_len=200)
        assert call(good, pool=None) == pk.KVP_ERR_INVALID_ARG
        assert b"pool is NULL" in lib.kvp_last_error()
        assert call(_desc(max_context_len=200, d_k=64, d_v=64)) == pk.KVP_ERR_INVALID_ARG
        assert b"differs from desc" in lib.kvp_last_error()
        assert call(good, k_new=None) == pk.KVP_ERR_INVALID_ARG
        assert call(good, v_new=P(4100)) == pk.KVP_ERR_INVALID_ARG
        assert b"16-byte aligned" in lib.kvp_last_error()
        latent = _desc(n_h=16, n_kv=1, d_k=576, d_v=512, max_context_len=200)
        assert call(latent) == pk.KVP_ERR_INVALID_ARG
    finally:
        lib.kv_pool_destroy(handle)


def _r256(n):
    return -(-n // 256) * 256


def test_ragged_planning_with_total_hint():
    """Host planning for ragged batches with a total-context hint (no GPU: the
    library plans for 256 compute units).  bf16, g = 4: the stream grid, two
    workgroups per compute unit over the 4 KV-head pairs (at most one per 256
    tokens of the hint), workspace = pieces (workgroups + B) x heads x
    (d_v + 2) fp32 plus a [B, 2] record.  A forced split leaves the split
    grid.  INT8: the compact split grid, split = the shortest that fits one
    round of two workgroups per compute unit, counting half a partial split
    per sequence and KV-head pair."""
    B, n_h, n_kv, d, mc, total = 32, 32, 8, 128, 4096, 73728
    kw = dict(B=B, n_h=n_h, n_kv=n_kv, max_blocks_per_seq=256, max_context_len=mc)
    d_bf = _desc(total_context_len=total, **kw)
    w = min(2 * 256 // 4, -(-total // 256))
    assert pk.decode_workspace_size(d_bf) == (_r256((w + B) * n_h * d * 4) + _r256((w + B) * n_h * 2 * 4)
                                            + _r256(B * 2 * 4))
    t = (total + 15 * B + w - 1) // w
    assert pk.decode_split_tokens(d_bf) == -(-t // 16) * 16
    d_one = _desc(total_context_len=1, **kw)                   # one workgroup per KV-head pair
    assert pk.decode_workspace_size(d_one) == (_r256((1 + B) * n_h * d * 4) + _r256((1 + B) * n_h * 2 * 4)
                                             + _r256(B * 2 * 4))
    d_forced = _desc(total_context_len=total, split_tokens=512, **kw)
    ns = mc // 512
    assert pk.decode_workspace_size(d_forced) == _r256(B * n_h * ns * d * 4) + _r256(B * n_h * ns * 2 * 4)
    d_q8 = _desc(total_context_len=total, kv_dtype=pk.KVP_INT8, **kw)
    avail = 2 * 256 - ((B + 1) // 2) * (n_kv // 2)
    split = -(-(total * (n_kv // 2)) // avail)
    split = -(-split // 256) * 256
    assert pk.decode_split_tokens(d_q8) == split
    ns = -(-mc // split)
    assert pk.decode_workspace_size(d_q8) == _r256(B * n_h * ns * d * 4) + _r256(B * n_h * ns * 2 * 4)


def test_shared_prefix_planning():
    """The shared-prefix plan on the host (256 compute units without a GPU):
    the 8B-shaped layer with a 2048-token hint takes 11 chunks of 192 tokens,
    two prefix workgroups per chunk (one per KV head of a pair) for its one
    group of 32 sequences, and the stream workgroups fill the rest of one
    round of two per compute unit; the workspace holds the stream pieces
    (workgroups + B) and the prefix pieces (chunks x B).  The hint is
    rounded down to a multiple of 64, and it is ignored (the plain plan) for
    INT8 pools, d = 64 and forced splits."""
    B, n_h, n_kv, mc, total = 32, 32, 8, 4060, 77726
    kw = dict(B=B, n_h=n_h, n_kv=n_kv, max_blocks_per_seq=254, max_context_len=mc, total_context_len=total)
    plain = pk.decode_workspace_size(_desc(**kw))
    for hint, S in ((2048, 2048), (2100, 2048), (5000, 4032)):
        nc = -(-S // 192)
        wgs = 2 * nc
        w = min(2 * 256 // 4 - wgs, -(-total // 256))
        rows = (w + B + nc * B) * n_h
        want = _r256(rows * 128 * 4) + _r256(rows * 8) + _r256(B * 8)
        assert pk.decode_workspace_size(_desc(shared_prefix_tokens=hint, **kw)) == max(plain, want), hint
    assert pk.decode_workspace_size(_desc(shared_prefix_tokens=63, **kw)) == plain
    q8 = dict(kw, kv_dtype=pk.KVP_INT8)
    assert pk.decode_workspace_size(_desc(shared_prefix_tokens=2048, **q8)) == pk.decode_workspace_size(_desc(**q8))
    assert (pk.decode_workspace_size(_desc(shared_prefix_tokens=2048, split_tokens=512, **kw)) ==
            pk.decode_workspace_size(_desc(split_tokens=512, **kw)))
    d64 = dict(kw, d_k=64, d_v=64)
    assert pk.decode_workspace_size(_desc(shared_prefix_tokens=2048, **d64)) == pk.decode_workspace_size(_desc(**d64))
    # g = 16 (128 query heads on 8 KV heads): eight sequences per prefix
    # workgroup, so four sequence groups per chunk and KV head
    g16 = dict(kw, n_h=128)
    nc, ncg = -(-2048 // 192), B // 8
    w = min(2 * 256 // 4 - 2 * nc * ncg, -(-total // 256))
    rows = (w + B + nc * B) * 128
    want = _r256(rows * 128 * 4) + _r256(rows * 8) + _r256(B * 8)
    assert pk.decode_workspace_size(_desc(shared_prefix_tokens=2048, **g16)) == \
        max(pk.decode_workspace_size(_desc(**g16)), want)
    assert _call_decode(_desc(shared_prefix_tokens=-1, max_context_len=200)) == pk.KVP_ERR_INVALID_ARG
