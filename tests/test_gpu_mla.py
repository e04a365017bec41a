"""GPU parity of absorbed MLA decode (matrix-core kernel) against the fp64
oracle.

The latent pool holds one 576-wide bf16 row ``[c (512) | k_rope (64)]`` per
token; the value is the first 512 columns of the same row.  The kernel cuts
the batch's context into 32-token tiles shared out to persistent
workgroups; sequences cut between workgroups are merged by log-sum-exp.
Tolerance: max |gpu - oracle| <= 2e-2 (bf16 inputs).  Slots no token owns
hold NaN, so a read past a context length shows up in the output.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure, device_normal_
from synth.workloads import custom_structure

from parity_support import TOL_BF16, host, max_err, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")

D_K, D_V = 576, 512


def _latent_case(s, bs, n_h, seed, poison=True):
    B = len(s.context_lens)
    pool = pk.kv_pool_create(s.num_blocks, bs, 1, D_K, D_V, torch.bfloat16, latent=True)
    device_normal_(pool.k, seed)
    if poison:
        poison_unowned_(pool.k, owned_slots(s.block_table, s.context_lens, bs))
    q = device_normal_(torch.empty((B, n_h, D_K), dtype=torch.bfloat16, device="cuda"), seed + 1)
    return pool, q


def _mla(pool, q, bt, ctx, s, scale, **kw):
    return pk.paged_decode_attention_mla(q, pool.k, bt, ctx, scale, D_V,
                                         max_context_len=s.max_context_len, **kw)


def _oracle(q, pool, s, scale, rows=None):
    qh, kh = host(q), host(pool.k)
    if rows is None:
        return oracle.paged_decode_attention_mla(qh, kh, s.block_table, s.context_lens, scale, D_V)
    return np.stack([oracle.paged_decode_attention_mla(qh[b:b + 1], kh, s.block_table[b:b + 1],
                                                       s.context_lens[b:b + 1], scale, D_V)[0]
                     for b in rows])


RAGGED = [1, 31, 32, 33, 0, 64, 65, 100, 257, 2]


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("n_h", [128, 16, 160, 19])
@pytest.mark.parametrize("workgroups", [0, 1, 3, 7])
def test_mla_ragged_against_oracle(bs, n_h, workgroups):
    s = custom_structure(RAGGED, bs, seed=bs + n_h + workgroups, pad_blocks=1)
    pool, q = _latent_case(s, bs, n_h, seed=100 + n_h + workgroups)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(192.0)
    out = _mla(pool, q, bt, ctx, s, scale, workgroups=workgroups)
    torch.cuda.synchronize()
    ref = _oracle(q, pool, s, scale)
    err = max_err(out, ref)
    assert err <= TOL_BF16, err
    # the empty sequence gives zeros
    assert torch.count_nonzero(out[4]) == 0


@pytest.mark.parametrize("scale", [-1.0 / math.sqrt(192.0), 0.0])
def test_mla_negative_and_zero_scale(scale):
    """The softmax takes scale * q.k for any finite scale: a negative scale
    favours the lowest scores, a zero scale averages the context."""
    s = custom_structure([1, 31, 32, 33, 100, 257], 64, seed=23)
    pool, q = _latent_case(s, 64, 128, seed=24)
    bt, ctx = tables_to_device(s)
    out = _mla(pool, q, bt, ctx, s, scale, workgroups=3)
    torch.cuda.synchronize()
    assert max_err(out, _oracle(q, pool, s, scale)) <= TOL_BF16


def test_mla_single_token_returns_latent_values_exactly():
    """One context token: its weight is exactly 1, so the output is the
    first 512 columns of its latent row, bit for bit."""
    s = custom_structure([1, 1, 1], 64, seed=5)
    pool, q = _latent_case(s, 64, 128, seed=9)
    bt, ctx = tables_to_device(s)
    out = _mla(pool, q, bt, ctx, s, 0.07, workgroups=2)
    torch.cuda.synchronize()
    o, k = host(out), host(pool.k)
    for b in range(3):
        row = k[s.block_table[b, 0], 0, 0, :D_V]
        assert np.array_equal(o[b], np.broadcast_to(row, (128, D_V))), b


def test_mla_workgroup_count_invariance():
    """The result does not depend on how the tiles are shared out (up to
    fp32 summation order), and a repeated call gives the same bits."""
    ctxs = [700, 33, 1500, 64, 999, 1]
    s = custom_structure(ctxs, 64, seed=11)
    pool, q = _latent_case(s, 64, 128, seed=12)
    bt, ctx = tables_to_device(s)
    scale = 1.0 / math.sqrt(192.0)
    outs = [_mla(pool, q, bt, ctx, s, scale, workgroups=w).float() for w in (1, 5, 17, 0, 200)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) <= TOL_BF16
    again = _mla(pool, q, bt, ctx, s, scale, workgroups=17).float()
    assert torch.equal(again, outs[2])
    ref = _oracle(q, pool, s, scale)
    assert max_err(outs[3].to(torch.bfloat16), ref) <= TOL_BF16


def test_mla_full_size_every_sequence():
    """The MLA workload at full size (B=64, n_h=128, contexts uniform in
    [1024, 8192], block 64, permuted blocks) in the launch configuration the
    bench times (one persistent workgroup per compute unit); every output
    element of all 64 sequences against the oracle."""
    cfg = CONFIGS["mla"]
    s = structure(cfg)
    pool, q = _latent_case(s, cfg.block_size, cfg.n_h, seed=cfg.seed)
    bt, ctx = tables_to_device(s)
    out = _mla(pool, q, bt, ctx, s, cfg.scale, total_context_len=int(s.context_lens.sum()))
    torch.cuda.synchronize()
    ref = _oracle(q, pool, s, cfg.scale)
    assert ref.shape == (cfg.B, cfg.n_h, D_V)
    assert max_err(out, ref) <= TOL_BF16


@pytest.mark.parametrize("B", [1300, 4096])
def test_mla_large_batch_of_short_contexts(B):
    """Batches past 512 sequences (each of the 512 threads of the tile-prefix
    scan sums several sequences' tile counts; 4096 is the largest batch),
    contexts of 0 to 80 tokens with empty sequences among them, block 16:
    every output row against the oracle, empty sequences zero."""
    rng = np.random.default_rng(B)
    ctxs = rng.integers(0, 81, B)
    ctxs[::97] = 0
    s = custom_structure(list(ctxs), 16, seed=B + 1, pad_blocks=1)
    pool, q = _latent_case(s, 16, 16, seed=B + 2)
    bt, ctx = tables_to_device(s)
    out = _mla(pool, q, bt, ctx, s, 0.07, total_context_len=int(ctxs.sum()))
    torch.cuda.synchronize()
    assert max_err(out, _oracle(q, pool, s, 0.07)) <= TOL_BF16
    assert torch.count_nonzero(out[::97]) == 0
