"""GPU parity of the cache-side kernels: slot mapping, reshape_and_cache (bit
copy and INT8 quantize-on-write) and the block-table gather, against the
oracle, bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, structure
from synth.workloads import custom_structure, prefill_tokens, decode_positions

from parity_support import host, device_from_host, owned_slots, poison_unowned_, tables_to_device

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


def _slots_gpu(bt_np, seq, pos, bs):
    return pk.paged_slot_mapping(torch.from_numpy(bt_np).cuda(), torch.from_numpy(seq).cuda(),
                                 torch.from_numpy(pos).cuda(), bs)


@pytest.mark.parametrize("name", ["tiny", "llama8b", "int8_70b", "mla"])
def test_slot_mapping_matches_oracle(name):
    cfg = CONFIGS[name]
    s = structure(cfg)
    seq, pos = prefill_tokens(s.context_lens)
    got = _slots_gpu(s.block_table, seq, pos, cfg.block_size).cpu().numpy()
    ref = oracle.slot_mapping(s.block_table, seq, pos, cfg.block_size)
    assert np.array_equal(got, ref)


def test_slot_mapping_marks_invalid_tokens():
    bt = np.array([[3, 7, 1, 12], [5, -1, -1, -1]], dtype=np.int32)
    seq = np.array([0, 0, 1, 1, -1, 0, 0], dtype=np.int32)
    pos = np.array([49, 0, 3, 16, 2, -4, 64], dtype=np.int32)
    got = _slots_gpu(bt, seq, pos, 16).cpu().numpy()
    assert got.tolist() == [12 * 16 + 1, 3 * 16, 5 * 16 + 3, -1, -1, -1, -1]


def _write_case(dtype, bs, n_kv, d_k, d_v, ctxs, latent=False, seed=0):
    s = custom_structure(ctxs, bs, seed=seed, pad_blocks=1)
    nb = s.num_blocks + 2
    rng = np.random.default_rng(seed)
    pool = pk.kv_pool_create(nb, bs, n_kv, d_k, d_v, dtype, latent=latent)
    pool.storage.fill_(0xFF)                       # NaN bit patterns everywhere
    seq, pos = prefill_tokens(s.context_lens)
    seq = np.concatenate([seq, [0, 0]]).astype(np.int32)      # two padding tokens
    pos = np.concatenate([pos, [-1, -1]]).astype(np.int32)
    T = len(seq)
    kind = "bf16" if dtype == torch.bfloat16 else "f32"
    from parity_support import host_normal
    k_new = host_normal(rng, (T, n_kv, d_k), kind)
    v_new = host_normal(rng, (T, n_kv, d_v), kind)
    slots = _slots_gpu(s.block_table, seq, pos, bs)
    k0, v0 = host(pool.k).copy(), host(pool.v).copy()
    pk.reshape_and_cache(pool, device_from_host(k_new), None if latent else device_from_host(v_new), slots)
    torch.cuda.synchronize()
    ref_slots = oracle.slot_mapping(s.block_table, seq[:-2], pos[:-2], bs)
    ref_slots = np.concatenate([ref_slots, [-1, -1]])
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    k_ref = oracle.reshape_and_cache(k0, k_new, ref_slots)
    assert np.array_equal(host(pool.k).view(np.uint8), k_ref.view(np.uint8))
    if not latent:
        v_ref = oracle.reshape_and_cache(v0, v_new, ref_slots)
        assert np.array_equal(host(pool.v).view(np.uint8), v_ref.view(np.uint8))
    return pool, s


@pytest.mark.parametrize("dtype,bs,n_kv,d", [(torch.float32, 16, 2, 64), (torch.bfloat16, 16, 8, 128),
                                             (torch.bfloat16, 1, 2, 64), (torch.float32, 4, 3, 5)])
def test_reshape_and_cache_bit_exact(dtype, bs, n_kv, d):
    _write_case(dtype, bs, n_kv, d, d, [37, 50, 1, 16])


def test_reshape_and_cache_latent_bit_exact():
    _write_case(torch.bfloat16, 64, 1, 576, 512, [65, 3, 128], latent=True)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_int8_quantize_on_write_bit_exact(src):
    rng = np.random.default_rng(5)
    bs, n_kv, d = 16, 8, 128
    s = custom_structure([37, 20], bs, seed=3)
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8)
    pool.storage.zero_()
    seq, pos = prefill_tokens(s.context_lens)
    T = len(seq)
    from parity_support import host_normal
    k_new = host_normal(rng, (T, n_kv, d), src)
    v_new = host_normal(rng, (T, n_kv, d), src)
    if src == "f32":
        k_new[0, 0] = 0.0                        # an all-zero row
        k_new[1, 1] *= 1e-3
        v_new[2, 3, :] = np.float32(7.0)
        v_new[2, 3, 5] = np.float32(-127.0)       # exact halves/quotients
    slots = _slots_gpu(s.block_table, seq, pos, bs)
    pk.reshape_and_cache(pool, device_from_host(k_new), device_from_host(v_new), slots)
    torch.cuda.synchronize()
    ref_slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    for new, codes_t, scales_t in [(k_new, pool.k, pool.k_scale), (v_new, pool.v, pool.v_scale)]:
        c_ref, s_ref = oracle.quantize_int8_rows(new)
        codes = host(codes_t).reshape(-1, n_kv, d)
        scales = host(scales_t).transpose(0, 2, 1).reshape(-1, n_kv)   # [NB, n_kv, bs] -> per slot
        assert np.array_equal(codes[ref_slots], c_ref)
        assert np.array_equal(scales[ref_slots].view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("dtype,bs", [(torch.bfloat16, 16), (torch.float32, 1), (torch.bfloat16, 64)])
def test_gather_bit_exact(dtype, bs):
    rng = np.random.default_rng(9)
    ctxs = [37, 50, 0, 129]
    s = custom_structure(ctxs, bs, seed=11, pad_blocks=1)
    pool = torch.randn((s.num_blocks + 1, bs, 2, 64), device="cuda").to(dtype)
    bt, ctx = tables_to_device(s)
    out = torch.full((4, 129, 2, 64), float("nan"), device="cuda", dtype=dtype)
    pk.paged_gather(pool, bt, ctx, 129, out=out)
    got = host(out)
    ph = host(pool)
    for b, c in enumerate(ctxs):
        ref = oracle.gather_sequence(ph, s.block_table[b], c)
        assert np.array_equal(got[b, :c].view(np.uint8), np.asarray(ref).view(np.uint8))
        tail = got[b, c:]
        if dtype == torch.float32:
            assert np.all(np.isnan(tail))
        else:
            assert np.all(np.isnan(oracle.widen(tail)))
