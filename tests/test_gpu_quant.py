"""GPU parity of quantize-on-write over row widths and sources (guijiagi 4.2,
8-bit and 4-bit branches): codes and scales bit-exact against the oracle's
binary32 quantizer at every written slot, for widths the vectorised
quantizer takes (64 ... 512) and the per-row one (32, 96), with rows of one
wavefront spanning several tokens (n_kv = 3), a ragged tail, all-zero,
tiny and exact-quotient rows, and tokens whose slot is -1 (nothing written)."""

import numpy as np
import pytest
import torch

import oracle
from synth import host_normal
from synth.workloads import custom_structure, prefill_tokens

from parity_support import device_from_host, host

pytestmark = pytest.mark.gpu

pk = pytest.importorskip("pagedattention_decode_paged_amd")


@pytest.mark.parametrize("kind", ["int8", "int4"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256, 512])
def test_quantize_on_write_bit_exact(kind, src, d):
    rng = np.random.default_rng(1000 + d)
    bs, n_kv = 16, 3
    s = custom_structure([37, 1, 20, 5], bs, seed=d, pad_blocks=1)
    seq, pos = prefill_tokens(s.context_lens)
    T = len(seq)
    k_new = host_normal(rng, (T, n_kv, d), src)
    v_new = host_normal(rng, (T, n_kv, d), src)
    zero = np.uint16(0) if src == "bf16" else np.float32(0.0)
    k_new[0, 0] = zero                                      # an all-zero row
    if src == "f32":
        k_new[1, 1] *= np.float32(1e-30)                    # tiny values
        v_new[2, 2, :] = np.float32(7.0)
        v_new[2, 2, 5] = np.float32(-127.0)                 # exact quotients
    ref_slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    slots = ref_slots.copy()
    dropped = [3, T - 1]
    slots[dropped] = -1                                     # tokens that write nothing
    pool = pk.kv_pool_create(s.num_blocks, bs, n_kv, d, d, torch.int8 if kind == "int8" else pk.INT4)
    pool.storage.fill_(0x5A)
    pk.reshape_and_cache(pool, device_from_host(k_new), device_from_host(v_new),
                         torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    keep = np.ones(T, dtype=bool)
    keep[dropped] = False
    for new, codes_t, scales_t in [(k_new, pool.k, pool.k_scale), (v_new, pool.v, pool.v_scale)]:
        if kind == "int8":
            c_ref, s_ref = oracle.quantize_int8_rows(new)
            width = d
        else:
            c4, s_ref = oracle.quantize_int4_rows(new)
            c_ref = oracle.pack_int4(c4)
            width = d // 2
        codes = codes_t.cpu().numpy().reshape(-1, n_kv, width)
        scales = scales_t.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_kv)   # [NB, n_kv, bs] -> per slot
        assert np.array_equal(codes[ref_slots[keep]], c_ref[keep])
        assert np.array_equal(scales[ref_slots[keep]].view(np.uint32), s_ref[keep].view(np.uint32))
        # the dropped tokens' slots keep the fill
        assert np.all(codes[ref_slots[dropped]].view(np.uint8) == 0x5A)
        assert np.all(scales[ref_slots[dropped]].view(np.uint32) == 0x5A5A5A5A)
