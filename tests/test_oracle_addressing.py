"""Pins of the oracle's addressing, write and gather against the pages'
worked examples and against structural invariants (CPU only)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from synth import CONFIGS, structure
from synth.workloads import custom_structure, prefill_tokens


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_talentme_write_kv_example(golden_dir):
    g = _load(golden_dir, "talentme_write_kv.json")
    nb, bs, nh, hd = g["num_blocks"], g["block_size"], g["num_heads"], g["head_dim"]
    k_pool = np.zeros((nb, bs, nh, hd), dtype=np.float32)
    v_pool = np.zeros_like(k_pool)
    free = list(range(nb))                         # handed out front first
    table = [free.pop(0) for _ in range(g["blocks_for_request"])]
    assert table == g["expected_block_table"]
    j = g["token_idx"]
    phys, off = oracle.logical_position(table, j, bs)
    assert j // bs == g["expected_logical_block"]
    assert (phys, off) == (g["expected_physical_block"], g["expected_offset"])
    slot = oracle.slot_of(table, j, bs)
    k_new = np.full((1, nh, hd), g["k_value"], dtype=np.float32)
    v_new = np.full((1, nh, hd), g["v_value"], dtype=np.float32)
    k2 = oracle.reshape_and_cache(k_pool, k_new, [slot])
    v2 = oracle.reshape_and_cache(v_pool, v_new, [slot])
    row = k2[table[1], 1]
    assert np.isclose(row.mean(), g["expected_k_mean"], rtol=0, atol=1e-6)
    assert np.all(v2[table[1], 1] == np.float32(g["v_value"]))
    # exactly one row changed in each pool
    assert np.count_nonzero(k2.reshape(nb * bs, -1).any(axis=1)) == 1
    assert np.count_nonzero(v2.reshape(nb * bs, -1).any(axis=1)) == 1


@pytest.mark.parametrize("fixture", ["qwbw_block_table.json", "guijiagi_mapping.json"])
def test_block_table_walkthroughs(golden_dir, fixture):
    g = _load(golden_dir, fixture)
    bt, bs = g["block_table"], g["block_size"]
    for j, phys, off in g["spot_checks"]:
        assert oracle.logical_position(bt, j, bs) == (phys, off)
        assert oracle.slot_of(bt, j, bs) == phys * bs + off
    for lo, hi, phys in g.get("ranges", []):
        for j in range(lo, hi + 1):
            assert oracle.logical_position(bt, j, bs) == (phys, j - lo)
    if "grown_table" in g:
        for j, phys, off in g["grown_spot_checks"]:
            assert oracle.logical_position(g["grown_table"], j, bs) == (phys, off)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(0, 70), min_size=1, max_size=5),
       st.sampled_from([1, 2, 4, 16]), st.integers(0, 2**31 - 1))
def test_slots_are_a_bijection_onto_used_cells(ctxs, bs, seed):
    s = custom_structure(ctxs, bs, seed=seed, pad_blocks=1)
    seq, pos = prefill_tokens(s.context_lens)
    slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    assert len(set(slots.tolist())) == len(slots)          # no two tokens share a cell
    assert np.all(slots >= 0) and np.all(slots < s.num_blocks * bs)
    # consecutive positions inside one block are consecutive cells
    for t in range(1, len(slots)):
        if seq[t] == seq[t - 1] and pos[t] % bs != 0:
            assert slots[t] == slots[t - 1] + 1
    # a block boundary jumps to the next table entry's first cell
    for t in range(len(slots)):
        if pos[t] % bs == 0:
            assert slots[t] == s.block_table[seq[t], pos[t] // bs] * bs


@settings(max_examples=40, deadline=None)
@given(st.lists(st.integers(0, 40), min_size=1, max_size=4),
       st.sampled_from([1, 3, 4, 16]), st.integers(0, 2**31 - 1))
def test_gather_inverts_the_write(ctxs, bs, seed):
    """Writing logical-order rows through the slots and gathering them back
    through the table returns the rows bit for bit; cells no token owns keep
    their NaN poison."""
    rng = np.random.default_rng(seed)
    s = custom_structure(ctxs, bs, seed=seed, num_blocks=None, pad_blocks=2)
    nb = s.num_blocks + 2
    pool = np.full((nb, bs, 2, 3), np.nan, dtype=np.float32)
    seq, pos = prefill_tokens(s.context_lens)
    rows = rng.standard_normal((len(seq), 2, 3)).astype(np.float32)
    slots = oracle.slot_mapping(s.block_table, seq, pos, bs)
    pool2 = oracle.reshape_and_cache(pool, rows, slots)
    t = 0
    for b, c in enumerate(s.context_lens):
        got = oracle.gather_sequence(pool2, s.block_table[b], int(c))
        assert got.shape == (int(c), 2, 3)
        assert np.array_equal(got.view(np.uint32), rows[t:t + c].view(np.uint32))
        t += c
    written = np.zeros(nb * bs, dtype=bool)
    written[slots] = True
    assert np.all(np.isnan(pool2.reshape(nb * bs, -1)[~written]))


def test_negative_slots_are_skipped():
    pool = np.zeros((2, 4, 1, 2), dtype=np.float32)
    new = np.ones((3, 1, 2), dtype=np.float32)
    out = oracle.reshape_and_cache(pool, new, [-1, 5, -7])
    assert out[1, 1].tolist() == [[1.0, 1.0]]
    assert np.count_nonzero(out) == 2


def test_workload_structures_are_consistent():
    """Every table entry a sequence uses is a valid, distinct block (except the
    deliberately shared prefix of the 8B-shaped workload)."""
    for name in ["tiny", "tiny_mha", "llama8b", "int8_70b", "mla"]:
        cfg = CONFIGS[name]
        s = structure(cfg)
        bs = cfg.block_size
        used = []
        for b, c in enumerate(s.context_lens):
            nb = -(-int(c) // bs)
            row = s.block_table[b, :nb]
            assert np.all((row >= 0) & (row < s.num_blocks))
            used.append(row[s.shared_blocks:] if s.shared_blocks else row)
        allu = np.concatenate(used)
        assert len(np.unique(allu)) == len(allu)
    s = structure(CONFIGS["tiny"])
    assert s.context_lens.tolist() == [37, 50]
    s70 = structure(CONFIGS["llama70b"], layer=3)
    assert s70.block_table.shape == (16, 512)
    assert sorted(s70.block_table.ravel().tolist()) == list(range(8192))
