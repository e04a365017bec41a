"""Workload definitions and seeded generators.

Six workloads, named by what they are:

* ``tiny``      fp32, B=2, n_h=4, n_kv=2, d=64, block 16, contexts {37, 50},
                a pool of 16 blocks handed out by a seeded permutation.
* ``tiny_mha``  the same with n_kv = n_h = 4 (multi-head attention, g = 1).
* ``llama8b``   bf16 layer of an 8B-shaped model: B=32, n_h=32, n_kv=8,
                d=128, block 16, contexts uniform in [512, 4096]; the first
                128 logical blocks of every sequence are one shared set of
                physical blocks (a 2K common prefix).
* ``llama70b``  bf16, B=16, n_h=64, n_kv=8, d=128, block 16, every context
                8192, 80 layers, each layer its own pool of 8192 blocks in a
                random permutation (40 GiB of K+V in total).
* ``int8_70b``  INT8 cache, B=32, n_h=64, n_kv=8, d=128, block 16, contexts
                log-uniform in [50, 32768].
* ``mla``       absorbed MLA, B=64, n_h=128, one 576-wide latent head
                (512 latent + 64 rope), values = first 512 columns, block 64,
                contexts uniform in [1024, 8192], scale 1/sqrt(192).

Host structure uses ``numpy.random.Generator(PCG64(seed))``; tensor contents
are N(0, 1), drawn on the host for the small workloads and on the device
(``torch.Generator``) for the large ones.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    kv_dtype: str          # "f32", "bf16", "int8"
    q_dtype: str           # "f32", "bf16"
    B: int
    n_h: int
    n_kv: int
    d_k: int
    d_v: int
    block_size: int
    scale: float
    seed: int
    layers: int = 1
    latent: bool = False   # V aliases the first d_v columns of K
    desc: str = ""


CONFIGS: dict[str, Config] = {
    "tiny": Config("tiny", "f32", "f32", 2, 4, 2, 64, 64, 16, 1.0 / 8.0, 1001,
                   desc="fp32 B=2 n_h=4 n_kv=2 d=64 bs=16 ctx={37,50} pool=16"),
    "tiny_mha": Config("tiny_mha", "f32", "f32", 2, 4, 4, 64, 64, 16, 1.0 / 8.0, 1006,
                       desc="fp32 MHA B=2 n_h=n_kv=4 d=64 bs=16 ctx={37,50} pool=16"),
    "llama8b": Config("llama8b", "bf16", "bf16", 32, 32, 8, 128, 128, 16,
                      1.0 / math.sqrt(128.0), 1002,
                      desc="bf16 B=32 n_h=32 n_kv=8 d=128 bs=16 ctx~U[512,4096] 2K shared prefix"),
    "llama70b": Config("llama70b", "bf16", "bf16", 16, 64, 8, 128, 128, 16,
                       1.0 / math.sqrt(128.0), 1003, layers=80,
                       desc="bf16 B=16 n_h=64 n_kv=8 d=128 bs=16 S=8192 x 80 layers"),
    "int8_70b": Config("int8_70b", "int8", "bf16", 32, 64, 8, 128, 128, 16,
                       1.0 / math.sqrt(128.0), 1004,
                       desc="int8 KV B=32 n_h=64 n_kv=8 d=128 bs=16 ctx log-U[50,32768]"),
    "mla": Config("mla", "bf16", "bf16", 64, 128, 1, 576, 512, 64,
                  1.0 / math.sqrt(192.0), 1005, latent=True,
                  desc="MLA absorbed B=64 n_h=128 d_k=576 d_v=512 bs=64 ctx~U[1024,8192]"),
}


@dataclass
class Structure:
    """Block tables and context lengths of one layer of a workload."""
    context_lens: np.ndarray            # int32 [B]
    block_table: np.ndarray             # int32 [B, max_blocks_per_seq], -1 padded
    num_blocks: int                     # physical blocks in the pool
    shared_blocks: int = 0              # leading logical blocks shared by all
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def _blocks_needed(ctx: int, bs: int) -> int:
    # Sequence length in whole blocks (how many pool blocks a sequence holds).
    return -(-int(ctx) // bs)


def _tables_from_counts(counts, perm, bs, max_blocks=None):
    """Deal ``perm`` out to sequences in order, ``counts[b]`` blocks each."""
    mb = max(counts) if max_blocks is None else max_blocks
    bt = np.full((len(counts), max(mb, 1)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(counts):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def structure(cfg: Config, layer: int = 0, seed: int | None = None) -> Structure:
    """Context lengths and block tables of one layer of ``cfg``."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    bs = cfg.block_size
    name = cfg.name
    if name in ("tiny", "tiny_mha"):
        ctx = np.array([37, 50], dtype=np.int32)
        perm = rng.permutation(16).astype(np.int32)
        counts = [_blocks_needed(c, bs) for c in ctx]          # 3 and 4
        bt = _tables_from_counts(counts, perm, bs)
        return Structure(ctx, bt, 16)
    if name == "llama8b":
        ctx = rng.integers(512, 4097, size=cfg.B).astype(np.int32)
        shared = 128
        private = [max(0, _blocks_needed(c, bs) - shared) for c in ctx]
        n_blocks = shared + int(sum(private))
        perm = rng.permutation(n_blocks).astype(np.int32)
        mb = max(_blocks_needed(c, bs) for c in ctx)
        bt = np.full((cfg.B, mb), -1, dtype=np.int32)
        pos = shared
        for b, c in enumerate(ctx):
            nb = _blocks_needed(c, bs)
            k = min(nb, shared)
            bt[b, :k] = perm[:k]
            bt[b, k:nb] = perm[pos:pos + private[b]]
            pos += private[b]
        return Structure(ctx, bt, n_blocks, shared_blocks=shared)
    if name == "llama70b":
        # one independent pool and permutation per layer
        lrng = np.random.Generator(np.random.PCG64([cfg.seed, layer]))
        S = 8192
        ctx = np.full(cfg.B, S, dtype=np.int32)
        per_seq = S // bs
        n_blocks = cfg.B * per_seq
        perm = lrng.permutation(n_blocks).astype(np.int32)
        bt = perm.reshape(cfg.B, per_seq).copy()
        return Structure(ctx, bt, n_blocks)
    if name == "int8_70b":
        u = rng.uniform(math.log(50.0), math.log(32768.0), size=cfg.B)
        ctx = np.clip(np.round(np.exp(u)), 50, 32768).astype(np.int32)
        counts = [_blocks_needed(c, bs) for c in ctx]
        n_blocks = int(sum(counts))
        perm = rng.permutation(n_blocks).astype(np.int32)
        return Structure(ctx, _tables_from_counts(counts, perm, bs), n_blocks)
    if name == "mla":
        ctx = rng.integers(1024, 8193, size=cfg.B).astype(np.int32)
        counts = [_blocks_needed(c, bs) for c in ctx]
        n_blocks = int(sum(counts))
        perm = rng.permutation(n_blocks).astype(np.int32)
        return Structure(ctx, _tables_from_counts(counts, perm, bs), n_blocks)
    raise KeyError(name)


def layer_structures(cfg: Config) -> list[Structure]:
    return [structure(cfg, layer=l) for l in range(cfg.layers)]


def custom_structure(context_lens, block_size: int, num_blocks: int | None = None,
                     seed: int = 7, pad_blocks: int = 0) -> Structure:
    """Random-permutation tables for arbitrary context lengths (edge cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int32)
    counts = [_blocks_needed(c, block_size) for c in ctx]
    need = int(sum(counts))
    nb = need if num_blocks is None else num_blocks
    if nb < need:
        raise ValueError("pool too small")
    perm = rng.permutation(nb).astype(np.int32)
    mb = max(max(counts) if counts else 1, 1) + pad_blocks
    return Structure(ctx, _tables_from_counts(counts, perm, block_size, mb), nb)


def shared_prefix_structure(context_lens, block_size: int, shared_blocks: int, seed: int = 11,
                            diverge=(), pad_blocks: int = 0) -> Structure:
    """Tables whose first ``shared_blocks`` logical blocks are one shared set
    of physical blocks (as in the 8B-shaped workload), a random permutation
    of a pool sized to the total.  ``diverge`` lists (sequence, logical
    block) pairs inside the shared range that get a block of their own
    instead (a sequence that only partly shares the prefix)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int32)
    nbs = [_blocks_needed(c, block_size) for c in ctx]
    own = set((int(b), int(j)) for b, j in diverge)
    private = [sum(1 for j in range(n) if j >= shared_blocks or (b, j) in own) for b, n in enumerate(nbs)]
    n_blocks = shared_blocks + int(sum(private))
    perm = rng.permutation(n_blocks).astype(np.int32)
    mb = max(max(nbs) if nbs else 1, 1) + pad_blocks
    bt = np.full((len(ctx), mb), -1, dtype=np.int32)
    pos = shared_blocks
    for b, n in enumerate(nbs):
        for j in range(n):
            if j < shared_blocks and (b, j) not in own:
                bt[b, j] = perm[j]
            else:
                bt[b, j] = perm[pos]
                pos += 1
    return Structure(ctx, bt, n_blocks, shared_blocks=shared_blocks)


def shared_prefix_prompts(cfg: Config, prefix_tokens: int = 2048, vocab: int = 32000):
    """Token ids of the 8B-shaped batch, for building its tables with a
    block allocator: the context lengths of ``structure(cfg)``; every prompt
    starts with one shared ``prefix_tokens``-token system prompt (a shorter
    prompt is that prompt's first tokens) followed by its own random ids.
    Also the allocator's initial free order (a seeded permutation of the
    pool, so physical placement is random) and a pool size with one block of
    headroom per sequence (a partly filled last block is never shared)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    ctx = rng.integers(512, 4097, size=cfg.B).astype(np.int32)          # as structure(cfg)
    trng = np.random.Generator(np.random.PCG64([cfg.seed, 7]))
    shared = trng.integers(0, vocab, size=prefix_tokens).astype(np.int32)
    prompts = [np.concatenate([shared[:min(int(c), prefix_tokens)],
                               trng.integers(0, vocab, size=max(0, int(c) - prefix_tokens)).astype(np.int32)])
               for c in ctx]
    bs = cfg.block_size
    n_blocks = _blocks_needed(prefix_tokens, bs) + sum(_blocks_needed(max(0, int(c) - prefix_tokens), bs)
                                                       for c in ctx) + cfg.B
    order = np.random.Generator(np.random.PCG64([cfg.seed, 8])).permutation(n_blocks).astype(np.int32)
    return prompts, n_blocks, order


# --------------------------------------------------------------------------
# token lists (structure only: which sequence and position each token has)
# --------------------------------------------------------------------------

def prefill_tokens(context_lens) -> tuple[np.ndarray, np.ndarray]:
    """(seq id, position) of every cached token, sequence-major."""
    seq, pos = [], []
    for b, c in enumerate(np.asarray(context_lens)):
        seq.extend([b] * int(c))
        pos.extend(range(int(c)))
    return np.asarray(seq, dtype=np.int32), np.asarray(pos, dtype=np.int32)


def decode_positions(context_lens) -> tuple[np.ndarray, np.ndarray]:
    """(seq id, position) of the token being decoded: the last one."""
    ctx = np.asarray(context_lens)
    return (np.arange(len(ctx), dtype=np.int32),
            np.maximum(ctx.astype(np.int32) - 1, 0))


# --------------------------------------------------------------------------
# tensor contents
# --------------------------------------------------------------------------

def host_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) draws on the host: float32 array, or bf16 bit patterns (uint16)
    rounded to nearest even from the float32 draw."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(dtype)


def device_normal_(t, seed: int, chunk_elems: int = 1 << 26):
    """Fill a device tensor with N(0,1) draws from ``torch.Generator``.

    Drawn in float32 in fixed chunks and cast to the tensor's dtype (for
    bfloat16, round-to-nearest-even), so a given seed gives the same bits
    whatever the device memory state.
    """
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    flat = t.view(-1)
    n = flat.numel()
    for lo in range(0, n, chunk_elems):
        hi = min(n, lo + chunk_elems)
        tmp = torch.randn(hi - lo, generator=g, device=t.device, dtype=torch.float32)
        flat[lo:hi].copy_(tmp.to(t.dtype))
    return t
