"""Plain, slow fp64 definitions of what paged decode attention computes.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No blocking, no
fusion, no online softmax: each function is the definition on the page it
cites, written out with numpy.  Array conventions:

* float32 / float64 arrays are taken as they are;
* uint16 arrays hold bfloat16 bit patterns (the top half of an IEEE fp32);
* int8 arrays hold quantized codes (with a separate fp32 scale array).

Pool layout: ``[num_blocks, block_size, n_kv, d]`` (talentme, chapter 3,
the NumPy pool class: one pool for K and one for V with that shape).
Block table: ``int32 [B, max_blocks_per_seq]``; entries past the blocks a
sequence uses are never read.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# element widening
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly.

    A bfloat16 value is an IEEE binary32 value whose low 16 mantissa bits are
    zero, so shifting the 16 stored bits into the high half of a 32-bit word
    gives the binary32 value, and binary32 -> binary64 is exact.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 data must be passed as uint16 bit patterns")
    as32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return as32.astype(np.float64)


def widen(x: np.ndarray) -> np.ndarray:
    """Any supported element type -> float64, exactly (no rounding)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported element type {x.dtype}")


# --------------------------------------------------------------------------
# logical -> physical addressing
# --------------------------------------------------------------------------

def logical_position(block_table_row, j: int, block_size: int) -> tuple[int, int]:
    """Physical (block, offset) that holds token ``j`` of a sequence.

    faulkner, section 逻辑块与物理块映射 (logical/physical block mapping):
    the logical block index is the floor of j over the block size, the
    in-block offset is j modulo the block size, and the physical block is
    the block table's entry at the logical block index.  qwbw section 3.3
    gives the same lookup with a worked table.
    """
    if j < 0:
        raise ValueError("token index must be non-negative")
    block_idx = j // block_size
    offset = j % block_size
    phys = int(block_table_row[block_idx])
    return phys, offset


def slot_of(block_table_row, j: int, block_size: int) -> int:
    """Flat slot id ``phys * block_size + offset`` of token ``j``.

    The pages address the pool as ``pool[phys, offset]`` (talentme,
    chapter 3, the ``write_kv`` lookup); numbering the (block, offset) cells
    of the pool row-major gives this flat slot.
    """
    phys, offset = logical_position(block_table_row, j, block_size)
    return phys * block_size + offset


def slot_mapping(block_table, seq_ids, positions, block_size: int) -> np.ndarray:
    """Slots of tokens given as (sequence id, position) pairs; int64."""
    out = np.empty(len(seq_ids), dtype=np.int64)
    for t, (b, j) in enumerate(zip(seq_ids, positions)):
        out[t] = slot_of(block_table[int(b)], int(j), block_size)
    return out


def reshape_and_cache(pool: np.ndarray, new: np.ndarray, slots) -> np.ndarray:
    """Scatter new per-token rows into a copy of the pool.

    talentme, chapter 3 (``write_kv``): the row of token t goes to
    ``pool[phys, offset]``.  Here the (phys, offset) pair arrives as a flat
    slot; a negative slot means "no write" (a padding token).  Bits are
    copied unchanged: the result is compared bit for bit.
    """
    out = pool.copy()
    bs = pool.shape[1]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        out[s // bs, s % bs] = new[t]
    return out


def gather_sequence(pool: np.ndarray, block_table_row, ctx: int) -> np.ndarray:
    """Rows 0 .. ctx-1 of one sequence, in logical order: ``[ctx, n_kv, d]``.

    qwbw section 3.4: attention walks the block table and reads each
    physical block in turn; only the K/V addresses are non-contiguous.
    Positions at or beyond ``ctx`` are never touched (the tail block may be
    partly filled, faulkner 逻辑块与物理块映射), so poisoned slots there
    cannot leak into the result.
    """
    bs = pool.shape[1]
    rows = []
    for j in range(ctx):
        phys, off = logical_position(block_table_row, j, bs)
        rows.append(pool[phys, off])
    if not rows:
        return pool[:0, 0]
    return np.stack(rows, axis=0)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Attention weights of one query over ``L`` keys, float64.

    faulkner, first section, equation for o_t: the weights are the softmax
    of the scaled dot products of the query with every cached key.  Plain
    softmax: subtract the maximum, exponentiate, divide by the sum.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    s = np.float64(scale) * (K @ q)
    s = s - s.max()
    e = np.exp(s)
    return e / e.sum()


def decode_attention_contiguous(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                                scale: float) -> np.ndarray:
    """One sequence, contiguous (unpaged) K/V.

    ``q [n_h, d_k]``, ``K [L, n_kv, d_k]``, ``V [L, n_kv, d_v]`` ->
    ``o [n_h, d_v]`` in float64.

    faulkner, section on the Roofline intensity of decode and the MHA/GQA/MLA
    table: ``g = n_h / n_kv`` query heads share one (K, V) head.  Query head
    ``h`` reads KV head ``h // g`` (consecutive groups; the pages give no
    index rule, this is the plainest reading).  ``L = 0`` gives zeros.
    """
    q = widen(q)
    K = widen(K)
    V = widen(V)
    n_h = q.shape[0]
    n_kv = K.shape[1]
    if n_h % n_kv:
        raise ValueError("n_h must be a multiple of n_kv")
    g = n_h // n_kv
    L = K.shape[0]
    out = np.zeros((n_h, V.shape[2]), dtype=np.float64)
    if L == 0:
        return out
    for h in range(n_h):
        kvh = h // g
        w = softmax_weights(q[h], K[:, kvh, :], scale)
        out[h] = w @ V[:, kvh, :]
    return out


def window_start(L: int, window: int) -> int:
    """First position a query at the end of a sequence of ``L`` tokens sees.

    guijiagi section 5.1 (sliding window cache): with window size w only
    the most recent w tokens are kept and attended, i.e. positions
    ``L - w .. L - 1`` (all of them when ``L <= w``).  ``window = 0`` means
    no window (the whole context).
    """
    if window < 0:
        raise ValueError("window must be >= 0")
    return max(0, L - window) if window > 0 else 0


def paged_decode_attention(q, k_pool, v_pool, block_table, context_lens,
                           scale: float, window: int = 0) -> np.ndarray:
    """Decode attention over a paged KV cache, float64 ``[B, n_h, d_v]``.

    qwbw section 3.4: for each sequence, gather its K and V through the
    block table, then run ordinary attention (scores, softmax, weighted sum
    of V).  The result equals attention over the contiguous cache because
    paging changes only where rows live (hx section 4.2: physical
    non-contiguity is invisible to the kernel).  ``context_lens[b]`` counts
    every cached token of sequence b, the token being decoded included
    (qwbw section 1.2 appends K/V before attending).  With ``window > 0``
    only the last ``window`` positions take part (:func:`window_start`).
    """
    q = np.asarray(q)
    B = q.shape[0]
    out = []
    for b in range(B):
        L = int(context_lens[b])
        K = gather_sequence(k_pool, block_table[b], L)
        V = gather_sequence(v_pool, block_table[b], L)
        w0 = window_start(L, window)
        out.append(decode_attention_contiguous(q[b], K[w0:], V[w0:], scale))
    return np.stack(out, axis=0)


# --------------------------------------------------------------------------
# INT8 KV cache
# --------------------------------------------------------------------------

def quantize_int8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row INT8 quantization in IEEE binary32 arithmetic.

    guijiagi section 4.2 (quantization method, 8-bit branch): the scale is the
    absolute maximum over the last dimension divided by 127; the code is
    x / scale rounded to nearest and clamped to [-128, 127].  The steps are
    taken in float32 exactly as written (a correctly rounded fp32 division
    for the scale, a correctly rounded fp32 division for each quotient,
    round-half-to-even), so that the codes are reproducible bit for bit.
    A row that is all zeros has no defined scale on the page; here its
    scale is 0 and its codes are 0.

    Returns ``(codes int8 [..., d], scale float32 [...])``.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x32 = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif x.dtype == np.float32:
        x32 = x
    else:
        raise TypeError("quantizer input must be float32 or bf16 bits")
    amax = np.abs(x32).max(axis=-1)                      # exact in fp32
    scale = (amax / np.float32(127.0)).astype(np.float32)  # fp32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = (x32 / safe[..., None]).astype(np.float32)   # fp32 division
    codes = np.clip(np.rint(ratio), -128, 127)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale.astype(np.float32)


def dequantize_int8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """``code * scale`` in float64 (guijiagi section 4.2, dequantize).

    The product of an int8 and a binary32 value is exact in binary64.
    """
    return codes.astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


def paged_decode_attention_int8(q, k_codes, k_scales, v_codes, v_scales,
                                block_table, context_lens, scale: float,
                                window: int = 0) -> np.ndarray:
    """Decode attention over an INT8 paged cache with per-(slot, head) scales.

    Pools: codes ``int8 [NB, bs, n_kv, d]``, scales ``float32 [NB, n_kv, bs]``
    (one scale per token per KV head, paged like the codes: the block is the
    page, and inside it one head's scales are adjacent).  The cache is
    dequantized (guijiagi section 4.2) and then attended exactly as
    :func:`paged_decode_attention`.
    """
    k = dequantize_int8(k_codes, np.swapaxes(np.asarray(k_scales), 1, 2))
    v = dequantize_int8(v_codes, np.swapaxes(np.asarray(v_scales), 1, 2))
    return paged_decode_attention(q, k, v, block_table, context_lens, scale, window)


# --------------------------------------------------------------------------
# INT4 KV cache with an unquantized attention sink
# --------------------------------------------------------------------------

def quantize_int4_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row INT4 quantization in IEEE binary32 arithmetic.

    guijiagi section 4.2 (quantization method, 4-bit branch): the scale is
    the absolute maximum over the last dimension divided by 7; the code is
    x / scale rounded to nearest and clamped to [-8, 7].  Taken in float32
    step by step as in :func:`quantize_int8_rows` (correctly rounded
    divisions, round-half-to-even); an all-zero row gets scale 0 and codes
    0.  Returns ``(codes int8 [..., d] in [-8, 7], scale float32 [...])``.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x32 = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        x32 = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x32), axis=-1)
    scale = (a / np.float32(7.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quo = (x32 / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(quo), -8, 7)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale.astype(np.float32)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte (guijiagi section 4.2 gives the 4x memory
    saving of 4-bit storage but no byte order): element 2i in the low
    nibble and element 2i + 1 in the high nibble of byte i, each as a 4-bit
    two's complement value.  ``[..., d]`` int8 -> ``[..., d / 2]`` uint8."""
    c = np.asarray(codes, dtype=np.int8)
    if c.shape[-1] % 2:
        raise ValueError("an even number of codes per row")
    u = c.astype(np.uint8) & np.uint8(0x0F)
    return (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4`: ``[..., d / 2]`` uint8 -> ``[..., d]`` int8."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & np.uint8(0x0F)).astype(np.int16)
    hi = (p >> np.uint8(4)).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def paged_decode_attention_int4(q, k_packed, k_scales, v_packed, v_scales, sink_k, sink_v,
                                block_table, context_lens, scale: float) -> np.ndarray:
    """Decode attention over an INT4 paged cache whose first tokens are kept
    unquantized.

    guijiagi section 4.3 (attention sink): the first k tokens of a sequence
    draw attention from every later token, so their quantization error is
    amplified; they are kept at full precision (k = 4 is typical).  Here
    ``sink_k``/``sink_v`` ``[B, n_sink, n_kv, d]`` hold positions
    ``0 .. n_sink - 1`` of each sequence (bf16 bits or floats); every other
    position comes from the paged INT4 pool (codes packed by
    :func:`pack_int4` ``[NB, bs, n_kv, d / 2]``, scales ``float32 [NB, n_kv,
    bs]``), dequantized as ``code * scale``.  The pool's rows at sink
    positions are not read.
    """
    q = np.asarray(q)
    k = dequantize_int8(unpack_int4(k_packed), np.swapaxes(np.asarray(k_scales), 1, 2))
    v = dequantize_int8(unpack_int4(v_packed), np.swapaxes(np.asarray(v_scales), 1, 2))
    sk, sv = widen(sink_k), widen(sink_v)
    n_sink = sk.shape[1]
    out = []
    for b in range(q.shape[0]):
        L = int(context_lens[b])
        K = gather_sequence(k, block_table[b], L).copy()
        V = gather_sequence(v, block_table[b], L).copy()
        ns = min(L, n_sink)
        K[:ns] = sk[b, :ns]
        V[:ns] = sv[b, :ns]
        out.append(decode_attention_contiguous(q[b], K, V, scale))
    return np.stack(out, axis=0)


# --------------------------------------------------------------------------
# chunked prefill over the paged cache
# --------------------------------------------------------------------------

def paged_prefill_attention(q, k_pool, v_pool, block_table, start_pos, chunk_lens,
                            scale: float) -> np.ndarray:
    """Causal attention of a chunk of new tokens over a paged cache.

    faulkner, continuous batching section (chunked prefill): a long prompt
    is processed a fixed number of tokens per step, each chunk attending to
    everything cached before it plus itself, causally.  Sequence b's chunk
    holds ``chunk_lens[b]`` query tokens at positions ``start_pos[b] + i``;
    their K/V are already in the cache (written before the attention, as
    in qwbw section 1.2), and query i sees positions ``0 .. start_pos[b] +
    i``.  ``q [B, C, n_h, d_k]`` -> ``[B, C, n_h, d_v]`` float64 (rows past
    a chunk's length are zero).
    """
    q = np.asarray(q)
    B, C = q.shape[0], q.shape[1]
    out = np.zeros((B, C, q.shape[2], np.asarray(v_pool).shape[3]), dtype=np.float64)
    for b in range(B):
        p0, n = int(start_pos[b]), int(chunk_lens[b])
        if n == 0:
            continue
        K = gather_sequence(k_pool, block_table[b], p0 + n)
        V = gather_sequence(v_pool, block_table[b], p0 + n)
        for i in range(n):
            out[b, i] = decode_attention_contiguous(q[b, i], K[:p0 + i + 1], V[:p0 + i + 1], scale)
    return out


# --------------------------------------------------------------------------
# MLA (absorbed) decode
# --------------------------------------------------------------------------

def paged_decode_attention_mla(q, latent_pool, block_table, context_lens,
                               scale: float, d_v: int) -> np.ndarray:
    """Absorbed MLA decode over a paged latent cache.

    faulkner, section on matrix absorption: with W^UK folded into the query
    side, every head scores the cached vector (c, k^R) of each token
    directly, and with W^UV folded into the output projection the value of
    a token is its latent c.  The cache holds one 576-wide vector per token
    shared by all heads (one KV head), ordered ``[c | k^R]``; the value is
    the first ``d_v`` columns of the same row.  Output is in latent space.
    """
    latent_pool = np.asarray(latent_pool)
    if latent_pool.shape[2] != 1:
        raise ValueError("the latent pool has a single KV head")
    v_pool = latent_pool[..., :d_v]
    return paged_decode_attention(q, latent_pool, v_pool, block_table,
                                  context_lens, scale)


# --------------------------------------------------------------------------
# split-context partials (for checking a split/merge decomposition)
# --------------------------------------------------------------------------

def split_partials(q_h, K, V, scale: float, bounds):
    """Per-split (max score, weight sum, normalised output) of one head.

    A split is a contiguous token range ``[lo, hi)``; over it the partial
    result is the row maximum m, the sum l of exp(s - m) and the output
    normalised by l.  Empty splits give ``(-inf, 0, 0)``.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    parts = []
    for lo, hi in bounds:
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        s = np.float64(scale) * (K[lo:hi] @ q_h)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        parts.append((m, l, (e @ V[lo:hi]) / l))
    return parts


def merge_partials(parts):
    """Merge split partials into the full softmax-weighted output.

    With M the largest split maximum, each split's weight is
    exp(m_s - M) * l_s; the output is the weight-averaged split output.
    This is the exact identity exp(s - M) = exp(s - m_s) * exp(m_s - M)
    applied to the softmax of faulkner's o_t equation.
    """
    M = max(p[0] for p in parts)
    wsum = 0.0
    acc = None
    for m, l, o in parts:
        if l == 0.0:
            continue
        w = np.exp(m - M) * l
        wsum += w
        acc = w * o if acc is None else acc + w * o
    return acc / wsum


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def kv_cache_bytes(L: int, n_kv: int, d_h: int, S: int, B: int,
                   bytes_per_elem: float) -> float:
    """Total KV bytes: 2 * L * n_kv * d_h * S * B * bytes.

    faulkner, KV Cache 容量公式 (capacity formula); the same product is
    given by guijiagi section 2.1 and talentme chapter 2.  The leading 2 is
    one copy for K and one for V.
    """
    return 2 * L * n_kv * d_h * S * B * bytes_per_elem


def decode_attention_intensity(g: int, S: int, d_h: int) -> float:
    """FLOP per byte of one KV head's decode attention in bf16.

    faulkner, Prefill/Decode intensity section: 4 g S d_h FLOPs over
    4 S d_h + 2 g d_h bytes, which tends to g.
    """
    return (4.0 * g * S * d_h) / (4.0 * S * d_h + 2.0 * g * d_h)
