"""Plain float64 CPU oracle for paged decode attention, prefill attention over the paged
cache, reshape_and_cache, copy_blocks and swap_blocks.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import, call or run anything here.  The GPU library never calls it,
and nothing here imports the GPU library.  It is deliberately slow: one sequence and one
head at a time, no blocking, no fusion, no reordering.

What is computed, and where the pages say so
--------------------------------------------
* Paged KV cache: K and V of each sequence live in fixed-size blocks of a shared physical
  pool; a per-sequence block table maps logical block j (tokens j*bs .. j*bs+bs-1) to a
  physical block.  PyTorch-CUDA-v2.9 PagedAttention page (jsqmd.com), section on paged memory
  for the KV cache; "GPT-OSS显存管理技巧：PagedAttention机制解析" (yongjin360.com) §2.2;
  UltraLAB summary of Kwon et al., SOSP 2023 (xasun.com) §一.
* The attention kernel fetches K/V block by block through the block table (xasun.com summary
  §二, attention-algorithm item), and paging does not change the result (same page, §一,
  "lossless" claim).  So the oracle resolves the table into contiguous K/V and then applies
  the plain definition.
* The definition is scaled dot-product attention with a softmax over the scores
  ("PagedAttention技术：加速GPT推理的利器" (yunthe.com) §1.1).  For one decoded query:
      z_t = scale * <q, k_t>,   p_t = exp(z_t - max z) / sum_u exp(z_u - max z),
      out = sum_t p_t v_t.
* Each decode step appends the new token's K/V into the cache (jsqmd.com page, paged-memory
  section and serving-workflow list).  reshape_and_cache_ref writes it at its physical slot.
* Blocks shared between sequences are reference-counted and copied before a write
  (copy-on-write; xasun.com summary §一 and §二, sharing item).  copy_blocks_ref is that copy.
* Per-token KV size (xasun.com summary §三, memory-capacity row: about 800 KB per token for
  OPT-13B) and block counts (yunthe.com §1.2: 2048 tokens in 128-token pages is 16 pages).

Readings where the pages are silent (each is listed with its reason in the design notes):
* ``scale`` is a caller argument (1/sqrt(head_dim) in every workload).
* ``context_lens`` counts the token being decoded (its K/V is written first).
* A context of 0 tokens gives an all-zero output (softmax over an empty set is undefined).
* Grouped-query attention maps query head h to KV head floor(h / G), G = Hq / Hkv.
* Slots past the context, unused blocks and unused table entries are never read.
* Split-KV partitions cover tokens [p*P, min((p+1)*P, n)) and are merged by their
  log-sum-exp weights; exact arithmetic gives the unsplit result.
* A slot or block id outside the pool is skipped by the cache writers.

Parity pins (``tests/test_oracle_pins.py``): brute-force contiguous attention and torch's
float64 SDPA on tiny inputs; paged == contiguous; invariance under any permutation of the
physical placement; all-equal keys and scale 0 give mean(V); one-token context gives V
exactly; poisoned unused slots/blocks/table entries change nothing; split+merge == unsplit;
the pages' per-token KV and page-count arithmetic (``tests/golden/``); reshape/copy against a
flat-slot formulation and a per-element loop; copy-on-write round trips; for prefill, decimal
brute force over the causal prefix, torch's float64 causal SDPA on whole prompts, every row
equal to a decode at its position, and invariance under re-chunking.  A mutation test
plants mistakes in a copy of this file and checks that some pin fails for each.
"""

from __future__ import annotations

import math

import numpy as np

_BF16_MIN_EXP = -133  # quantum of bfloat16 subnormals: 2**-133


# ---------------------------------------------------------------------------------------
# element types
# ---------------------------------------------------------------------------------------
def storage_to_f64(x, dtype: str) -> np.ndarray:
    """Exact float64 value of a storage array ("f64": float64, "f32": float32, "f16": float16,
    "bf16": uint16 raw bits)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to bfloat16 (nearest, ties to even) in one step: scale each value so
    its bfloat16 quantum is 1, round with rint (ties-to-even), scale back."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    qexp = np.maximum(e - 8, _BF16_MIN_EXP)   # 8 significant bits for normal values
    r = np.ldexp(np.rint(np.ldexp(xf, -qexp)), qexp)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)            # exact, or +-inf past the bfloat16 range
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    big = np.abs(r) >= 2.0 ** 128
    bits = np.where(big, np.where(r > 0, np.uint16(0x7F80), np.uint16(0xFF80)), bits)
    out[...] = bits
    out[np.isnan(x)] = 0x7FC0
    out[np.isposinf(x)] = 0x7F80
    out[np.isneginf(x)] = 0xFF80
    return out


def f64_to_storage(x, dtype: str) -> np.ndarray:
    """Round float64 to the storage type, nearest-even, in a single rounding."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return _f64_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------------------
# paging arithmetic
# ---------------------------------------------------------------------------------------
def num_blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(n / bs)."""
    return -(-int(num_tokens) // int(block_size))


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one token across all layers: 2 * L * H_kv * d * e bytes."""
    return 2 * int(num_layers) * int(num_kv_heads) * int(head_dim) * int(elem_bytes)


def slot_utilization(lengths, block_size: int) -> float:
    """Fraction of reserved slots holding a token: sum(n) / sum(ceil(n/bs) * bs)."""
    lengths = [int(n) for n in lengths]
    reserved = sum(num_blocks_for(n, block_size) * block_size for n in lengths)
    return sum(lengths) / reserved if reserved else 1.0


def resolve_sequence(cache, table_row, num_tokens: int, block_size: int, dtype: str) -> np.ndarray:
    """Logical K (or V) of one sequence: float64 ``[H_kv, n, d]``.

    Follows the block table: logical block j is physical block ``table_row[j]``; within a
    block, token t sits at offset t mod bs.  Only the first ceil(n/bs) table entries are
    read, and only the first n tokens are kept.
    """
    n = int(num_tokens)
    nb = num_blocks_for(n, block_size)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = storage_to_f64(cache[phys], dtype)          # [nb, H, bs, d]
    h, d = blocks.shape[1], blocks.shape[3]
    seq = blocks.transpose(1, 0, 2, 3).reshape(h, nb * block_size, d)
    return seq[:, :n, :]


# ---------------------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------------------
def _softmax_weighted_sum(K, V, q, scale):
    """Attention of one query over n keys/values (all float64)."""
    z = scale * (K @ q)
    z = z - z.max()
    p = np.exp(z)
    return (p @ V) / p.sum()


def decode_ref(query, key_cache, value_cache, block_tables, context_lens, block_size, scale,
               dtype: str) -> np.ndarray:
    """Single-query paged decode attention, float64 ``[S, Hq, d]``.

    ``query`` [S, Hq, d], ``key_cache``/``value_cache`` [NB, Hkv, bs, d] (storage arrays),
    ``block_tables`` [S, max_blocks], ``context_lens`` [S], ``scale`` a float32 value.
    """
    S, Hq, d = query.shape
    Hkv = key_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        n = int(context_lens[s])
        if n <= 0:
            continue
        K = resolve_sequence(key_cache, block_tables[s], n, block_size, dtype)
        V = resolve_sequence(value_cache, block_tables[s], n, block_size, dtype)
        q = storage_to_f64(query[s], dtype)
        for h in range(Hq):
            kv = h // G
            out[s, h] = _softmax_weighted_sum(K[kv], V[kv], q[h], sc)
    return out


def decode_split_ref(query, key_cache, value_cache, block_tables, context_lens, block_size, scale,
                     dtype: str, partition_size: int):
    """Split-KV decode: per partition (m, l, o) then a log-sum-exp merge.

    Partition p of a sequence with n tokens covers tokens [p*P, min((p+1)*P, n)).  For each
    partition: m = max z, l = sum exp(z - m), o = sum exp(z - m) v / l.  Merge:
    M = max_p m_p, w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p.
    Returns (out [S, Hq, d], partials) with partials[s][h] a list of (m, l, o).
    """
    S, Hq, d = query.shape
    Hkv = key_cache.shape[1]
    G = Hq // Hkv
    P = int(partition_size)
    if P <= 0:
        raise ValueError("partition_size must be positive")
    sc = float(np.float32(scale))
    out = np.zeros((S, Hq, d), dtype=np.float64)
    partials = []
    for s in range(S):
        n = int(context_lens[s])
        row = []
        if n <= 0:
            partials.append([[] for _ in range(Hq)])
            continue
        K = resolve_sequence(key_cache, block_tables[s], n, block_size, dtype)
        V = resolve_sequence(value_cache, block_tables[s], n, block_size, dtype)
        q = storage_to_f64(query[s], dtype)
        for h in range(Hq):
            kv = h // G
            parts = []
            for t0 in range(0, n, P):
                t1 = min(t0 + P, n)
                z = sc * (K[kv, t0:t1] @ q[h])
                m = z.max()
                e = np.exp(z - m)
                l = e.sum()
                parts.append((m, l, (e @ V[kv, t0:t1]) / l))
            M = max(m for m, _, _ in parts)
            w = np.array([l * math.exp(m - M) for m, l, _ in parts])
            o = np.stack([o for _, _, o in parts])
            out[s, h] = (w @ o) / w.sum()
            row.append(parts)
        partials.append(row)
    return out, partials


# ---------------------------------------------------------------------------------------
# cache writers
# ---------------------------------------------------------------------------------------
def reshape_and_cache_ref(key, value, key_cache, value_cache, slot_mapping, block_size):
    """Copies of the pools with token i's K/V [Hkv, d] stored at physical slot
    ``slot_mapping[i]``: block slot // bs, offset slot % bs.  Negative or out-of-pool slots
    are skipped.  Bits are copied unchanged."""
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    nb = kc.shape[0]
    bs = int(block_size)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0 or slot >= nb * bs:
            continue
        b, o = divmod(slot, bs)
        kc[b, :, o, :] = key[i]
        vc[b, :, o, :] = value[i]
    return kc, vc


def swap_blocks_ref(src_key, src_value, dst_key, dst_value, block_mapping):
    """Copies of the destination pools where block dst receives the whole of source block src
    (every head, every slot) for each (src, dst) pair.  Source and destination are different
    pools (the GPU pool and the host pool used to swap preempted sequences out and back in:
    xasun.com summary §二, block-engine and scheduler items).  Pairs with an id outside its
    pool are skipped; bits are copied unchanged."""
    kd = np.array(dst_key, copy=True)
    vd = np.array(dst_value, copy=True)
    ns, nd = src_key.shape[0], kd.shape[0]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        src, dst = int(src), int(dst)
        if not (0 <= src < ns and 0 <= dst < nd):
            continue
        kd[dst] = src_key[src]
        vd[dst] = src_value[src]
    return kd, vd


def copy_blocks_ref(key_cache, value_cache, block_mapping):
    """Copies of the pools where block dst receives the whole of block src (every head,
    every slot) for each (src, dst) pair, all read from the pools as they were before the
    call.  Pairs with an id outside the pool are skipped."""
    k0 = np.array(key_cache, copy=True)
    v0 = np.array(value_cache, copy=True)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    nb = kc.shape[0]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        src, dst = int(src), int(dst)
        if not (0 <= src < nb and 0 <= dst < nb):
            continue
        kc[dst] = k0[src]
        vc[dst] = v0[src]
    return kc, vc


# ---------------------------------------------------------------------------------------
# prefill attention over the paged cache
# ---------------------------------------------------------------------------------------
def prefill_ref(query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
                block_size, scale, dtype: str) -> np.ndarray:
    """Causal attention of a chunk of new tokens per sequence over the paged cache, float64
    ``[T, Hq, d]``.

    Prefill is the compute-heavy phase that precedes decoding (xasun.com summary §三, table row
    on the compute pattern), and it may be cut into chunks (the chunked-prefill switch in the
    jsqmd.com page's vLLM usage example).  Sequence s owns query rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1`` (L rows).  Its ``context_lens[s]`` = n
    cached tokens already include those rows' own K/V (reshape_and_cache runs first), so the
    chunk's token i sits at position n - L + i and, as a decoded token at that position would,
    attends to the positions 0 .. n - L + i.  A sequence with n < L has no valid placement:
    its rows are zero.  Rows no sequence owns are zero.
    """
    T, Hq, d = query.shape
    Hkv = key_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    sc = float(np.float32(scale))
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    out = np.zeros((T, Hq, d), dtype=np.float64)
    for s in range(len(qsl) - 1):
        q0, q1 = int(qsl[s]), int(qsl[s + 1])
        L, n = q1 - q0, int(context_lens[s])
        if L <= 0 or n < L:
            continue
        K = resolve_sequence(key_cache, block_tables[s], n, block_size, dtype)
        V = resolve_sequence(value_cache, block_tables[s], n, block_size, dtype)
        q = storage_to_f64(query[q0:q1], dtype)
        for i in range(L):
            last = n - L + i               # the token's own position
            for h in range(Hq):
                kv = h // G
                out[q0 + i, h] = _softmax_weighted_sum(K[kv, :last + 1], V[kv, :last + 1],
                                                       q[i, h], sc)
    return out


# ---------------------------------------------------------------------------------------
# 8-bit floating-point KV cache
# ---------------------------------------------------------------------------------------
# The cache element type is a serving choice (kv_cache_dtype in the vLLM configuration example
# of yongjin360.com, §3.2); an 8-bit cache halves the bytes decode streams.  The format is the
# OCP 8-bit E4M3 ("FN") encoding: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
# infinities, S.1111.111 is NaN, largest finite value 448, subnormals m * 2^-9.  A cache keeps
# one float scale per pool: the stored code is E4M3(x / scale), read back as code * scale.
FP8_MAX = 448.0


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of E4M3 codes (uint8 array)."""
    c = np.asarray(codes).view(np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where((c & 0x80) != 0, -mag, mag)
    val[(e == 15) & (c & 0x7 == 7)] = np.nan
    return val


def f64_to_fp8_e4m3(x) -> np.ndarray:
    """Round to E4M3, nearest with ties to even.  Values that round past 448 (|x| > 464) and
    NaN give the NaN code; the sign of zero is kept.  Callers that saturate clamp first."""
    x = np.asarray(x, dtype=np.float64)
    a = np.where(np.isfinite(x), np.abs(x), 0.0)
    _, ex = np.frexp(a)                            # a = f * 2^ex, 0.5 <= f < 1
    qexp = np.maximum(ex - 4, -9)                  # 3 mantissa bits; subnormal quantum 2^-9
    r = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)
    _, rex = np.frexp(r)
    sub = r < 2.0 ** -6
    e = np.where(sub, 0, rex - 1 + 7)
    m = np.where(sub, np.ldexp(r, 9), np.ldexp(r, -(rex - 1)) * 8 - 8)
    code = (e.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(r > FP8_MAX, 0x7F, code)
    code = np.where(np.isnan(x) | np.isinf(x), 0x7F, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def quantize_fp8(x, dtype: str, scale) -> np.ndarray:
    """Codes a cache writer stores for values ``x`` (storage of type ``dtype``): y = x * (1 /
    scale) in float32 (the reciprocal rounded to float32 once), clamped to +-448 (saturation),
    then rounded to E4M3."""
    inv = np.float32(1.0) / np.float32(scale)
    y = storage_to_f64(x, dtype).astype(np.float32) * inv        # float32 product, nearest
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return f64_to_fp8_e4m3(y.astype(np.float64))


def dequantize_fp8(codes, scale) -> np.ndarray:
    """float64 values code * scale of an 8-bit cache."""
    return fp8_e4m3_to_f64(codes) * float(np.float32(scale))


def reshape_and_cache_fp8_ref(key, value, key_cache, value_cache, slot_mapping, block_size,
                              dtype: str, k_scale, v_scale):
    """reshape_and_cache_ref for an 8-bit cache: token i's K/V (storage of type ``dtype``) are
    quantized with the pool's scale and stored at slot ``slot_mapping[i]``."""
    return reshape_and_cache_ref(quantize_fp8(key, dtype, k_scale),
                                 quantize_fp8(value, dtype, v_scale),
                                 key_cache, value_cache, slot_mapping, block_size)


def decode_fp8_ref(query, key_cache, value_cache, block_tables, context_lens, block_size, scale,
                   dtype: str, k_scale, v_scale) -> np.ndarray:
    """Paged decode attention over an 8-bit cache: decode_ref on the dequantized pools (codes
    times the pool's scale, exactly); ``dtype`` is the query's type."""
    kc = dequantize_fp8(key_cache, k_scale)
    vc = dequantize_fp8(value_cache, v_scale)
    qf = storage_to_f64(query, dtype)
    return decode_ref(qf, kc, vc, block_tables, context_lens, block_size, scale, "f64")


def prefill_fp8_ref(query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
                    block_size, scale, dtype: str, k_scale, v_scale) -> np.ndarray:
    """Chunked prefill over an 8-bit cache: prefill_ref on the dequantized pools (codes times
    each pool's scale, exactly); ``dtype`` is the query's type."""
    keys = dequantize_fp8(key_cache, k_scale)
    values = dequantize_fp8(value_cache, v_scale)
    return prefill_ref(storage_to_f64(query, dtype), keys, values, block_tables, query_start_loc,
                       context_lens, block_size, scale, "f64")


# ---------------------------------------------------------------------------------------
# block engine: append with copy-on-write, fork, free, prefix-block hashes
# ---------------------------------------------------------------------------------------
# The KV cache manager maps each sequence's logical blocks to physical blocks, allocates on
# demand and reclaims freed blocks (xasun.com summary §二, block-engine item); shared blocks
# carry reference counts and are copied before a sharer writes into them (same page, sharing
# item).  The state below is the one the GPU keeps: tables, context lengths, one reference
# count per block, and a stack of free block ids whose top ``free_top`` entries are free.
def append_slots_ref(tables, ctx, refs, stack, free_top, seq_ids, block_size):
    """Append one token to each listed sequence, in list order.

    For a sequence with n tokens: if n is a multiple of the block size, a fresh block is taken
    from the top of the free stack; else, if its last block is shared (reference count > 1),
    a fresh block is taken, the pair (old, new) is recorded for copying, the old block loses a
    reference and the table points at the new one; else the token goes into the last block.
    The token's slot is block * bs + n mod bs, and n grows by one.  A sequence whose table is
    full, or that needs a block when none is free, is left unchanged with slot -1 and raises
    a status (1: out of blocks, 2: table full).

    Returns (tables, ctx, refs, stack, free_top, slots, pairs, status), all copies."""
    tables = np.array(tables, dtype=np.int32, copy=True)
    ctx = np.array(ctx, dtype=np.int32, copy=True)
    refs = np.array(refs, dtype=np.int32, copy=True)
    stack = np.array(stack, dtype=np.int32, copy=True)
    top = int(free_top)
    bs = int(block_size)
    slots, pairs, status = [], [], 0
    for s in np.asarray(seq_ids, dtype=np.int64):
        n = int(ctx[s])
        j, off = divmod(n, bs)
        if off == 0:
            if j >= tables.shape[1]:
                slots.append(-1)
                status = max(status, 2)
                continue
            if top == 0:
                slots.append(-1)
                status = max(status, 1)
                continue
            top -= 1
            new = int(stack[top])
            tables[s, j] = new
            refs[new] = 1
            block = new
        else:
            block = int(tables[s, j])
            if refs[block] > 1:
                if top == 0:
                    slots.append(-1)
                    status = max(status, 1)
                    continue
                top -= 1
                new = int(stack[top])
                pairs.append((block, new))
                refs[block] -= 1
                refs[new] = 1
                tables[s, j] = new
                block = new
        slots.append(block * bs + off)
        ctx[s] = n + 1
    return (tables, ctx, refs, stack, top, np.array(slots, np.int64),
            np.array(pairs, np.int64).reshape(-1, 2), status)


def fork_ref(tables, ctx, refs, parent_child, block_size):
    """Each child gets the parent's table entries and length; every shared block gains one
    reference (parallel sampling forks a sequence this way)."""
    tables = np.array(tables, dtype=np.int32, copy=True)
    ctx = np.array(ctx, dtype=np.int32, copy=True)
    refs = np.array(refs, dtype=np.int32, copy=True)
    for parent, child in np.asarray(parent_child, dtype=np.int64).reshape(-1, 2):
        nb = num_blocks_for(int(ctx[parent]), block_size)
        tables[child, :nb] = tables[parent, :nb]
        ctx[child] = ctx[parent]
        for b in tables[parent, :nb]:
            refs[b] += 1
    return tables, ctx, refs


def free_seqs_ref(tables, ctx, refs, stack, free_top, seq_ids, block_size):
    """Drop each listed sequence: every block loses a reference and blocks left with none go
    back on the free stack (in table order, sequence by sequence); the length becomes 0 and
    the freed table entries -1."""
    tables = np.array(tables, dtype=np.int32, copy=True)
    ctx = np.array(ctx, dtype=np.int32, copy=True)
    refs = np.array(refs, dtype=np.int32, copy=True)
    stack = np.array(stack, dtype=np.int32, copy=True)
    top = int(free_top)
    for s in np.asarray(seq_ids, dtype=np.int64):
        nb = num_blocks_for(int(ctx[s]), block_size)
        for j in range(nb):
            b = int(tables[s, j])
            refs[b] -= 1
            if refs[b] == 0:
                stack[top] = b
                top += 1
            tables[s, j] = -1
        ctx[s] = 0
    return tables, ctx, refs, stack, top


_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = _FNV_OFFSET) -> int:
    """64-bit FNV-1a (Fowler, Noll, Vo): for each byte, h ^= byte, then h *= 2^40 + 2^8 + 0xb3
    modulo 2^64, from the offset basis 0xcbf29ce484222325."""
    for byte in data:
        h ^= byte
        h = (h * _FNV_PRIME) & _MASK64
    return h


def block_hashes_ref(token_ids, num_tokens, block_size) -> np.ndarray:
    """Prefix hashes of full blocks, uint64 [S, max_tokens // bs]: block j's hash covers the
    sequence's tokens 0 .. (j+1)*bs - 1, so two sequences share block j's hash exactly when
    (up to collisions) they share that whole prefix, which is what lets a fixed system prompt's
    blocks be reused (yongjin360.com §5.1, prefix caching).  g_j = FNV-1a-64 of the block's
    token ids (int32, little-endian); h_j = FNV-1a-64 of the 16 bytes h_{j-1} || g_j
    (little-endian, h_{-1} = 0).  Blocks that are not full get 0."""
    tok = np.asarray(token_ids, dtype=np.int32)
    S, T = tok.shape
    bs = int(block_size)
    out = np.zeros((S, T // bs), dtype=np.uint64)
    for s in range(S):
        h = 0
        for j in range(int(num_tokens[s]) // bs):
            g = fnv1a64(tok[s, j * bs:(j + 1) * bs].astype('<i4').tobytes())
            h = fnv1a64(int(h).to_bytes(8, "little") + int(g).to_bytes(8, "little"))
            out[s, j] = h
    return out
