"""GPU parity of the 8-bit (E4M3) KV cache: pa_reshape_and_cache_fp8 bit-exact against the
oracle's quantisation, pa_decode_fp8 against the float64 oracle on the dequantized pools
(attention bar of ``gpu_helpers``: the quantisation is in the stored data, identical for both
sides), and the block copies on 8-bit pools.  All calls go through the C ABI."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

from gpu_helpers import assert_attention_close, compare_every_sequence, need_gpu, say, snapshot_seq

pytestmark = pytest.mark.gpu

K_SCALE = np.float32(W.FP8_DRAW_SCALE)       # pools drawn as N(0,1) / (1/64)
V_SCALE = np.float32(W.FP8_DRAW_SCALE * 0.5)


def _spec(dtype, bs, Hq, Hkv, lengths, seed, D=128, **kw):
    kw.setdefault("new_tokens", ("free", 0))
    return W.CaseSpec("fp8", seed, len(lengths), Hq, Hkv, D, dtype, bs, ("fixed", list(lengths)),
                      kv_dtype="fp8", **kw)


def _upload(case, dev):
    import torch
    kc = W.to_torch(case.key_cache, "fp8", dev)
    vc = W.to_torch(case.value_cache, "fp8", dev)
    bt = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).to(dev)
    cl = torch.from_numpy(np.ascontiguousarray(case.context_lens, np.int32)).to(dev)
    q = W.to_torch(case.query, case.dtype, dev)
    return q, kc, vc, bt, cl


def _vmax(case, vc=None):
    vc = case.value_cache if vc is None else vc
    m = 0.0
    for s in range(case.spec.num_seqs):
        n = int(case.context_lens[s])
        if n > 0:
            V = oracle.resolve_sequence(vc, case.block_tables[s], n, case.block_size, "f64")
            m = max(m, float(np.nanmax(np.abs(V))))
    return m


def _oracle(case, kc=None, vc=None):
    return oracle.decode_fp8_ref(case.query, case.key_cache if kc is None else kc,
                                 case.value_cache if vc is None else vc, case.block_tables,
                                 case.context_lens, case.block_size, case.scale, case.dtype,
                                 K_SCALE, V_SCALE)


MATRIX = [
    ("bf16", 16, 8, 8, (1, 15, 16, 17, 200, 1000), 0),
    ("f16", 16, 4, 4, (3, 64, 333, 70), 48),
    ("bf16", 32, 8, 2, (1, 31, 500, 90), 0),          # GQA, 2 heads per workgroup
    ("f16", 32, 6, 2, (40, 1, 129), 64),              # G = 3
    ("bf16", 16, 4, 1, (2048, 1500), 256),            # G = 4, many partitions
    ("bf16", 64, 8, 8, (1, 63, 64, 65, 700), 128),    # 64-token blocks
    ("f16", 128, 4, 2, (1, 127, 129, 900), 0),        # 128-token blocks
    ("bf16", 8, 8, 2, (1, 7, 8, 9, 300), 16),         # 8-token blocks, one-chunk partitions
    ("f16", 16, 16, 4, (1, 15, 17, 640, 333), 64),    # G = 4 with f16 queries (matrix cores)
    ("bf16", 32, 16, 2, (5, 100, 1100), 0),           # G = 8: 8 heads per workgroup
    ("bf16", 16, 12, 1, (1, 16, 300, 777), 128),      # G = 12: three 4-head workgroups per KV head
    ("bf16", 16, 32, 1, (17, 513, 1500), 0),          # G = 32: two 16-head workgroups
]


@pytest.mark.parametrize("dtype,bs,Hq,Hkv,lengths,P", MATRIX)
def test_decode_fp8_matches_oracle(dtype, bs, Hq, Hkv, lengths, P):
    import torch
    dev = need_gpu()
    case = W.build_case(_spec(dtype, bs, Hq, Hkv, lengths, seed=200 + len(lengths) + bs + Hq))
    say(f"decode_fp8 {dtype} bs{bs} Hq{Hq} Hkv{Hkv} lengths={lengths} P={P}")
    q, kc, vc, bt, cl = _upload(case, dev)
    out = torch.empty_like(q)
    ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE),
                   partition_size=P)
    torch.cuda.synchronize()
    got = W.from_torch(out, dtype)
    vdeq = oracle.dequantize_fp8(case.value_cache, V_SCALE)
    assert_attention_close(got, _oracle(case), dtype, _vmax(case, vdeq), "decode_fp8")


@pytest.mark.parametrize("D", [64, 80, 256])
@pytest.mark.parametrize("dtype,bs,Hq,Hkv,P", [("bf16", 16, 8, 8, 0), ("f16", 8, 8, 2, 64),
                                               ("bf16", 64, 4, 1, 128), ("bf16", 16, 16, 4, 256)])
def test_decode_fp8_head_dims(D, dtype, bs, Hq, Hkv, P):
    """8-bit caches at head dims 64, 80 (rows of 5 sixteen-byte vectors: 3 idle lanes per 8-lane
    row) and 256, on the vector ALUs for every head grouping: against the oracle on the
    dequantized pools, and bit-identical when every unread slot holds a NaN code and unused
    table entries hold junk."""
    import torch
    dev = need_gpu()
    lengths = (1, 15, 16, 17, 200, 1000, 2049)
    spec = _spec(dtype, bs, Hq, Hkv, lengths, seed=240 + D + bs + Hq, D=D)
    say(f"decode_fp8 D={D} {dtype} bs{bs} Hq{Hq} Hkv{Hkv} P={P}")
    outs = []
    for kw in ({}, {"poison": True, "table_fill": 2**31 - 1}):
        case = W.build_case(spec, **kw)
        q, kc, vc, bt, cl = _upload(case, dev)
        out = torch.empty_like(q)
        ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE),
                       partition_size=P)
        torch.cuda.synchronize()
        outs.append(W.from_torch(out, dtype))
        if not kw:
            vdeq = oracle.dequantize_fp8(case.value_cache, V_SCALE)
            assert_attention_close(outs[0], _oracle(case), dtype, _vmax(case, vdeq),
                                   f"decode_fp8 D={D}")
    assert np.array_equal(outs[1].view(np.uint16), outs[0].view(np.uint16))


@pytest.mark.parametrize("D", [64, 80, 256])
def test_fp8_step_head_dims(D):
    """reshape_and_cache_fp8 then decode at head dims 64 / 80 / 256: the quantised writes are
    bit-exact over the whole pool and the decode meets the bar against the oracle chain."""
    import torch
    dev = need_gpu()
    spec = W.CaseSpec("fp8step", 250 + D, 5, 8, 2, D, "bf16", 16, ("fixed", [1, 16, 17, 300, 64]),
                      kv_dtype="fp8")
    case = W.build_case(spec)
    q, kc, vc, bt, cl = _upload(case, dev)
    nk, nv = W.to_torch(case.new_key, "bf16", dev), W.to_torch(case.new_value, "bf16", dev)
    ops.reshape_and_cache_fp8(nk, nv, kc, vc, torch.from_numpy(case.slot_mapping).to(dev),
                              float(K_SCALE), float(V_SCALE))
    out = torch.empty_like(q)
    ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE))
    torch.cuda.synchronize()
    k2, v2 = oracle.reshape_and_cache_fp8_ref(case.new_key, case.new_value, case.key_cache,
                                              case.value_cache, case.slot_mapping, 16, "bf16",
                                              K_SCALE, V_SCALE)
    assert np.array_equal(W.from_torch(kc, "fp8"), k2)
    assert np.array_equal(W.from_torch(vc, "fp8"), v2)
    assert_attention_close(W.from_torch(out, "bf16"), _oracle(case, k2, v2), "bf16",
                           _vmax(case, oracle.dequantize_fp8(v2, V_SCALE)), f"fp8 step D={D}")


@pytest.mark.parametrize("heads", [(4, 4), (8, 2)])
def test_decode_fp8_poison_and_junk_tables(heads):
    """NaN codes in every slot no sequence reads and junk table entries: same bits as the clean
    run (vector-ALU kernel for G = 1, matrix cores for G = 4)."""
    import torch
    dev = need_gpu()
    spec = _spec("bf16", 16, heads[0], heads[1], (1, 15, 16, 33, 100), seed=210, max_blocks_per_seq=12)
    outs = []
    for kw in ({}, {"poison": True, "table_fill": -1}, {"poison": True, "table_fill": 2**31 - 1}):
        case = W.build_case(spec, **kw)
        q, kc, vc, bt, cl = _upload(case, dev)
        out = torch.empty_like(q)
        ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE))
        torch.cuda.synchronize()
        outs.append(W.from_torch(out, "bf16"))
    assert np.all(np.isfinite(oracle.storage_to_f64(outs[0], "bf16")))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_reshape_and_cache_fp8_bit_exact(dtype):
    """Quantised writes equal the oracle's bit for bit, including saturated values (inputs up
    to ~40 / scale 0.05 = 800 > 448), skipped (-1) and out-of-pool slots."""
    import torch
    dev = need_gpu()
    rng = np.random.default_rng(5)
    NB, Hkv, bs, d, N = 40, 4, 16, 128, 37
    kc0 = rng.integers(0, 0x7E, size=(NB, Hkv, bs, d), dtype=np.uint8)
    vc0 = rng.integers(0, 0x7E, size=(NB, Hkv, bs, d), dtype=np.uint8)
    key = W.round_to_storage(rng.standard_normal((N, Hkv, d)).astype(np.float32) * 10, dtype)
    val = W.round_to_storage(rng.standard_normal((N, Hkv, d)).astype(np.float32) * 0.01, dtype)
    slots = rng.choice(NB * bs, size=N, replace=False).astype(np.int64)
    slots[3], slots[9] = -1, NB * bs + 5
    ks, vs = np.float32(0.05), np.float32(1e-4)
    want_k, want_v = oracle.reshape_and_cache_fp8_ref(key, val, kc0, vc0, slots, bs, dtype, ks, vs)
    kc, vc = W.to_torch(kc0, "fp8", dev), W.to_torch(vc0, "fp8", dev)
    ops.reshape_and_cache_fp8(W.to_torch(key, dtype, dev), W.to_torch(val, dtype, dev), kc, vc,
                              torch.from_numpy(slots).to(dev), float(ks), float(vs))
    torch.cuda.synchronize()
    got_k, got_v = W.from_torch(kc, "fp8"), W.from_torch(vc, "fp8")
    say(f"  reshape_fp8 {dtype}: saturated codes {int(np.sum((want_k & 0x7F) == 0x7E))}")
    assert np.array_equal(got_k, want_k)
    assert np.array_equal(got_v, want_v)


def test_fp8_step_append_then_decode():
    """reshape_and_cache_fp8 of each sequence's new token, then decode over the updated 8-bit
    pools, against the oracle chain (quantise -> store -> dequantise -> attend)."""
    import torch
    dev = need_gpu()
    spec = W.CaseSpec("fp8step", 220, 5, 8, 2, 128, "bf16", 16, ("fixed", [1, 16, 17, 300, 64]),
                      kv_dtype="fp8")
    case = W.build_case(spec)
    q, kc, vc, bt, cl = _upload(case, dev)
    nk, nv = W.to_torch(case.new_key, "bf16", dev), W.to_torch(case.new_value, "bf16", dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    ops.reshape_and_cache_fp8(nk, nv, kc, vc, slots, float(K_SCALE), float(V_SCALE))
    out = torch.empty_like(q)
    ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE))
    torch.cuda.synchronize()
    k2, v2 = oracle.reshape_and_cache_fp8_ref(case.new_key, case.new_value, case.key_cache,
                                              case.value_cache, case.slot_mapping, 16, "bf16",
                                              K_SCALE, V_SCALE)
    assert np.array_equal(W.from_torch(kc, "fp8"), k2)
    ref = _oracle(case, k2, v2)
    assert_attention_close(W.from_torch(out, "bf16"), ref, "bf16",
                           _vmax(case, oracle.dequantize_fp8(v2, V_SCALE)), "fp8 step")


def test_fp8_block_copies():
    """copy_blocks and swap_blocks move 8-bit blocks bit for bit."""
    import torch
    dev = need_gpu()
    rng = np.random.default_rng(7)
    pool = rng.integers(0, 256, size=(20, 8, 16, 128), dtype=np.uint8)
    kc, vc = W.to_torch(pool, "fp8", dev), W.to_torch(pool[::-1].copy(), "fp8", dev)
    pairs = np.array([[1, 5], [7, 2], [19, 0]], np.int64)
    ops.copy_blocks(kc, vc, torch.from_numpy(pairs).to(dev))
    host_k = torch.zeros((6, 8, 16, 128), dtype=torch.uint8).pin_memory()
    host_v = torch.zeros_like(host_k).pin_memory()
    sw = np.array([[5, 0], [2, 3]], np.int64)
    ops.swap_blocks(kc, vc, host_k, host_v, torch.from_numpy(sw).to(dev))
    torch.cuda.synchronize()
    wk, wv = oracle.copy_blocks_ref(pool, pool[::-1].copy(), pairs)
    assert np.array_equal(W.from_torch(kc, "fp8"), wk)
    assert np.array_equal(W.from_torch(vc, "fp8"), wv)
    hk, hv = oracle.swap_blocks_ref(wk, wv, np.zeros((6, 8, 16, 128), np.uint8),
                                    np.zeros((6, 8, 16, 128), np.uint8), sw)
    assert np.array_equal(host_k.numpy(), hk) and np.array_equal(host_v.numpy(), hv)


@pytest.mark.parametrize("name", ["llama7b_bs16_fp8", "gqa_long_fp8"])
def test_decode_fp8_full_size_every_sequence(name):
    """The Llama-7B-shaped (vector ALUs) and GQA long-context (matrix cores, 512-token
    partitions) steps over an 8-bit cache, pools drawn on the GPU, in the benchmark's launch
    configuration: reshape_and_cache_fp8 of each sequence's new token, then pa_decode_fp8.
    Every sequence is checked against the oracle chain (quantise -> store -> dequantise ->
    attend), the whole output at the attention bar, and every block a sequence reads after the
    step (its new token's block among them) bit for bit."""
    import torch
    dev = need_gpu()
    spec = W.CONFIGS[name]
    case = W.build_case(spec, device=dev)
    say(f"decode_fp8 full size {name}: {case.num_blocks} blocks")
    kc, vc = case.key_cache, case.value_cache
    snaps = [snapshot_seq(case, s, kc, vc, pool_dtype="fp8") for s in range(spec.num_seqs)]
    q = W.to_torch(case.query, "bf16", dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    ops.reshape_and_cache_fp8(W.to_torch(case.new_key, "bf16", dev),
                              W.to_torch(case.new_value, "bf16", dev), kc, vc,
                              torch.from_numpy(case.slot_mapping).to(dev), float(K_SCALE),
                              float(V_SCALE))
    ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE),
                   partition_size=spec.partition_size)
    torch.cuda.synchronize()

    def oracle_seq(snap):
        s = snap["s"]
        k2, v2 = oracle.reshape_and_cache_fp8_ref(case.new_key[s:s + 1], case.new_value[s:s + 1],
                                                  snap["mk"], snap["mv"], snap["slot"],
                                                  case.block_size, "bf16", K_SCALE, V_SCALE)
        ref = oracle.decode_fp8_ref(case.query[s:s + 1], k2, v2, snap["table"],
                                    np.array([snap["n"]], np.int32), case.block_size, case.scale,
                                    "bf16", K_SCALE, V_SCALE)
        V = oracle.resolve_sequence(oracle.dequantize_fp8(v2, V_SCALE), snap["table"][0],
                                    snap["n"], case.block_size, "f64")
        return ref[0], k2, v2, float(np.max(np.abs(V)))

    compare_every_sequence(case, W.from_torch(out, "bf16"), kc, vc, snaps, oracle_seq,
                           f"fp8 full size {name}", pool_dtype="fp8")
    del kc, vc, case, snaps
    torch.cuda.empty_cache()


@pytest.mark.parametrize("heads", [(8, 8), (8, 2)])
def test_decode_fp8_two_launches_equal_one(heads):
    """pa_decode_fp8_partitions followed by pa_decode_merge (the two launches the benchmark
    brackets with events) give the same bits as pa_decode_fp8, for the vector-ALU (G = 1) and
    matrix-core (G = 4) paths, split and single pass."""
    import torch
    dev = need_gpu()
    case = W.build_case(_spec("bf16", 16, heads[0], heads[1], (5, 300, 1200, 17), seed=230))
    q, kc, vc, bt, cl = _upload(case, dev)
    sp = case.spec
    for P in (0, 64, 256):
        say(f"fp8 two launches: Hq={heads[0]} Hkv={heads[1]} P={P}")
        one = torch.empty_like(q)
        ops.decode_fp8(one, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE),
                       partition_size=P)
        nb = ops.workspace_bytes(sp.num_seqs, sp.num_heads, sp.num_kv_heads, 128, 16,
                                 case.max_blocks_per_seq, P)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        two = torch.empty_like(q)
        ops.decode_fp8_partitions(two, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE),
                                  float(V_SCALE), ws, partition_size=P)
        ops.decode_merge(two, cl, sp.num_kv_heads, 16, case.max_blocks_per_seq, ws, partition_size=P)
        torch.cuda.synchronize()
        assert np.array_equal(W.from_torch(one, "bf16").view(np.uint16),
                              W.from_torch(two, "bf16").view(np.uint16)), P


@pytest.mark.parametrize("dtype,Hq,Hkv", [("bf16", 4, 4), ("f16", 4, 4), ("bf16", 16, 4),
                                          ("f16", 16, 4)])
def test_decode_fp8_every_code_one_token(dtype, Hq, Hkv):
    """Every finite E4M3 code as a value, in one-token contexts: the output is that token's
    dequantized V row, exactly (a code times the power-of-two value scale is exact in both
    16-bit types), on the vector-ALU kernel (G = 1) and the matrix-core kernel (G = 4)."""
    import torch
    dev = need_gpu()
    S = 8
    case = W.build_case(_spec(dtype, 16, Hq, Hkv, [1] * S, seed=4242))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 finite
    vc = case.value_cache.copy()
    D = case.spec.head_dim
    for s in range(S):
        blk = int(case.block_tables[s][0])
        for g in range(Hkv):
            start = ((s * Hkv + g) * D) % len(codes)
            vc[blk, g, 0, :] = np.resize(np.roll(codes, -start), D)
    say(f"decode_fp8 every code {dtype} Hq{Hq} Hkv{Hkv}")
    case.value_cache = vc
    q, kc, vct, bt, cl = _upload(case, dev)
    out = torch.empty_like(q)
    ops.decode_fp8(out, q, kc, vct, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE))
    torch.cuda.synchronize()
    got = W.from_torch(out, dtype)
    ref = oracle.f64_to_storage(_oracle(case), dtype)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    seen = set()
    for s in range(S):
        seen.update(vc[int(case.block_tables[s][0]), :, 0, :].ravel().tolist())
    assert seen == set(codes.tolist())


@pytest.mark.parametrize("scale", [0.0, -0.0883883, -2.0])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_fp8_zero_and_negative_scale(scale, D):
    """Grouped heads over an 8-bit cache (the matrix-core kernel, which compares raw scores and
    carries a negative scale in the query signs): scale 0 gives the mean of V, a negative scale
    reverses the ordering of the scores -- against the oracle, single pass and split."""
    import torch
    dev = need_gpu()
    case = W.build_case(_spec("bf16", 16, 16, 4, (1, 17, 300, 1000), seed=260 + D, D=D))
    case.scale = np.float32(scale)
    q, kc, vc, bt, cl = _upload(case, dev)
    ref = _oracle(case)
    vmax = _vmax(case, oracle.dequantize_fp8(case.value_cache, V_SCALE))
    for P in (0, 64):
        say(f"decode_fp8 D={D} scale={scale} P={P}")
        out = torch.empty_like(q)
        ops.decode_fp8(out, q, kc, vc, bt, cl, float(case.scale), float(K_SCALE), float(V_SCALE),
                       partition_size=P)
        torch.cuda.synchronize()
        assert_attention_close(W.from_torch(out, "bf16"), ref, "bf16", vmax,
                               f"fp8 scale {scale} D={D} P={P}")
