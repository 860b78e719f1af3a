"""The matrix-core decode with one workgroup walking several consecutive partitions of a
(sequence, KV head).

The library lets a workgroup walk partitions of a multiple of 128 tokens, up to about 1024
tokens and at most 4 / 2 / 1 partitions at 4 / 8 / 16 query heads per workgroup, while the grid
keeps at least 2048 workgroups; the shapes below make it walk 4, 2 and 1.  Each wave leaves its
state in the partition's LDS slot when it ends a partition, and the last wave to finish the
workgroup merges every partition.  Lengths fall on and around partition, chunk and block edges,
and the table is sized for the longest.  Each sequence's result must meet the attention bar
against the oracle, and must be bit-identical to the same sequences decoded four at a time (a
grid far below 2048 workgroups, so one partition per workgroup): every partition's partial is
the same whichever workgroup computes it."""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_attention_close, need_gpu, say
from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

pytestmark = pytest.mark.gpu

K_SCALE = np.float32(W.FP8_DRAW_SCALE)
V_SCALE = np.float32(W.FP8_DRAW_SCALE * 0.5)


def _lengths(S, width, P, seed):
    edges = [1, 15, 16, 17, P - 1, P, P + 1, 2 * P - 1, 2 * P, 2 * P + 1, 4 * P, 4 * P + 1,
             width - 1, width]
    rng = np.random.default_rng(seed)
    rest = rng.integers(1, width + 1, size=S - len(edges))
    return [int(x) for x in edges + list(rest) if 1 <= int(x) <= width][:S]


# (Hq, Hkv, S, table tokens, P, head dim) and the partitions per workgroup the library picks
SHAPES = [
    (32, 8, 64, 1664, 128, 128),    # 4 heads per workgroup, 13 partitions -> 4 per workgroup
    (32, 8, 64, 1664, 256, 128),    # 7 partitions -> 2 per workgroup
    (32, 8, 64, 1664, 384, 128),    # 5 partitions -> 1 per workgroup (the grid would be too small)
    (64, 8, 64, 1664, 128, 128),    # 8 heads per workgroup -> 2 (LDS slots for 2)
    (32, 2, 128, 3712, 128, 128),   # 16 heads per workgroup -> 1
    (32, 8, 64, 1664, 128, 64),     # head dim 64, 4 heads -> 4
    (64, 8, 64, 1664, 128, 64),     # head dim 64, 8 heads -> 4
    (32, 8, 64, 1664, 128, 256),    # head dim 256, 4 heads -> 2
    (32, 8, 64, 1664, 128, 80),     # head dim 80 (128-dim products), 4 heads -> 4
]


CASES = [(*shape, kv) for shape in SHAPES for kv in ("bf16", "f16", "fp8")]


@pytest.mark.parametrize("Hq,Hkv,S,width,P,D,kv", CASES)
def test_partition_groups(Hq, Hkv, S, width, P, D, kv):
    import torch
    dev = need_gpu()
    dtype = "f16" if kv == "f16" else "bf16"
    lens = _lengths(S, width, P, seed=Hq * 1000 + P)
    S = len(lens)
    spec = W.CaseSpec("pgroups", 700 + P + Hq + D, S, Hq, Hkv, D, dtype, 16, ("fixed", lens),
                      new_tokens=("free", 0), max_blocks_per_seq=width // 16,
                      kv_dtype="fp8" if kv == "fp8" else None)
    case = W.build_case(spec)
    pdt = "fp8" if kv == "fp8" else dtype
    kc = W.to_torch(case.key_cache, pdt, dev)
    vc = W.to_torch(case.value_cache, pdt, dev)
    q = W.to_torch(case.query, dtype, dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    say(f"partition groups {kv}: S={S} Hq={Hq} Hkv={Hkv} width={width} P={P}")

    def run(rows):
        out = torch.empty((len(rows), Hq, D), dtype=q.dtype, device=dev)
        idx = torch.tensor(rows, dtype=torch.int64, device=dev)
        qs, bts, cls = q.index_select(0, idx), bt.index_select(0, idx), cl.index_select(0, idx)
        if kv == "fp8":
            ops.decode_fp8(out, qs, kc, vc, bts, cls, float(case.scale), float(K_SCALE),
                           float(V_SCALE), partition_size=P)
        else:
            ops.decode(out, qs, kc, vc, bts, cls, float(case.scale), partition_size=P,
                       kernel="mfma")
        torch.cuda.synchronize()
        return W.from_torch(out, dtype)

    full = run(list(range(S)))
    if kv == "fp8":
        ref = oracle.decode_fp8_ref(case.query, case.key_cache, case.value_cache, case.block_tables,
                                    case.context_lens, 16, case.scale, dtype, K_SCALE, V_SCALE)
        vpool, vdt = oracle.dequantize_fp8(case.value_cache, V_SCALE), "f64"
    else:
        ref = oracle.decode_ref(case.query, case.key_cache, case.value_cache, case.block_tables,
                                case.context_lens, 16, case.scale, dtype)
        vpool, vdt = case.value_cache, dtype
    vmax = max(float(np.max(np.abs(oracle.resolve_sequence(vpool, case.block_tables[s], n, 16, vdt))))
               for s, n in enumerate(lens))
    assert_attention_close(full, ref, dtype, vmax, f"partition groups {kv} Hq{Hq}/Hkv{Hkv} P{P}")
    # the same sequences four at a time: one partition per workgroup, the same bits
    for b0 in range(0, S, S // 4):
        rows = [b0, b0 + 1, b0 + 2, b0 + 3]
        sub = run(rows)
        assert np.array_equal(sub.view(np.uint16), full[rows].view(np.uint16)), rows
