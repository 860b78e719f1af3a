"""The decode step and prefill captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches): the library allocates nothing, never synchronises and records no memset, so a
serving loop can replay a captured step.  Every replay, with unrelated eager work and
synchronisations between replays, gives the eager result bit for bit."""

from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

from gpu_helpers import Uploaded, assert_attention_close, bits, live_vmax, need_gpu, oracle_decode, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_decode_step_graph_replays(kernel):
    import torch
    dev = need_gpu()
    spec = W.scaled(W.CONFIGS["shared_prefix"], num_seqs=8, num_heads=8, num_kv_heads=2,
                    dtype="bf16", shared_prefix=64, lengths=("uniform", 1, 200))
    case = W.build_case(spec)
    say(f"graph replay: decode step, {kernel}, {len(case.block_mapping)} copy pairs, "
        f"{len(case.slot_mapping)} new tokens")
    u = Uploaded(case, dev)
    P = 64
    ws = torch.empty(max(256, ops.workspace_bytes(spec.num_seqs, spec.num_heads, spec.num_kv_heads,
                                                  spec.head_dim, spec.block_size,
                                                  case.max_blocks_per_seq, P)),
                     dtype=torch.uint8, device=dev)

    def step():
        if len(case.block_mapping):
            ops.copy_blocks(u.kc, u.vc, u.pairs)
        ops.reshape_and_cache(u.nk, u.nv, u.kc, u.vc, u.slots)
        ops.decode_partitions(u.out, u.q, u.kc, u.vc, u.bt, u.cl, float(case.scale), ws,
                              partition_size=P, kernel=kernel, shared_blocks=True)
        ops.decode_merge(u.out, u.cl, spec.num_kv_heads, spec.block_size, case.max_blocks_per_seq,
                         ws, partition_size=P)

    step()                       # eager (copy-on-write and the append are idempotent)
    torch.cuda.synchronize()
    eager = W.from_torch(u.out, "bf16").copy()
    kc_eager = u.kc.clone()

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()                   # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        u.out.view(torch.int16).fill_(-1)                           # NaN pattern
        junk = torch.randn(1 << 20, device=dev).sum()               # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        got = W.from_torch(u.out, "bf16")
        assert np.array_equal(bits(got, "bf16"), bits(eager, "bf16")), f"replay {r}"
        assert torch.equal(u.kc, kc_eager), f"replay {r}: pool changed"
        del junk
    assert_attention_close(eager, _oracle_after_step(case), "bf16", live_vmax(case), "eager step")


def _oracle_after_step(case):
    import oracle
    kc, vc = case.key_cache, case.value_cache
    if len(case.block_mapping):
        kc, vc = oracle.copy_blocks_ref(kc, vc, case.block_mapping)
    kc, vc = oracle.reshape_and_cache_ref(case.new_key, case.new_value, kc, vc, case.slot_mapping,
                                          case.block_size)
    return oracle_decode(case, kc, vc)


def test_prefill_graph_replays():
    import torch
    dev = need_gpu()
    spec = W.PrefillSpec("g", 31, 3, 8, 2, 128, "bf16", 16, ("fixed", [0, 40, 300]),
                         ("fixed", [70, 1, 129]))
    case = W.build_prefill_case(spec)
    say("graph replay: prefill")
    q = W.to_torch(case.query, "bf16", dev)
    kc = W.to_torch(case.pool.key_cache, "bf16", dev)
    vc = W.to_torch(case.pool.value_cache, "bf16", dev)
    bt = torch.from_numpy(np.ascontiguousarray(case.pool.block_tables, np.int32)).to(dev)
    qsl = torch.from_numpy(np.ascontiguousarray(case.query_start_loc, np.int32)).to(dev)
    cl = torch.from_numpy(np.ascontiguousarray(case.context_lens, np.int32)).to(dev)
    out = torch.empty_like(q)

    def run():
        ops.prefill(out, q, kc, vc, bt, qsl, cl, float(case.scale), case.max_query_len)

    run()
    torch.cuda.synchronize()
    eager = W.from_torch(out, "bf16").copy()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(dev).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(3):
        out.view(torch.int16).fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(W.from_torch(out, "bf16"), "bf16"), bits(eager, "bf16")), r


def test_prefill_fp8_split_graph_replays():
    """pa_prefill_fp8 with its keys split (two launches: the partials, then the merge) over
    E4M3 pools, captured and replayed with unrelated eager work between replays: every replay
    gives the eager bits."""
    import torch
    dev = need_gpu()
    spec = W.PrefillSpec("g8", 32, 3, 8, 2, 128, "bf16", 16, ("fixed", [0, 300, 700]),
                         ("fixed", [70, 40, 129]), kv_dtype="fp8")
    case = W.build_prefill_case(spec)
    say("graph replay: prefill_fp8 with key splits")
    q = W.to_torch(case.query, "bf16", dev)
    kc = W.to_torch(case.pool.key_cache, "fp8", dev)
    vc = W.to_torch(case.pool.value_cache, "fp8", dev)
    bt = torch.from_numpy(np.ascontiguousarray(case.pool.block_tables, np.int32)).to(dev)
    qsl = torch.from_numpy(np.ascontiguousarray(case.query_start_loc, np.int32)).to(dev)
    cl = torch.from_numpy(np.ascontiguousarray(case.context_lens, np.int32)).to(dev)
    out = torch.empty_like(q)
    need = ops.prefill_workspace_bytes(3, q.shape[0], 8, 2, 128, 16, bt.shape[1],
                                       case.max_query_len, 128)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ks, vs = W.FP8_DRAW_SCALE, W.FP8_DRAW_SCALE * 0.5

    def run():
        ops.prefill_fp8(out, q, kc, vc, bt, qsl, cl, float(case.scale), case.max_query_len,
                        ks, vs, kv_split=128, workspace=ws)

    run()
    torch.cuda.synchronize()
    eager = W.from_torch(out, "bf16").copy()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(dev).wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    junk = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    for r in range(3):
        out.view(torch.int16).fill_(-1)
        ws.fill_(0xFF)
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(W.from_torch(out, "bf16"), "bf16"), bits(eager, "bf16")), r
