"""pa_decode_noalloc, the decode entry point for callers that cannot allocate: its split-KV
partials live in the library's fixed per-GPU array instead of a caller's workspace.

Through the C ABI: two calls in a row on one GPU (the second smaller, so it runs over what the
first left in the array) give the same bits as pa_decode_ex with a workspace of its own, for the
vector-ALU and the matrix-core kernels, and both meet the attention bar against the oracle.
Shapes whose partials do not fit the array are refused on the host."""

import ctypes

import numpy as np
import pytest

from gpu_helpers import Uploaded, assert_attention_close, live_vmax, need_gpu, oracle_decode, say
from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

SCRATCH_BYTES = 32 << 20   # PA_DECODE_NOALLOC_SCRATCH_BYTES
_p, _i = ctypes.c_void_p, ctypes.c_int32


def _fn(lib):
    fn = lib.pa_decode_noalloc
    fn.restype = _i
    fn.argtypes = [_p] * 6 + [_i] * 7 + [ctypes.c_float, _i, _i, _i, ctypes.c_uint32, _p]
    return fn


def _call(lib, up: Uploaded, partition_size, kernel):
    import torch
    sp = up.case.spec
    NB, Hkv, BS, D = up.kc.shape
    st = _fn(lib)(_p(up.out.data_ptr()), _p(up.q.data_ptr()), _p(up.kc.data_ptr()),
                  _p(up.vc.data_ptr()), _p(up.bt.data_ptr()), _p(up.cl.data_ptr()), sp.num_seqs,
                  sp.num_heads, Hkv, D, BS, NB, up.bt.shape[1], float(up.case.scale),
                  {"f32": 0, "f16": 1, "bf16": 2}[sp.dtype], partition_size,
                  ops.KERNELS[kernel], 0, _p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_refuses_oversized_partials():
    """A shape whose partials exceed the array returns PA_ERR_WORKSPACE (host-side check)."""
    lib = ops.load()
    # 4096 sequences x 32 heads x 16 partitions x (128 + 2) floats = 1.06 GB of partials
    need = lib.pa_decode_workspace_bytes(4096, 32, 32, 128, 16, 512, 512)
    assert need > SCRATCH_BYTES
    st = _fn(lib)(_p(1), _p(1), _p(1), _p(1), _p(1), _p(1), 4096, 32, 32, 128, 16, 100000, 512,
                  0.1, 2, 512, 0, 0, None)
    assert st == 4
    assert _fn(lib)(None, None, None, None, None, None, 0, 32, 32, 128, 16, 1, 4, 0.1, 2, 0, 0, 0,
                    None) == 0                   # empty batch: no-op
    assert _fn(lib)(None, _p(1), _p(1), _p(1), _p(1), _p(1), 4, 8, 2, 128, 16, 10, 4, 0.1, 2, 0,
                    0, 0, None) == 1             # null output


def _case(seed, lengths, Hq, Hkv, dtype="bf16", bs=16, D=128):
    return W.build_case(W.CaseSpec("noalloc", seed, len(lengths), Hq, Hkv, D, dtype, bs,
                                   ("fixed", list(lengths)), new_tokens=("free", 0)))


@pytest.mark.gpu
@pytest.mark.parametrize("kernel,Hq,Hkv,D", [("valu", 8, 8, 128), ("mfma", 16, 4, 128),
                                            ("mfma", 16, 4, 80)])
def test_noalloc_two_calls_match_workspace_path(kernel, Hq, Hkv, D):
    import torch
    dev = need_gpu()
    lib = ops.load()
    big = _case(400, (3000, 1, 17, 2049, 512, 777), Hq, Hkv, D=D)
    small = _case(401, (100, 700, 5), Hq, Hkv, D=D)
    for label, case, P in (("first (larger)", big, 256), ("second (smaller)", small, 64)):
        up = Uploaded(case, dev)
        sp = case.spec
        need = lib.pa_decode_workspace_bytes(sp.num_seqs, Hq, Hkv, D, 16, up.bt.shape[1], P)
        say(f"noalloc {kernel} {label}: S={sp.num_seqs} Hq={Hq} Hkv={Hkv} D={D} P={P} "
            f"partials={need} B")
        assert 0 < need <= SCRATCH_BYTES
        up.out.fill_(float("nan"))
        st = _call(lib, up, P, kernel)
        assert st == 0, ops.status_string(st)
        torch.cuda.synchronize()
        got = W.from_torch(up.out, sp.dtype).copy()
        want = up.decode(kernel=kernel, partition_size=P)   # pa_decode_ex, its own workspace
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), label
        assert_attention_close(got, oracle_decode(case), sp.dtype, live_vmax(case),
                               f"noalloc {kernel} {label}")
