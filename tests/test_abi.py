"""The C-ABI library: it loads, exports every symbol include/pa.h declares, and rejects bad
arguments with the documented status codes before launching anything (no GPU needed: every
call here returns during host-side validation)."""

import ctypes
import subprocess

import pytest

from paged_kv_cache_05_amd import ops


@pytest.fixture(scope="module")
def lib():
    if not ops.LIB_PATH.exists():
        from paged_kv_cache_05_amd.build import build
        build()
    return ops.load()


def test_exports_every_declared_symbol(lib):
    declared = ops.header_symbols()
    assert len(declared) >= 10
    nm = subprocess.run(["nm", "-D", "--defined-only", str(ops.LIB_PATH)], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert getattr(lib, s) is not None


def test_status_strings_and_version(lib):
    for code in range(6):
        s = ops.status_string(code)
        assert s.startswith("PA_")
    assert lib.pa_version() >= 10000


def _decode(lib, **kw):
    a = dict(out=1, q=1, kc=1, vc=1, bt=1, cl=1, S=4, Hq=8, Hkv=2, D=128, BS=16, NB=100, maxb=8,
             scale=0.1, dtype=2, P=0, ws=None, wsb=0, kernel=0, flags=0)
    a.update(kw)
    p = lambda v: ctypes.c_void_p(v) if v else None
    return lib.pa_decode_ex(p(a["out"]), p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), p(a["cl"]),
                            a["S"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"], a["maxb"],
                            a["scale"], a["dtype"], a["P"], p(a["ws"]), a["wsb"], a["kernel"],
                            a["flags"], None)


def test_decode_argument_errors(lib):
    assert _decode(lib, out=0) == 1                  # PA_ERR_NULL_PTR
    assert _decode(lib, bt=0) == 1
    assert _decode(lib, Hq=6, Hkv=4) == 2            # PA_ERR_BAD_SHAPE: heads not a multiple
    assert _decode(lib, S=-1) == 2
    assert _decode(lib, S=2**26, Hq=64, Hkv=64) == 2   # (sequence, head) ids past int32
    assert _decode(lib, maxb=0) == 2
    assert _decode(lib, NB=0) == 2
    assert _decode(lib, P=24) == 2                   # not a multiple of block_size
    assert _decode(lib, scale=float("nan")) == 2
    assert _decode(lib, D=96) == 3                   # PA_ERR_UNSUPPORTED
    assert _decode(lib, BS=4) == 3
    assert _decode(lib, BS=48) == 3
    assert _decode(lib, BS=8, out=0) == 1             # 8-token blocks accepted
    assert _decode(lib, BS=8, P=24) == 2              # partitions hold whole 16-token chunks
    assert _decode(lib, BS=8, P=32, out=0) == 1
    assert _decode(lib, D=80, dtype=0) == 3          # fp32 rows: head_dim 64 or 128 only
    assert _decode(lib, D=256, BS=128, out=0) == 1   # 256 dims and 128-token blocks accepted
    assert _decode(lib, dtype=7) == 3
    assert _decode(lib, kernel=9) == 3
    assert _decode(lib, kernel=2, dtype=0) == 3      # matrix-core path needs f16/bf16
    assert _decode(lib, kernel=2, Hq=6, Hkv=3) == 3  # group of 2
    assert _decode(lib, kernel=2, D=80, out=0) == 1  # matrix cores: head dims 64, 80, 128, 256
    assert _decode(lib, kernel=2, D=64, out=0) == 1
    assert _decode(lib, kernel=2, D=256, out=0) == 1
    assert _decode(lib, flags=0x2) == 3              # unknown flag bit
    assert _decode(lib, flags=0x1, out=0) == 1       # the shared-blocks flag itself is accepted
    assert _decode(lib, maxb=64, P=64) == 4          # split needs a workspace
    assert _decode(lib, maxb=64, P=64, ws=1, wsb=16) == 4
    assert _decode(lib, S=0, out=0, q=0) == 0        # empty batch: no-op


def test_workspace_and_partition_sizes(lib):
    # one pass when the table fits one partition: no workspace
    assert ops.workspace_bytes(4, 2, 2, 64, 16, 7) == 0
    # 256 seqs x 32 heads x 8 partitions x (2 + 128) floats, each region 256-byte aligned
    assert ops.workspace_bytes(256, 32, 32, 128, 16, 256, 512) == 256 * 32 * 8 * 2 * 4 + 256 * 32 * 8 * 128 * 4
    # many (sequence, KV head) units: long partitions, capped at 2048 tokens
    assert ops.auto_partition(256, 32, 32, 128, 16, 256) == 2048
    # few units -> smaller partitions so the grid still fills the GPU (floor 256)
    assert ops.auto_partition(1, 8, 8, 128, 16, 2048) == 256
    assert ops.auto_partition(16, 32, 8, 128, 16, 2048) == 2048
    assert ops.auto_partition(4, 2, 2, 64, 16, 7) >= 7 * 16
    # 112-token table in 48-token partitions: 3 partitions -> 256 B (ml) + 6144 B (o)
    assert ops.workspace_bytes(4, 2, 2, 64, 16, 7, 48) == 256 + 4 * 2 * 3 * 64 * 4
    assert ops.workspace_bytes(4, 2, 2, 96, 16, 7) == 0    # unsupported -> 0


def test_cache_kernel_argument_errors(lib):
    p = ctypes.c_void_p(1)
    assert lib.pa_reshape_and_cache(None, p, p, p, p, 4, 2, 64, 16, 64, 0, None) == 1
    assert lib.pa_reshape_and_cache(p, p, p, p, p, -1, 2, 64, 16, 64, 0, None) == 2
    assert lib.pa_reshape_and_cache(p, p, p, p, p, 4, 2, 3, 16, 64, 1, None) == 3   # 6-byte rows
    assert lib.pa_reshape_and_cache(None, None, None, None, None, 0, 2, 64, 16, 64, 0, None) == 0
    assert lib.pa_copy_blocks(p, p, None, 3, 2, 64, 16, 64, 0, None) == 1
    assert lib.pa_copy_blocks(p, p, p, -2, 2, 64, 16, 64, 0, None) == 2
    assert lib.pa_copy_blocks(p, p, p, 1, 2, 64, 16, 64, 5, None) == 3
    assert lib.pa_copy_blocks(None, None, None, 0, 2, 64, 16, 64, 0, None) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(2, 2, 64)
    kc = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError):
        ops.decode(x, x, kc, kc, torch.zeros(2, 1, dtype=torch.int32),
                   torch.ones(2, dtype=torch.int32), 0.125)


def test_swap_blocks_argument_errors(lib):
    p = ctypes.c_void_p(1)
    assert lib.pa_swap_blocks(p, p, 4, p, None, 4, p, 2, 2, 64, 16, 0, None) == 1
    assert lib.pa_swap_blocks(p, p, -1, p, p, 4, p, 2, 2, 64, 16, 0, None) == 2
    assert lib.pa_swap_blocks(p, p, 4, p, p, 4, p, 2, 1, 3, 1, 1, None) == 3     # 6-byte blocks
    assert lib.pa_swap_blocks(None, None, 4, None, None, 4, None, 0, 2, 64, 16, 0, None) == 0


def _prefill(lib, **kw):
    a = dict(out=1, q=1, kc=1, vc=1, bt=1, qsl=1, cl=1, S=4, Hq=8, Hkv=2, D=128, BS=16, NB=100,
             maxb=8, maxq=64, scale=0.1, dtype=2, flags=0)
    a.update(kw)
    p = lambda v: ctypes.c_void_p(v) if v else None
    return lib.pa_prefill(p(a["out"]), p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), p(a["qsl"]),
                          p(a["cl"]), a["S"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"],
                          a["maxb"], a["maxq"], a["scale"], a["dtype"], a["flags"], None)


def _prefill_ex(lib, **kw):
    a = dict(out=1, q=1, kc=1, vc=1, bt=1, qsl=1, cl=1, S=4, T=100, Hq=8, Hkv=2, D=128, BS=16,
             NB=100, maxb=64, maxq=64, scale=0.1, dtype=2, split=0, ws=0, wsb=0, flags=0)
    a.update(kw)
    p = lambda v: ctypes.c_void_p(v) if v else None
    return lib.pa_prefill_ex(p(a["out"]), p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]),
                             p(a["qsl"]), p(a["cl"]), a["S"], a["T"], a["Hq"], a["Hkv"], a["D"],
                             a["BS"], a["NB"], a["maxb"], a["maxq"], a["scale"], a["dtype"],
                             a["split"], p(a["ws"]), a["wsb"], a["flags"], None)


def _prefill_fp8(lib, **kw):
    a = dict(out=1, q=1, kc=1, vc=1, bt=1, qsl=1, cl=1, S=4, T=100, Hq=8, Hkv=2, D=128, BS=16,
             NB=100, maxb=8, maxq=64, scale=0.1, dtype=2, ks=0.5, vs=0.25, split=1024, ws=0,
             wsb=0, flags=0)
    a.update(kw)
    p = lambda v: ctypes.c_void_p(v) if v else None
    return lib.pa_prefill_fp8(p(a["out"]), p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]),
                              p(a["qsl"]), p(a["cl"]), a["S"], a["T"], a["Hq"], a["Hkv"], a["D"],
                              a["BS"], a["NB"], a["maxb"], a["maxq"], a["scale"], a["dtype"],
                              a["ks"], a["vs"], a["split"], p(a["ws"]), a["wsb"], a["flags"], None)


def test_prefill_fp8_argument_errors(lib):
    """pa_prefill_fp8 checks its arguments like pa_prefill_ex, and its pool scales."""
    assert _prefill_fp8(lib, ks=0.0) == 2                       # PA_ERR_BAD_SHAPE
    assert _prefill_fp8(lib, vs=-1.0) == 2
    assert _prefill_fp8(lib, ks=float("inf")) == 2
    assert _prefill_fp8(lib, vs=float("nan")) == 2
    assert _prefill_fp8(lib, out=0) == 1                        # PA_ERR_NULL_PTR
    assert _prefill_fp8(lib, dtype=0) == 3                      # f32 queries: unsupported
    assert _prefill_fp8(lib, D=256) == 3
    assert _prefill_fp8(lib, D=64, out=0) == 1
    assert _prefill_fp8(lib, flags=0x2) == 3
    assert _prefill_fp8(lib, flags=0x1, out=0) == 1             # bf16 probabilities accepted
    assert _prefill_fp8(lib, split=512, maxb=64) == 4           # a split needs the workspace
    assert _prefill_fp8(lib, S=0, out=0) == 0


def test_plain_decode_argument_errors(lib):
    """pa_decode (the basic entry) checks its arguments like pa_decode_ex."""
    p = lambda v: ctypes.c_void_p(v) if v else None

    def call(**kw):
        a = dict(out=1, q=1, kc=1, vc=1, bt=1, cl=1, S=4, Hq=8, Hkv=2, D=128, BS=16, NB=100,
                 maxb=8, scale=0.1, dtype=2, P=0, ws=0, wsb=0)
        a.update(kw)
        return lib.pa_decode(p(a["out"]), p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), p(a["cl"]),
                             a["S"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"], a["maxb"],
                             a["scale"], a["dtype"], a["P"], p(a["ws"]), a["wsb"], None)
    assert call(out=0) == 1
    assert call(Hq=6, Hkv=4) == 2
    assert call(D=96) == 3
    assert call(P=16, maxb=64) == 4                 # split: a workspace is needed
    assert call(S=0) == 0


def test_prefill_split_plan_and_errors(lib):
    """Key splits: the workspace query, the library's choice (split only small grids), an
    explicit split length, and the argument errors of pa_prefill_ex."""
    ws = lib.pa_prefill_workspace_bytes
    # 4 seqs x 2 KV heads x 2 row tiles = 16 workgroups over 1024-token tables: split
    auto = ws(4, 100, 8, 2, 128, 16, 64, 64, 0)
    assert auto > 0
    # 256 x 32 heads x 4 row tiles: the grid fills the GPU, no split
    assert ws(256, 100, 32, 32, 128, 16, 64, 512, 0) == 0
    assert ws(4, 100, 8, 2, 128, 16, 64, 64, 1024) == 0          # one split covers the table
    two = ws(4, 100, 8, 2, 128, 16, 64, 64, 512)                 # two splits: 100 x 8 x 2 slots
    # token lengths (400 B -> 512), (max, denominator) pairs, fp32 partial outputs
    assert two == 512 + 1600 * 2 * 4 + 1600 * 128 * 4
    # head dim 80: the partials are 80 floats a row; other head dims get no workspace
    assert ws(4, 100, 8, 2, 80, 16, 64, 64, 512) == 512 + 1600 * 2 * 4 + 1600 * 80 * 4
    assert ws(4, 100, 8, 2, 256, 16, 64, 64, 512) == 0
    assert ws(4, 100, 8, 2, 128, 16, 64, 64, 96) == 0            # not a multiple of 64
    assert _prefill_ex(lib, split=96) == 2                       # PA_ERR_BAD_SHAPE
    assert _prefill_ex(lib, split=-64) == 2
    assert _prefill_ex(lib, T=0) == 2                            # splitting needs the token count
    assert _prefill_ex(lib, T=0, split=1024, out=0) == 1         # no split: T unused
    assert _prefill_ex(lib, split=512, ws=1, wsb=two - 1) == 4   # PA_ERR_WORKSPACE
    assert _prefill_ex(lib, split=512) == 4                      # no workspace at all
    assert _prefill_ex(lib, split=512, ws=1, wsb=two, out=0) == 1


def test_prefill_argument_errors(lib):
    assert _prefill(lib, qsl=0) == 1                 # PA_ERR_NULL_PTR
    assert _prefill(lib, out=0) == 1
    assert _prefill(lib, Hq=6, Hkv=4) == 2           # PA_ERR_BAD_SHAPE
    assert _prefill(lib, maxq=-1) == 2
    assert _prefill(lib, NB=0) == 2
    assert _prefill(lib, scale=float("inf")) == 2
    assert _prefill(lib, dtype=0) == 3               # PA_ERR_UNSUPPORTED: f32
    assert _prefill(lib, D=80, out=0) == 1          # head dim 80 accepted
    assert _prefill(lib, D=256) == 3
    assert _prefill(lib, D=64, out=0) == 1          # head dim 64 accepted
    assert _prefill(lib, BS=4) == 3
    assert _prefill(lib, BS=8, out=0) == 1            # 8-token blocks accepted
    assert _prefill(lib, flags=0x2) == 3
    assert _prefill(lib, flags=0x1, out=0) == 1      # the bf16-probabilities flag is accepted
    assert _prefill(lib, S=0, out=0) == 0            # nothing to do
    assert _prefill(lib, maxq=0, out=0) == 0


def test_fp8_argument_errors(lib):
    p = ctypes.c_void_p(1)
    f = lib.pa_reshape_and_cache_fp8
    assert f(p, p, p, p, None, 4, 2, 128, 16, 64, 2, 0.1, 0.1, None) == 1
    assert f(p, p, p, p, p, 4, 2, 128, 16, 64, 0, 0.1, 0.1, None) == 3      # f32 source
    assert f(p, p, p, p, p, 4, 2, 12, 16, 64, 2, 0.1, 0.1, None) == 3       # head_dim % 8
    assert f(p, p, p, p, p, 4, 2, 128, 16, 64, 2, 0.0, 0.1, None) == 2      # scale must be > 0
    assert f(p, p, p, p, p, 4, 2, 128, 16, 64, 2, 0.1, float("nan"), None) == 2
    assert f(None, None, None, None, None, 0, 2, 128, 16, 64, 2, 0.1, 0.1, None) == 0
    d = lib.pa_decode_fp8
    args = [p, p, p, p, p, p, 4, 8, 2, 128, 16, 100, 8, 0.1, 2, 0.1, 0.1, 0, None, 0, 0, None]
    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return d(*a)
    assert call({0: None}) == 1
    assert call({14: 0}) == 3               # f32 queries
    assert call({14: 3}) == 3               # an 8-bit query type
    assert call({9: 96}) == 3               # head_dim 96
    assert call({9: 64, 0: None}) == 1      # head dims 64, 80, 256 accepted (then null output)
    assert call({9: 80, 0: None}) == 1
    assert call({9: 256, 0: None}) == 1
    assert call({20: 2}) == 3               # unknown flag
    assert call({15: float("inf")}) == 2
    assert call({12: 64, 17: 64}) == 4      # split needs a workspace
    assert call({6: 0, 0: None}) == 0
    c = lib.pa_copy_blocks
    assert c(p, p, None, 1, 2, 64, 16, 64, 3, None) == 1   # 8-bit pools accepted (then null map)


def test_block_engine_argument_errors(lib):
    p = ctypes.c_void_p(1)
    a = lib.pa_append_slots
    assert a(p, p, p, p, None, 4, 8, 16, 64, p, 2, p, p, p, p, None) == 1      # no free_top
    assert a(p, p, p, p, p, 4, 8, 16, 64, p, 2, p, p, None, p, None) == 1      # no counter
    assert a(p, p, p, p, p, 4, 0, 16, 64, p, 2, p, p, p, p, None) == 2         # no table width
    assert a(p, p, p, p, p, 4, 8, 16, 64, p, -1, p, p, p, p, None) == 2
    f = lib.pa_fork_seqs
    assert f(p, p, p, 4, 8, 16, 64, None, 2, None) == 1
    assert f(p, p, p, 4, 8, 16, 64, None, 0, None) == 0
    r = lib.pa_free_seqs
    assert r(p, p, p, None, p, 4, 8, 16, 64, p, 1, None) == 1
    assert r(p, p, p, p, p, 4, 8, 16, 64, None, 0, None) == 0
    c = lib.pa_copy_blocks_counted
    assert c(p, p, p, None, 4, 2, 64, 16, 64, 1, None) == 1
    assert c(p, p, p, p, 0, 2, 64, 16, 64, 1, None) == 0
    h = lib.pa_block_hashes
    assert h(p, p, 4, 64, 0, p, None) == 2
    assert h(p, None, 4, 64, 16, p, None) == 1
    assert h(None, None, 4, 8, 16, None, None) == 0                            # no full block


def test_read_tiles_argument_errors(lib):
    p = lambda v: ctypes.c_void_p(v) if v else None
    f = lib.pa_read_tiles
    assert f(p(1), 10, 4096, None, 4, None, None) == 1          # PA_ERR_NULL_PTR
    assert f(None, 10, 4096, None, 4, p(1), None) == 1
    assert f(p(1), 10, 4096, None, -1, p(1), None) == 2         # PA_ERR_BAD_SHAPE
    assert f(p(1), 0, 4096, None, 4, p(1), None) == 2
    assert f(p(1), 10, 4096, None, 11, p(1), None) == 2         # contiguous run past the buffer
    assert f(p(1), 10, 4096, p(1), 11, None, None) == 1         # scattered ids may repeat tiles
    assert f(p(1), 10, 3000, None, 4, p(1), None) == 3          # PA_ERR_UNSUPPORTED tile size
    assert f(p(1), 10, 16384, None, 4, p(1), None) == 3
    assert f(None, 10, 4096, None, 0, None, None) == 0          # nothing to read: no-op


def test_empty_batch_sizes(lib):
    """An empty batch needs no workspace and no split (no division by the unit count)."""
    assert lib.pa_decode_workspace_bytes(0, 32, 32, 128, 16, 64, 0) == 0
    assert lib.pa_decode_auto_partition(0, 32, 8, 128, 16, 64) >= 64 * 16   # one pass
    assert lib.pa_decode_workspace_bytes(0, 32, 32, 128, 16, 64, 256) == 0


def test_one_hip_runtime_per_process(lib):
    """libpa.so binds to torch's copy of the HIP runtime even when the binding is loaded before
    anything imports torch: a second copy would take the library's calls to a runtime that has
    none of torch's device state."""
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from paged_kv_cache_05_amd import ops\n"
            "ops.load()\n"
            "import torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n"
            % str(ops.LIB_PATH.parents[1]))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         timeout=300).stdout
    mapped = eval(out.strip().splitlines()[-1])
    assert len(mapped) == 1, mapped
