"""Seeded synthetic inputs for paged decode attention and the two cache kernels.

This module draws numbers and builds index structures (context lengths, block tables, slot
mappings, copy-on-write pairs); it contains none of the attention arithmetic.  Both the CPU
oracle and the GPU library consume what it produces.

Storage conventions (host arrays):
  ``"f32"``  -> numpy float32
  ``"f16"``  -> numpy float16
  ``"bf16"`` -> numpy uint16 holding the raw bfloat16 bits
Values are drawn as float32 N(0, 1) and rounded once, round-to-nearest-even, to the storage
type, so the oracle and the GPU read identical inputs.

Random streams: ``numpy.random.SeedSequence(seed)`` spawns six children used, in order, for
context lengths, physical placement, queries, keys, values and the step's new tokens.

Workloads follow the shapes the pages discuss (16-token pages, 128-dim heads, Llama-7B /
OPT-13B / GQA shapes, shared prompt prefixes with parallel sampling); the pages' own data sets
(ShareGPT/Alpaca, a Chinese summarisation set) are not available, and these synthetic
draws stand in for them.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

from .block_manager import BlockManager

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}
# 8-bit caches hold E4M3 codes of N(0,1) draws divided by this scale (and clipped to +-6.5
# sigma so no draw leaves the format's +-448 range): 6.5 * 64 = 416.
FP8_DRAW_SCALE = 1.0 / 64.0


# ---------------------------------------------------------------------------------------
# rounding of generated float32 values to the storage type
# ---------------------------------------------------------------------------------------
def float32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, on the integer bit pattern."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r = np.where(nan, np.uint16(NAN_BITS["bf16"]), r)
    return r


def round_to_storage(x32, dtype: str) -> np.ndarray:
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.copy()
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return float32_to_bf16_bits(x32)
    if dtype == "fp8":   # random E4M3 codes: torch's cast of the clipped, scaled draw
        import torch
        y = np.clip(x32, -6.5, 6.5) / np.float32(FP8_DRAW_SCALE)
        return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_storage(dtype: str):
    if dtype == "fp8":
        return np.uint8(NAN_BITS["fp8"])
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.uint16(NAN_BITS["f16"]).view(np.float16)
    return np.uint16(NAN_BITS["bf16"])


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[dtype]


# ---------------------------------------------------------------------------------------
# workload specs
# ---------------------------------------------------------------------------------------
@dataclass(frozen=True)
class CaseSpec:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("fixed", [n0, n1, ...])
    lengths: tuple
    num_blocks: int | None = None      # None: live blocks fill ``pool_fill`` of the pool
    pool_fill: float = 0.9
    new_tokens: object = "next"        # "next": one appended token per sequence; ("free", n)
    partition_size: int = 0            # 0: the library chooses
    shared_prefix: int = 0             # tokens of a prompt prefix shared by every sequence
    fork: bool = False                 # parallel-sampling sibling per sequence before the step
    q_scale: float = 1.0               # multiplies q (peaky-softmax stress when large)
    max_blocks_per_seq: int | None = None  # table width; None: the widest sequence
    kv_dtype: str | None = None        # pool element type when it differs ("fp8")


def scaled(spec: CaseSpec, **kw) -> CaseSpec:
    return dataclasses.replace(spec, **kw)


CONFIGS = {
    "tiny": CaseSpec("tiny", 1, 4, 2, 2, 64, "f32", 16, ("uniform", 1, 100),
                     num_blocks=64, new_tokens=("free", 4)),
    "opt13b": CaseSpec("opt13b", 2, 64, 40, 40, 128, "f16", 16, ("uniform", 1, 2048),
                       num_blocks=16384),
    "llama7b_bs16": CaseSpec("llama7b_bs16", 3, 256, 32, 32, 128, "bf16", 16,
                             ("lognormal", 700.0, 1.0, 16, 4096)),
    "llama7b_bs32": CaseSpec("llama7b_bs32", 3, 256, 32, 32, 128, "bf16", 32,
                             ("lognormal", 700.0, 1.0, 16, 4096)),
    "llama7b_bs8": CaseSpec("llama7b_bs8", 3, 256, 32, 32, 128, "bf16", 8,
                            ("lognormal", 700.0, 1.0, 16, 4096)),
    "gqa_long": CaseSpec("gqa_long", 4, 16, 32, 8, 128, "bf16", 16, ("uniform", 8192, 32768),
                         partition_size=512),
    "shared_prefix": CaseSpec("shared_prefix", 5, 64, 32, 32, 128, "f16", 16,
                              ("uniform", 1, 512), shared_prefix=1024, fork=True),
    # the Llama-7B-shaped decode step over an 8-bit E4M3 cache (bf16 queries and new tokens)
    "llama7b_bs16_fp8": CaseSpec("llama7b_bs16_fp8", 3, 256, 32, 32, 128, "bf16", 16,
                                 ("lognormal", 700.0, 1.0, 16, 4096), kv_dtype="fp8"),
    # the GQA long-context step over an 8-bit E4M3 cache
    "gqa_long_fp8": CaseSpec("gqa_long_fp8", 4, 16, 32, 8, 128, "bf16", 16, ("uniform", 8192, 32768),
                             partition_size=512, kv_dtype="fp8"),
    # the GQA long-context step with heads of 80 dims (16-bit and E4M3 caches), which the
    # matrix-core kernel runs as 128-dim products on zero-padded rows
    "gqa_long_d80": CaseSpec("gqa_long_d80", 4, 16, 32, 8, 80, "bf16", 16, ("uniform", 8192, 32768),
                             partition_size=512),
    "gqa_long_fp8_d80": CaseSpec("gqa_long_fp8_d80", 4, 16, 32, 8, 80, "bf16", 16,
                                 ("uniform", 8192, 32768), partition_size=512, kv_dtype="fp8"),
}


def draw_from(lengths: tuple, count: int, rng: np.random.Generator) -> np.ndarray:
    """``count`` integers from a length spec: ("uniform", lo, hi) inclusive,
    ("lognormal", median, sigma, lo, hi) rounded and clipped, ("fixed", [n0, n1, ...])."""
    kind = lengths[0]
    if kind == "uniform":
        lo, hi = lengths[1], lengths[2]
        return rng.integers(lo, hi + 1, size=count).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = lengths[1:]
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=count)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind == "fixed":
        v = np.asarray(lengths[1], dtype=np.int64)
        if v.shape != (count,):
            raise ValueError("fixed lengths must have one entry per sequence")
        return v.copy()
    raise ValueError(f"unknown length spec {lengths!r}")


def draw_lengths(spec: CaseSpec, rng: np.random.Generator) -> np.ndarray:
    return draw_from(spec.lengths, spec.num_seqs, rng)


# ---------------------------------------------------------------------------------------
# a generated case
# ---------------------------------------------------------------------------------------
@dataclass
class DecodeCase:
    spec: CaseSpec
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    query: np.ndarray                 # [S, Hq, d] storage
    block_tables: np.ndarray          # int32 [S, max_blocks_per_seq]
    context_lens: np.ndarray          # int32 [S]  (after this step's append)
    new_key: np.ndarray               # [N, Hkv, d] storage
    new_value: np.ndarray
    slot_mapping: np.ndarray          # int64 [N]
    block_mapping: np.ndarray         # int64 [P, 2] (src, dst)
    key_cache: object = None          # [NB, Hkv, bs, d]: numpy storage, or a torch tensor on GPU
    value_cache: object = None
    token_slots: list = field(default_factory=list)   # per sequence: slot of every token
    contiguous: list | None = None    # per sequence: (K, V) storage [Hkv, n, d] after the step
    sibling_tables: np.ndarray | None = None
    sibling_lens: np.ndarray | None = None
    live_slots: np.ndarray | None = None

    @property
    def dtype(self):
        return self.spec.dtype

    @property
    def block_size(self):
        return self.spec.block_size


def _build_layout(spec: CaseSpec, rng_len, perm_seed):
    """Lengths, placement and the step's slots; returns a dict of host index arrays."""
    bs = spec.block_size
    lens = draw_lengths(spec, rng_len)
    S = spec.num_seqs
    free_mode = isinstance(spec.new_tokens, tuple) and spec.new_tokens[0] == "free"

    if spec.shared_prefix:
        P = int(spec.shared_prefix)
        need = -(-P // bs) + int(sum(-(-int(n) // bs) for n in lens)) + S
        nb_pool = spec.num_blocks or int(math.ceil(need / spec.pool_fill))
        bm = BlockManager(nb_pool, bs, seed=perm_seed)
        holder = bm.new_sequence()
        bm.append_tokens(holder, P)
        seqs = []
        for s in range(S):
            sid = bm.fork(holder)
            bm.append_tokens(sid, int(lens[s]))
            seqs.append(sid)
        bm.free_sequence(holder)
        sibs = [bm.fork(sid) for sid in seqs] if spec.fork else []
        pre_tables = [bm.table(sid) for sid in seqs]
        slots, pairs = [], []
        for sid in seqs:
            slot, cow = bm.append_token(sid)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        ctx = bm.context_lens(seqs)
        width = spec.max_blocks_per_seq or max(len(bm.table(s)) for s in seqs)
        out = dict(bm=bm, seqs=seqs, ctx=ctx, width=width, slots=np.array(slots, np.int64),
                   pairs=np.array(pairs, np.int64).reshape(-1, 2), num_blocks=nb_pool,
                   pre_tables=pre_tables)
        if sibs:
            out["sibs"] = sibs
            out["sib_tables"] = bm.block_tables(sibs, width=width)
            out["sib_lens"] = bm.context_lens(sibs)
        return out

    if np.any(lens < (0 if free_mode else 1)):
        raise ValueError("a sequence needs at least one token to append")
    total = int(sum(-(-int(n) // bs) for n in lens))
    nb_pool = spec.num_blocks or int(math.ceil(total / spec.pool_fill))
    bm = BlockManager(nb_pool, bs, seed=perm_seed)
    seqs, token_slots, step_slots = [], [], []
    for s in range(S):
        sid = bm.new_sequence()
        n = int(lens[s])
        if free_mode:
            sl, _ = bm.append_tokens(sid, n)
        else:
            sl, _ = bm.append_tokens(sid, n - 1)
            slot, _ = bm.append_token(sid)
            sl.append(slot)
            step_slots.append(slot)
        seqs.append(sid)
        token_slots.append(np.array(sl, np.int64))
    width = spec.max_blocks_per_seq or max(1, max(len(bm.table(s)) for s in seqs))
    return dict(bm=bm, seqs=seqs, ctx=bm.context_lens(seqs), width=width,
                slots=np.array(step_slots, np.int64), pairs=np.zeros((0, 2), np.int64),
                num_blocks=nb_pool, token_slots=token_slots)


def _slot_view(pool):
    """[NB, H, bs, d] -> [H, NB*bs, d]: slot ``b*bs + o`` is row ``b*bs + o``."""
    nb, h, bs, d = pool.shape
    return pool.transpose(1, 0, 2, 3).reshape(h, nb * bs, d)


def build_case(spec: CaseSpec, *, device=None, poison=False, table_fill=-1,
               keep_contiguous=False) -> DecodeCase:
    """Generate one decode step of ``spec``.

    ``device=None`` draws the K/V pools on the host (numpy storage arrays).  ``device="cuda"``
    draws them on the GPU with a seeded torch generator (for pools of several GB); the host
    then holds only the index arrays, queries and new tokens.

    ``poison=True`` fills every slot that holds no live token with NaN, so a kernel that reads
    a masked slot, an unused block or an unused table entry shows it.  ``table_fill`` is
    written into the table entries past each sequence's last block.
    """
    if spec.dtype not in DTYPES:
        raise ValueError(spec.dtype)
    ss = np.random.SeedSequence(spec.seed)
    c_len, c_perm, c_q, c_k, c_v, c_new = ss.spawn(6)
    lay = _build_layout(spec, np.random.default_rng(c_len), np.random.default_rng(c_perm))
    S, Hq, Hkv, d, bs = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    NB = lay["num_blocks"]
    dt = spec.dtype
    scale = np.float32(1.0 / math.sqrt(d))

    q32 = np.random.default_rng(c_q).standard_normal((S, Hq, d), dtype=np.float32)
    query = round_to_storage(q32 * np.float32(spec.q_scale), dt)

    free_mode = isinstance(spec.new_tokens, tuple) and spec.new_tokens[0] == "free"
    bm = lay["bm"]
    tables = bm.block_tables(lay["seqs"], width=lay["width"], fill=table_fill)

    # live slots: every slot a sequence (or its sibling) can read
    live = np.zeros(NB * bs, dtype=bool)
    all_tables = [bm.table(s) for s in lay["seqs"]] + [bm.table(s) for s in lay.get("sibs", [])]
    lens_all = list(lay["ctx"]) + [bm.length(s) for s in lay.get("sibs", [])]
    for tbl, n in zip(all_tables, lens_all):
        for j, b in enumerate(tbl):
            k = min(bs, int(n) - j * bs)
            if k > 0:
                live[b * bs: b * bs + k] = True
    if "pre_tables" in lay:
        for tbl, n in zip(lay["pre_tables"], lay["ctx"] - 1):
            for j, b in enumerate(tbl):
                k = min(bs, int(n) - j * bs)
                if k > 0:
                    live[b * bs: b * bs + k] = True

    rng_new = np.random.default_rng(c_new)
    if free_mode:
        nnew = int(spec.new_tokens[1])
        free_slots = np.flatnonzero(~live)
        slots = np.sort(rng_new.choice(free_slots, size=nnew, replace=False)).astype(np.int64)
    else:
        slots = lay["slots"]
        nnew = len(slots)
    nk32 = rng_new.standard_normal((nnew, Hkv, d), dtype=np.float32)
    nv32 = rng_new.standard_normal((nnew, Hkv, d), dtype=np.float32)

    case = DecodeCase(spec=spec, num_blocks=NB, max_blocks_per_seq=tables.shape[1], scale=scale,
                      query=query, block_tables=tables, context_lens=lay["ctx"].astype(np.int32),
                      new_key=round_to_storage(nk32, dt), new_value=round_to_storage(nv32, dt),
                      slot_mapping=slots, block_mapping=lay["pairs"],
                      token_slots=lay.get("token_slots", []), live_slots=np.flatnonzero(live))
    if "sib_tables" in lay:
        case.sibling_tables = lay["sib_tables"]
        case.sibling_lens = lay["sib_lens"]

    shape = (NB, Hkv, bs, d)
    pdt = spec.kv_dtype or dt          # pool element type
    if device is None:
        kc = round_to_storage(np.random.default_rng(c_k).standard_normal(shape, dtype=np.float32), pdt)
        vc = round_to_storage(np.random.default_rng(c_v).standard_normal(shape, dtype=np.float32), pdt)
        if poison:
            dead = ~live
            if not free_mode and len(slots):
                # the step's own slots are written by reshape_and_cache before decode reads them
                dead[slots] = True
            # slot b*bs + o is pool[b, :, o, :]; index the pool itself (a reshaped
            # transpose would be a copy, and writing into it would leave the pool clean)
            db, do = np.divmod(np.flatnonzero(dead), bs)
            for pool in (kc, vc):
                pool[db, :, do, :] = nan_storage(pdt)
        case.key_cache, case.value_cache = kc, vc
        if keep_contiguous and not spec.shared_prefix:
            case.contiguous = []
            kv_view, vv_view = _slot_view(kc), _slot_view(vc)
            for s in range(S):
                ts = case.token_slots[s]
                K = kv_view[:, ts, :].copy()
                V = vv_view[:, ts, :].copy()
                if not free_mode:
                    if pdt != dt:
                        raise ValueError("contiguous K/V of a quantized cache need free-slot mode")
                    K[:, -1, :] = case.new_key[s]
                    V[:, -1, :] = case.new_value[s]
                case.contiguous.append((K, V))
    else:
        case.key_cache = _device_pool(shape, pdt, c_k, device)
        case.value_cache = _device_pool(shape, pdt, c_v, device)
        if poison:
            raise ValueError("poisoned pools are host-generated only")
    return case


# ---------------------------------------------------------------------------------------
# torch plumbing (device memory only)
# ---------------------------------------------------------------------------------------
def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.uint8}[dtype]


def to_torch(arr, dtype: str, device):
    """Host storage array -> torch tensor of the element type on ``device`` (bit-exact)."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(a.view(np.float16))
    elif dtype == "f32":
        t = torch.from_numpy(a.view(np.float32))
    elif dtype == "fp8":
        t = torch.from_numpy(a.view(np.uint8))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """torch tensor -> host storage array (bit-exact)."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return t.numpy().view(np.float16)
    if dtype == "f32":
        return t.numpy().view(np.float32)
    if dtype == "fp8":
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _device_pool(shape, dtype, seed_seq, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed_seq.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF))
    out = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    step = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for b0 in range(0, shape[0], step):
        b1 = min(shape[0], b0 + step)
        x = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if dtype == "fp8":
            out[b0:b1] = (x.clamp(-6.5, 6.5) / FP8_DRAW_SCALE).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            out[b0:b1] = x.to(out.dtype)
    return out


# ---------------------------------------------------------------------------------------
# prefill (a chunk of new tokens per sequence, attending causally over the paged cache)
# ---------------------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillSpec:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    prefix_lengths: tuple              # tokens cached before this chunk (length-spec forms)
    chunk_lengths: tuple               # new tokens in this chunk
    pool_fill: float = 0.9
    max_blocks_per_seq: int | None = None
    kv_dtype: str | None = None        # pool element type when it differs ("fp8")


PREFILL_CONFIGS = {
    # Llama-7B-shaped chunked prefill: 512-token chunks on top of 0..1536 cached tokens
    "prefill_llama7b": PrefillSpec("prefill_llama7b", 6, 32, 32, 32, 128, "bf16", 16,
                                   ("uniform", 0, 1536), ("fixed", [512] * 32)),
    # grouped-query heads, ragged chunks, long prefixes
    "prefill_gqa": PrefillSpec("prefill_gqa", 7, 8, 32, 8, 128, "bf16", 16,
                               ("uniform", 0, 3000), ("uniform", 1, 700)),
    # GPT-OSS-shaped heads (64 query heads on 8 KV heads of 64 dims, the published gpt-oss-20b
    # attention shape): 512-token chunks on 0..1536 cached tokens
    "prefill_gptoss_d64": PrefillSpec("prefill_gptoss_d64", 8, 16, 64, 8, 64, "bf16", 16,
                                      ("uniform", 0, 1536), ("fixed", [512] * 16)),
    # heads of 80 dims, which the kernel runs as 128-dim products on zero-padded rows: the
    # Llama-7B-shaped prefill with 32 heads of 80 dims
    "prefill_d80": PrefillSpec("prefill_d80", 9, 32, 32, 32, 80, "bf16", 16,
                               ("uniform", 0, 1536), ("fixed", [512] * 32)),
    # the Llama-7B-shaped chunked prefill over an E4M3 cache
    "prefill_llama7b_fp8": PrefillSpec("prefill_llama7b_fp8", 6, 32, 32, 32, 128, "bf16", 16,
                                       ("uniform", 0, 1536), ("fixed", [512] * 32), kv_dtype="fp8"),
}


@dataclass
class PrefillCase:
    spec: PrefillSpec
    pool: DecodeCase                   # pools, tables, context lengths (its query is unused)
    query: np.ndarray                  # [T, Hq, d] storage, the chunks packed back to back
    query_start_loc: np.ndarray        # int32 [S + 1]
    query_lens: np.ndarray             # int64 [S]
    context_lens: np.ndarray           # int32 [S]: prefix + chunk (the chunk is already cached)
    max_query_len: int

    @property
    def dtype(self):
        return self.spec.dtype

    @property
    def block_size(self):
        return self.spec.block_size

    @property
    def scale(self):
        return self.pool.scale


def build_prefill_case(spec: PrefillSpec, *, device=None, poison=False, table_fill=-1,
                       keep_contiguous=False) -> PrefillCase:
    """Generate one chunked-prefill call: every sequence's prefix and chunk are in the pool
    (the chunk written by reshape_and_cache beforehand), and the chunk's queries are packed
    into ``query`` in sequence order."""
    ss = np.random.SeedSequence(spec.seed)
    c_pre, c_chunk, c_q, c_pool = ss.spawn(4)
    S = spec.num_seqs
    pre = draw_from(spec.prefix_lengths, S, np.random.default_rng(c_pre))
    chunk = draw_from(spec.chunk_lengths, S, np.random.default_rng(c_chunk))
    if np.any(pre < 0) or np.any(chunk < 0):
        raise ValueError("lengths must be non-negative")
    ctx = pre + chunk
    pool_spec = CaseSpec(spec.name, int(c_pool.generate_state(1)[0]), S, spec.num_heads,
                         spec.num_kv_heads, spec.head_dim, spec.dtype, spec.block_size,
                         ("fixed", [int(n) for n in ctx]), pool_fill=spec.pool_fill,
                         new_tokens=("free", 0), max_blocks_per_seq=spec.max_blocks_per_seq,
                         kv_dtype=spec.kv_dtype)
    pool = build_case(pool_spec, device=device, poison=poison, table_fill=table_fill,
                      keep_contiguous=keep_contiguous)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(chunk)
    T = int(qsl[-1])
    q32 = np.random.default_rng(c_q).standard_normal((T, spec.num_heads, spec.head_dim),
                                                     dtype=np.float32)
    return PrefillCase(spec=spec, pool=pool, query=round_to_storage(q32, spec.dtype),
                       query_start_loc=qsl, query_lens=chunk.astype(np.int64),
                       context_lens=ctx.astype(np.int32),
                       max_query_len=int(chunk.max()) if S else 0)
