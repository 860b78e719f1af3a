"""Every plausible mistake planted in a copy of the oracle must make some pin fail.

The real oracle file is never modified: its source is read, one substring is replaced, and
the result is executed as a fresh module that the pins then run against.
"""

import pathlib
import types

import pytest

import oracle_pins

SRC = (pathlib.Path(__file__).resolve().parents[1] / "oracle" / "pa_oracle.py").read_text()

# (name, original substring, planted mistake)
MUTATIONS = [
    ("dropped scale", "z = scale * (K @ q)", "z = (K @ q)"),
    ("wrong GQA head map", "            kv = h // G\n            out[s, h]",
     "            kv = h % Hkv\n            out[s, h]"),
    ("wrong query head", "_softmax_weighted_sum(K[kv], V[kv], q[h], sc)",
     "_softmax_weighted_sum(K[kv], V[kv], q[kv], sc)"),
    ("token/block order transposed", "seq = blocks.transpose(1, 0, 2, 3)",
     "seq = blocks.transpose(1, 2, 0, 3)"),
    ("table read off by one", "phys = np.asarray(table_row[:nb]", "phys = np.asarray(table_row[1:nb + 1]"),
    ("context shifted", "return seq[:, :n, :]", "return seq[:, 1:n + 1, :]"),
    ("floor block count", "    nb = num_blocks_for(n, block_size)\n    phys",
     "    nb = max(1, n // block_size)\n    phys"),
    ("unstable shift", "z = z - z.max()\n    p = np.exp(z)", "z = z - z.min()\n    p = np.exp(z)"),
    ("exp sign", "    p = np.exp(z)\n    return", "    p = np.exp(-z)\n    return"),
    ("wrong normaliser", "return (p @ V) / p.sum()", "return (p @ V) / p.max()"),
    ("keys used as values", "return (p @ V) / p.sum()", "return (p @ K) / p.sum()"),
    ("empty context not handled", "        if n <= 0:\n            continue\n        K = resolve",
     "        K = resolve"),
    ("divmod swapped", "b, o = divmod(slot, bs)", "o, b = divmod(slot, bs)"),
    ("negative slot written", "if slot < 0 or slot >= nb * bs:", "if slot >= nb * bs:"),
    ("value not written", "        vc[b, :, o, :] = value[i]\n", "        vc[b, :, o, :] = key[i]\n"),
    ("copy direction", "kc[dst] = k0[src]", "kc[src] = k0[dst]"),
    ("V block not copied", "        vc[dst] = v0[src]\n", "        pass\n"),
    ("bf16 truncation", "r = np.ldexp(np.rint(np.ldexp(xf,", "r = np.ldexp(np.trunc(np.ldexp(xf,"),
    ("bf16 precision", "qexp = np.maximum(e - 8,", "qexp = np.maximum(e - 9,"),
    ("bf16 decode shift", "<< np.uint32(16)\n        return bits", "<< np.uint32(15)\n        return bits"),
    ("merge weight", "w = np.array([l * math.exp(m - M) for m, l, _ in parts])",
     "w = np.array([l for m, l, _ in parts])"),
    ("partition bound", "t1 = min(t0 + P, n)", "t1 = min(t0 + P - 1, n)"),
    ("kv bytes factor", "return 2 * int(num_layers)", "return int(num_layers)"),
    ("floor page count", "return -(-int(num_tokens) // int(block_size))",
     "return int(num_tokens) // int(block_size)"),
    ("utilisation denominator", "reserved = sum(num_blocks_for(n, block_size) * block_size for n in lengths)",
     "reserved = sum(lengths)"),
    ("swap writes the source", "        kd[dst] = src_key[src]\n", "        kd[src % nd] = src_key[dst % ns]\n"),
    ("swap bounds use one pool", "if not (0 <= src < ns and 0 <= dst < nd):", "if not (0 <= src < nd and 0 <= dst < nd):"),
    ("prefill strict causal", "_softmax_weighted_sum(K[kv, :last + 1], V[kv, :last + 1],",
     "_softmax_weighted_sum(K[kv, :last + 2], V[kv, :last + 2],"),
    ("prefill excludes itself", "            last = n - L + i ", "            last = n - L + i - 1 "),
    ("prefill ignores cached prefix", "            last = n - L + i ", "            last = i "),
    ("prefill sees whole chunk", "            last = n - L + i ", "            last = n - 1 "),
    ("prefill GQA map", "                kv = h // G\n                out[q0 + i, h]",
     "                kv = h % Hkv\n                out[q0 + i, h]"),
    ("prefill row offset", "q = storage_to_f64(query[q0:q1], dtype)", "q = storage_to_f64(query[0:L], dtype)"),
    ("prefill no length guard", "if L <= 0 or n < L:", "if L <= 0:"),
    ("fp8 exponent bias", "np.exp2((e - 7).astype(np.float64))", "np.exp2((e - 8).astype(np.float64))"),
    ("fp8 subnormal quantum", "mag = np.where(e == 0, m * 2.0 ** -9,", "mag = np.where(e == 0, m * 2.0 ** -10,"),
    ("fp8 sign dropped", "    val = np.where((c & 0x80) != 0, -mag, mag)\n", "    val = mag\n"),
    ("fp8 rounding truncates", "r = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)\n    _, rex",
     "r = np.ldexp(np.floor(np.ldexp(a, -qexp)), qexp)\n    _, rex"),
    ("fp8 mantissa width", "qexp = np.maximum(ex - 4, -9)", "qexp = np.maximum(ex - 3, -9)"),
    ("fp8 no saturation", "    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))\n", ""),
    ("fp8 scale multiplies", "inv = np.float32(1.0) / np.float32(scale)", "inv = np.float32(scale)"),
    ("fp8 value scale for keys", "    kc = dequantize_fp8(key_cache, k_scale)", "    kc = dequantize_fp8(key_cache, v_scale)"),
    ("fp8 prefill key scale", "    keys = dequantize_fp8(key_cache, k_scale)", "    keys = dequantize_fp8(key_cache, v_scale)"),
    ("fp8 prefill values from keys", "    values = dequantize_fp8(value_cache, v_scale)",
     "    values = dequantize_fp8(key_cache, v_scale)"),
    ("CoW on any reference", "            if refs[block] > 1:", "            if refs[block] >= 1:"),
    ("CoW keeps the old reference", "                refs[block] -= 1\n", "                pass\n"),
    ("fresh block unreferenced", "            tables[s, j] = new\n            refs[new] = 1\n", "            tables[s, j] = new\n"),
    ("append slot offset", "        slots.append(block * bs + off)", "        slots.append(block * bs + off + 1)"),
    ("fork without reference", "        for b in tables[parent, :nb]:\n            refs[b] += 1", "        for b in tables[parent, :nb]:\n            pass"),
    ("free pushes shared blocks", "            if refs[b] == 0:\n                stack[top] = b", "            if refs[b] <= 1:\n                stack[top] = b"),
    ("FNV prime", "_FNV_PRIME = 0x100000001B3", "_FNV_PRIME = 0x100000001B5"),
    ("FNV order", "        h ^= byte\n        h = (h * _FNV_PRIME) & _MASK64", "        h = (h * _FNV_PRIME) & _MASK64\n        h ^= byte"),
    ("hash chain ignores the prefix", "            h = fnv1a64(int(h).to_bytes(8, \"little\") + int(g).to_bytes(8, \"little\"))",
     "            h = fnv1a64(int(0).to_bytes(8, \"little\") + int(g).to_bytes(8, \"little\"))"),
]


def _mutant(orig, new):
    assert SRC.count(orig) == 1, f"mutation anchor must occur exactly once: {orig!r}"
    mod = types.ModuleType("pa_oracle_mutant")
    exec(compile(SRC.replace(orig, new), "pa_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, orig, new):
    mod = _mutant(orig, new)
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail(f"no pin caught the planted mistake: {name}")


def test_unmutated_copy_passes():
    mod = _mutant("z = scale * (K @ q)", "z = scale * (K @ q)")
    for pin in oracle_pins.ALL_PINS:
        pin(mod)
