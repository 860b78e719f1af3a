"""CPU oracle for paged decode attention — test infrastructure only.

Only the test-suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import this package.  It imports nothing from the GPU library.
"""

from .pa_oracle import (  # noqa: F401
    append_slots_ref,
    block_hashes_ref,
    copy_blocks_ref,
    decode_ref,
    decode_fp8_ref,
    decode_split_ref,
    dequantize_fp8,
    f64_to_fp8_e4m3,
    f64_to_storage,
    fnv1a64,
    fork_ref,
    free_seqs_ref,
    fp8_e4m3_to_f64,
    kv_bytes_per_token,
    prefill_fp8_ref,
    prefill_ref,
    quantize_fp8,
    num_blocks_for,
    reshape_and_cache_fp8_ref,
    reshape_and_cache_ref,
    resolve_sequence,
    slot_utilization,
    storage_to_f64,
    swap_blocks_ref,
)
