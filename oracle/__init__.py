"""CPU oracle for paged KV-cache attention (test infrastructure only).

This package is the slow, obviously correct reference the HIP path is checked
against.  Only the test suite, the smoke check of the package entry file and
the CPU-baseline leg of the benchmark may import it; the product path never
does, and it shares no code with the HIP library (no kernels, headers,
helpers or tables in common).

Modules
  paged_attention  numpy fp64 implementation of the operator: scatter the
                   step's K/V into copies of the caches, gather each sequence's
                   history through block_table, brute-force causal GQA softmax
                   attention, optionally with each row's attention-domain
                   lse.  Also the partial (out, lse) state over a key subset
                   and the fixed-order merge of such states, and the fused
                   prologue (Q/K OffsetRMSNorm, interleaved partial MRoPE,
                   cast to the data type).
  scalar           a second, independent formulation in plain Python scalars
                   (nested loops, math.fsum) for tiny inputs, used to pin the
                   numpy version.

Every function cites the passage of the pages it follows; the pins that tie it
to something other than itself live in tests/test_oracle_pins.py.  Parity is
pinned for every function here (no function is "parity unpinned").
"""
from .paged_attention import (  # noqa: F401
    paged_attention,
    scatter_kv,
    gather_history,
    attend_sequence,
    partial_state,
    merge_partials,
    merge_states,
    resolve_call,
    values,
    quantize_int8,
    quantize_int4,
    pack_int4,
    unpack_int4,
    dequantize,
    output_gate,
    qk_prologue,
    offset_rms_norm,
    mrope_components,
    rotary_angles,
    apply_rotary,
    round_to_format,
    to_dtype_bits,
)
