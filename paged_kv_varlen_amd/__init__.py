"""Python binding of libpagedattn.so (the MI355X paged KV-cache attention library).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is not built, every call raises.

    out = paged_attention(query, key, value, key_cache, value_cache,
                          cumulative_sequence_length, past_seqlens, block_table,
                          slot_mapping=None, num_heads=H, kv_num_heads=Hkv,
                          scale=0.0)
    out, lse = paged_attention(..., return_lse=True)      # + fp32 lse [N, H]
    out, lse = merge_states(state_out, state_lse)          # fixed-order merge

Argument meaning follows the com.microsoft PagedAttention operator (model-card
README "com.microsoft.PagedAttention", sections Inputs, Outputs, Attributes);
key_cache and value_cache are updated in place.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["paged_attention", "paged_attention_noalloc", "merge_states", "workspace_bytes",
           "PagedAttentionError", "PaArgs", "PaMergeArgs", "library", "library_path", "STATUS",
           "NOALLOC_SCRATCH_BYTES"]

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_DTYPE_F16 = 1
PA_DTYPE_BF16 = 2
PA_KV_SAME, PA_KV_INT8, PA_KV_INT4 = 0, 1, 2
PA_ROPE_ADJACENT, PA_ROPE_CONTIGUOUS = 1, 2
_CODE_DTYPES = {torch.int8: PA_KV_INT8, torch.uint8: PA_KV_INT4}  # cache dtype -> kv_quant
_DTYPE_CODES = {torch.float16: PA_DTYPE_F16, torch.bfloat16: PA_DTYPE_BF16}
ABI_VERSION = 5
KERNELS = ("scatter_plan", "decode", "merge", "prefill")  # enum pa_kernel order
NOALLOC_SCRATCH_BYTES = 128 << 20  # PA_NOALLOC_SCRATCH_BYTES
STATUS = {
    0: "PA_OK", 1: "PA_ERR_NULL_ARG", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
    4: "PA_ERR_WORKSPACE", 5: "PA_ERR_ALIGNMENT", 6: "PA_ERR_ABI", 7: "PA_ERR_METADATA",
    8: "PA_ERR_HIP",
}


class PaArgs(ctypes.Structure):
    """Mirror of pa_args in include/pagedattn.h (same order and types)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("query", ctypes.c_void_p),
        ("key", ctypes.c_void_p),
        ("value", ctypes.c_void_p),
        ("key_cache", ctypes.c_void_p),
        ("value_cache", ctypes.c_void_p),
        ("cumulative_sequence_length", ctypes.c_void_p),
        ("past_seqlens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("output", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int64),
        ("query_width", ctypes.c_int64),
        ("batch_size", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("kv_num_heads", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("cache_kv_heads", ctypes.c_int32),
        ("cache_head_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("is_causal", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("kernel_events", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("output_f32", ctypes.c_void_p),
        ("kv_quant", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("gate", ctypes.c_void_p),
        ("q_norm_weight", ctypes.c_void_p),
        ("k_norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("rotary_dim", ctypes.c_int32),
        ("position_ids", ctypes.c_void_p),
        ("rope_theta", ctypes.c_float),
        ("mrope_section", ctypes.c_int32 * 3),
        ("rope_flags", ctypes.c_int32),
    ]


class PaMergeArgs(ctypes.Structure):
    """Mirror of pa_merge_args in include/pagedattn.h."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("num_states", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("num_rows", ctypes.c_int64),
        ("state_out", ctypes.c_void_p),
        ("state_lse", ctypes.c_void_p),
        ("output", ctypes.c_void_p),
        ("output_f32", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
    ]


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_LIB = None


def library() -> ctypes.CDLL:
    """Load libpagedattn.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m paged_kv_varlen_amd.build`")
        lib = ctypes.CDLL(library_path)
        lib.pa_paged_attention.argtypes = [ctypes.POINTER(PaArgs), ctypes.c_void_p]
        lib.pa_paged_attention.restype = ctypes.c_int
        lib.pa_paged_attention_noalloc.argtypes = [ctypes.POINTER(PaArgs), ctypes.c_void_p]
        lib.pa_paged_attention_noalloc.restype = ctypes.c_int
        lib.pa_workspace_bytes.argtypes = [ctypes.POINTER(PaArgs)]
        lib.pa_workspace_bytes.restype = ctypes.c_size_t
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_merge_states.argtypes = [ctypes.POINTER(PaMergeArgs), ctypes.c_void_p]
        lib.pa_merge_states.restype = ctypes.c_int
        lib.pa_abi_version.argtypes = []
        lib.pa_abi_version.restype = ctypes.c_int32
        if lib.pa_abi_version() != ABI_VERSION:
            raise RuntimeError("libpagedattn.so ABI version mismatch")
        _LIB = lib
    return _LIB


_EMPTY_ADDR = 256  # aligned stand-in for a present but empty tensor; never dereferenced


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of a tensor; None (NULL) only for an absent input.
    torch gives empty tensors address 0, which the ABI would read as
    "absent" (e.g. key/value NULL = packed [Q|K|V]), so a present empty
    tensor gets a non-NULL stand-in: with no elements nothing is read."""
    if t is None:
        return None
    return t.data_ptr() if t.data_ptr() != 0 or t.numel() > 0 else _EMPTY_ADDR


def _dtype_code(t: torch.Tensor) -> int:
    """pa_dtype of a tensor (0, which the library rejects, for other types)."""
    return _DTYPE_CODES.get(t.dtype, 0)


def make_args(query, key, value, key_cache, value_cache, cumulative_sequence_length,
              past_seqlens, block_table, slot_mapping, output, *, num_heads: int,
              kv_num_heads: int, scale: float = 0.0, is_causal: int = 1,
              workspace: Optional[torch.Tensor] = None,
              k_scale: Optional[torch.Tensor] = None,
              v_scale: Optional[torch.Tensor] = None,
              gate: Optional[torch.Tensor] = None,
              prologue: Optional[dict] = None) -> PaArgs:
    """Fill a PaArgs from tensors (no checks beyond what marshalling needs:
    the library validates shapes, dtypes and alignment itself).  int8 (INT8)
    or uint8 (INT4, two codes per byte) caches with fp32 ``k_scale``/``v_scale``
    [kv_num_heads, head_size] select a quantized cache path.  ``prologue``:
    the fused Q/K norm and rotation (see set_prologue)."""
    for name, t in (("query", query), ("key", key), ("value", value), ("key_cache", key_cache),
                    ("value_cache", value_cache),
                    ("cumulative_sequence_length", cumulative_sequence_length),
                    ("past_seqlens", past_seqlens), ("block_table", block_table),
                    ("slot_mapping", slot_mapping), ("output", output)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("cumulative_sequence_length", cumulative_sequence_length),
                    ("past_seqlens", past_seqlens), ("block_table", block_table),
                    ("slot_mapping", slot_mapping)):
        if t is not None and t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32 (type constraint S)")
    a = PaArgs()
    a.struct_size = ctypes.sizeof(PaArgs)
    kv_quant = _CODE_DTYPES.get(key_cache.dtype, PA_KV_SAME)
    caches = () if kv_quant != PA_KV_SAME else (key_cache, value_cache)
    same = all(t is None or t.dtype == query.dtype for t in (key, value, output) + caches)
    if kv_quant != PA_KV_SAME and value_cache.dtype != key_cache.dtype:
        same = False
    a.dtype = _dtype_code(query) if same else 0
    if kv_quant != PA_KV_SAME:
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError(f"quantized caches need a contiguous float32 {name}")
        a.kv_quant = kv_quant
        a.k_scale = _ptr(k_scale)
        a.v_scale = _ptr(v_scale)
    if gate is not None and (gate.dtype != query.dtype or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous tensor of the query's dtype")
    a.gate = _ptr(gate)
    a.query = _ptr(query)
    a.key = _ptr(key)
    a.value = _ptr(value)
    a.key_cache = _ptr(key_cache)
    a.value_cache = _ptr(value_cache)
    a.cumulative_sequence_length = _ptr(cumulative_sequence_length)
    a.past_seqlens = _ptr(past_seqlens)
    a.block_table = _ptr(block_table)
    a.slot_mapping = _ptr(slot_mapping)
    a.output = _ptr(output)
    a.num_tokens = query.shape[0]
    a.query_width = query.shape[1]
    a.batch_size = past_seqlens.shape[0]
    a.num_heads = num_heads
    a.kv_num_heads = kv_num_heads
    a.num_blocks, a.block_size, a.cache_kv_heads, a.cache_head_size = key_cache.shape
    if value_cache.shape != key_cache.shape:
        raise ValueError("value_cache must have key_cache's shape")
    a.max_blocks_per_seq = block_table.shape[1] if block_table.dim() == 2 else 0
    a.scale = float(scale)
    a.is_causal = int(is_causal)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    if prologue is not None:
        set_prologue(a, **prologue)
    return a


def set_prologue(a: PaArgs, *, position_ids: Optional[torch.Tensor] = None, rotary_dim: int = 0,
                 theta: float = 1.0e6, sections=(0, 0, 0), interleaved: bool = True,
                 adjacent: bool = False, q_norm_weight: Optional[torch.Tensor] = None,
                 k_norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6) -> None:
    """The fused prologue's fields of pa_args: OffsetRMSNorm of the query and
    key heads (fp32 weights [head_size], either may be None), then the partial
    MRoPE of the first ``rotary_dim`` channels (0: none) with int64
    ``position_ids`` [3, num_tokens], base ``theta``, pairs per position row
    ``sections``, interleaved or contiguous sections, half-split or adjacent
    pairs.  Keyword names follow the oracle's qk_prologue."""
    for name, t, dt in (("position_ids", position_ids, torch.int64), ("q_norm_weight", q_norm_weight, torch.float32),
                        ("k_norm_weight", k_norm_weight, torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    a.q_norm_weight = _ptr(q_norm_weight)
    a.k_norm_weight = _ptr(k_norm_weight)
    a.norm_eps = float(eps)
    a.rotary_dim = int(rotary_dim)
    a.position_ids = _ptr(position_ids)
    a.rope_theta = float(theta)
    a.mrope_section = (ctypes.c_int32 * 3)(*[int(x) for x in sections])
    a.rope_flags = (PA_ROPE_ADJACENT if adjacent else 0) | (0 if interleaved else PA_ROPE_CONTIGUOUS)


def workspace_bytes(args: PaArgs) -> int:
    return int(library().pa_workspace_bytes(ctypes.byref(args)))


def call(args: PaArgs, stream: Optional[int] = None, noalloc: bool = False) -> None:
    """Run the library's entry point (pa_paged_attention, or with ``noalloc``
    pa_paged_attention_noalloc) on a filled PaArgs; raise on error."""
    lib = library()
    fn = lib.pa_paged_attention_noalloc if noalloc else lib.pa_paged_attention
    st = fn(ctypes.byref(args), stream)
    if st != 0:
        raise PagedAttentionError(st, lib.pa_status_string(st).decode())


def paged_attention_noalloc(query, key, value, key_cache, value_cache, cumulative_sequence_length,
                            past_seqlens, block_table, slot_mapping=None, *, num_heads: int,
                            kv_num_heads: int, output: torch.Tensor, scale: float = 0.0,
                            is_causal: int = 1, lse: Optional[torch.Tensor] = None,
                            output_f32: Optional[torch.Tensor] = None,
                            k_scale: Optional[torch.Tensor] = None,
                            v_scale: Optional[torch.Tensor] = None,
                            gate: Optional[torch.Tensor] = None,
                            prologue: Optional[dict] = None,
                            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """pa_paged_attention_noalloc: paged_attention() with the library's own
    per-GPU scratch as workspace.  Nothing is allocated here either: the
    caller passes ``output`` (and ``lse`` / ``output_f32`` if wanted).  Calls
    that may overlap on one GPU race on the scratch and must be ordered."""
    args = make_args(query, key, value, key_cache, value_cache, cumulative_sequence_length,
                     past_seqlens, block_table, slot_mapping, output, num_heads=num_heads,
                     kv_num_heads=kv_num_heads, scale=scale, is_causal=is_causal,
                     k_scale=k_scale, v_scale=v_scale, gate=gate, prologue=prologue)
    for name, t in (("lse", lse), ("output_f32", output_f32)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    args.lse = _ptr(lse)
    args.output_f32 = _ptr(output_f32)
    s = stream if stream is not None else torch.cuda.current_stream(query.device)
    call(args, s.cuda_stream, noalloc=True)
    return output


def paged_attention(query: torch.Tensor, key: Optional[torch.Tensor],
                    value: Optional[torch.Tensor], key_cache: torch.Tensor,
                    value_cache: torch.Tensor, cumulative_sequence_length: torch.Tensor,
                    past_seqlens: torch.Tensor, block_table: torch.Tensor,
                    slot_mapping: Optional[torch.Tensor] = None, *, num_heads: int,
                    kv_num_heads: int, scale: float = 0.0, is_causal: int = 1,
                    output: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None,
                    kernel_events=None, return_lse: bool = False,
                    lse: Optional[torch.Tensor] = None,
                    output_f32: Optional[torch.Tensor] = None,
                    k_scale: Optional[torch.Tensor] = None,
                    v_scale: Optional[torch.Tensor] = None,
                    gate: Optional[torch.Tensor] = None,
                    prologue: Optional[dict] = None):
    """Scatter the step's K/V into the caches (in place) and return the
    attention output [num_tokens, num_heads * head_size].

    With ``return_lse`` (or a given ``lse`` tensor, fp32 [num_tokens,
    num_heads]) the call also writes each row's attention-domain lse and
    returns (output, lse).  ``output_f32`` (fp32 [num_tokens, num_heads *
    head_size]) receives the output before its rounding; together with lse it
    is the row's partial state for merge_states().

    ``kernel_events``: optional sequence of 2*len(KERNELS) torch.cuda.Event
    (enable_timing=True); the library records pair k around its k-th kernel.

    INT8 caches: int8 ``key_cache``/``value_cache`` with fp32 ``k_scale`` and
    ``v_scale`` [kv_num_heads, head_size] (per-channel scales).  INT4 caches:
    uint8 [num_blocks, block_size, kv_num_heads, head_size / 2], two codes per
    byte (the even element in bits 0-3), with the same scales.

    ``gate``: optional [num_tokens, num_heads * head_size] tensor of the
    query's dtype; the output is then the attention times sigmoid(gate),
    rounded once (``lse`` and ``output_f32`` stay ungated).

    ``prologue``: optional dict of the fused Q/K OffsetRMSNorm and partial
    MRoPE applied to the step's query and key rows first (set_prologue's
    keyword arguments, device tensors for position_ids and the weights)."""
    lib = library()
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    packed = key is None
    heads = num_heads + 2 * kv_num_heads if packed else num_heads
    D = query.shape[1] // heads if heads > 0 else 0
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    # Tensors made here are allocated on the stream the kernels run on: the
    # caching allocator then hands a freed block (the workspace, dropped on
    # return) only to later work on that stream, which runs after the kernels.
    with torch.cuda.stream(s):
        if output is None:
            output = torch.empty((query.shape[0], num_heads * D), dtype=query.dtype, device=dev)
        args = make_args(query, key, value, key_cache, value_cache, cumulative_sequence_length,
                         past_seqlens, block_table, slot_mapping, output, num_heads=num_heads,
                         kv_num_heads=kv_num_heads, scale=scale, is_causal=is_causal,
                         k_scale=k_scale, v_scale=v_scale, gate=gate, prologue=prologue)
        if return_lse and lse is None:
            lse = torch.empty((query.shape[0], num_heads), dtype=torch.float32, device=dev)
        for name, t in (("lse", lse), ("output_f32", output_f32)):
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous float32 tensor")
        args.lse = _ptr(lse)
        args.output_f32 = _ptr(output_f32)
        need = int(lib.pa_workspace_bytes(ctypes.byref(args)))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    ev_array = None
    if kernel_events is not None:
        if len(kernel_events) != 2 * len(KERNELS):
            raise ValueError(f"kernel_events needs {2 * len(KERNELS)} events")
        ev_array = (ctypes.c_void_p * len(kernel_events))(*[e.cuda_event for e in kernel_events])
        args.kernel_events = ctypes.cast(ev_array, ctypes.c_void_p)
    call(args, s.cuda_stream)
    return (output, lse) if lse is not None else output


def merge_states(state_out: torch.Tensor, state_lse: torch.Tensor, *,
                 output: Optional[torch.Tensor] = None,
                 output_f32: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None,
                 dtype: torch.dtype = torch.float16,
                 stream: Optional[torch.cuda.Stream] = None):
    """Fixed-order merge of partial states (library entry pa_merge_states).

    state_out fp32 [P, R, D], state_lse fp32 [P, R] (natural log, -inf =
    empty); states fold in index order.  Returns (output [R, D] in ``dtype``
    (fp16 or bf16; the type of ``output`` when given), lse fp32 [R]);
    ``output_f32`` optionally receives the unrounded output."""
    lib = library()
    if state_out.dim() != 3 or state_lse.shape != state_out.shape[:2]:
        raise ValueError("state_out must be [P, R, D] and state_lse [P, R]")
    for name, t in (("state_out", state_out), ("state_lse", state_lse)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    P, R, D = state_out.shape
    dev = state_out.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(s):  # results belong to the stream that writes them
        if output is None:
            output = torch.empty((R, D), dtype=dtype, device=dev)
        if lse is None:
            lse = torch.empty((R,), dtype=torch.float32, device=dev)
    a = PaMergeArgs()
    a.struct_size = ctypes.sizeof(PaMergeArgs)
    a.dtype = _dtype_code(output)
    a.num_states = P
    a.head_size = D
    a.num_rows = R
    a.state_out = _ptr(state_out)
    a.state_lse = _ptr(state_lse)
    a.output = _ptr(output)
    a.output_f32 = _ptr(output_f32)
    a.lse = _ptr(lse)
    st = lib.pa_merge_states(ctypes.byref(a), s.cuda_stream)
    if st != 0:
        raise PagedAttentionError(st, lib.pa_status_string(st).decode())
    return output, lse
