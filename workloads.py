"""Seeded synthetic inputs for the paged KV-cache attention path.

This module only *builds inputs*: lengths, page tables, page-id permutations,
N(0,1) tensors in fp16 or bf16 and the slot list a page allocator hands out.  It holds no
attention arithmetic (no scatter, gather, softmax or merge), so both the oracle
tests and the HIP path can draw their inputs from it without sharing any of the
method's computation.

Shapes follow the com.microsoft PagedAttention operator contract
("com.microsoft.PagedAttention" model-card README, sections Inputs/Attributes):
  query        [N, H*D]  or packed [N, (H+2*Hkv)*D] when key/value are absent
  key, value   [N, Hkv*D]
  key_cache,
  value_cache  [num_blocks, block_size, Hkv, D]
  cumulative_sequence_length [B+1], past_seqlens [B], block_table [B, MB],
  slot_mapping [N] (optional, -1 = no write).

Page-table rules follow the KVCacheSpec paragraph of "WS2 CP-Aware Attention
Contract" (section Mode-Specific Metadata): padding is trailing, the number of
active pages is ceil(kv_len/page_size), a sequence never repeats a page id, and
pages are shared across sequences only as a declared, fully populated,
read-only prefix.

Draw order for one batch (fixed so that a seed names one input exactly):
  1. per-sequence new-token counts (order permutation), 2. past lengths,
  3. physical page permutation, 4. slot_mapping entries switched to -1,
  5. query / key / value (or packed query), 6. key_cache, 7. value_cache.
With ``meta_only=True`` the draws stop after step 4 and the data tensors are
left uninitialised (only their shapes are meaningful).

INT8 caches (``kv_quant="int8"``): the cache tensors are int8 codes and the
batch carries per-(kv head, channel) scales; the step's K/V stay in dtype.
INT4 caches (``kv_quant="int4"``): uint8 tensors [NB, bs, Hkv, D/2] whose two
nibbles per byte are independent codes (the even element in bits 0-3), with
scales as for INT8.

Data type: every workload takes ``dtype`` "f16" (default) or "bf16", and
``head_size`` (0 = its own; 256 for the head_size-256 variant: same heads,
lengths and pages, wider heads).  The
float32 draws are the same for both; they are rounded to nearest (ties to
even) to the type.  numpy has no bfloat16, so bf16 tensors are numpy uint16
arrays holding the bit patterns (the upper half of the float32 pattern).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

_CHUNK = 1 << 24  # elements per draw when filling large fp16 tensors


def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp16 tensor, drawn in float32 chunks so multi-GB caches fit."""
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        flat[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 (finite) -> bfloat16 bit patterns as uint16, round to nearest,
    ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) bf16 tensor (uint16 bit patterns), same float32 draws as
    normal_f16."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        flat[s:e] = round_bf16(rng.standard_normal(e - s, dtype=np.float32))
    return out


# INT8 caches: synthetic codes round(28 * N(0,1)) clipped to [-127, 127], and
# per-(kv head, channel) scales 4.5/127 * 2^U(-1/4, 1/4) that cover about
# 4.5 standard deviations of the step's N(0,1) rows
INT8_CODE_GAIN = 28.0
INT8_SCALE = 4.5 / 127.0


def int8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.int8)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32) * np.float32(INT8_CODE_GAIN)
        flat[s:e] = np.clip(np.rint(x), -127, 127).astype(np.int8)
    return out


def int8_scales(rng: np.random.Generator, Hkv: int, D: int) -> np.ndarray:
    return (INT8_SCALE * np.exp2(rng.uniform(-0.25, 0.25, (Hkv, D)))).astype(np.float32)


# INT4 caches: codes round(1.6 * N(0,1)) clipped to [-7, 7], each stored as the
# 4-bit two's complement nibble (code & 15), two per byte; scales
# 4.5/7 * 2^U(-1/4, 1/4), so a cached value is about N(0,1) and the step's
# N(0,1) rows use about two thirds of the code range on each side
INT4_CODE_GAIN = 1.6
INT4_SCALE = 4.5 / 7.0


def int4_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    """uint8 [..., D/2] for a logical shape [..., D]."""
    *lead, D = shape
    out = np.empty((*lead, D // 2), dtype=np.uint8)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        c = np.clip(np.rint(rng.standard_normal((e - s, 2), dtype=np.float32) * np.float32(INT4_CODE_GAIN)),
                    -7, 7).astype(np.int16) & 15
        flat[s:e] = (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)
    return out


def int4_scales(rng: np.random.Generator, Hkv: int, D: int) -> np.ndarray:
    return (INT4_SCALE * np.exp2(rng.uniform(-0.25, 0.25, (Hkv, D)))).astype(np.float32)


def storage_dtype(dtype: str):
    """numpy dtype that holds tensors of data type ``dtype``."""
    return {"f16": np.float16, "bf16": np.uint16}[dtype]


@dataclasses.dataclass
class Batch:
    """One call's worth of operator inputs (numpy, host side)."""

    name: str
    seed: int
    query: np.ndarray                 # fp16 [N, H*D] or [N, (H+2Hkv)*D]
    key: Optional[np.ndarray]         # fp16 [N, Hkv*D] or None (packed)
    value: Optional[np.ndarray]       # fp16 [N, Hkv*D] or None (packed)
    key_cache: np.ndarray             # fp16 [NB, bs, Hkv, D]
    value_cache: np.ndarray           # fp16 [NB, bs, Hkv, D]
    cum: np.ndarray                   # int32 [B+1]
    past: np.ndarray                  # int32 [B]
    block_table: np.ndarray           # int32 [B, MB], -1 padding
    slot_mapping: Optional[np.ndarray]  # int32 [N] or None
    num_heads: int
    kv_num_heads: int
    head_size: int
    block_size: int
    scale: float = 0.0
    note: str = ""
    dtype: str = "f16"                # "f16" (float16 arrays) or "bf16" (uint16 bit patterns)
    kv_quant: str = "none"            # "none" (caches in dtype), "int8" or "int4" (codes + scales)
    k_scale: Optional[np.ndarray] = None  # fp32 [Hkv, D] with kv_quant "int8" / "int4"
    v_scale: Optional[np.ndarray] = None

    @property
    def num_tokens(self) -> int:
        return int(self.cum[-1])

    @property
    def batch_size(self) -> int:
        return int(self.past.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cum).astype(np.int64)

    @property
    def kv_lens(self) -> np.ndarray:
        return self.past.astype(np.int64) + self.q_lens

    @property
    def packed(self) -> bool:
        return self.key is None


# ---------------------------------------------------------------------------
# page allocation
# ---------------------------------------------------------------------------

def pages_needed(total_len: int, block_size: int) -> int:
    """Active pages for a sequence of total_len tokens: ceil(len/page)."""
    return -(-int(total_len) // int(block_size))


def allocate_pages(rng: np.random.Generator, kv_lens: Sequence[int], block_size: int,
                   num_blocks: Optional[int] = None, max_blocks: Optional[int] = None,
                   shared_prefix: Optional[Sequence[int]] = None,
                   group_size: int = 4):
    """Hand out physical pages to sequences.

    Without ``shared_prefix`` every logical page of every sequence gets its own
    physical page; the ids are ``rng.permutation(num_blocks)`` taken in order.
    With ``shared_prefix`` (pages each sequence may take from a prefix chain
    shared by its group of ``group_size`` consecutive rows), each group owns one
    chain of ``max`` shared pages and every sequence adds exclusive pages
    after its shared ones.  Returns (block_table [B, MB] int32 with -1 padding,
    num_blocks, pages_used).
    """
    kv_lens = [int(x) for x in kv_lens]
    n = [pages_needed(L, block_size) for L in kv_lens]
    B = len(kv_lens)
    mb = max([1] + n) if max_blocks is None else int(max_blocks)
    if shared_prefix is None:
        used = sum(n)
        nb = used if num_blocks is None else int(num_blocks)
        if used > nb:
            raise ValueError(f"pool of {nb} pages cannot hold {used}")
        ids = rng.permutation(nb)
        table = np.full((B, mb), -1, dtype=np.int32)
        cursor = 0
        for b in range(B):
            table[b, :n[b]] = ids[cursor:cursor + n[b]]
            cursor += n[b]
        return table, nb, used
    shared = [int(x) for x in shared_prefix]
    groups = [list(range(s, min(B, s + group_size))) for s in range(0, B, group_size)]
    chain_len = [max(shared[b] for b in g) for g in groups]
    used = sum(chain_len) + sum(n[b] - shared[b] for b in range(B))
    nb = used if num_blocks is None else int(num_blocks)
    if used > nb:
        raise ValueError(f"pool of {nb} pages cannot hold {used}")
    ids = rng.permutation(nb)
    table = np.full((B, mb), -1, dtype=np.int32)
    cursor = 0
    for g, members in enumerate(groups):
        chain = ids[cursor:cursor + chain_len[g]]
        cursor += chain_len[g]
        for b in members:
            table[b, :shared[b]] = chain[:shared[b]]
    for b in range(B):
        k = n[b] - shared[b]
        table[b, shared[b]:n[b]] = ids[cursor:cursor + k]
        cursor += k
    return table, nb, used


def allocator_slots(block_table: np.ndarray, past: np.ndarray, q_lens: np.ndarray,
                    block_size: int) -> np.ndarray:
    """The flat cache slot a page allocator hands each new token.

    For each sequence the allocator lays its pages end to end (page p covers
    slots p*block_size .. p*block_size+block_size-1) into one list of slots,
    one per logical position, and gives new token i the entry at position
    past+i.  This is the allocator's own bookkeeping, built by enumeration.
    """
    out = []
    for b in range(block_table.shape[0]):
        q = int(q_lens[b])
        if q == 0:
            continue
        p = int(past[b])
        n = pages_needed(p + q, block_size)
        row = block_table[b, :n].astype(np.int64)
        layout = np.concatenate([np.arange(pg * block_size, (pg + 1) * block_size)
                                 for pg in row])
        out.append(layout[p:p + q])
    if not out:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(out).astype(np.int32)


def cum_from_lens(q_lens: Sequence[int]) -> np.ndarray:
    c = np.zeros(len(q_lens) + 1, dtype=np.int64)
    c[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    return c.astype(np.int32)


# ---------------------------------------------------------------------------
# generic builder
# ---------------------------------------------------------------------------

def make_batch(q_lens: Sequence[int], past_lens: Sequence[int], *, num_heads: int,
               kv_num_heads: int, head_size: int, block_size: int, seed: int = 0,
               rng: Optional[np.random.Generator] = None, packed: bool = False,
               slot_mode: Optional[str] = None, drop_count: int = 0,
               num_blocks: Optional[int] = None, max_blocks: Optional[int] = None,
               shared_prefix: Optional[Sequence[int]] = None, scale: float = 0.0,
               name: str = "custom", note: str = "", dtype: str = "f16",
               kv_quant: str = "none") -> Batch:
    """Build one batch.  ``slot_mode``: None (omit slot_mapping), "derived"
    (allocator slots), or "drop" (allocator slots with ``drop_count`` entries
    set to -1, chosen by ``rng.choice(N, drop_count, replace=False)``)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    q_lens = np.asarray(q_lens, dtype=np.int64)
    past = np.asarray(past_lens, dtype=np.int64)
    kv = past + q_lens
    table, nb, _ = allocate_pages(rng, kv, block_size, num_blocks=num_blocks,
                                  max_blocks=max_blocks, shared_prefix=shared_prefix)
    return _fill(rng, name, seed, q_lens, past, table, nb, num_heads, kv_num_heads,
                 head_size, block_size, packed, slot_mode, drop_count, scale, note, dtype=dtype,
                 kv_quant=kv_quant)


def _fill(rng, name, seed, q_lens, past, table, nb, H, Hkv, D, bs, packed, slot_mode,
          drop_count, scale, note, meta_only=False, dtype="f16", kv_quant="none") -> Batch:
    cum = cum_from_lens(q_lens)
    N = int(cum[-1])
    slots = None
    if slot_mode is not None:
        slots = allocator_slots(table, past, q_lens, bs)
        if slot_mode == "drop" and drop_count > 0:
            idx = rng.choice(N, drop_count, replace=False)
            slots[idx] = -1
        elif slot_mode not in ("derived", "drop"):
            raise ValueError(slot_mode)
    normal = {"f16": normal_f16, "bf16": normal_bf16}[dtype]
    draw = (lambda shape: np.empty(shape, storage_dtype(dtype))) if meta_only else \
        (lambda shape: normal(rng, shape))
    if packed:
        query = draw((N, (H + 2 * Hkv) * D))
        key = value = None
    else:
        query = draw((N, H * D))
        key = draw((N, Hkv * D))
        value = draw((N, Hkv * D))
    k_scale = v_scale = None
    if kv_quant == "int8":
        if meta_only:
            key_cache = np.empty((nb, bs, Hkv, D), np.int8)
            value_cache = np.empty((nb, bs, Hkv, D), np.int8)
        else:
            key_cache = int8_codes(rng, (nb, bs, Hkv, D))
            value_cache = int8_codes(rng, (nb, bs, Hkv, D))
        k_scale = int8_scales(rng, Hkv, D)
        v_scale = int8_scales(rng, Hkv, D)
    elif kv_quant == "int4":
        if meta_only:
            key_cache = np.empty((nb, bs, Hkv, D // 2), np.uint8)
            value_cache = np.empty((nb, bs, Hkv, D // 2), np.uint8)
        else:
            key_cache = int4_bytes(rng, (nb, bs, Hkv, D))
            value_cache = int4_bytes(rng, (nb, bs, Hkv, D))
        k_scale = int4_scales(rng, Hkv, D)
        v_scale = int4_scales(rng, Hkv, D)
    elif kv_quant == "none":
        key_cache = draw((nb, bs, Hkv, D))
        value_cache = draw((nb, bs, Hkv, D))
    else:
        raise ValueError(kv_quant)
    return Batch(name=name, seed=seed, query=query, key=key, value=value,
                 key_cache=key_cache, value_cache=value_cache, cum=cum,
                 past=past.astype(np.int32), block_table=table, slot_mapping=slots,
                 num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                 scale=float(scale), note=note, dtype=dtype, kv_quant=kv_quant,
                 k_scale=k_scale, v_scale=v_scale)


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def tiny(seed: int = 0, meta_only: bool = False, dtype: str = "f16", head_size: int = 0,
         kv_quant: str = "none") -> Batch:
    """B=2, H/Hkv=4/2, D=64, block_size 16, 8 pages, past [5,20], new [3,1];
    block_table is a random permutation of all 8 pages, no slot_mapping."""
    rng = np.random.default_rng(seed)
    q_lens = np.array([3, 1])
    past = np.array([5, 20])
    table = rng.permutation(8).astype(np.int32).reshape(2, 4)
    return _fill(rng, "tiny", seed, q_lens, past, table, 8, 4, 2, head_size or 64, 16, False, None,
                 0, 0.0, "B=2 4/2 heads D=64 bs=16 NB=8 past=[5,20] q=[3,1]", meta_only, dtype,
                 kv_quant)


def pure_decode(seed: int = 0, meta_only: bool = False, dtype: str = "f16", head_size: int = 0,
                kv_quant: str = "none") -> Batch:
    """B=64 single-token decodes, past ~ U[512,4096], 32/8 heads, D=128,
    block_size 16, pool sized to fit, shuffled page ids."""
    rng = np.random.default_rng(seed)
    q_lens = np.ones(64, dtype=np.int64)
    past = rng.integers(512, 4096 + 1, size=64)
    table, nb, _ = allocate_pages(rng, past + q_lens, 16)
    return _fill(rng, "pure_decode", seed, q_lens, past, table, nb, 32, 8, head_size or 128, 16, False,
                 None, 0, 0.0, "B=64 q=1 past~U[512,4096] 32/8 D=128 bs=16", meta_only, dtype, kv_quant)


def mixed(seed: int = 0, meta_only: bool = False, dtype: str = "f16", head_size: int = 0,
          kv_quant: str = "none") -> Batch:
    """B=16: 8 decodes + 8 chunks of 512 new tokens (order shuffled), past ~
    U[0,8192], 32/8 heads, D=128, block_size 256, random page table."""
    rng = np.random.default_rng(seed)
    q_lens = rng.permutation(np.array([1] * 8 + [512] * 8))
    past = rng.integers(0, 8192 + 1, size=16)
    table, nb, _ = allocate_pages(rng, past + q_lens, 256)
    return _fill(rng, "mixed", seed, q_lens, past, table, nb, 32, 8, head_size or 128, 256, False, None,
                 0, 0.0, "B=16 (8x1 + 8x512) past~U[0,8192] 32/8 D=128 bs=256", meta_only, dtype, kv_quant)


def long_prefill(seed: int = 0, meta_only: bool = False, dtype: str = "f16", head_size: int = 0,
                 kv_quant: str = "none") -> Batch:
    """One sequence, 2048 new tokens on top of 2048 cached (second half of a
    4096-token sequence), 16/4 heads (one of two tensor-parallel ranks of a
    32/8 model), D=128, block_size 256, 16 pages in shuffled order."""
    rng = np.random.default_rng(seed)
    q_lens = np.array([2048])
    past = np.array([2048])
    table = rng.permutation(16).astype(np.int32)[None, :]
    return _fill(rng, "long_prefill", seed, q_lens, past, table, 16, 16, 4, head_size or 128, 256,
                 False, None, 0, 0.0, "B=1 q=2048 past=2048 16/4 D=128 bs=256", meta_only, dtype, kv_quant)


def serving(seed: int = 0, meta_only: bool = False, dtype: str = "f16", head_size: int = 0,
            kv_quant: str = "none") -> Batch:
    """B=256: 224 decodes + 32 chunks of 128 (order shuffled), past ~
    U[256,16384], 32/8 heads, D=128, block_size 256, 4096 pages, packed
    [Q|K|V] query, explicit slot_mapping with 5% of entries -1.

    4096 pages cannot hold 256 disjoint histories of up to 16.5k tokens, so
    consecutive rows form groups of 4 that share a read-only, fully populated
    prefix chain (each row takes floor(past/256) pages of it), as allowed for
    declared shared-prefix pages; every page a new token lands in is
    exclusive.  Redraws (same rng stream) if a draw would need >4096 pages.
    """
    rng = np.random.default_rng(seed)
    bs, nb, B = 256, 4096, 256
    while True:
        q_lens = rng.permutation(np.array([1] * 224 + [128] * 32))
        past = rng.integers(256, 16384 + 1, size=B)
        shared = past // bs
        try:
            table, nb_, _ = allocate_pages(rng, past + q_lens, bs, num_blocks=nb,
                                           max_blocks=65, shared_prefix=shared)
            break
        except ValueError:
            continue
    N = int(q_lens.sum())
    return _fill(rng, "serving", seed, q_lens, past, table, nb_, 32, 8, head_size or 128, bs, True,
                 "drop", int(round(0.05 * N)), 0.0,
                 "B=256 (224x1 + 32x128) past~U[256,16384] 32/8 D=128 bs=256 NB=4096 "
                 "packed QKV, slot_mapping 5% -1, groups of 4 share prefix pages", meta_only, dtype,
                 kv_quant)


WORKLOADS = {
    "tiny": tiny,
    "pure_decode": pure_decode,
    "mixed": mixed,
    "long_prefill": long_prefill,
    "serving": serving,
}


def workload(name: str, seed: int = 0, meta_only: bool = False, dtype: str = "f16",
             head_size: int = 0, kv_quant: str = "none") -> Batch:
    """A named workload; ``head_size`` (0: the workload's own) replaces only
    the head size, for the head_size-256 variants of the same shapes."""
    return WORKLOADS[name](seed, meta_only, dtype, head_size, kv_quant)


def output_gate_input(batch: "Batch", seed: int) -> np.ndarray:
    """An output-gate tensor [N, H*D] for the batch: N(0,1) in the batch's data
    type (its own seeded stream, so the batch's other draws do not move)."""
    rng = np.random.default_rng(seed)
    normal = {"f16": normal_f16, "bf16": normal_bf16}[batch.dtype]
    return normal(rng, (batch.num_tokens, batch.num_heads * batch.head_size))


def token_positions(batch: "Batch") -> np.ndarray:
    """Logical position past_b + i of every packed token (int64 [N])."""
    return np.concatenate([np.arange(int(batch.past[i]), int(batch.past[i]) + int(q))
                           for i, q in enumerate(batch.q_lens)] or [np.zeros(0)]).astype(np.int64)


def prologue_inputs(batch: "Batch", seed: int, rotary_dim: int = 0, norm: bool = True,
                    spatial: bool = False, theta: float = 1.0e6, adjacent: bool = False,
                    interleaved: bool = True) -> dict:
    """Inputs of the fused Q/K prologue for a batch (own seeded stream).

    position_ids int64 [3, N]: every row is the token's logical position
    (text tokens); with ``spatial`` rows 1 and 2 are drawn in [0, 64) instead
    (a spatial grid position).  Norm weights fp32 [D]: offsets N(0, 0.1^2).
    rotary_dim 0: the head size.  Sections: rotary_dim / 2 pairs split as
    evenly as possible over the three rows, the remainder to row 0.  Returns
    the keyword arguments of the oracle's qk_prologue."""
    rng = np.random.default_rng(seed)
    D = batch.head_size
    rd = rotary_dim or D
    half = rd // 2
    pos = token_positions(batch)
    ids = np.stack([pos, pos, pos]).astype(np.int64)
    if spatial:
        ids[1] = rng.integers(0, 64, pos.size)
        ids[2] = rng.integers(0, 64, pos.size)
    out = dict(position_ids=ids, rotary_dim=rd, theta=theta,
               sections=(half - 2 * (half // 3), half // 3, half // 3),
               interleaved=interleaved, adjacent=adjacent, eps=1e-6)
    if norm:
        out["q_norm_weight"] = (rng.standard_normal(D) * 0.1).astype(np.float32)
        out["k_norm_weight"] = (rng.standard_normal(D) * 0.1).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# algorithmic work of a call (what a roofline is measured against)
# ---------------------------------------------------------------------------

def work(batch: Batch) -> dict:
    """Bytes and flops a call must move / perform at minimum.

    flops  = 4*D*H * sum_b sum_{i<q_b} (past_b + i + 1)   (QK^T and PV over
             causally visible pairs, 2 flop per multiply-add)
    kv_hist = sum_b L_b * 2 * Hkv * D * e bytes (logical history read; e = 2
             for 16-bit caches, 1 for INT8 codes, 1/2 for INT4 codes)
    plus query, output, the step's K/V, the cache writes and (quantized
    caches) the two scale tables.
    """
    H, Hkv, D = batch.num_heads, batch.kv_num_heads, batch.head_size
    q = batch.q_lens
    p = batch.past.astype(np.int64)
    L = p + q
    pairs = int(np.sum(q * p + q * (q + 1) // 2))
    dec = q == 1
    quant = batch.kv_quant in ("int8", "int4")
    row = {"none": 2 * Hkv * D * 2, "int8": 2 * Hkv * D, "int4": Hkv * D}[batch.kv_quant]  # a slot, both caches
    n_write = int(batch.num_tokens if batch.slot_mapping is None
                  else np.count_nonzero(batch.slot_mapping >= 0))
    out = {
        "flops": 4 * D * H * pairs,
        "kv_hist_bytes": int(L.sum()) * row,
        "decode_kv_hist_bytes": int(L[dec].sum()) * row,
        "prefill_flops": 4 * D * H * int(np.sum((q * p + q * (q + 1) // 2)[~dec])),
        "q_bytes": batch.num_tokens * H * D * 2,
        "o_bytes": batch.num_tokens * H * D * 2,
        "step_kv_bytes": batch.num_tokens * 2 * Hkv * D * 2,
        "cache_write_bytes": n_write * row,
        "scale_bytes": 2 * Hkv * D * 4 if quant else 0,
        "tokens": batch.num_tokens,
        "kv_tokens": int(L.sum()),
    }
    out["bytes"] = (out["kv_hist_bytes"] + out["q_bytes"] + out["o_bytes"]
                    + out["step_kv_bytes"] + out["cache_write_bytes"] + out["scale_bytes"])
    if batch.name == "serving":
        # unique pages actually referenced (shared prefix pages count once),
        # over all rows and over the single-token (decode) rows alone
        used, used_dec = set(), set()
        for b in range(batch.batch_size):
            n = pages_needed(int(L[b]), batch.block_size)
            used.update(batch.block_table[b, :n].tolist())
            if dec[b]:
                used_dec.update(batch.block_table[b, :n].tolist())
        out["kv_unique_bytes"] = len(used) * batch.block_size * row
        out["decode_kv_unique_bytes"] = len(used_dec) * batch.block_size * row
    return out
