"""numpy fp64 oracle of the com.microsoft PagedAttention operator (SEPARATE K/V).

Test infrastructure: imported only by the test suite, the package entry file's
smoke check and the benchmark's CPU-baseline leg.  Nothing here is shared with
the HIP library.

What the operator computes (model-card README "com.microsoft.PagedAttention",
sections Description, Inputs, Outputs, Attributes, Type constraints): the
step's keys and values are written into the block caches, then every packed
query row attends, causally, to its sequence's history read back through
block_table.  Grouped-query heads share a key/value head; scale 0 means
1/sqrt(head_size); only is_causal=1 exists.

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):
  * Everything is read back from the cache *after* the writes, through
    block_table, including the step's own positions; a token whose slot is -1
    sees whatever the cache already held at its position (README,
    Description: "scattered into the cache, then attended"; Inputs,
    slot_mapping: block_table "defines the read path").
  * Query head h uses key/value head h // (H/Hkv) (contiguous groups): in the
    Qwen3-8B example of "WS2 CP-Aware Attention Contract" one rank owns query
    heads 0-15 together with KV heads 0-3 only.
  * Causal alignment is bottom-right: new row i of sequence b sits at logical
    position past_b + i and sees keys 0..past_b+i ("WS2 ...", Scope and
    Mode-Specific Metadata: chunked prefill / decode have query lengths
    shorter than their KV context, one causal offset per packed sequence).
  * Packed rows are [Q | K | V], each head-major [heads, D].
  * Slot writes are applied in token order (two tokens naming one slot is
    outside the contract, so the order only makes the oracle definite).

All floating point is fp64; the caches returned hold the input bits copied,
never converted.  Data tensors are fp16 (numpy float16) or bf16 (numpy uint16
arrays of bfloat16 bit patterns, since numpy has no bfloat16); ``values``
turns either into fp64 exactly.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def values(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of a data tensor: float16 as is; uint16 as bfloat16
    bit patterns, which are the upper 16 bits of an IEEE binary32 (the lower
    16 are zero), so widening the pattern gives the number exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype != np.float16:
        raise TypeError("data tensors are float16, or uint16 holding bfloat16 bits")
    return x.astype(np.float64)


def quantize_int8(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """INT8 code of each element of x with its per-channel scale s (the
    Qwen3.8 export issue's "INT8/INT4 per-channel paged KV cache and
    calibrated scale loading", read plainly as symmetric scales given by the
    caller, one per (kv head, channel)): code = clamp(rint(x / s), -127, 127),
    the quotient taken in fp32 (x is exact there) and rounded half to even."""
    q = values(x).astype(np.float32) / np.asarray(s, dtype=np.float32)
    return np.clip(np.rint(q), -127, 127).astype(np.int8)


def quantize_int4(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """INT4 code of each element: the INT8 reading with the symmetric 4-bit
    range, clamp(rint(x / s), -7, 7), the quotient in fp32, ties to even."""
    q = values(x).astype(np.float32) / np.asarray(s, dtype=np.float32)
    return np.clip(np.rint(q), -7, 7).astype(np.int8)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Codes [..., D] (D even) as bytes [..., D/2]: element 2i in bits 0-3 and
    element 2i+1 in bits 4-7, each as a 4-bit two's complement number (the
    plainest packing of two per-channel codes into a byte, low channel
    first)."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: bytes [..., D/2] -> int8 codes [..., D] in [-8, 7]."""
    w = np.asarray(b, dtype=np.uint8).astype(np.int16)
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), dtype=np.int8)
    out[..., 0::2] = ((w & 0xF) ^ 8) - 8
    out[..., 1::2] = ((w >> 4) ^ 8) - 8
    return out


def dequantize(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact fp64 value code * s of every cached element (s broadcasts over
    the trailing [Hkv, D])."""
    return codes.astype(np.float64) * np.asarray(s, dtype=np.float32).astype(np.float64)


def resolve_call(query: np.ndarray, key: Optional[np.ndarray], value: Optional[np.ndarray],
                 num_heads: int, kv_num_heads: int, scale: float):
    """Split the query input and fix head_size and scale.

    README, Inputs (query, key, value) and Attributes (scale): query is
    [N, H*D], or [N, (H+2*Hkv)*D] carrying [Q|K|V] when key and value are both
    absent; scale == 0 selects 1/sqrt(D).  Returns (Q, K, V, D, scale) with Q
    [N, H, D], K and V [N, Hkv, D], still in the input's type.
    """
    if (key is None) != (value is None):
        raise ValueError("key and value must be given together")
    H, Hkv = int(num_heads), int(kv_num_heads)
    if H <= 0 or Hkv <= 0 or H % Hkv:
        raise ValueError("num_heads must be a positive multiple of kv_num_heads")
    N, width = query.shape
    if key is None:
        if width % (H + 2 * Hkv):
            raise ValueError("packed query width is not (H+2*Hkv)*D")
        D = width // (H + 2 * Hkv)
        Q = query[:, :H * D]
        K = query[:, H * D:(H + Hkv) * D]
        V = query[:, (H + Hkv) * D:]
    else:
        if width % H:
            raise ValueError("query width is not H*D")
        D = width // H
        Q, K, V = query, key, value
        if K.shape != (N, Hkv * D) or V.shape != (N, Hkv * D):
            raise ValueError("key/value must be [N, Hkv*D]")
    s = 1.0 / math.sqrt(D) if scale == 0 else float(scale)
    return (Q.reshape(N, H, D), K.reshape(N, Hkv, D), V.reshape(N, Hkv, D), D, s)


def scatter_kv(key_cache: np.ndarray, value_cache: np.ndarray, K: np.ndarray, V: np.ndarray,
               cum: np.ndarray, past: np.ndarray, block_table: np.ndarray,
               slot_mapping: Optional[np.ndarray], k_scale=None, v_scale=None):
    """Write each new token's K/V rows into copies of the caches.

    README, Inputs (slot_mapping): token t goes to flat slot
    block_id*block_size + offset; -1 suppresses the write; without
    slot_mapping the slot follows from past_seqlens (token i of sequence b is
    at position past_b + i, found through block_table).  The copy is bit
    exact: the stored bits are the input's bits.  With quantized caches
    (scales given) each row is stored as its codes: int8 caches hold INT8
    codes (quantize_int8), uint8 caches two INT4 codes per byte
    (quantize_int4, pack_int4).
    """
    kc = key_cache.copy()
    vc = value_cache.copy()
    NB, bs, Hkv, Dc = kc.shape
    kslots = kc.reshape(NB * bs, Hkv, Dc)
    vslots = vc.reshape(NB * bs, Hkv, Dc)

    def stored(row, sc):
        if sc is None:
            return row
        if kc.dtype == np.uint8:
            return pack_int4(quantize_int4(row, sc))
        return quantize_int8(row, sc)

    for b in range(past.shape[0]):
        for i in range(int(cum[b + 1]) - int(cum[b])):
            t = int(cum[b]) + i
            if slot_mapping is not None:
                slot = int(slot_mapping[t])
            else:
                pos = int(past[b]) + i
                slot = int(block_table[b, pos // bs]) * bs + pos % bs
            if slot >= 0:
                kslots[slot] = stored(K[t], k_scale)
                vslots[slot] = stored(V[t], v_scale)
    return kc, vc


def gather_history(kc: np.ndarray, vc: np.ndarray, block_table: np.ndarray, b: int,
                   length: int, k_scale=None, v_scale=None):
    """Contiguous fp64 copies [length, Hkv, D] of sequence b's positions
    0..length-1, each read at slot block_table[b, j // bs]*bs + j % bs
    (README, Inputs: block_table maps a sequence's logical blocks to
    physical blocks and defines the read path).  Quantized caches read as
    code * scale (uint8 caches: two INT4 codes per byte, unpack_int4)."""
    NB, bs, Hkv, Dc = kc.shape
    j = np.arange(int(length), dtype=np.int64)
    idx = block_table[b, j // bs].astype(np.int64) * bs + j % bs
    kr = kc.reshape(NB * bs, Hkv, Dc)[idx]
    vr = vc.reshape(NB * bs, Hkv, Dc)[idx]
    if kc.dtype == np.uint8 and k_scale is not None:
        kr, vr = unpack_int4(kr), unpack_int4(vr)
    Kb = values(kr) if k_scale is None else dequantize(kr, k_scale)
    Vb = values(vr) if v_scale is None else dequantize(vr, v_scale)
    return Kb, Vb


def attend_sequence(Qb: np.ndarray, Kb: np.ndarray, Vb: np.ndarray, past_b: int,
                    scale: float, rows: Optional[Sequence[int]] = None, with_lse: bool = False):
    """Causal grouped-query softmax attention of one sequence, brute force.

    Qb [q, H, D], Kb/Vb [L, Hkv, D] (fp64, L = past_b + q).  For head h with
    kv head k = h // (H/Hkv): S = scale * Q_h K_k^T, entries with key
    position j > past_b + i set to -inf, P = softmax over keys, O = P V_k.
    ``rows`` restricts the work to those new-token rows (others are NaN).
    Returns [q, H, D] fp64; with ``with_lse`` also the attention-domain lse
    [q, H] = log sum_j exp(S_j) over the visible keys (natural log; "WS2
    CP-Aware Attention Contract", Reduction Semantics: the partial state of a
    row is (out, lse)).
    """
    q, H, D = Qb.shape
    L, Hkv, _ = Kb.shape
    G = H // Hkv
    sel = np.arange(q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((q, H, D), np.nan)
    lse = np.full((q, H), np.nan)
    if sel.size == 0:
        return (out, lse) if with_lse else out
    pos = int(past_b) + sel
    masked = np.arange(L)[None, :] > pos[:, None]
    for h in range(H):
        k = h // G
        S = scale * (Qb[sel, h, :] @ Kb[:, k, :].T)
        S[masked] = -np.inf
        mx = S.max(axis=1, keepdims=True)
        P = np.exp(S - mx)
        den = P.sum(axis=1, keepdims=True)
        out[sel, h, :] = (P / den) @ Vb[:, k, :]
        lse[sel, h] = (mx + np.log(den))[:, 0]
    return (out, lse) if with_lse else out


def output_gate(out: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """The attention output times sigmoid(gate), elementwise, in fp64.

    "Add Qwen3.8 packed hybrid PagedAttention export for ORT GenAI Engine",
    Per-layer behavior (Full attention): the doubled Q projection is split per
    head into the query and an output gate, and sigmoid(gate) is applied to
    the attention output; read plainly, the gate has the output's shape
    [N, H*D] and sigmoid(g) = 1 / (1 + exp(-g)) multiplies each element."""
    g = values(gate)
    return out * (1.0 / (1.0 + np.exp(-g)))


# ---------------------------------------------------------------------------
# Fused prologue: Q/K OffsetRMSNorm, then interleaved partial MRoPE
# ---------------------------------------------------------------------------
#
# "Add Qwen3.8 packed hybrid PagedAttention export for ORT GenAI Engine",
# Per-layer behavior (Full attention, step 3): the query and key heads get an
# OffsetRMSNorm and then an interleaved partial MRoPE, norm before RoPE, once
# ("do not normalize twice"); the positions are position_ids INT64 [3, N]
# (Packed graph contract, Shared inputs).  "WS2 CP-Aware Attention Contract",
# RoPE / Position Semantics and the Qwen3-8B example: the cached K is
# post-RoPE, the rotation has a base theta and a rotary_dim that fits the head
# dimension, and the result is cast to the data type after RoPE.  Readings of
# what the pages leave open (each a parameter here):
#   * OffsetRMSNorm of a head row x [D] with weights w [D]:
#     y = x * (1 + w) / sqrt(mean(x^2) + eps)  (the weight is an offset from 1);
#   * partial: the first rotary_dim channels of each head rotate, the rest
#     pass through; frequency pair i < rotary_dim / 2 has inverse frequency
#     theta^(-2i / rotary_dim) and angle position * inverse frequency;
#   * pairing: pair i is channels (i, i + rotary_dim/2) ("half"), or channels
#     (2i, 2i+1) ("adjacent"), rotated as y1 = x1 cos - x2 sin,
#     y2 = x2 cos + x1 sin;
#   * MRoPE sections: pair i takes its position from component c(i) of the
#     three rows of position_ids, with section sizes (s0, s1, s2) summing to
#     rotary_dim / 2; "interleaved": c(i) = i mod 3 while that component still
#     has room, else the first component that has; "contiguous": the first s0
#     pairs use component 0, the next s1 component 1, the rest component 2.


def round_to_format(x: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round fp64 values to the nearest number with mant_bits significant
    bits and minimum normal exponent emin (ties to even), as fp64: fp16 is
    (11, -14), bf16 is (8, -126).  Quantum 2^(max(e, emin) - mant_bits + 1)
    for |x| in [2^e, 2^(e+1)).  Finite inputs of moderate size only."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                    # x = m 2^e, m in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e - 1, emin) - mant_bits + 1)
    return np.rint(x / q) * q


def to_dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values -> storage of the data type, rounded to nearest even:
    float16 arrays for "f16", uint16 bfloat16 bit patterns for "bf16"."""
    if dtype == "bf16":
        r = round_to_format(x, 8, -126).astype(np.float32)  # exact in fp32
        return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return round_to_format(x, 11, -14).astype(np.float16)   # exact in fp16


def offset_rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """OffsetRMSNorm over the last axis: x * (1 + w) / sqrt(mean(x^2) + eps),
    fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * (1.0 + np.asarray(w, dtype=np.float64))


def mrope_components(rotary_dim: int, sections, interleaved: bool = True) -> np.ndarray:
    """Position component (0, 1 or 2) of each frequency pair i < rotary_dim/2."""
    half = rotary_dim // 2
    sections = [int(v) for v in sections]
    if len(sections) != 3 or sum(sections) != half or min(sections) < 0:
        raise ValueError("mrope sections must be three counts summing to rotary_dim / 2")
    comp = np.empty(half, dtype=np.int64)
    if interleaved:
        used = [0, 0, 0]
        for i in range(half):
            c = i % 3
            if used[c] >= sections[c]:
                c = next(k for k in range(3) if used[k] < sections[k])
            comp[i] = c
            used[c] += 1
    else:
        comp[:] = np.repeat(np.arange(3), sections)
    return comp


def rotary_angles(position_ids: np.ndarray, rotary_dim: int, theta: float,
                  components: np.ndarray) -> np.ndarray:
    """Angles [N, rotary_dim/2] (fp64): position_ids[c(i), t] * theta^(-2i/rotary_dim)."""
    half = rotary_dim // 2
    inv = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    pos = np.asarray(position_ids, dtype=np.int64)[components, :].T.astype(np.float64)  # [N, half]
    return pos * inv[None, :]


def apply_rotary(x: np.ndarray, angles: np.ndarray, rotary_dim: int,
                 adjacent: bool = False) -> np.ndarray:
    """Rotate the first rotary_dim channels of x [N, heads, D] (fp64) by
    angles [N, rotary_dim/2]; the other channels are returned unchanged."""
    y = np.array(x, dtype=np.float64, copy=True)
    half = rotary_dim // 2
    if adjacent:
        i1, i2 = np.arange(0, rotary_dim, 2), np.arange(1, rotary_dim, 2)
    else:
        i1, i2 = np.arange(half), np.arange(half, rotary_dim)
    cos = np.cos(angles)[:, None, :]
    sin = np.sin(angles)[:, None, :]
    x1, x2 = y[:, :, i1].copy(), y[:, :, i2].copy()
    y[:, :, i1] = x1 * cos - x2 * sin
    y[:, :, i2] = x2 * cos + x1 * sin
    return y


def qk_prologue(Q: np.ndarray, K: np.ndarray, *, position_ids=None, rotary_dim: int = 0,
                theta: float = 1.0e6, sections=None, interleaved: bool = True,
                adjacent: bool = False, q_norm_weight=None, k_norm_weight=None,
                eps: float = 1e-6, rounded: bool = True):
    """The fused prologue on Q [N, H, D] and K [N, Hkv, D] (data-type storage):
    OffsetRMSNorm of every head (when its weights are given), then the
    partial MRoPE (when rotary_dim > 0), then the cast to the data type.
    Returns (Q', K') in the data type's storage, or fp64 with rounded=False."""
    dtype = "bf16" if np.asarray(Q).dtype == np.uint16 else "f16"
    q, k = values(Q), values(K)
    if q_norm_weight is not None:
        q = offset_rms_norm(q, q_norm_weight, eps)
    if k_norm_weight is not None:
        k = offset_rms_norm(k, k_norm_weight, eps)
    if rotary_dim:
        D = q.shape[-1]
        if rotary_dim % 2 or not 0 < rotary_dim <= D:
            raise ValueError("rotary_dim must be even and fit the head size")
        if sections is None:
            raise ValueError("rotary needs the three section sizes")
        ang = rotary_angles(position_ids, rotary_dim, theta,
                            mrope_components(rotary_dim, sections, interleaved))
        q = apply_rotary(q, ang, rotary_dim, adjacent)
        k = apply_rotary(k, ang, rotary_dim, adjacent)
    if not rounded:
        return q, k
    return to_dtype_bits(q, dtype), to_dtype_bits(k, dtype)


def paged_attention(query, key, value, key_cache, value_cache, cum, past, block_table,
                    slot_mapping=None, *, num_heads: int, kv_num_heads: int,
                    scale: float = 0.0, is_causal: int = 1, rows=None, with_lse: bool = False,
                    k_scale=None, v_scale=None, gate=None, prologue=None):
    """The whole operator: returns (output fp64 [N, H*D], key_cache', value_cache').

    README, Description/Outputs: the caches are updated (here: copies are
    returned) and output holds one row of H*D values per packed token.
    ``rows``: optional sorted token indices to compute (others are NaN), so
    that full-size workloads can be checked on a sample.  ``with_lse``: also
    return the attention-domain lse [N, H] of every row (see attend_sequence)
    as a fourth value.  ``k_scale``/``v_scale`` ([Hkv, D] fp32, both or
    neither): the caches hold codes, INT8 (int8 caches) or INT4 (uint8
    caches, [NB, bs, Hkv, D/2], two codes per byte); the step's rows are
    quantized on write and every cached element reads as code * scale.
    ``gate`` ([N, H*D] in the data type): the returned output is
    output_gate(attention, gate); the lse (the row's state) is unchanged.
    ``prologue`` (a dict of qk_prologue's keyword arguments): the step's
    query and key rows are first normalised and rotated (qk_prologue), and
    those rows are what is cached and attended.
    """
    if (k_scale is None) != (v_scale is None):
        raise ValueError("k_scale and v_scale go together")
    if int(is_causal) != 1:
        raise ValueError("only is_causal=1 is defined")
    Q, K, V, D, s = resolve_call(query, key, value, num_heads, kv_num_heads, scale)
    if prologue is not None:
        Q, K = qk_prologue(Q, K, **prologue)
    cum = np.asarray(cum, dtype=np.int64)
    past = np.asarray(past, dtype=np.int64)
    N = Q.shape[0]
    if cum[0] != 0 or cum[-1] != N or np.any(np.diff(cum) < 0):
        raise ValueError("cumulative_sequence_length must run from 0 to N")
    kc, vc = scatter_kv(key_cache, value_cache, K, V, cum, past, block_table, slot_mapping,
                        k_scale, v_scale)
    out = np.full((N, num_heads, D), np.nan)
    lse = np.full((N, num_heads), np.nan)
    want = None if rows is None else np.zeros(N, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True
    for b in range(past.shape[0]):
        t0, t1 = int(cum[b]), int(cum[b + 1])
        if t1 == t0:
            continue
        local = None
        if want is not None:
            local = np.nonzero(want[t0:t1])[0]
            if local.size == 0:
                continue
        L = int(past[b]) + (t1 - t0)
        Kb, Vb = gather_history(kc, vc, block_table, b, L, k_scale, v_scale)
        Qb = values(Q[t0:t1])
        if with_lse:
            out[t0:t1], lse[t0:t1] = attend_sequence(Qb, Kb, Vb, int(past[b]), s, rows=local,
                                                     with_lse=True)
        else:
            out[t0:t1] = attend_sequence(Qb, Kb, Vb, int(past[b]), s, rows=local)
    out = out.reshape(N, num_heads * D)
    if gate is not None:
        out = output_gate(out, gate)
    if with_lse:
        return out, kc, vc, lse
    return out, kc, vc


def partial_state(q_row: np.ndarray, Kk: np.ndarray, Vk: np.ndarray, scale: float,
                  keys: Sequence[int]):
    """Partial attention state of one query row and head over a key subset.

    "WS2 CP-Aware Attention Contract", Reduction Semantics: a partial state is
    (out, attention-domain lse).  Here out = sum_j softmax_J(s)_j v_j and
    lse = log sum_{j in J} exp(s_j) with s_j = scale <q, k_j>, natural log,
    fp64.  q_row [D], Kk/Vk [L, D].
    """
    J = np.asarray(keys, dtype=np.int64)
    s = scale * (Kk[J] @ q_row)
    m = s.max()
    w = np.exp(s - m)
    return (w @ Vk[J]) / w.sum(), m + math.log(w.sum())


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[float]) -> np.ndarray:
    """Fixed-order merge of partial states ("WS2 CP-Aware Attention Contract",
    Reduction Semantics: online-softmax merge by lse, fp32-or-wider
    accumulation, fixed global block order, downcast only at the final write).
    out = sum_s e^{lse_s - M} out_s / sum_s e^{lse_s - M}, M = max_s lse_s,
    summed in the given order."""
    M = max(lses)
    num = np.zeros_like(np.asarray(outs[0], dtype=np.float64))
    den = 0.0
    for o, l in zip(outs, lses):
        w = math.exp(l - M)
        num = num + w * np.asarray(o, dtype=np.float64)
        den += w
    return num / den


def merge_states(outs: np.ndarray, lses: np.ndarray):
    """Merge of partial states, whole tensors at once ("WS2 CP-Aware Attention
    Contract", Reduction Semantics: partial state (out, attention-domain lse),
    online-softmax merge, fixed order, one downcast at the final write).

    outs [P, R, D], lses [P, R] (R rows, P states per row, in merge order).
    The merged state of a row is the state of the union of the key sets:
    lse = log sum_p exp(lse_p) and out = sum_p exp(lse_p - lse) out_p, here
    evaluated with the shift M = max_p lse_p, in fp64.  A state with lse =
    -inf (no keys) has weight 0; a row whose states are all empty merges to
    out = 0, lse = -inf.  Returns (out [R, D], lse [R]) fp64.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    empty = ~np.isfinite(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(lses - Ms[None, :])            # [P, R], 0 for empty states
    den = w.sum(axis=0)
    out = np.zeros(outs.shape[1:])
    for p in range(outs.shape[0]):             # summed in the given order
        out += w[p][:, None] * outs[p]
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(empty[:, None], 0.0, out / np.where(empty, 1.0, den)[:, None])
        lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, den)))
    return out, lse
