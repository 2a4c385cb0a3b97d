"""Second oracle formulation in plain Python scalars (test infrastructure only).

Independent of paged_attention.py: no numpy arithmetic, no array gathers.  The
cache is modelled as a dict from flat slot to a per-head list of element
values (as Python floats: fp16 values, or bf16 values decoded from their bit
patterns with struct); each output element is a sum over visible keys taken with
math.fsum.  Used only on tiny inputs to pin the numpy oracle (same operator:
model-card README "com.microsoft.PagedAttention", Description and Inputs;
causal offsets and GQA grouping as read from "WS2 CP-Aware Attention
Contract").
"""
from __future__ import annotations

import math
import struct


def _num(x) -> float:
    """Value of one element: a float16 as is; a uint16 as a bfloat16 bit
    pattern, i.e. the upper half of an IEEE binary32 whose lower half is 0."""
    if getattr(x, "dtype", None) is not None and x.dtype.kind == "u":
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    return float(x)


def _row(arr, t, start, count):
    return [_num(x) for x in arr[t][start:start + count]]


def _f32(x: float) -> float:
    """x rounded to the nearest binary32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _code(x: float, s: float) -> int:
    """INT8 code clamp(round(x / s), -127, 127) with x / s rounded to binary32
    first (x, s are binary32 values, so the binary64 quotient rounded once
    more is the correctly rounded binary32 quotient); round() is half to
    even."""
    return max(-127, min(127, round(_f32(x / s))))


def _code4(x: float, s: float) -> int:
    """INT4 code clamp(round(x / s), -7, 7), the quotient rounded as in _code."""
    return max(-7, min(7, round(_f32(x / s))))


def _nibbles(byte: int):
    """The two INT4 codes of a cache byte: bits 0-3 (the even element), then
    bits 4-7, each a 4-bit two's complement number."""
    lo, hi = byte & 15, (byte >> 4) & 15
    return [lo - 16 if lo >= 8 else lo, hi - 16 if hi >= 8 else hi]


def paged_attention_scalar(query, key, value, key_cache, value_cache, cum, past,
                           block_table, slot_mapping, num_heads, kv_num_heads, scale,
                           with_lse=False, k_scale=None, v_scale=None):
    """Returns (out as nested lists [N][H*D], dict slot->(krow, vrow) of the
    slots written), and with ``with_lse`` also lse as nested lists [N][H]
    (log of the fsum of exp(score) over the visible keys, natural log).
    Inputs are numpy arrays only as containers.  With ``k_scale``/``v_scale``
    ([Hkv, D]) the caches hold codes (int8 caches: INT8; uint8 caches: two
    INT4 codes per byte): written rows are stored as codes (the dict holds
    them one per element), and a cached element reads as code * scale."""
    H, Hkv = int(num_heads), int(kv_num_heads)
    N, width = query.shape
    packed = key is None
    D = width // (H + 2 * Hkv) if packed else width // H
    sc = 1.0 / math.sqrt(D) if scale == 0 else float(scale)
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    B = len(past)

    quant = k_scale is not None
    int4 = quant and str(key_cache.dtype) == "uint8"
    code = _code4 if int4 else _code
    scales = None
    if quant:
        scales = ([float(x) for x in k_scale.reshape(-1)], [float(x) for x in v_scale.reshape(-1)])

    def k_of(t):
        return _row(query, t, H * D, Hkv * D) if packed else _row(key, t, 0, Hkv * D)

    def v_of(t):
        return _row(query, t, (H + Hkv) * D, Hkv * D) if packed else _row(value, t, 0, Hkv * D)

    # token -> (sequence, index inside the sequence)
    owner = {}
    for b in range(B):
        for t in range(int(cum[b]), int(cum[b + 1])):
            owner[t] = (b, t - int(cum[b]))

    # writes, in token order
    written = {}
    for t in range(N):
        b, i = owner[t]
        if slot_mapping is not None:
            slot = int(slot_mapping[t])
        else:
            pos = int(past[b]) + i
            blk, off = divmod(pos, bs)
            slot = int(block_table[b][blk]) * bs + off
        if slot >= 0:
            if quant:
                written[slot] = ([code(x, sv) for x, sv in zip(k_of(t), scales[0])],
                                 [code(x, sv) for x, sv in zip(v_of(t), scales[1])])
            else:
                written[slot] = (k_of(t), v_of(t))

    def cache_row(slot, which):
        if slot in written:
            row = written[slot][which]
        else:
            blk, off = divmod(slot, bs)
            src = key_cache if which == 0 else value_cache
            if int4:
                row = [c for x in src[blk][off].reshape(-1) for c in _nibbles(int(x))]
            else:
                row = [_num(x) if not quant else int(x) for x in src[blk][off].reshape(-1)]
        if quant:
            return [c * sv for c, sv in zip(row, scales[which])]
        return row

    out = []
    lse = []
    for t in range(N):
        b, i = owner[t]
        pos = int(past[b]) + i
        qrow = _row(query, t, 0, H * D)
        orow = []
        lrow = []
        for h in range(H):
            kvh = h * Hkv // H  # = h // (H/Hkv)
            scores = []
            vals = []
            for j in range(pos + 1):
                blk, off = divmod(j, bs)
                slot = int(block_table[b][blk]) * bs + off
                kr = cache_row(slot, 0)[kvh * D:(kvh + 1) * D]
                vr = cache_row(slot, 1)[kvh * D:(kvh + 1) * D]
                scores.append(sc * math.fsum(qrow[h * D + d] * kr[d] for d in range(D)))
                vals.append(vr)
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            z = math.fsum(w)
            for d in range(D):
                orow.append(math.fsum(w[j] * vals[j][d] for j in range(len(w))) / z)
            lrow.append(top + math.log(z))
        out.append(orow)
        lse.append(lrow)
    return (out, written, lse) if with_lse else (out, written)


def qk_prologue_scalar(q_rows, k_rows, D, *, position_ids=None, rotary_dim=0, theta=1.0e6,
                       sections=None, interleaved=True, adjacent=False, q_norm_weight=None,
                       k_norm_weight=None, eps=1e-6):
    """The fused prologue written out per element with Python floats ("Add
    Qwen3.8 packed hybrid PagedAttention export for ORT GenAI Engine",
    Per-layer behavior, Full attention, step 3: OffsetRMSNorm, then
    interleaved partial MRoPE; "WS2 CP-Aware Attention Contract", RoPE /
    Position Semantics: theta, rotary_dim).  q_rows / k_rows: lists over
    tokens of lists over heads of D element values.  Returns the unrounded
    (q, k) in the same nested form.

    Independent of the numpy formulation: the section of each frequency pair
    is found by counting per component, the angle is taken per element with
    math.cos / math.sin, the mean square with math.fsum."""
    half = rotary_dim // 2

    def component(i):
        if not interleaved:
            if i < sections[0]:
                return 0
            return 1 if i < sections[0] + sections[1] else 2
        used = [0, 0, 0]
        c = 0
        for j in range(i + 1):
            c = j % 3
            if used[c] >= sections[c]:
                c = [k for k in range(3) if used[k] < sections[k]][0]
            used[c] += 1
        return c

    comps = [component(i) for i in range(half)]

    def one(row, w, t):
        x = list(row)
        if w is not None:
            ms = math.fsum(v * v for v in x) / D
            r = 1.0 / math.sqrt(ms + eps)
            x = [x[d] * r * (1.0 + float(w[d])) for d in range(D)]
        if rotary_dim:
            y = list(x)
            for i in range(half):
                pos = float(position_ids[comps[i]][t])
                ang = pos * theta ** (-2.0 * i / rotary_dim)
                a, b = (2 * i, 2 * i + 1) if adjacent else (i, i + half)
                y[a] = x[a] * math.cos(ang) - x[b] * math.sin(ang)
                y[b] = x[b] * math.cos(ang) + x[a] * math.sin(ang)
            x = y
        return x

    q = [[one(h, q_norm_weight, t) for h in heads] for t, heads in enumerate(q_rows)]
    k = [[one(h, k_norm_weight, t) for h in heads] for t, heads in enumerate(k_rows)]
    return q, k
