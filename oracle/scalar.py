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


def paged_attention_scalar(query, key, value, key_cache, value_cache, cum, past,
                           block_table, slot_mapping, num_heads, kv_num_heads, scale,
                           with_lse=False):
    """Returns (out as nested lists [N][H*D], dict slot->(krow, vrow) of the
    slots written), and with ``with_lse`` also lse as nested lists [N][H]
    (log of the fsum of exp(score) over the visible keys, natural log).
    Inputs are numpy arrays only as containers."""
    H, Hkv = int(num_heads), int(kv_num_heads)
    N, width = query.shape
    packed = key is None
    D = width // (H + 2 * Hkv) if packed else width // H
    sc = 1.0 / math.sqrt(D) if scale == 0 else float(scale)
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    B = len(past)

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
            written[slot] = (k_of(t), v_of(t))

    def cache_row(slot, which):
        if slot in written:
            return written[slot][which]
        blk, off = divmod(slot, bs)
        src = key_cache if which == 0 else value_cache
        return [_num(x) for x in src[blk][off].reshape(-1)]

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
