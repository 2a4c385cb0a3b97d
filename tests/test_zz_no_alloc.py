"""pa_paged_attention_noalloc against pa_paged_attention (needs an MI355X).

The no-alloc entry point runs the same kernels with the library's own
per-GPU scratch as workspace, so on the same inputs it must give the same
bits as the entry point with a caller workspace: caches bit-exact and
outputs bit-identical (and, as every call, within the bar of the fp64
oracle).  Two calls in a row, the second smaller than the first, check that
what the first call leaves in the scratch does not leak into the second.
Every call goes through the C ABI.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_varlen_amd as pa
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 4e-3


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run(b, noalloc, prologue=None):
    t = {k: dev(getattr(b, k)) for k in ("query", "key", "value", "key_cache", "value_cache", "cum",
                                         "past", "block_table", "slot_mapping", "k_scale",
                                         "v_scale")}
    out = torch.empty((b.num_tokens, b.num_heads * b.head_size), dtype=torch.float16, device=DEV)
    lse = torch.empty((b.num_tokens, b.num_heads), dtype=torch.float32, device=DEV)
    common = (t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"], t["cum"],
              t["past"], t["block_table"], t["slot_mapping"])
    kw = dict(num_heads=b.num_heads, kv_num_heads=b.kv_num_heads, scale=b.scale, output=out,
              lse=lse, k_scale=t["k_scale"], v_scale=t["v_scale"])
    if prologue is not None:  # the fused Q/K prologue (its query rows live in the scratch too)
        kw["prologue"] = {k: dev(v) if isinstance(v, np.ndarray) else v for k, v in prologue.items()}
    if noalloc:
        pa.paged_attention_noalloc(*common, **kw)
    else:
        pa.paged_attention(*common, **kw)
    torch.cuda.synchronize()
    return out, lse, t["key_cache"], t["value_cache"]


def compare(b, prologue=None):
    say(f"[gpu] noalloc {b.name} N={b.num_tokens} B={b.batch_size} kv={b.kv_quant}"
        + (" with the fused prologue" if prologue else ""))
    o1, l1, k1, v1 = run(b, noalloc=False, prologue=prologue)
    o2, l2, k2, v2 = run(b, noalloc=True, prologue=prologue)
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    ref, rkc, rvc = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                           b.cum, b.past, b.block_table, b.slot_mapping,
                                           num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                           scale=b.scale, k_scale=b.k_scale, v_scale=b.v_scale,
                                           prologue=prologue)
    raw = lambda x: x.view(np.uint8 if x.itemsize == 1 else np.uint16)
    if prologue is None:  # (written key rows carry the kernel's fp32 rounding: the parity tests bound them)
        assert np.array_equal(raw(k2.cpu().numpy()), raw(rkc))
    assert np.array_equal(raw(v2.cpu().numpy()), raw(rvc))
    err = float(np.max(np.abs(o2.double().cpu().numpy() - ref)))
    say(f"      identical to the workspace entry point; max|err| vs oracle {err:.3e}")
    assert err <= TOL


def test_noalloc_matches_workspace_entry_two_calls():
    # a large call (decodes cut across waves, prefill chunks, INT8 caches),
    # then a smaller one that reuses the scratch
    big = W.make_batch([1, 1, 300, 1, 64, 1], [9000, 12000, 40, 7, 3000, 16383], num_heads=32,
                       kv_num_heads=8, head_size=128, block_size=16, seed=900, name="noalloc_big",
                       kv_quant="int8")
    small = W.make_batch([1, 5, 1], [33, 70, 500], num_heads=8, kv_num_heads=2, head_size=128,
                         block_size=16, seed=901, name="noalloc_small", packed=True,
                         slot_mode="drop", drop_count=1)
    compare(big)
    compare(small)


def test_noalloc_full_workload_then_smaller():
    compare(W.mixed(0))
    compare(W.tiny(0))


def test_noalloc_with_the_fused_prologue_then_without():
    # the prologue's transformed query rows sit in the scratch; the next call
    # (no prologue) must not read them
    b = W.make_batch([1, 120, 1, 33], [3000, 200, 40, 900], num_heads=16, kv_num_heads=4, head_size=128,
                     block_size=16, seed=902, name="noalloc_prologue")
    compare(b, prologue=W.prologue_inputs(b, 903, rotary_dim=64, spatial=True))
    compare(W.tiny(0))
