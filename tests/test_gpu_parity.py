"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bar (stated with the workloads): both caches bit-exact over every slot,
written or untouched; outputs within max-abs 4e-3 of the fp64 oracle (fp16
inputs, fp32 accumulation, O(1) data).  For bf16 data the bar scales with the
unit roundoff: bf16 keeps 8 significant bits to fp16's 11, so every rounding
in the path (P before the PV product, the output) is 8 times coarser and the
bar is 8 * 4e-3 = 3.2e-2.  INT8 caches keep the bar of their data type: the
codes are bit-exact, and the one extra rounding (the K scales folded into the
query, rounded to the data type) moves the scores by about 3e-4 (fp16) or
2e-3 (bf16) of a unit, far inside it.  Every workload, full-size ones
included, is checked on every cache slot and on every output element against
the fp64 oracle.  Every call goes through the C ABI (libpagedattn.so via
ctypes).
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import paged_kv_varlen_amd as pa
import workloads as W

pytestmark = pytest.mark.gpu
TOL = 4e-3
TOL_BF16 = 8 * TOL
DEV = "cuda:0"


def tol(b) -> float:
    return TOL_BF16 if b.dtype == "bf16" else TOL


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(x, dtype=None):
    """numpy -> device tensor; uint16 arrays hold bf16 bit patterns."""
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    t = torch.from_numpy(x)
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def to_host(t):
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(x):
    """Values of host data: float16 as is, uint16 as bf16 bits (torch's decode)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double().numpy()
    return x.astype(np.float64)


class DevBatch:
    def __init__(self, b: W.Batch):
        self.q = to_dev(b.query)
        self.k = to_dev(b.key)
        self.v = to_dev(b.value)
        self.kc = to_dev(b.key_cache)
        self.vc = to_dev(b.value_cache)
        self.cum = to_dev(b.cum)
        self.past = to_dev(b.past)
        self.table = to_dev(b.block_table)
        self.slots = to_dev(b.slot_mapping)
        self.ks = to_dev(b.k_scale)
        self.vs = to_dev(b.v_scale)
        self.b = b

    def run(self, **kw):
        b = self.b
        return pa.paged_attention(self.q, self.k, self.v, self.kc, self.vc, self.cum, self.past,
                                  self.table, self.slots, num_heads=b.num_heads,
                                  kv_num_heads=b.kv_num_heads, scale=b.scale,
                                  k_scale=self.ks, v_scale=self.vs, **kw)


def gpu_run(b: W.Batch):
    say(f"[gpu] {b.name} {b.dtype} kv={b.kv_quant} seed={b.seed} N={b.num_tokens} B={b.batch_size} "
        f"H={b.num_heads}/{b.kv_num_heads} D={b.head_size} bs={b.block_size} NB={b.num_blocks}")
    d = DevBatch(b)
    out = d.run()
    torch.cuda.synchronize()
    return (to_host(out), to_host(d.kc), to_host(d.vc))


def raw_bits(x):
    """Cache contents as unsigned integers of their width (int8 codes or 16-bit values)."""
    return x.view(np.uint8 if x.itemsize == 1 else np.uint16)


def check(b: W.Batch, rows=None, gpu=None):
    out, kc, vc = gpu if gpu is not None else gpu_run(b)
    t0 = time.perf_counter()
    ref, rkc, rvc = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                           b.cum, b.past, b.block_table, b.slot_mapping,
                                           num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                           scale=b.scale, rows=rows, k_scale=b.k_scale,
                                           v_scale=b.v_scale)
    assert kc.dtype == rkc.dtype and vc.dtype == rvc.dtype
    assert np.array_equal(raw_bits(kc), raw_bits(rkc)), "key_cache differs"
    assert np.array_equal(raw_bits(vc), raw_bits(rvc)), "value_cache differs"
    sel = np.arange(b.num_tokens) if rows is None else rows
    got = as_f64(out[sel])
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref[sel])) if sel.size else 0.0
    say(f"      rows checked {sel.size} of {b.num_tokens}, max|err| {err:.3e} "
        f"(oracle {time.perf_counter() - t0:.1f} s)")
    assert err <= tol(b), f"max abs error {err}"
    return err


# ------------------------------------------------------------------ the five workloads

def test_tiny():
    check(W.tiny(0))


@pytest.mark.parametrize("seed", [0, 1])
def test_pure_decode_full(seed):
    check(W.pure_decode(seed))


def test_mixed():
    check(W.mixed(0))


def test_long_prefill():
    check(W.long_prefill(0))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,kvq", [("f16", "none"), ("bf16", "none"), ("f16", "int8")])
def test_serving(dtype, kvq):
    check(W.serving(0, dtype=dtype, kv_quant=kvq))


# ------------------------------------------------------------------ shape and edge sweeps

SWEEP = [
    # (q_lens, past_lens, H, Hkv, D, bs)
    ([1, 2, 17, 128, 129, 0, 300], [0, 1, 15, 16, 17, 5, 1000], 8, 2, 128, 16),
    ([1, 1, 64, 3, 200], [255, 256, 257, 0, 511], 8, 8, 128, 256),
    ([5, 1, 33, 1], [31, 32, 64, 700], 16, 2, 64, 32),
    ([1, 40, 1, 7], [4000, 90, 9000, 1], 32, 4, 128, 64),
    ([2, 1, 70], [0, 0, 0], 12, 4, 64, 16),      # G=3
    ([1, 9, 1], [100, 100, 5000], 64, 1, 128, 16),  # G=64
    ([1, 16, 1], [17, 3, 2000], 20, 4, 128, 48),  # G=5, block_size 48
    # three kv heads: an odd unit count (16-bit: split pairs of waves; quantized:
    # one plan start per wave)
    ([1, 1, 40, 1, 3], [3000, 700, 50, 9000, 17], 3, 3, 128, 16),
    ([1, 25, 1, 1], [1500, 40, 4000, 33], 12, 6, 64, 32),  # six kv heads: unit groups of two
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
@pytest.mark.parametrize("packed,slots", [(False, None), (True, "drop")])
def test_sweep(case, packed, slots):
    q, p, H, Hkv, D, bs = SWEEP[case]
    n = sum(q)
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=100 + case, packed=packed, slot_mode=slots,
                     drop_count=max(1, n // 20) if slots else 0, num_blocks=None,
                     name=f"sweep{case}")
    check(b)


# Large pages: the ABI accepts block sizes up to 4096.  Pasts sit on and
# around page boundaries (bs - 1, bs, bs + 1), with packed [Q|K|V] rows,
# dropped slots, decodes cut across decode waves and multi-token chunks that
# span pages.
BIG_PAGES = [
    # (q_lens, past_lens, H, Hkv, D, bs, dtype, kv_quant)
    ([1, 1, 300, 1, 64, 2], [1023, 1024, 1025, 5000, 2047, 0], 8, 2, 128, 1024, "f16", "none"),
    ([1, 129, 1, 2, 1], [4095, 4000, 9000, 4096, 4097], 16, 4, 128, 4096, "f16", "none"),
    ([1, 70, 1], [4095, 4090, 12000], 8, 2, 256, 4096, "bf16", "none"),
    ([1, 33, 1, 1], [1023, 1000, 8191, 1025], 8, 2, 128, 1024, "f16", "int8"),
    ([1, 40, 1, 1], [4095, 3000, 12000, 4097], 16, 4, 128, 4096, "f16", "int4"),
    ([1, 17, 1], [2047, 100, 3000], 8, 2, 64, 1024, "bf16", "int8"),
]


@pytest.mark.parametrize("case", range(len(BIG_PAGES)))
def test_block_sizes_1024_and_4096(case):
    q, p, H, Hkv, D, bs, dtype, kvq = BIG_PAGES[case]
    n = sum(q)
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=700 + case, packed=True, slot_mode="drop", drop_count=max(1, n // 20),
                     num_blocks=None, name=f"pages{bs}_{case}", dtype=dtype, kv_quant=kvq)
    check(b)


def test_custom_scale_and_spare_pages():
    b = W.make_batch([1, 30, 1], [77, 12, 3000], num_heads=8, kv_num_heads=2, head_size=128,
                     block_size=16, seed=7, scale=-0.21, num_blocks=400, name="scale")
    check(b)


def test_first_token_returns_its_value_row_exactly():
    # past 0, one new token: the only weight is exactly 1
    b = W.make_batch([1, 1, 1], [0, 0, 0], num_heads=8, kv_num_heads=2, head_size=128,
                     block_size=16, seed=8, name="first")
    out, _, _ = gpu_run(b)
    G = 4
    for t in range(3):
        for h in range(8):
            k = h // G
            assert np.array_equal(out[t, h * 128:(h + 1) * 128].view(np.uint16),
                                  b.value[t, k * 128:(k + 1) * 128].view(np.uint16))


def test_garbage_outside_history_is_never_used():
    # every cache slot the call must not read holds NaN: results are unchanged
    b = W.make_batch([1, 37, 1, 5], [50, 20, 4095, 0], num_heads=8, kv_num_heads=2,
                     head_size=128, block_size=64, seed=9, num_blocks=200, name="nan")
    keep = np.zeros(b.num_blocks * b.block_size, dtype=bool)
    for i in range(b.batch_size):
        L = int(b.kv_lens[i])
        for j in range(L):
            keep[int(b.block_table[i, j // b.block_size]) * b.block_size + j % b.block_size] = True
    for cache in (b.key_cache, b.value_cache):
        flat = cache.reshape(b.num_blocks * b.block_size, -1)
        flat[~keep] = np.float16(np.nan)
    check(b)


def test_empty_sequences_and_empty_call():
    b = W.make_batch([0, 3, 0, 1, 0], [4, 10, 0, 33, 2], num_heads=4, kv_num_heads=2,
                     head_size=64, block_size=16, seed=10, name="empties")
    check(b)
    e = W.make_batch([0, 0], [3, 9], num_heads=4, kv_num_heads=2, head_size=64, block_size=16,
                     seed=11, name="no_tokens")
    out, kc, vc = gpu_run(e)
    assert out.shape == (0, 256)
    assert np.array_equal(kc.view(np.uint16), e.key_cache.view(np.uint16))


def test_long_decode_many_splits():
    b = W.make_batch([1, 1, 1, 2], [16383, 9000, 511, 12000], num_heads=32, kv_num_heads=8,
                     head_size=128, block_size=256, seed=12, name="long_decode")
    check(b)


def test_long_history_prefill():
    # a chunk on top of 40000 cached tokens: the prefill reads more than
    # 32768 keys, past what one window of cache slots covers; an odd number
    # of half-tiles leaves one item with a single half
    b = W.make_batch([37, 1, 20], [40000, 100, 33000], num_heads=8, kv_num_heads=1,
                     head_size=128, block_size=16, seed=13, name="long_history")
    check(b)


def many_sequences(B, mixed, kv_quant="none"):
    # B sequences of one new token each over pasts in [0, 300); with mixed, one
    # sequence in 50 is a chunk of 2..40 new tokens and one in 37 is empty
    rng = np.random.default_rng(14)
    q = np.ones(B, dtype=np.int64)
    if mixed:
        q[::50] = rng.integers(2, 41, size=q[::50].size)
        q[7::37] = 0
    p = rng.integers(0, 300, size=B)
    return W.make_batch(q, p, num_heads=8, kv_num_heads=2, head_size=128, block_size=16,
                        seed=14, name=f"many_sequences_{B}", kv_quant=kv_quant)


# The plan keeps up to 1024 decode records in LDS and the scatter stages up to
# 2047 sequences' offsets in LDS for its token -> sequence search; past those
# counts both read global memory.  1024 and 2047 are the largest staged cases,
# 2300 sequences take both global paths.
@pytest.mark.parametrize("B,mixed,kvq", [(1024, False, "none"), (2047, False, "none"),
                                         (2300, True, "none"), (2300, True, "int8")])
def test_many_sequences(B, mixed, kvq):
    b = many_sequences(B, mixed, kvq)
    check(b)


def test_deterministic_bits():
    b = W.mixed(1)
    d = DevBatch(b)
    o1 = d.run().clone()
    o2 = d.run().clone()  # idempotent: the second call rewrites the same cache bits
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("kv_quant", ["int8", "int4"])
def test_deterministic_bits_quantized_decode(kv_quant):
    # two waves per SIMD take turns at the higher issue priority by progress:
    # the schedule changes from run to run, the cut points and bits must not
    b = W.workload("pure_decode", 2, kv_quant=kv_quant)
    d = DevBatch(b)
    runs = []
    for _ in range(3):
        out, lse = d.run(return_lse=True)
        runs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for out, lse in runs[1:]:
        assert torch.equal(out.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), runs[0][1].view(torch.int32))


def test_chunked_continuation_matches_one_shot():
    H, Hkv, D, bs = 8, 2, 128, 16
    b = W.make_batch([150], [37], num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=13, name="chunks")
    one = DevBatch(b)
    o_full = one.run()
    two = DevBatch(b)
    cut = 61
    mk = lambda x: x.contiguous()
    o_a = pa.paged_attention(mk(two.q[:cut]), mk(two.k[:cut]), mk(two.v[:cut]), two.kc, two.vc,
                             to_dev(np.array([0, cut], np.int32)), two.past, two.table,
                             num_heads=H, kv_num_heads=Hkv)
    o_b = pa.paged_attention(mk(two.q[cut:]), mk(two.k[cut:]), mk(two.v[cut:]), two.kc, two.vc,
                             to_dev(np.array([0, 150 - cut], np.int32)), two.past + cut,
                             two.table, num_heads=H, kv_num_heads=Hkv)
    torch.cuda.synchronize()
    assert torch.equal(one.kc.view(torch.int16), two.kc.view(torch.int16))
    assert torch.equal(one.vc.view(torch.int16), two.vc.view(torch.int16))
    diff = (torch.cat([o_a, o_b]).float() - o_full.float()).abs().max().item()
    assert diff <= 2 * TOL


def test_unsupported_example_shape_is_typed_error():
    # README example call: H=2, Hkv=1, D=2, block_size 2 -> typed PA_ERR_UNSUPPORTED
    q = torch.zeros(2, 4, dtype=torch.float16, device=DEV)
    k = torch.zeros(2, 2, dtype=torch.float16, device=DEV)
    kc = torch.zeros(3, 2, 1, 2, dtype=torch.float16, device=DEV)
    with pytest.raises(pa.PagedAttentionError) as ei:
        pa.paged_attention(q, k, k.clone(), kc, kc.clone(), to_dev(np.array([0, 2], np.int32)),
                           to_dev(np.array([1], np.int32)), to_dev(np.array([[0, 1, 2]], np.int32)),
                           num_heads=2, kv_num_heads=1)
    assert ei.value.status == 3


def test_hip_graph_replay_matches_eager():
    b = W.mixed(2)
    d = DevBatch(b)
    ref = d.run().clone()
    torch.cuda.synchronize()
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(output=out, workspace=ws, stream=s)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(output=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ partial states: lse export and merge

# lse tolerance: P is rounded to fp16 before it is summed (relative error at
# most 2^-11 per weight), so log(sum) is off by at most about 2^-11 = 4.9e-4
# in natural-log units; fp32 score and sum rounding add ~1e-6.  bf16 weights
# round 8 times coarser.
LSE_TOL = 1e-3
LSE_TOL_BF16 = 8 * LSE_TOL


def rounding_of(f32, low):
    """``low`` (fp16, or bf16 bits as uint16) is a nearest value of f32
    elementwise.  The packed fp32->fp16 conversion of gfx950
    (v_cvt_pk_f16_f32) may break an exact tie away from the even neighbour,
    where numpy rounds to even; both are nearest."""
    if low.dtype == np.uint16:
        r = W.round_bf16(f32)
        diff = r != low
    else:
        r = f32.astype(np.float16)
        diff = r.view(np.uint16) != low.view(np.uint16)
    x = f32.astype(np.float64)
    tie = np.abs(x - as_f64(r)) == np.abs(x - as_f64(low))
    if np.any(diff & ~tie):
        i = np.argwhere(diff & ~tie)[0]
        say(f"      not a rounding at {tuple(i)}: f32 {f32[tuple(i)]!r} low {low[tuple(i)]!r}")
    say(f"      rounded output == rounding of fp32 output ({int(np.sum(diff))} ties broken the other way)")
    return not np.any(diff & ~tie)


@pytest.mark.parametrize("name,dtype", [("tiny", "f16"), ("sweep0", "f16"), ("long_decode", "f16"),
                                        ("mixed", "f16"), ("tiny", "bf16"), ("long_decode", "bf16"),
                                        ("mixed", "bf16")])
def test_lse_and_fp32_output(name, dtype):
    if name == "tiny":
        b = W.tiny(0, dtype=dtype)
    elif name == "sweep0":
        q, p, H, Hkv, D, bs = SWEEP[0]
        b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                         seed=100, name="sweep0", dtype=dtype)
    elif name == "long_decode":  # decode segments cut across waves: merged states
        b = W.make_batch([1, 1, 1, 2], [16383, 9000, 511, 12000], num_heads=32, kv_num_heads=8,
                         head_size=128, block_size=256, seed=12, name="long_decode", dtype=dtype)
    else:
        b = W.mixed(0, dtype=dtype)
    say(f"[gpu] lse {b.name} {b.dtype} N={b.num_tokens} B={b.batch_size}")
    d = DevBatch(b)
    f32 = torch.empty((b.num_tokens, b.num_heads * b.head_size), dtype=torch.float32, device=DEV)
    out, lse = d.run(return_lse=True, output_f32=f32)
    torch.cuda.synchronize()
    rows = None
    ref, _, _, rlse = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                             b.cum, b.past, b.block_table, b.slot_mapping,
                                             num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                             scale=b.scale, rows=rows, with_lse=True)
    sel = np.arange(b.num_tokens) if rows is None else rows
    o16, o32, l32 = to_host(out), f32.cpu().numpy(), lse.cpu().numpy()
    assert rounding_of(o32, o16)
    e_o = np.max(np.abs(o32[sel].astype(np.float64) - ref[sel]))
    e_l = np.max(np.abs(l32[sel].astype(np.float64) - rlse[sel]))
    say(f"      rows {sel.size}: max|err| out_f32 {e_o:.3e}, lse {e_l:.3e}")
    assert e_o <= tol(b) and e_l <= (LSE_TOL_BF16 if dtype == "bf16" else LSE_TOL)


@pytest.mark.parametrize("P,R,D,dtype", [(1, 37, 128, torch.float16), (3, 1000, 128, torch.float16),
                                         (5, 777, 64, torch.float16), (2, 4096, 256, torch.float16),
                                         (3, 1000, 128, torch.bfloat16)])
def test_merge_states(P, R, D, dtype):
    rng = np.random.default_rng(P * 1000 + R)
    outs = rng.standard_normal((P, R, D)).astype(np.float32)
    lses = (rng.standard_normal((P, R)) * 4).astype(np.float32)
    lses[rng.random((P, R)) < 0.2] = -np.inf      # empty states
    lses[:, :3] = -np.inf                           # rows with no keys at all
    ref_o, ref_l = oracle.merge_states(outs, lses)
    so, sl = torch.from_numpy(outs).to(DEV), torch.from_numpy(lses).to(DEV)
    f32 = torch.empty((R, D), dtype=torch.float32, device=DEV)
    o16, l32 = pa.merge_states(so, sl, output_f32=f32, dtype=dtype)
    o16b, l32b = pa.merge_states(so, sl, dtype=dtype)
    torch.cuda.synchronize()
    assert o16.dtype == dtype
    o16, o32, l32 = to_host(o16), f32.cpu().numpy(), l32.cpu().numpy()
    assert np.array_equal(o16.view(np.uint16), to_host(o16b).view(np.uint16))   # deterministic
    assert np.array_equal(l32.view(np.uint32), l32b.cpu().numpy().view(np.uint32))
    assert rounding_of(o32, o16)
    fin = np.isfinite(ref_l)
    assert np.all(o32[~fin] == 0) and np.all(l32[~fin] == -np.inf)
    # fp32 sequential merge of O(1) states: relative rounding ~P * 2^-24
    e_o = np.max(np.abs(o32 - ref_o) / (1.0 + np.abs(ref_o)))
    e_l = np.max(np.abs(l32[fin] - ref_l[fin]) / (1.0 + np.abs(ref_l[fin])))
    say(f"[gpu] merge P={P} R={R} D={D}: max rel err out {e_o:.2e}, lse {e_l:.2e}")
    assert e_o <= 1e-5 and e_l <= 1e-6
    t = TOL_BF16 if dtype == torch.bfloat16 else TOL
    assert np.max(np.abs(as_f64(o16) - ref_o)) <= t * (1 + np.abs(ref_o).max())


# ------------------------------------------------------------------ bf16 data

@pytest.mark.parametrize("case", ["tiny"] + [f"sweep{i}" for i in range(len(SWEEP))] + ["packed3"])
def test_bf16_shapes(case):
    if case == "tiny":
        b = W.tiny(0, dtype="bf16")
    elif case == "packed3":
        q, p, H, Hkv, D, bs = SWEEP[3]
        b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                         seed=203, packed=True, slot_mode="drop", drop_count=2, name="packed3",
                         dtype="bf16")
    else:
        i = int(case[5:])
        q, p, H, Hkv, D, bs = SWEEP[i]
        b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                         seed=200 + i, name=case, dtype="bf16")
    check(b)


def test_bf16_pure_decode_full():
    check(W.pure_decode(0, dtype="bf16"))


def test_bf16_mixed():
    check(W.mixed(0, dtype="bf16"))


def test_bf16_long_prefill():
    check(W.long_prefill(0, dtype="bf16"))


def test_bf16_first_token_and_determinism():
    b = W.make_batch([1, 1, 1], [0, 0, 0], num_heads=8, kv_num_heads=2, head_size=128,
                     block_size=16, seed=8, name="first", dtype="bf16")
    out, _, _ = gpu_run(b)
    for t in range(3):
        for h in range(8):
            k = h // 4
            assert np.array_equal(out[t, h * 128:(h + 1) * 128], b.value[t, k * 128:(k + 1) * 128])
    d = DevBatch(W.mixed(1, dtype="bf16"))
    o1 = d.run().clone()
    o2 = d.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------------------------ head_size 256

HD256 = [
    # (q_lens, past_lens, H, Hkv, bs)
    ([1, 5, 1, 70, 200, 1, 0, 33], [0, 33, 4000, 17, 300, 1500, 9, 64], 16, 2, 16),  # G=8
    ([1, 1, 1, 1, 2, 130], [9000, 12000, 700, 1, 3, 0], 4, 4, 64),                  # MHA, cut decodes
    ([1, 17, 1, 64], [2500, 100, 31, 6000], 16, 1, 256),                              # G=16
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", range(len(HD256)))
def test_head_size_256(case, dtype):
    q, p, H, Hkv, bs = HD256[case]
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=256, block_size=bs,
                     seed=300 + case, name=f"hd256_{case}", dtype=dtype)
    check(b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_size_256_long_prefill_and_state(dtype):
    b = W.make_batch([700, 1, 1], [1100, 20000, 3], num_heads=8, kv_num_heads=2, head_size=256,
                     block_size=256, seed=310, name="hd256_long", dtype=dtype, packed=True,
                     slot_mode="drop", drop_count=7)
    rows = np.arange(b.num_tokens)
    check(b)
    d = DevBatch(b)
    f32 = torch.empty((b.num_tokens, b.num_heads * 256), dtype=torch.float32, device=DEV)
    out, lse = d.run(return_lse=True, output_f32=f32)
    torch.cuda.synchronize()
    ref, _, _, rlse = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                             b.cum, b.past, b.block_table, b.slot_mapping,
                                             num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                             scale=b.scale, rows=rows, with_lse=True)
    o_low, o32, l32 = to_host(out), f32.cpu().numpy(), lse.cpu().numpy()
    assert rounding_of(o32, o_low)
    e_o = np.max(np.abs(o32[rows].astype(np.float64) - ref[rows]))
    e_l = np.max(np.abs(l32[rows].astype(np.float64) - rlse[rows]))
    say(f"      state: max|err| out_f32 {e_o:.3e}, lse {e_l:.3e}")
    assert e_o <= tol(b) and e_l <= (LSE_TOL_BF16 if dtype == "bf16" else LSE_TOL)


# ------------------------------------------------------------------ adversarial cases for the wider paths

@pytest.mark.parametrize("D,dtype", [(256, "f16"), (256, "bf16"), (128, "bf16")])
def test_garbage_outside_history_wide(D, dtype):
    # every slot the call must not read holds a NaN pattern (fp16 0x7E00, bf16
    # 0x7FC0): keys past a history come from the zero page, never the cache
    b = W.make_batch([1, 37, 1, 5, 70], [50, 20, 4095, 0, 190], num_heads=8, kv_num_heads=2,
                     head_size=D, block_size=64, seed=40 + D, num_blocks=200, name=f"nan{D}",
                     dtype=dtype)
    keep = np.zeros(b.num_blocks * b.block_size, dtype=bool)
    for i in range(b.batch_size):
        for j in range(int(b.kv_lens[i])):
            keep[int(b.block_table[i, j // b.block_size]) * b.block_size + j % b.block_size] = True
    nan_bits = np.uint16(0x7FC0 if dtype == "bf16" else 0x7E00)
    for cache in (b.key_cache, b.value_cache):
        flat = cache.reshape(b.num_blocks * b.block_size, -1).view(np.uint16)
        flat[~keep] = nan_bits
    check(b)


@pytest.mark.parametrize("D,dtype", [(256, "bf16"), (128, "bf16")])
def test_hip_graph_replay_wide(D, dtype):
    b = W.make_batch([1, 1, 300, 1, 64], [900, 5000, 40, 7, 3000], num_heads=16, kv_num_heads=2,
                     head_size=D, block_size=16, seed=50 + D, name=f"graph{D}", dtype=dtype)
    d = DevBatch(b)
    ref = d.run().clone()
    torch.cuda.synchronize()
    ws = torch.empty(1 << 27, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(output=out, workspace=ws, stream=s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(output=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ INT8 / INT4 caches (codes + per-channel scales)

QUANT = ["int8", "int4"]


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quant_tiny(dtype, kvq):
    check(W.tiny(0, dtype=dtype, kv_quant=kvq))


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("case", range(len(SWEEP)))
@pytest.mark.parametrize("dtype,packed,slots", [("f16", False, None), ("bf16", True, "drop")])
def test_quant_sweep(case, dtype, packed, slots, kvq):
    q, p, H, Hkv, D, bs = SWEEP[case]
    n = sum(q)
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=500 + case, packed=packed, slot_mode=slots,
                     drop_count=max(1, n // 20) if slots else 0, num_blocks=None,
                     name=f"{kvq}_sweep{case}", dtype=dtype, kv_quant=kvq)
    check(b)


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quant_pure_decode_full(dtype, kvq):
    check(W.pure_decode(0, dtype=dtype, kv_quant=kvq))


@pytest.mark.parametrize("kvq", QUANT)
def test_quant_mixed(kvq):
    check(W.mixed(0, kv_quant=kvq))


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quant_long_prefill(dtype, kvq):
    check(W.long_prefill(0, dtype=dtype, kv_quant=kvq))


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", range(len(HD256)))
def test_quant_head_size_256(case, dtype, kvq):
    q, p, H, Hkv, bs = HD256[case]
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=256, block_size=bs,
                     seed=520 + case, name=f"{kvq}_hd256_{case}", dtype=dtype, kv_quant=kvq)
    check(b)


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_quant_extreme_codes_outside_history(D, kvq):
    # every slot the call must not read holds the code 7 (INT8: 127): keys past
    # a history come from the zero page, never the cache (a read would move
    # the scores by many units)
    b = W.make_batch([1, 37, 1, 5, 70], [50, 20, 4095, 0, 190], num_heads=8, kv_num_heads=2,
                     head_size=D, block_size=64, seed=540 + D, num_blocks=200, name=f"{kvq}_far{D}",
                     kv_quant=kvq)
    keep = np.zeros(b.num_blocks * b.block_size, dtype=bool)
    for i in range(b.batch_size):
        for j in range(int(b.kv_lens[i])):
            keep[int(b.block_table[i, j // b.block_size]) * b.block_size + j % b.block_size] = True
    for cache in (b.key_cache, b.value_cache):
        flat = cache.reshape(b.num_blocks * b.block_size, -1)
        flat[~keep] = 127 if kvq == "int8" else 0x77
    check(b)


@pytest.mark.parametrize("kvq", QUANT)
def test_quant_state_and_determinism(kvq):
    b = W.make_batch([300, 1, 1, 64], [700, 9000, 3, 0], num_heads=16, kv_num_heads=4, head_size=128,
                     block_size=16, seed=550, name=f"{kvq}_state", kv_quant=kvq)
    rows = np.arange(b.num_tokens)
    d = DevBatch(b)
    f32 = torch.empty((b.num_tokens, b.num_heads * 128), dtype=torch.float32, device=DEV)
    out, lse = d.run(return_lse=True, output_f32=f32)
    out = out.clone()
    again = d.run()  # the second call rewrites the same codes: same bits
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    ref, _, _, rlse = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                             b.cum, b.past, b.block_table, b.slot_mapping,
                                             num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                             scale=b.scale, rows=rows, with_lse=True,
                                             k_scale=b.k_scale, v_scale=b.v_scale)
    o_low, o32, l32 = to_host(out), f32.cpu().numpy(), lse.cpu().numpy()
    assert rounding_of(o32, o_low)
    e_o = np.max(np.abs(o32[rows].astype(np.float64) - ref[rows]))
    e_l = np.max(np.abs(l32[rows].astype(np.float64) - rlse[rows]))
    say(f"      state: max|err| out_f32 {e_o:.3e}, lse {e_l:.3e}")
    assert e_o <= TOL and e_l <= LSE_TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_int4_every_nibble_value(dtype):
    # INT4 caches may hold any nibble, -8 included (the quantizer never writes
    # it, a cache filled elsewhere may): uniformly random bytes in every slot.
    # Uniform codes spread about 3 times wider than the recipe's, so the
    # scales are a quarter of the recipe's to keep the data O(1), as the bar
    # assumes.
    b = W.make_batch([1, 40, 1, 9], [300, 70, 2000, 5], num_heads=8, kv_num_heads=2, head_size=128,
                     block_size=16, seed=560, name="int4_nibbles", dtype=dtype, kv_quant="int4")
    rng = np.random.default_rng(561)
    for cache in (b.key_cache, b.value_cache):
        cache[...] = rng.integers(0, 256, cache.shape, dtype=np.uint8)
    b.k_scale *= np.float32(0.25)
    b.v_scale *= np.float32(0.25)
    check(b)


@pytest.mark.parametrize("kvq", QUANT)
@pytest.mark.parametrize("H,Hkv", [(8, 1), (12, 3), (40, 5)])
def test_quant_odd_unit_counts(H, Hkv, kvq):
    # an odd number of units per sequence (1, 3, 5 kv heads): INT4 at head size
    # 128 cannot pair units across waves then and streams one unit per wave
    b = W.make_batch([1, 1, 23, 1], [900, 4000, 60, 17], num_heads=H, kv_num_heads=Hkv, head_size=128,
                     block_size=32, seed=570 + Hkv, name=f"{kvq}_odd{Hkv}", kv_quant=kvq)
    check(b)


@pytest.mark.parametrize("kvq", QUANT)
def test_quant_hip_graph_replay(kvq):
    b = W.make_batch([1, 1, 300, 1, 64], [900, 5000, 40, 7, 3000], num_heads=16, kv_num_heads=4,
                     head_size=128, block_size=16, seed=580, name=f"{kvq}_graph", kv_quant=kvq)
    d = DevBatch(b)
    ref = d.run().clone()
    torch.cuda.synchronize()
    ws = torch.empty(1 << 27, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(output=out, workspace=ws, stream=s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(output=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ output gate: sigmoid(gate) on the output

def check_gated(b: W.Batch, rows=None, seed=1):
    gate = W.output_gate_input(b, seed)
    say(f"[gpu] gated {b.name} {b.dtype} kv={b.kv_quant} N={b.num_tokens} B={b.batch_size} "
        f"H={b.num_heads}/{b.kv_num_heads} D={b.head_size}")
    d = DevBatch(b)
    out = d.run(gate=to_dev(gate))
    torch.cuda.synchronize()
    ref, rkc, rvc = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache,
                                           b.cum, b.past, b.block_table, b.slot_mapping,
                                           num_heads=b.num_heads, kv_num_heads=b.kv_num_heads,
                                           scale=b.scale, rows=rows, k_scale=b.k_scale,
                                           v_scale=b.v_scale, gate=gate)
    assert np.array_equal(raw_bits(to_host(d.kc)), raw_bits(rkc)), "key_cache differs"
    assert np.array_equal(raw_bits(to_host(d.vc)), raw_bits(rvc)), "value_cache differs"
    sel = np.arange(b.num_tokens) if rows is None else rows
    got = as_f64(to_host(out)[sel])
    err = np.max(np.abs(got - ref[sel])) if sel.size else 0.0
    say(f"      rows checked {sel.size}, max|err| {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol(b), f"max abs error {err}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gate_tiny(dtype):
    check_gated(W.tiny(0, dtype=dtype))


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_gate_sweep(case):
    q, p, H, Hkv, D, bs = SWEEP[case]
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=600 + case, num_blocks=None, name=f"gate_sweep{case}")
    check_gated(b, seed=case)


def test_gate_pure_decode_full():
    check_gated(W.pure_decode(0))  # whole segments in the decode kernel, cut ones in the merge


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gate_long_prefill_and_mixed(dtype):
    check_gated(W.long_prefill(0, dtype=dtype))
    check_gated(W.mixed(0, dtype=dtype))


@pytest.mark.parametrize("kvq", ["none", "int8", "int4"])
def test_gate_head_size_256_and_quantized(kvq):
    q, p, H, Hkv, bs = HD256[0]
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=256, block_size=bs,
                     seed=610, name=f"gate_hd256_{kvq}", kv_quant=kvq)
    check_gated(b)
    s = W.make_batch([1, 40, 1, 9], [3000, 70, 9000, 5], num_heads=32, kv_num_heads=8, head_size=128,
                     block_size=16, seed=611, name=f"gate_q_{kvq}", kv_quant=kvq)
    check_gated(s)


def test_gate_leaves_the_state_ungated():
    b = W.make_batch([1, 300, 1, 64], [2000, 700, 9000, 0], num_heads=16, kv_num_heads=4, head_size=128,
                     block_size=16, seed=620, name="gate_state")
    gate = to_dev(W.output_gate_input(b, 3))
    d = DevBatch(b)
    f0 = torch.empty((b.num_tokens, b.num_heads * 128), dtype=torch.float32, device=DEV)
    f1 = torch.empty_like(f0)
    _, l0 = d.run(return_lse=True, output_f32=f0)
    _, l1 = d.run(return_lse=True, output_f32=f1, gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(f0, f1) and torch.equal(l0, l1)


# ------------------------------------------------------------------ binding: streams

def test_side_stream_without_workspace():
    # The binding makes the workspace and the output itself on the stream the
    # kernels run on.  Straight after the call, the default stream allocates a
    # block of the workspace's size and overwrites it: had the freed workspace
    # belonged to the default stream, that block would be the workspace while
    # the kernels on the side stream still read it.
    b = W.mixed(3)
    d = DevBatch(b)
    need = pa.workspace_bytes(pa.make_args(d.q, d.k, d.v, d.kc, d.vc, d.cum, d.past, d.table,
                                           d.slots, torch.empty(1, device=DEV),
                                           num_heads=b.num_heads, kv_num_heads=b.kv_num_heads))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = d.run(stream=s)
    junk = torch.empty(need, dtype=torch.uint8, device=DEV)
    junk.fill_(0xFF)
    torch.cuda.synchronize()
    check(b, gpu=(to_host(out), to_host(d.kc), to_host(d.vc)))


# ------------------------------------------------------------------ fused prologue: Q/K OffsetRMSNorm + partial MRoPE
#
# The kernels normalise and rotate in fp32 and round once to the data type;
# the oracle does the same steps in fp64.  So every cache slot the call does
# not write, and every value row, stays bit-exact.  A key element written
# through the prologue must lie within one unit in the last place of the
# exact (fp64) value plus the fp32 arithmetic's error: a handful of fp32
# units (2^-24) of the head row's largest element, bounded here by
# 2^-21 * max|row| (the products and sums of the norm and the rotation round
# at the row's scale, so a result that nearly cancels, x1 cos - x2 sin close
# to 0, carries an absolute error of that size, several units of its own
# last place).  With INT8 / INT4 caches the codes lie within one code.
# Outputs keep the bar of their data type.

def prologue_dev(kw):
    out = dict(kw)
    for n in ("position_ids", "q_norm_weight", "k_norm_weight"):
        if kw.get(n) is not None:
            out[n] = to_dev(np.ascontiguousarray(kw[n]))
    return out


def token_slots(b: W.Batch) -> np.ndarray:
    if b.slot_mapping is not None:
        return b.slot_mapping.astype(np.int64)
    pos = W.token_positions(b)
    seq = np.repeat(np.arange(b.batch_size), b.q_lens)
    return b.block_table[seq, pos // b.block_size].astype(np.int64) * b.block_size + pos % b.block_size


def unit_in_last_place(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the data type's numbers at |v| (fp64)."""
    a = np.maximum(np.abs(v), 2.0 ** -14 if dtype == "f16" else 2.0 ** -126)
    e = np.floor(np.log2(a))
    return np.exp2(e - (10 if dtype == "f16" else 7))


def check_prologue(b: W.Batch, kw: dict, tag=""):
    say(f"[gpu] prologue{tag} {b.name} {b.dtype} kv={b.kv_quant} N={b.num_tokens} D={b.head_size} "
        f"rd={kw.get('rotary_dim')} norm={kw.get('q_norm_weight') is not None} "
        f"adjacent={kw.get('adjacent')} interleaved={kw.get('interleaved')}")
    d = DevBatch(b)
    out = d.run(prologue=prologue_dev(kw))
    torch.cuda.synchronize()
    ref, rkc, rvc = oracle.paged_attention(b.query, b.key, b.value, b.key_cache, b.value_cache, b.cum,
                                           b.past, b.block_table, b.slot_mapping, num_heads=b.num_heads,
                                           kv_num_heads=b.kv_num_heads, scale=b.scale, k_scale=b.k_scale,
                                           v_scale=b.v_scale, prologue=kw)
    kc, vc = to_host(d.kc), to_host(d.vc)
    assert np.array_equal(raw_bits(vc), raw_bits(rvc)), "value_cache differs"
    nslot = b.num_blocks * b.block_size
    slots = token_slots(b)
    written = np.zeros(nslot, dtype=bool)
    written[slots[slots >= 0]] = True
    kg, kr = raw_bits(kc).reshape(nslot, -1), raw_bits(rkc).reshape(nslot, -1)
    assert np.array_equal(kg[~written], kr[~written]), "key_cache differs outside the written slots"
    toks = np.nonzero(slots >= 0)[0]
    if toks.size:
        Q, K, _, _, _ = oracle.resolve_call(b.query, b.key, b.value, b.num_heads, b.kv_num_heads, b.scale)
        _, kex = oracle.qk_prologue(Q, K, rounded=False, **kw)      # exact key rows [N, Hkv, D]
        rows = slots[toks]
        if b.kv_quant == "none":
            got = as_f64(kg[rows].view(np.uint16 if b.dtype == "bf16" else np.float16))
            exact = kex[toks].reshape(got.shape)
            D = b.head_size
            rowmax = np.repeat(np.max(np.abs(exact.reshape(-1, D)), axis=1), D).reshape(exact.shape)
            ulp = unit_in_last_place(exact, b.dtype)
            excess = np.abs(got - exact) - ulp
            worst = float(np.max(np.abs(got - exact) / ulp))
            flips = int(np.sum(kg[rows] != kr[rows]))
            i = np.unravel_index(np.argmax(excess / (2.0 ** -21 * rowmax)), exact.shape)
            say(f"      written key rows: {rows.size}, worst |gpu - exact| {worst:.3f} ulp, "
                f"{flips} of {kg[rows].size} roundings differ from the oracle's; "
                f"{int(np.sum(excess > 0))} beyond one ulp, largest at exact {exact[i]:.4g} "
                f"got {got[i]:.4g} (row max {rowmax[i]:.3g})")
            assert np.all(excess <= 2.0 ** -21 * rowmax)
        else:
            cg, cr = kc.reshape(nslot, -1)[rows], rkc.reshape(nslot, -1)[rows]
            if b.kv_quant == "int4":
                cg, cr = oracle.unpack_int4(cg), oracle.unpack_int4(cr)
            diff = np.abs(cg.astype(np.int64) - cr.astype(np.int64))
            say(f"      written key rows: {rows.size}, codes differing by one: {int(np.sum(diff == 1))}")
            assert diff.max() <= 1
    got = as_f64(to_host(out))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"      outputs: max|err| {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol(b)


PROLOGUE_SWEEP = [  # (sweep case, rotary_dim as a fraction of D, spatial, adjacent, interleaved, norm)
    (0, 0.5, False, False, True, True),
    (1, 1.0, True, False, True, True),
    (2, 0.25, True, True, True, True),
    (3, 0.5, False, False, False, True),
    (4, 1.0, True, True, False, False),   # rotation only (G=3)
    (5, 0.0, False, False, True, True),   # norm only (G=64)
    (6, 0.5, True, False, True, True),    # G=5, block_size 48
]


@pytest.mark.parametrize("case", range(len(PROLOGUE_SWEEP)))
@pytest.mark.parametrize("packed", [False, True])
def test_prologue_sweep(case, packed):
    i, frac, spatial, adjacent, interleaved, norm = PROLOGUE_SWEEP[case]
    q, p, H, Hkv, D, bs = SWEEP[i]
    n = sum(q)
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs, seed=800 + case,
                     packed=packed, slot_mode="drop" if packed else None,
                     drop_count=max(1, n // 20) if packed else 0, name=f"prologue_sweep{case}")
    kw = W.prologue_inputs(b, 810 + case, rotary_dim=int(D * frac), norm=norm, spatial=spatial,
                           adjacent=adjacent, interleaved=interleaved)
    if frac == 0.0:
        kw.update(rotary_dim=0)
    check_prologue(b, kw)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kvq", ["none", "int8", "int4"])
def test_prologue_tiny(dtype, kvq):
    b = W.tiny(0, dtype=dtype, kv_quant=kvq)
    check_prologue(b, W.prologue_inputs(b, 820, rotary_dim=32, spatial=True))


def test_prologue_long_prefill():
    # one rank's share of a 32/8 model, rotating half of each 128-wide head
    b = W.long_prefill(0)
    check_prologue(b, W.prologue_inputs(b, 830, rotary_dim=64))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prologue_mixed(dtype):
    b = W.mixed(0, dtype=dtype)
    check_prologue(b, W.prologue_inputs(b, 831, rotary_dim=128, adjacent=dtype == "bf16",
                                        interleaved=dtype == "f16"))


@pytest.mark.parametrize("kvq", ["none", "int8"])
def test_prologue_head_size_256(kvq):
    # head size 256 with a quarter of the channels rotating, spatial positions
    q, p, H, Hkv, bs = HD256[0]
    b = W.make_batch(q, p, num_heads=H, kv_num_heads=Hkv, head_size=256, block_size=bs, seed=840,
                     name=f"prologue_hd256_{kvq}", dtype="bf16", kv_quant=kvq, packed=True,
                     slot_mode="drop", drop_count=5)
    check_prologue(b, W.prologue_inputs(b, 841, rotary_dim=64, spatial=True))


def test_prologue_pure_decode_full():
    b = W.pure_decode(0)
    check_prologue(b, W.prologue_inputs(b, 850, rotary_dim=64))


# ------------------------------------------------------------------ fused prologue with the other features

def test_prologue_with_gate_and_state():
    # The prologue transforms the step's query and key rows; the output gate
    # multiplies the output only, and the exported (out, lse) state is the
    # ungated attention over the transformed rows.  Decode segments cut
    # across waves (merged) and whole ones, and chunked rows, in one call.
    b = W.make_batch([1, 300, 1, 64], [2000, 700, 9000, 0], num_heads=16, kv_num_heads=4, head_size=128,
                     block_size=16, seed=860, name="prologue_gate_state")
    kw = W.prologue_inputs(b, 861, rotary_dim=64, spatial=True)
    gate = W.output_gate_input(b, 862)
    say(f"[gpu] prologue + gate + state {b.name} N={b.num_tokens} B={b.batch_size}")
    d = DevBatch(b)
    f32 = torch.empty((b.num_tokens, b.num_heads * b.head_size), dtype=torch.float32, device=DEV)
    out, lse = d.run(return_lse=True, output_f32=f32, gate=to_dev(gate), prologue=prologue_dev(kw))
    torch.cuda.synchronize()
    args = (b.query, b.key, b.value, b.key_cache, b.value_cache, b.cum, b.past, b.block_table, b.slot_mapping)
    common = dict(num_heads=b.num_heads, kv_num_heads=b.kv_num_heads, scale=b.scale, prologue=kw)
    gated, _, _ = oracle.paged_attention(*args, gate=gate, **common)
    plain, _, _, rlse = oracle.paged_attention(*args, with_lse=True, **common)
    o16, o32, l32 = as_f64(to_host(out)), f32.cpu().numpy().astype(np.float64), lse.cpu().numpy()
    e_g = float(np.max(np.abs(o16 - gated)))
    e_o = float(np.max(np.abs(o32 - plain)))
    e_l = float(np.max(np.abs(l32.astype(np.float64) - rlse)))
    say(f"      max|err| gated output {e_g:.3e}, out_f32 {e_o:.3e}, lse {e_l:.3e}")
    assert e_g <= tol(b) and e_o <= tol(b) and e_l <= LSE_TOL


def test_prologue_hip_graph_replay_matches_eager():
    # the prologue's query rows live in the workspace: a captured call must
    # rebuild them on every replay (eager work on other data between replays)
    b = W.mixed(3)
    kw = prologue_dev(W.prologue_inputs(b, 870, rotary_dim=64))
    d = DevBatch(b)
    ref = d.run(prologue=kw).clone()
    torch.cuda.synchronize()
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(output=out, workspace=ws, stream=s, prologue=kw)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(output=out, workspace=ws, stream=s, prologue=kw)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
