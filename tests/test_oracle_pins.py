"""Pins of the CPU oracle to things other than itself (CPU only).

Each check_* function takes an oracle callable with the signature of
oracle.paged_attention and raises AssertionError when the callable breaks the
property.  The tests run every check on the real oracle; test_planted_mistakes
runs them on copies of the oracle with a typical mistake planted and requires
that each mistake is caught by at least one check.

What each pin rests on (pages cited by title and section):
  I1  slot_mapping -1 leaves the cache untouched; exactly the slots >= 0
      change (README "com.microsoft.PagedAttention", Inputs: slot_mapping).
  I2  explicit allocator slots == omitted slot_mapping (same passage: the
      derived slot follows past_seqlens).
  I3  relabelling physical pages leaves the result unchanged (README,
      Description: block_table maps a history onto scattered blocks).
  I4  paged == contiguous at several block sizes (same passage).
  I5  single contiguous sequence == torch scaled_dot_product_attention in
      float64 with an explicit bottom-right mask and repeated KV heads
      (library routine; bottom-right offset from "WS2 CP-Aware Attention
      Contract", Mode-Specific Metadata).
  I6  closed forms: a lone first token returns its own V row; a zero query or
      equal keys give the mean of the visible V rows.
  I7  hand computations: a two-key case in sigmoid form, and the README's
      example shape (tests/golden/p3_example.json).
  I8  GQA == MHA with each KV head repeated; packed [Q|K|V] == separate;
      scale 0 == 1/sqrt(D) (README, Inputs and Attributes).
  I9  a batch == independent calls; permuting sequences permutes rows;
      a chunked continuation == one shot ("Add Qwen3.8 packed hybrid
      PagedAttention export ...", Acceptance criteria).
  I10 partial (out, lse) states merged in fixed order == direct softmax
      ("WS2 CP-Aware Attention Contract", Reduction Semantics).
  I11 the scalar formulation (oracle/scalar.py) agrees within 1e-12.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import scalar
import importlib
import workloads as W

pa_mod = importlib.import_module("oracle.paged_attention")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def call(fn, b: W.Batch, **kw):
    args = dict(query=b.query, key=b.key, value=b.value, key_cache=b.key_cache,
                value_cache=b.value_cache, cum=b.cum, past=b.past, block_table=b.block_table,
                slot_mapping=b.slot_mapping, num_heads=b.num_heads,
                kv_num_heads=b.kv_num_heads, scale=b.scale)
    args.update(kw)
    return fn(args.pop("query"), args.pop("key"), args.pop("value"), args.pop("key_cache"),
              args.pop("value_cache"), args.pop("cum"), args.pop("past"),
              args.pop("block_table"), args.pop("slot_mapping"), **args)


def small(seed=0, **kw):
    base = dict(q_lens=[3, 1, 17, 5], past_lens=[5, 20, 0, 33], num_heads=4, kv_num_heads=2,
                head_size=8, block_size=4, seed=seed)
    base.update(kw)
    q, p = base.pop("q_lens"), base.pop("past_lens")
    return W.make_batch(q, p, **base)


def slot_view(cache):
    NB, bs, Hkv, D = cache.shape
    return cache.reshape(NB * bs, Hkv * D).view(np.uint16)


# ------------------------------------------------------------------ I1 / I2

def check_I1(fn):
    b = small(seed=1, slot_mode="drop", drop_count=3)
    _, kc, vc = call(fn, b)
    sm = b.slot_mapping
    written = {int(s): t for t, s in enumerate(sm) if s >= 0}
    K = b.key.view(np.uint16)
    V = b.value.view(np.uint16)
    for before, after, src in ((b.key_cache, kc, K), (b.value_cache, vc, V)):
        sb, sa = slot_view(before), slot_view(after)
        for s in range(sb.shape[0]):
            if s in written:
                assert np.array_equal(sa[s], src[written[s]]), f"slot {s} not written"
            else:
                assert np.array_equal(sa[s], sb[s]), f"slot {s} changed"


def check_I2(fn):
    b = small(seed=2)
    o1, k1, v1 = call(fn, b)
    slots = W.allocator_slots(b.block_table, b.past, b.q_lens, b.block_size)
    o2, k2, v2 = call(fn, b, slot_mapping=slots)
    assert np.array_equal(k1.view(np.uint16), k2.view(np.uint16))
    assert np.array_equal(v1.view(np.uint16), v2.view(np.uint16))
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------------ I3 / I4

def check_I3(fn):
    b = small(seed=3, num_blocks=40)
    o1, k1, v1 = call(fn, b)
    rng = np.random.default_rng(33)
    pi = rng.permutation(b.num_blocks)
    kc = np.empty_like(b.key_cache)
    vc = np.empty_like(b.value_cache)
    kc[pi] = b.key_cache
    vc[pi] = b.value_cache
    table = np.where(b.block_table >= 0, pi[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    o2, k2, v2 = call(fn, b, key_cache=kc, value_cache=vc, block_table=table)
    assert np.array_equal(o1, o2)
    assert np.array_equal(k2[pi].view(np.uint16), k1.view(np.uint16))
    assert np.array_equal(v2[pi].view(np.uint16), v1.view(np.uint16))


def layout(hist_k, hist_v, q_lens, bs, rng, spare=3):
    """Place logical histories (lists of [p_b, Hkv, D] fp16) into a paged
    cache with block size bs and a shuffled table; returns caches and table."""
    B = len(hist_k)
    Hkv, D = hist_k[0].shape[1:]
    n = [W.pages_needed(h.shape[0] + q, bs) for h, q in zip(hist_k, q_lens)]
    nb = sum(n) + spare
    ids = rng.permutation(nb)
    table = np.full((B, max(n)), -1, np.int32)
    kc = W.normal_f16(rng, (nb, bs, Hkv, D))
    vc = W.normal_f16(rng, (nb, bs, Hkv, D))
    cur = 0
    for i in range(B):
        table[i, :n[i]] = ids[cur:cur + n[i]]
        cur += n[i]
        for j in range(hist_k[i].shape[0]):
            pg = table[i, j // bs]
            kc[pg, j % bs] = hist_k[i][j]
            vc[pg, j % bs] = hist_v[i][j]
    return kc, vc, table


def check_I4(fn):
    rng = np.random.default_rng(4)
    q_lens, past = [2, 1, 6], [7, 19, 30]
    H, Hkv, D = 4, 2, 8
    hk = [W.normal_f16(rng, (p, Hkv, D)) for p in past]
    hv = [W.normal_f16(rng, (p, Hkv, D)) for p in past]
    N = sum(q_lens)
    Q = W.normal_f16(rng, (N, H * D))
    K = W.normal_f16(rng, (N, Hkv * D))
    V = W.normal_f16(rng, (N, Hkv * D))
    cum = W.cum_from_lens(q_lens)
    outs = []
    for bs in (1, 4, 16, 64):
        kc, vc, table = layout(hk, hv, q_lens, bs, np.random.default_rng(bs))
        o, _, _ = fn(Q, K, V, kc, vc, cum, np.array(past, np.int32), table, None,
                     num_heads=H, kv_num_heads=Hkv, scale=0.0)
        outs.append(o)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ------------------------------------------------------------------ I5

def check_I5(fn):
    rng = np.random.default_rng(5)
    H, Hkv, D, p, q = 6, 2, 16, 11, 7
    bs = 8
    L = p + q
    nb = W.pages_needed(L, bs)
    table = np.arange(nb, dtype=np.int32)[None, :]
    kc = W.normal_f16(rng, (nb, bs, Hkv, D))
    vc = W.normal_f16(rng, (nb, bs, Hkv, D))
    Q = W.normal_f16(rng, (q, H * D))
    K = W.normal_f16(rng, (q, Hkv * D))
    V = W.normal_f16(rng, (q, Hkv * D))
    scale = 0.37
    o, _, _ = fn(Q, K, V, kc, vc, np.array([0, q], np.int32), np.array([p], np.int32), table,
                 None, num_heads=H, kv_num_heads=Hkv, scale=scale)
    # contiguous history: the identity table puts position j at slot j
    kf = kc.reshape(-1, Hkv, D)[:L].astype(np.float64).copy()
    vf = vc.reshape(-1, Hkv, D)[:L].astype(np.float64).copy()
    kf[p:] = K.reshape(q, Hkv, D)
    vf[p:] = V.reshape(q, Hkv, D)
    G = H // Hkv
    qt = torch.from_numpy(Q.astype(np.float64).reshape(q, H, D)).permute(1, 0, 2)
    kt = torch.from_numpy(kf).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(vf).permute(1, 0, 2).repeat_interleave(G, dim=0)
    allow = torch.ones(q, L, dtype=torch.bool).tril(diagonal=p)  # row i sees j <= p+i
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow,
                                                           scale=scale)
    ref = ref.permute(1, 0, 2).reshape(q, H * D).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


# ------------------------------------------------------------------ I6

def check_I6(fn):
    rng = np.random.default_rng(6)
    H, Hkv, D, bs = 4, 2, 8, 4
    # (a) a sequence's very first token sees only itself: weight exactly 1
    b = small(seed=6, q_lens=[1, 1], past_lens=[0, 0])
    o, _, _ = call(fn, b)
    G = H // Hkv
    for t in range(2):
        for h in range(H):
            k = h // G
            want = b.value[t, k * D:(k + 1) * D].astype(np.float64)
            assert np.array_equal(o[t, h * D:(h + 1) * D], want)
    # (b) zero query: uniform weights -> mean of visible V rows
    # (c) all keys equal: uniform weights as well
    p, q = 9, 4
    L = p + q
    nb = W.pages_needed(L, bs)
    table = np.arange(nb, dtype=np.int32)[None, :]
    kc = W.normal_f16(rng, (nb, bs, Hkv, D))
    vc = W.normal_f16(rng, (nb, bs, Hkv, D))
    K = W.normal_f16(rng, (q, Hkv * D))
    V = W.normal_f16(rng, (q, Hkv * D))
    vf = vc.reshape(-1, Hkv, D)[:L].astype(np.float64).copy()
    vf[p:] = V.reshape(q, Hkv, D)
    args = (np.array([0, q], np.int32), np.array([p], np.int32), table, None)
    Qz = np.zeros((q, H * D), np.float16)
    o_b, _, _ = fn(Qz, K, V, kc, vc, *args, num_heads=H, kv_num_heads=Hkv, scale=0.0)
    kce = np.full_like(kc, 0.75)
    Ke = np.full_like(K, 0.75)
    Qr = W.normal_f16(rng, (q, H * D))
    o_c, _, _ = fn(Qr, Ke, V, kce, vc, *args, num_heads=H, kv_num_heads=Hkv, scale=0.0)
    for i in range(q):
        for h in range(H):
            mean = vf[:p + i + 1, h // G].mean(axis=0)
            assert np.max(np.abs(o_b[i, h * D:(h + 1) * D] - mean)) < 1e-14
            assert np.max(np.abs(o_c[i, h * D:(h + 1) * D] - mean)) < 1e-14


# ------------------------------------------------------------------ I7

def check_I7(fn):
    # two keys, one head, D=2: o = sig(s1-s0) v1 + (1 - sig(s1-s0)) v0
    rng = np.random.default_rng(7)
    for trial in range(5):
        kc = W.normal_f16(rng, (2, 2, 1, 2))
        vc = W.normal_f16(rng, (2, 2, 1, 2))
        Q = W.normal_f16(rng, (1, 2))
        K = W.normal_f16(rng, (1, 2))
        V = W.normal_f16(rng, (1, 2))
        table = np.array([[1, 0]], np.int32)  # position 0 at slot 2, position 1 at slot 3
        o, _, _ = fn(Q, K, V, kc, vc, np.array([0, 1], np.int32), np.array([1], np.int32),
                     table, None, num_heads=1, kv_num_heads=1, scale=0.0)
        q0, q1 = float(Q[0, 0]), float(Q[0, 1])
        k0 = [float(x) for x in kc[1, 0, 0]]
        v0 = [float(x) for x in vc[1, 0, 0]]
        k1 = [float(x) for x in K[0]]
        v1 = [float(x) for x in V[0]]
        c = 1 / math.sqrt(2)
        s0 = c * (q0 * k0[0] + q1 * k0[1])
        s1 = c * (q0 * k1[0] + q1 * k1[1])
        sig = 1 / (1 + math.exp(-(s1 - s0)))
        want = [sig * v1[d] + (1 - sig) * v0[d] for d in range(2)]
        assert np.max(np.abs(o[0] - np.array(want))) < 1e-14
    # the README's example shape with chosen data (exact expected values)
    with open(os.path.join(GOLDEN, "p3_example.json")) as f:
        g = json.load(f)
    c0, c1 = g["cases"]
    arr = lambda x: np.array(x, dtype=np.float16)
    args = [arr(c0["query"]), arr(c0["key"]), arr(c0["value"]), arr(c0["key_cache"]),
            arr(c0["value_cache"]), np.array(c0["cum"], np.int32),
            np.array(c0["past"], np.int32), np.array(c0["block_table"], np.int32)]
    o, kc, vc = fn(*args, None, num_heads=2, kv_num_heads=1, scale=c0["scale"])
    # exact rationals; thirds are not dyadic, so allow a few ulps
    assert np.max(np.abs(o - np.array(c0["expected_output"]))) < 1e-14
    assert np.array_equal(kc, arr(c0["expected_key_cache"]))
    assert np.array_equal(vc, arr(c0["expected_value_cache"]))
    o2, kc2, _ = fn(*args, np.array(c1["slot_mapping"], np.int32), num_heads=2,
                    kv_num_heads=1, scale=0.0)
    assert np.max(np.abs(o2[0] - np.array(c1["expected_output_row0"]))) < 1e-14
    assert kc2[0, 0, 0, 0] == 5.0
    for h, (qa, qb) in enumerate([(1.0, 1.0), (-0.5, 3.0)]):
        a = math.exp((qa * 5 + qb * 5) / math.sqrt(2))
        want = [(1 + 3 + 100 * a) / (2 + a), (-2 + 0.5 + 100 * a) / (2 + a)]
        assert np.max(np.abs(o2[1, 2 * h:2 * h + 2] - want)) < 1e-12


# ------------------------------------------------------------------ I8

def check_I8(fn):
    b = small(seed=8)
    o, kc, vc = call(fn, b)
    G = b.num_heads // b.kv_num_heads
    D = b.head_size
    # MHA with each KV head repeated G times
    rep = lambda x: np.repeat(x.reshape(x.shape[0], b.kv_num_heads, D), G, axis=1
                              ).reshape(x.shape[0], -1)
    kcm = np.repeat(b.key_cache, G, axis=2)
    vcm = np.repeat(b.value_cache, G, axis=2)
    om, _, _ = call(fn, b, key=rep(b.key), value=rep(b.value), key_cache=kcm, value_cache=vcm,
                    kv_num_heads=b.num_heads)
    assert np.array_equal(o, om)
    # packed [Q|K|V] == separate inputs
    packed = np.concatenate([b.query, b.key, b.value], axis=1)
    op, kcp, vcp = call(fn, b, query=packed, key=None, value=None)
    assert np.array_equal(o, op)
    assert np.array_equal(kc.view(np.uint16), kcp.view(np.uint16))
    assert np.array_equal(vc.view(np.uint16), vcp.view(np.uint16))
    # scale 0 selects 1/sqrt(D)
    os_, _, _ = call(fn, b, scale=1.0 / math.sqrt(D))
    assert np.array_equal(o, os_)


# ------------------------------------------------------------------ I9

def check_I9(fn):
    b = small(seed=9)
    o, kc, vc = call(fn, b)
    B = b.batch_size
    # independent single-sequence calls on the original caches
    for i in range(B):
        t0, t1 = int(b.cum[i]), int(b.cum[i + 1])
        oi, _, _ = call(fn, b, query=b.query[t0:t1], key=b.key[t0:t1], value=b.value[t0:t1],
                        cum=np.array([0, t1 - t0], np.int32), past=b.past[i:i + 1],
                        block_table=b.block_table[i:i + 1])
        assert np.array_equal(oi, o[t0:t1])
    # permuting the sequences permutes the output rows
    perm = np.array([2, 0, 3, 1])
    rows = np.concatenate([np.arange(b.cum[i], b.cum[i + 1]) for i in perm])
    qp = b.q_lens[perm]
    op, kcp, _ = call(fn, b, query=b.query[rows], key=b.key[rows], value=b.value[rows],
                      cum=W.cum_from_lens(qp), past=b.past[perm],
                      block_table=b.block_table[perm])
    assert np.array_equal(op, o[rows])
    assert np.array_equal(kcp.view(np.uint16), kc.view(np.uint16))
    # chunked continuation: sequence 2 (17 new tokens) in two calls
    i = 2
    t0, t1 = int(b.cum[i]), int(b.cum[i + 1])
    cut = 6
    one = dict(block_table=b.block_table[i:i + 1])
    oa, kca, vca = call(fn, b, query=b.query[t0:t0 + cut], key=b.key[t0:t0 + cut],
                        value=b.value[t0:t0 + cut], cum=np.array([0, cut], np.int32),
                        past=b.past[i:i + 1], **one)
    ob, kcb, vcb = call(fn, b, query=b.query[t0 + cut:t1], key=b.key[t0 + cut:t1],
                        value=b.value[t0 + cut:t1], key_cache=kca, value_cache=vca,
                        cum=np.array([0, t1 - t0 - cut], np.int32),
                        past=b.past[i:i + 1] + cut, **one)
    of, kcf, vcf = call(fn, b, query=b.query[t0:t1], key=b.key[t0:t1], value=b.value[t0:t1],
                        cum=np.array([0, t1 - t0], np.int32), past=b.past[i:i + 1], **one)
    # BLAS may block a matmul over 6 and 17 rows differently: allow rounding
    assert np.max(np.abs(np.concatenate([oa, ob]) - of)) < 1e-13
    assert np.array_equal(kcb.view(np.uint16), kcf.view(np.uint16))
    assert np.array_equal(vcb.view(np.uint16), vcf.view(np.uint16))


# ------------------------------------------------------------------ I10

def check_I10(fn):
    b = small(seed=10)
    o, kc, vc = call(fn, b)
    Q, K, V, D, s = oracle.resolve_call(b.query, b.key, b.value, b.num_heads,
                                        b.kv_num_heads, 0.0)
    rng = np.random.default_rng(10)
    G = b.num_heads // b.kv_num_heads
    for i in range(b.batch_size):
        L = int(b.kv_lens[i])
        Kb, Vb = oracle.gather_history(kc, vc, b.block_table, i, L)
        for r in range(int(b.q_lens[i])):
            t = int(b.cum[i]) + r
            vis = int(b.past[i]) + r + 1
            for h in range(b.num_heads):
                keys = np.arange(vis)
                for mode in ("contiguous", "shuffled"):
                    ks = keys if mode == "contiguous" else rng.permutation(keys)
                    cuts = np.sort(rng.choice(np.arange(1, vis), size=min(3, vis - 1),
                                              replace=False)) if vis > 1 else []
                    parts = np.split(ks, cuts)
                    st = [oracle.partial_state(Q[t, h].astype(np.float64), Kb[:, h // G],
                                               Vb[:, h // G], s, p) for p in parts]
                    m = oracle.merge_partials([x[0] for x in st], [x[1] for x in st])
                    assert np.max(np.abs(m - o[t, h * D:(h + 1) * D])) < 1e-12


# ------------------------------------------------------------------ I11

def check_I11(fn):
    cases = [W.tiny(0), small(seed=11, head_size=4), small(seed=12, head_size=4, packed=True,
                                                            slot_mode="drop", drop_count=2)]
    for b in cases:
        o, _, _ = call(fn, b)
        so, written = scalar.paged_attention_scalar(b.query, b.key, b.value, b.key_cache,
                                                    b.value_cache, b.cum, b.past,
                                                    b.block_table, b.slot_mapping,
                                                    b.num_heads, b.kv_num_heads, b.scale)
        assert np.max(np.abs(o - np.array(so))) < 1e-12


CHECKS = [check_I1, check_I2, check_I3, check_I4, check_I5, check_I6, check_I7, check_I8,
          check_I9, check_I10, check_I11]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.paged_attention)


# ------------------------------------------------------------------ planted mistakes

def _mutant(**patch):
    """A copy of oracle.paged_attention whose module-level helpers are replaced."""
    def fn(*a, **k):
        saved = {name: getattr(pa_mod, name) for name in patch}
        try:
            for name, f in patch.items():
                setattr(pa_mod, name, f)
            return pa_mod.paged_attention(*a, **k)
        finally:
            for name, f in saved.items():
                setattr(pa_mod, name, f)
    return fn


def _attend_variant(head_map=None, top_left=False, no_scale=False, off_by_one=False):
    def attend(Qb, Kb, Vb, past_b, scale, rows=None):
        q, H, D = Qb.shape
        L, Hkv, _ = Kb.shape
        G = H // Hkv
        sel = np.arange(q) if rows is None else np.asarray(rows)
        out = np.full((q, H, D), np.nan)
        pos = (0 if top_left else past_b) + sel + (1 if off_by_one else 0)
        masked = np.arange(L)[None, :] > pos[:, None]
        for h in range(H):
            k = head_map(h, H, Hkv) if head_map else h // G
            S = (1.0 if no_scale else scale) * (Qb[sel, h] @ Kb[:, k].T)
            S[masked] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[sel, h] = P @ Vb[:, k]
        return out
    return attend


def _scatter_ignoring_minus_one(kc, vc, K, V, cum, past, table, sm, k_scale=None, v_scale=None):
    sm2 = None if sm is None else np.where(sm < 0, 0, sm)
    return _orig_scatter(kc, vc, K, V, cum, past, table, sm2)


_orig_scatter = pa_mod.scatter_kv


def _scatter_nothing(kc, vc, K, V, cum, past, table, sm, k_scale=None, v_scale=None):
    return kc.copy(), vc.copy()


def _gather_wrong_offset(kc, vc, table, b, length, k_scale=None, v_scale=None):
    NB, bs, Hkv, D = kc.shape
    j = np.arange(int(length))
    idx = table[b, j // bs].astype(np.int64) * bs + (bs - 1 - j % bs)
    return (kc.reshape(-1, Hkv, D)[idx].astype(np.float64),
            vc.reshape(-1, Hkv, D)[idx].astype(np.float64))


MUTANTS = {
    "interleaved_head_map": dict(attend_sequence=_attend_variant(
        head_map=lambda h, H, Hkv: h % Hkv)),
    "top_left_causal": dict(attend_sequence=_attend_variant(top_left=True)),
    "scale_dropped": dict(attend_sequence=_attend_variant(no_scale=True)),
    "mask_off_by_one": dict(attend_sequence=_attend_variant(off_by_one=True)),
    "reads_pre_scatter_cache": dict(scatter_kv=_scatter_nothing),
    "minus_one_written": dict(scatter_kv=_scatter_ignoring_minus_one),
    "wrong_in_block_offset": dict(gather_history=_gather_wrong_offset),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name):
    fn = _mutant(**MUTANTS[name])
    caught = []
    for check in CHECKS:
        try:
            check(fn)
        except (AssertionError, IndexError, ValueError):
            caught.append(check.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# ------------------------------------------------------------------ lse and state merge

# Pins of the attention-domain lse the oracle exports with its output, and of
# its whole-tensor merge of partial states ("WS2 CP-Aware Attention Contract",
# Reduction Semantics: the partial state of a row is (out, lse); states merge
# by the online-softmax rule in a fixed order).
#   L1  lone first token: one visible key, lse = scale <q, k0>; zero query:
#       all scores 0, lse = log(number of visible keys).
#   L2  the scalar formulation's fsum lse agrees within 1e-12.
#   M1  splitting a row's visible keys into parts, the merged partial states
#       equal the direct (out, lse) of the row (union of the key sets).
#   M2  one state is returned unchanged; a state with lse = -inf is ignored;
#       all-empty rows give (0, -inf); permuting the states changes nothing
#       beyond rounding.


def _scale_of(b):
    return b.scale if b.scale != 0 else 1.0 / math.sqrt(b.head_size)


def check_L(fn_lse):
    b = W.make_batch([1, 1], [0, 9], num_heads=4, kv_num_heads=2, head_size=8, block_size=16,
                     seed=21, name="lse_pins")
    o, _, _, lse = fn_lse(b)
    # first sequence: past 0, one token: a single visible key (its own K row)
    Q = b.query.astype(np.float64).reshape(b.num_tokens, b.num_heads, -1)
    K = b.key.astype(np.float64).reshape(b.num_tokens, b.kv_num_heads, -1)
    D = Q.shape[2]
    for h in range(b.num_heads):
        assert abs(lse[0, h] - _scale_of(b) * Q[0, h] @ K[0, h // 2]) < 1e-12
    # zero query: every score is 0
    bz = W.make_batch([3], [13], num_heads=2, kv_num_heads=1, head_size=8, block_size=16, seed=22,
                      name="lse_zero")
    bz.query[:] = 0
    _, _, _, lz = fn_lse(bz)
    for i in range(3):
        assert np.all(np.abs(lz[i] - math.log(13 + i + 1)) < 1e-12)
    # scalar formulation
    for bb in (b, small(seed=23, head_size=4), small(seed=24, head_size=4, packed=True,
                                                     slot_mode="drop", drop_count=2)):
        _, _, _, l1 = fn_lse(bb)
        _, _, l2 = scalar.paged_attention_scalar(bb.query, bb.key, bb.value, bb.key_cache,
                                                 bb.value_cache, bb.cum, bb.past, bb.block_table,
                                                 bb.slot_mapping, bb.num_heads, bb.kv_num_heads,
                                                 bb.scale, with_lse=True)
        assert np.max(np.abs(l1 - np.array(l2))) < 1e-12


def _oracle_with_lse(b):
    return call(oracle.paged_attention, b, with_lse=True)


def test_oracle_lse_pins():
    check_L(_oracle_with_lse)


def check_M(merge):
    rng = np.random.default_rng(31)
    b = W.make_batch([5, 1], [40, 70], num_heads=4, kv_num_heads=2, head_size=16, block_size=16,
                     seed=32, name="merge_pins")
    o, kc, vc, lse = _oracle_with_lse(b)
    Q, _, _, D, s = oracle.resolve_call(b.query, b.key, b.value, b.num_heads, b.kv_num_heads,
                                        b.scale)
    G = b.num_heads // b.kv_num_heads
    for i in range(b.batch_size):
        L = int(b.kv_lens[i])
        Kb, Vb = oracle.gather_history(kc, vc, b.block_table, i, L)
        for r in range(int(b.q_lens[i])):
            t = int(b.cum[i]) + r
            vis = int(b.past[i]) + r + 1
            for h in range(b.num_heads):
                keys = rng.permutation(vis)
                parts = np.split(keys, np.sort(rng.choice(np.arange(1, vis), 3, replace=False)))
                st = [oracle.partial_state(Q[t, h].astype(np.float64), Kb[:, h // G], Vb[:, h // G],
                                           s, p) for p in parts]
                mo, ml = merge(np.stack([x[0] for x in st])[:, None, :],
                               np.array([x[1] for x in st])[:, None])
                assert np.max(np.abs(mo[0] - o[t, h * D:(h + 1) * D])) < 1e-12
                assert abs(ml[0] - lse[t, h]) < 1e-12
    # identities on random states
    P, R, Dm = 4, 6, 8
    outs = rng.standard_normal((P, R, Dm))
    lses = rng.standard_normal((P, R)) * 3
    mo, ml = merge(outs[:1], lses[:1])
    assert np.max(np.abs(mo - outs[0])) < 1e-15 and np.max(np.abs(ml - lses[0])) < 1e-15
    l2 = lses.copy()
    l2[2] = -np.inf
    a_o, a_l = merge(outs, l2)
    b_o, b_l = merge(np.delete(outs, 2, axis=0), np.delete(l2, 2, axis=0))
    assert np.max(np.abs(a_o - b_o)) < 1e-12 and np.max(np.abs(a_l - b_l)) < 1e-12
    e_o, e_l = merge(outs, np.full((P, R), -np.inf))
    assert np.all(e_o == 0) and np.all(e_l == -np.inf)
    perm = rng.permutation(P)
    p_o, p_l = merge(outs[perm], lses[perm])
    m_o, m_l = merge(outs, lses)
    assert np.max(np.abs(p_o - m_o)) < 1e-12 and np.max(np.abs(p_l - m_l)) < 1e-12


def test_oracle_merge_pins():
    check_M(oracle.merge_states)


def _merge_unnormalised(outs, lses):
    o, l = oracle.merge_states(outs, lses)
    return o * np.exp(l - np.max(lses, axis=0))[:, None], l


def _merge_lse_is_max(outs, lses):
    o, _ = oracle.merge_states(outs, lses)
    return o, np.max(lses, axis=0)


def _merge_last_state_only(outs, lses):
    return np.asarray(outs[-1], dtype=np.float64), np.asarray(lses[-1], dtype=np.float64)


def _lse_log2(b):
    o, kc, vc, lse = _oracle_with_lse(b)
    return o, kc, vc, lse / math.log(2)


def _lse_unscaled(b):
    o, kc, vc, lse = _oracle_with_lse(b)
    return o, kc, vc, lse / _scale_of(b)


@pytest.mark.parametrize("mutant", [_merge_unnormalised, _merge_lse_is_max, _merge_last_state_only],
                         ids=lambda f: f.__name__)
def test_merge_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        check_M(mutant)


@pytest.mark.parametrize("mutant", [_lse_log2, _lse_unscaled], ids=lambda f: f.__name__)
def test_lse_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        check_L(mutant)


# ------------------------------------------------------------------ bf16 data

# bf16 tensors travel as uint16 bit patterns (numpy has no bfloat16); the
# oracle decodes them exactly ("values").  Pins:
#   B1  hand-decoded bit patterns (closed forms of the binary32 layout);
#   B2  one contiguous bf16 sequence == torch's scaled_dot_product_attention
#       on torch's own bf16 -> float64 conversion of the same bits;
#   B3  the bf16 cache writes are bit copies (slot -1 untouched, every other
#       slot equal to its token's row) and the scalar formulation, which
#       decodes bits with struct, agrees within 1e-12.

def check_B1(values):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127, -0.0,
            3.140625]
    got = values(bits)
    assert got.dtype == np.float64
    assert [float(x) for x in got] == want
    assert np.signbit(got[5])
    h = np.array([1.5, -0.25, 65504.0], dtype=np.float16)
    assert [float(x) for x in values(h)] == [1.5, -0.25, 65504.0]


def check_B2(fn):
    rng = np.random.default_rng(21)
    H, Hkv, D, p, q, bs = 4, 2, 16, 9, 6, 4
    L = p + q
    nb = W.pages_needed(L, bs)
    table = np.arange(nb, dtype=np.int32)[None, :]
    kc = W.normal_bf16(rng, (nb, bs, Hkv, D))
    vc = W.normal_bf16(rng, (nb, bs, Hkv, D))
    Q = W.normal_bf16(rng, (q, H * D))
    K = W.normal_bf16(rng, (q, Hkv * D))
    V = W.normal_bf16(rng, (q, Hkv * D))
    scale = -0.29
    o, _, _ = fn(Q, K, V, kc, vc, np.array([0, q], np.int32), np.array([p], np.int32), table,
                 None, num_heads=H, kv_num_heads=Hkv, scale=scale)

    def t64(x):  # torch's own bf16 decode
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double()
    kf = t64(kc.reshape(-1, Hkv, D)[:L]).clone()
    vf = t64(vc.reshape(-1, Hkv, D)[:L]).clone()
    kf[p:] = t64(K.reshape(q, Hkv, D))
    vf[p:] = t64(V.reshape(q, Hkv, D))
    G = H // Hkv
    qt = t64(Q.reshape(q, H, D)).permute(1, 0, 2)
    kt = kf.permute(1, 0, 2).repeat_interleave(G, dim=0)
    vt = vf.permute(1, 0, 2).repeat_interleave(G, dim=0)
    allow = torch.ones(q, L, dtype=torch.bool).tril(diagonal=p)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow,
                                                           scale=scale)
    ref = ref.permute(1, 0, 2).reshape(q, H * D).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def check_B3(fn):
    b = small(seed=23, slot_mode="drop", drop_count=3, dtype="bf16")
    o, kc, vc = call(fn, b)
    assert kc.dtype == np.uint16 and vc.dtype == np.uint16
    slots = W.allocator_slots(b.block_table, b.past, b.q_lens, b.block_size)
    NB, bs, Hkv, D = b.key_cache.shape
    before_k = b.key_cache.reshape(NB * bs, Hkv * D)
    after_k = kc.reshape(NB * bs, Hkv * D)
    after_v = vc.reshape(NB * bs, Hkv * D)
    dropped = np.nonzero(b.slot_mapping < 0)[0]
    for t in range(b.num_tokens):
        s = int(slots[t])
        if t in dropped:
            assert np.array_equal(after_k[s], before_k[s])
        else:
            assert np.array_equal(after_k[s], b.key[t]) and np.array_equal(after_v[s], b.value[t])
    for case in (W.tiny(0, dtype="bf16"), small(seed=24, head_size=4, packed=True, dtype="bf16")):
        oo, _, _ = call(fn, case)
        so, _ = scalar.paged_attention_scalar(case.query, case.key, case.value, case.key_cache,
                                              case.value_cache, case.cum, case.past,
                                              case.block_table, case.slot_mapping,
                                              case.num_heads, case.kv_num_heads, case.scale)
        assert np.max(np.abs(oo - np.array(so))) < 1e-12


def test_oracle_bf16_pins():
    check_B1(oracle.values)
    check_B2(oracle.paged_attention)
    check_B3(oracle.paged_attention)


def _values_as_f16(x):
    x = np.asarray(x)
    return x.view(np.float16).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _values_shift15(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


@pytest.mark.parametrize("mutant", [_values_as_f16, _values_shift15], ids=lambda f: f.__name__)
def test_bf16_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        check_B1(mutant)
    saved = pa_mod.values
    pa_mod.values = mutant
    try:
        with pytest.raises(AssertionError):
            check_B2(oracle.paged_attention)
    finally:
        pa_mod.values = saved


# ------------------------------------------------------------------ INT8 caches

# INT8 per-channel caches (codes + fp32 scales per (kv head, channel)).  Pins:
#   Q1  hand values of the code clamp(rint(x / s), -127, 127): exact
#       multiples, ties to even, clamping, and two cases where the quotient
#       taken in fp32 rounds to a tie that the fp64 quotient does not reach;
#   Q2  with power-of-two scales every code * scale is an fp16 value: the
#       INT8 oracle equals the fp16 oracle run on those values (and on step
#       rows that quantize exactly), bit for bit;
#   Q3  the scalar formulation (its own binary32 rounding) agrees within 1e-12.

def check_Q1(quant):
    s = np.full((1, 8), 0.25, dtype=np.float32)
    x = np.array([[1.0, 0.375, 0.625, 0.875, -0.625, 40.0, -40.0, 0.0]], dtype=np.float16)
    assert quant(x, s).tolist() == [[4, 2, 2, 4, -2, 127, -127, 0]]
    # x / s in fp32 is exactly 48.5 (code 48) and 53.5 (code 54); in fp64 the
    # quotients are 48.5000003 and 53.4999993 (codes 49 and 53)
    xs = np.array([[0x3C7D, 0x40E1]], dtype=np.uint16).view(np.float16)
    ss = np.array([[1019053721, 1027261488]], dtype=np.uint32).view(np.float32)
    assert quant(xs, ss).tolist() == [[48, 54]]
    # bf16 input (uint16 bit patterns): 3.0 / 0.5 = 6, -1.5 / 1 = -2 (tie to even)
    xb = np.array([[0x4040, 0xBFC0]], dtype=np.uint16)
    assert quant(xb, np.array([[0.5, 1.0]], dtype=np.float32)).tolist() == [[6, -2]]


def check_Q2(fn):
    rng = np.random.default_rng(31)
    H, Hkv, D, bs = 4, 2, 16, 4
    q_lens, past = [3, 1, 6], [5, 11, 0]
    b = W.make_batch(q_lens, past, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=31, kv_quant="int8")
    s = np.full((Hkv, D), 2.0 ** -5, dtype=np.float32)
    # step rows that are exact multiples of the scale within the code range
    K = (rng.integers(-127, 128, b.key.shape) * 2.0 ** -5).astype(np.float16)
    V = (rng.integers(-127, 128, b.value.shape) * 2.0 ** -5).astype(np.float16)
    o8, kc8, vc8 = fn(b.query, K, V, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                      None, num_heads=H, kv_num_heads=Hkv, k_scale=s, v_scale=s)
    kf = (b.key_cache.astype(np.float64) * 2.0 ** -5).astype(np.float16)
    vf = (b.value_cache.astype(np.float64) * 2.0 ** -5).astype(np.float16)
    o16, kc16, vc16 = fn(b.query, K, V, kf, vf, b.cum, b.past, b.block_table, None,
                         num_heads=H, kv_num_heads=Hkv)
    assert np.array_equal(o8, o16)
    assert np.array_equal((kc8.astype(np.float64) * 2.0 ** -5).astype(np.float16), kc16)
    assert np.array_equal((vc8.astype(np.float64) * 2.0 ** -5).astype(np.float16), vc16)


def check_Q3(fn):
    for b in (W.tiny(0, kv_quant="int8"),
              small(seed=33, head_size=4, packed=True, slot_mode="drop", drop_count=2,
                    dtype="bf16", kv_quant="int8")):
        o, kc, _ = call(fn, b, k_scale=b.k_scale, v_scale=b.v_scale)
        so, written = scalar.paged_attention_scalar(b.query, b.key, b.value, b.key_cache,
                                                    b.value_cache, b.cum, b.past,
                                                    b.block_table, b.slot_mapping,
                                                    b.num_heads, b.kv_num_heads, b.scale,
                                                    k_scale=b.k_scale, v_scale=b.v_scale)
        assert np.max(np.abs(o - np.array(so))) < 1e-12
        NB, bs, Hkv, D = kc.shape
        for slot, (krow, _) in written.items():
            assert kc.reshape(NB * bs, Hkv * D)[slot].tolist() == krow


def test_oracle_int8_pins():
    check_Q1(oracle.quantize_int8)
    check_Q2(oracle.paged_attention)
    check_Q3(oracle.paged_attention)


def _quant_trunc(x, s):
    return np.clip(oracle.values(x).astype(np.float32) / np.asarray(s, np.float32), -127, 127).astype(np.int8)


def _quant_half_up(x, s):
    q = oracle.values(x).astype(np.float32) / np.asarray(s, np.float32)
    return np.clip(np.floor(q + np.float32(0.5)), -127, 127).astype(np.int8)


def _quant_fp64(x, s):
    q = oracle.values(x) / np.asarray(s, np.float32).astype(np.float64)
    return np.clip(np.rint(q), -127, 127).astype(np.int8)


def _quant_clamp128(x, s):
    q = oracle.values(x).astype(np.float32) / np.asarray(s, np.float32)
    return np.clip(np.rint(q), -128, 127).astype(np.int8)


def _quant_times(x, s):
    q = oracle.values(x).astype(np.float32) * np.asarray(s, np.float32)
    return np.clip(np.rint(q), -127, 127).astype(np.int8)


@pytest.mark.parametrize("mutant", [_quant_trunc, _quant_half_up, _quant_fp64, _quant_clamp128,
                                    _quant_times], ids=lambda f: f.__name__)
def test_int8_pins_catch_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        check_Q1(mutant)


def _dequant_no_scale(codes, s):
    return codes.astype(np.float64)


def test_int8_pins_catch_dequant_mistake():
    saved = pa_mod.dequantize
    pa_mod.dequantize = _dequant_no_scale
    try:
        with pytest.raises(AssertionError):
            check_Q2(oracle.paged_attention)
    finally:
        pa_mod.dequantize = saved


# ------------------------------------------------------------------ INT4 caches

# INT4 per-channel caches (uint8 [NB, bs, Hkv, D/2], two codes per byte, the
# even element in bits 0-3).  Pins:
#   Q4  hand values of the code clamp(rint(x / s), -7, 7) (ties to even, both
#       clamps, never -8) and hand-packed bytes; every pair of codes in
#       [-8, 7] survives pack/unpack;
#   Q5  with power-of-two scales every code * scale is an fp16 value: the
#       INT4 oracle equals the fp16 oracle run on those values, bit for bit;
#   Q6  the scalar formulation (its own nibble decoding) agrees within 1e-12.

def check_Q4(quant, pack, unpack):
    s = np.full((1, 8), 0.25, dtype=np.float32)
    x = np.array([[1.0, 0.375, 0.625, 0.875, -0.625, 40.0, -40.0, -1.875]], dtype=np.float16)
    assert quant(x, s).tolist() == [[4, 2, 2, 4, -2, 7, -7, -7]]
    c = np.array([[1, -1, 7, -7, 0, 3, -2, 5]], dtype=np.int8)
    assert pack(c).tolist() == [[0xF1, 0x97, 0x30, 0x5E]]
    allc = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int8)
    assert np.array_equal(unpack(pack(allc)), allc)
    assert unpack(np.array([[0x8F]], dtype=np.uint8)).tolist() == [[-1, -8]]


def check_Q5(fn):
    rng = np.random.default_rng(35)
    H, Hkv, D, bs = 4, 2, 16, 4
    q_lens, past = [3, 1, 6], [5, 11, 0]
    b = W.make_batch(q_lens, past, num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs,
                     seed=35, kv_quant="int4")
    s = np.full((Hkv, D), 0.25, dtype=np.float32)
    K = (rng.integers(-7, 8, b.key.shape) * 0.25).astype(np.float16)
    V = (rng.integers(-7, 8, b.value.shape) * 0.25).astype(np.float16)
    o4, kc4, vc4 = fn(b.query, K, V, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                      None, num_heads=H, kv_num_heads=Hkv, k_scale=s, v_scale=s)
    # the same caches written out as fp16 values (nibble codes read by hand)
    def as_f16(cache):
        lo = (cache & 15).astype(np.int16)
        hi = (cache >> 4).astype(np.int16)
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        codes = np.stack([lo, hi], axis=-1).reshape(cache.shape[:-1] + (2 * cache.shape[-1],))
        return (codes * 0.25).astype(np.float16)
    o16, kc16, vc16 = fn(b.query, K, V, as_f16(b.key_cache), as_f16(b.value_cache), b.cum, b.past,
                         b.block_table, None, num_heads=H, kv_num_heads=Hkv)
    assert np.array_equal(o4, o16)
    assert np.array_equal(as_f16(kc4), kc16)
    assert np.array_equal(as_f16(vc4), vc16)


def check_Q6(fn):
    for b in (W.tiny(0, kv_quant="int4"),
              small(seed=37, head_size=4, packed=True, slot_mode="drop", drop_count=2,
                    dtype="bf16", kv_quant="int4")):
        o, kc, _ = call(fn, b, k_scale=b.k_scale, v_scale=b.v_scale)
        so, written = scalar.paged_attention_scalar(b.query, b.key, b.value, b.key_cache,
                                                    b.value_cache, b.cum, b.past,
                                                    b.block_table, b.slot_mapping,
                                                    b.num_heads, b.kv_num_heads, b.scale,
                                                    k_scale=b.k_scale, v_scale=b.v_scale)
        assert np.max(np.abs(o - np.array(so))) < 1e-12
        NB, bs, Hkv, Dh = kc.shape
        for slot, (krow, _) in written.items():
            row = kc.reshape(NB * bs, Hkv * Dh)[slot]
            got = [(v ^ 8) - 8 for byte in row.tolist() for v in (byte & 15, byte >> 4)]
            assert got == krow


def test_oracle_int4_pins():
    check_Q4(oracle.quantize_int4, oracle.pack_int4, oracle.unpack_int4)
    check_Q5(oracle.paged_attention)
    check_Q6(oracle.paged_attention)


def _quant4_clamp8(x, s):
    q = oracle.values(x).astype(np.float32) / np.asarray(s, np.float32)
    return np.clip(np.rint(q), -8, 7).astype(np.int8)


def _pack_high_first(codes):
    c = np.asarray(codes).astype(np.int16) & 0xF
    return ((c[..., 0::2] << 4) | c[..., 1::2]).astype(np.uint8)


def _unpack_unsigned(b):
    w = np.asarray(b, dtype=np.uint8).astype(np.int16)
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), dtype=np.int8)
    out[..., 0::2] = w & 0xF
    out[..., 1::2] = w >> 4
    return out


@pytest.mark.parametrize("which", ["clamp8", "high_first", "unsigned"])
def test_int4_pins_catch_planted_mistakes(which):
    quant, pack, unpack = oracle.quantize_int4, oracle.pack_int4, oracle.unpack_int4
    if which == "clamp8":
        quant = _quant4_clamp8
    elif which == "high_first":
        pack = _pack_high_first
    else:
        unpack = _unpack_unsigned
    with pytest.raises(AssertionError):
        check_Q4(quant, pack, unpack)


def test_int4_pins_catch_oracle_mistakes():
    # the oracle itself with a nibble-order or sign mistake fails Q5 or Q6
    for name, bad in (("pack_int4", _pack_high_first), ("unpack_int4", _unpack_unsigned)):
        saved = getattr(pa_mod, name)
        setattr(pa_mod, name, bad)
        try:
            with pytest.raises(AssertionError):
                check_Q5(oracle.paged_attention)
                check_Q6(oracle.paged_attention)
        finally:
            setattr(pa_mod, name, saved)


# ------------------------------------------------------------------ output gate

# sigmoid(gate) on the attention output.  Pins:
#   G1  gate 0 halves the output exactly (sigmoid(0) = 1/2);
#   G2  gates g and -g sum to the ungated output (sigmoid(g) + sigmoid(-g) = 1);
#   G3  the gated output equals the ungated one times scipy.special.expit of
#       the gate values;
#   G4  a gate of +20 leaves the output within 1e-8, -20 brings it within 1e-8
#       of zero; the lse is the ungated one in every case.

def check_G(fn):
    import scipy.special
    b = small(seed=41)
    o0, _, _, l0 = call(fn, b, with_lse=True)
    zero = np.zeros((b.num_tokens, b.num_heads * b.head_size), dtype=np.float16)
    o, _, _, l = call(fn, b, with_lse=True, gate=zero)
    assert np.array_equal(o, 0.5 * o0) and np.array_equal(l, l0)              # G1
    g = W.output_gate_input(b, 42)
    op, _, _ = call(fn, b, gate=g)
    om, _, _ = call(fn, b, gate=(-g.astype(np.float32)).astype(np.float16))
    assert np.max(np.abs(op + om - o0)) < 1e-12                               # G2
    assert np.max(np.abs(op - o0 * scipy.special.expit(g.astype(np.float64)))) < 1e-12  # G3
    big = np.full_like(zero, 20.0)
    oh, _, _ = call(fn, b, gate=big)
    ol, _, _ = call(fn, b, gate=-big)
    assert np.max(np.abs(oh - o0)) < 1e-8 * max(1.0, np.max(np.abs(o0)))     # G4
    assert np.max(np.abs(ol)) < 1e-8 * max(1.0, np.max(np.abs(o0)))
    gb = W.output_gate_input(small(seed=43, dtype="bf16"), 44)
    bb = small(seed=43, dtype="bf16")
    ob0, _, _ = call(fn, bb)
    ob, _, _ = call(fn, bb, gate=gb)
    assert np.max(np.abs(ob - ob0 * scipy.special.expit(oracle.values(gb)))) < 1e-12  # G3, bf16 gate


def test_oracle_gate_pins():
    check_G(oracle.paged_attention)


@pytest.mark.parametrize("which", ["sign", "exp", "tanh"])
def test_gate_pins_catch_planted_mistakes(which):
    wrong = {"sign": lambda out, gate: out / (1.0 + np.exp(oracle.values(gate))),
             "exp": lambda out, gate: out * np.exp(-oracle.values(gate)),
             "tanh": lambda out, gate: out * np.tanh(oracle.values(gate))}[which]
    saved = pa_mod.output_gate
    pa_mod.output_gate = wrong
    try:
        with pytest.raises(AssertionError):
            check_G(oracle.paged_attention)
    finally:
        pa_mod.output_gate = saved
