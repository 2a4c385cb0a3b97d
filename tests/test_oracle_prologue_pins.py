"""Pins of the oracle's fused prologue (CPU only): Q/K OffsetRMSNorm, then
interleaved partial MRoPE, then the cast to the data type.

Source: "Add Qwen3.8 packed hybrid PagedAttention export for ORT GenAI Engine",
Per-layer behavior (Full attention, step 3: norm before RoPE, normalised once)
and Packed graph contract (position_ids INT64 [3, N]); "WS2 CP-Aware Attention
Contract", RoPE / Position Semantics and the Qwen3-8B example (theta,
rotary_dim, post-RoPE cached K, cast after RoPE).

Every check takes the implementation as an argument; test_planted_mistakes
runs them on copies with a typical mistake planted and requires each copy to
fail at least one check.  Pins:
  P1  rounding to the data type: fp16 == numpy's float16 conversion of the
      fp64 value; bf16 == torch's float32 -> bfloat16 conversion on values
      that are exact in float32; hand values (ties to even, a value just
      above a tie that a rounding through float32 would break to even)
  P2  OffsetRMSNorm closed forms: unit RMS with zero offsets and eps 0, the
      hand row [3, 4, 0, 0] -> [1.2, 1.6, 0, 0], the factor (1 + w), scale
      invariance
  P3  rotation: each pair keeps its length, position 0 is the identity,
      channels past rotary_dim only pass through, pair 0 turns by exactly
      the position (theta^0 = 1), and both pairings equal a complex product
      (x1 + i x2) e^(i angle) (numpy complex arithmetic)
  P4  text tokens (three equal position rows): q'.k' depends only on the
      position difference
  P5  MRoPE section maps: hand-listed interleaved maps for (11, 11, 10) and
      (22, 21, 21), a contiguous map, and a position in one component turns
      exactly the pairs of that component
  P6  the scalar formulation (oracle/scalar.py) agrees within 1e-12, and
      bit for bit after rounding
  P7  in the operator: without a prologue nothing changes; with one, the
      result equals the plain operator applied to the prologue's rows
"""
import importlib
import types

import numpy as np
import pytest
import torch

import oracle
OP = importlib.import_module("oracle.paged_attention")  # the module (the package re-exports a function of that name)
from oracle import scalar
import workloads as W


def impl(**patch):
    ns = types.SimpleNamespace(round_to_format=OP.round_to_format, to_dtype_bits=OP.to_dtype_bits,
                               offset_rms_norm=OP.offset_rms_norm,
                               mrope_components=OP.mrope_components,
                               rotary_angles=OP.rotary_angles, apply_rotary=OP.apply_rotary,
                               qk_prologue=OP.qk_prologue)
    for k, v in patch.items():
        setattr(ns, k, v)
    return ns


# ------------------------------------------------------------------ P1 rounding

def check_P1(m):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-12, 12, 4000))
    got = m.to_dtype_bits(x, "f16")
    assert np.array_equal(got.view(np.uint16), x.astype(np.float16).view(np.uint16))
    x32 = (rng.standard_normal(4000) * 3).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(m.to_dtype_bits(x32, "bf16"), ref)
    # hand values: ties to even, and a value just above a bf16 tie (exact in
    # fp64, not in fp32: rounding through fp32 would make it a tie)
    hand = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 2.0 ** -8 + 2.0 ** -30)])
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -(1 + 2.0 ** -7)])
    got = m.to_dtype_bits(hand, "bf16")
    assert np.array_equal(((got.astype(np.uint32)) << 16).view(np.float32).astype(np.float64), want)
    h16 = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2048 + 1.0, 65504.0])
    assert np.array_equal(m.to_dtype_bits(h16, "f16").astype(np.float64),
                          np.array([1.0, 1 + 2.0 ** -9, 2048.0, 65504.0]))


# ------------------------------------------------------------------ P2 OffsetRMSNorm

def check_P2(m):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 64)) * 3
    y = m.offset_rms_norm(x, np.zeros(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-12)
    y = m.offset_rms_norm(np.array([3.0, 4.0, 0.0, 0.0]), np.zeros(4), 0.0)
    assert np.allclose(y, [1.2, 1.6, 0.0, 0.0], rtol=0, atol=1e-15)
    y = m.offset_rms_norm(np.array([3.0, 4.0, 0.0, 0.0]), np.array([1.0, -0.5, 2.0, 0.0]), 0.0)
    assert np.allclose(y, [2.4, 0.8, 0.0, 0.0], rtol=0, atol=1e-15)
    w = rng.standard_normal(64) * 0.1
    assert np.allclose(m.offset_rms_norm(x * 7.5, w, 0.0), m.offset_rms_norm(x, w, 0.0), rtol=1e-12, atol=1e-12)
    # eps inside the root: mean square 1 with eps 3 divides by 2
    y = m.offset_rms_norm(np.ones(16), np.zeros(16), 3.0)
    assert np.allclose(y, 0.5, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ P3 rotation

def check_P3(m):
    rng = np.random.default_rng(3)
    N, Hh, D = 6, 3, 64
    x = rng.standard_normal((N, Hh, D))
    for rd in (16, 32, 64):
        for adjacent in (False, True):
            ang = rng.uniform(-50, 50, (N, rd // 2))
            y = m.apply_rotary(x, ang, rd, adjacent)
            if adjacent:
                i1, i2 = np.arange(0, rd, 2), np.arange(1, rd, 2)
            else:
                i1, i2 = np.arange(rd // 2), np.arange(rd // 2, rd)
            # complex product (numpy complex arithmetic)
            z = (x[:, :, i1] + 1j * x[:, :, i2]) * np.exp(1j * ang)[:, None, :]
            assert np.allclose(y[:, :, i1], z.real, rtol=0, atol=1e-12)
            assert np.allclose(y[:, :, i2], z.imag, rtol=0, atol=1e-12)
            # lengths of the pairs, untouched channels
            assert np.allclose(y[:, :, i1] ** 2 + y[:, :, i2] ** 2, x[:, :, i1] ** 2 + x[:, :, i2] ** 2,
                               rtol=1e-12, atol=1e-12)
            assert np.array_equal(y[:, :, rd:], x[:, :, rd:])
            # position 0 is the identity
            assert np.array_equal(m.apply_rotary(x, np.zeros((N, rd // 2)), rd, adjacent), x)
    # pair 0 turns by the position itself; pair i by position * theta^(-2i/rd)
    pos = np.array([[5, 0, 1234], [5, 0, 1234], [5, 0, 1234]])
    comps = m.mrope_components(32, (6, 5, 5))
    ang = m.rotary_angles(pos, 32, 1.0e6, comps)
    assert np.array_equal(ang[:, 0], [5.0, 0.0, 1234.0])
    assert np.allclose(ang[2, 7], 1234.0 * 1.0e6 ** (-14.0 / 32), rtol=1e-15, atol=0)
    assert np.allclose(ang[2, 15], 1234.0 * 10.0 ** (-6 * 30 / 32), rtol=1e-14, atol=0)


# ------------------------------------------------------------------ P4 relative positions

def check_P4(m):
    rng = np.random.default_rng(4)
    D, rd = 128, 64
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    comps = m.mrope_components(rd, (11, 11, 10))

    def dot(pq, pk, shift):
        a = m.apply_rotary(q, m.rotary_angles(np.full((3, 1), pq + shift), rd, 1.0e6, comps), rd, False)
        b = m.apply_rotary(k, m.rotary_angles(np.full((3, 1), pk + shift), rd, 1.0e6, comps), rd, False)
        return float(np.sum(a * b))

    base = dot(700, 650, 0)
    for shift in (1, 37, 4096, 15000):
        assert abs(dot(700, 650, shift) - base) <= 1e-9 * (1 + abs(base))
    assert abs(dot(701, 650, 0) - base) > 1e-6  # a different difference changes it


# ------------------------------------------------------------------ P5 MRoPE sections

def check_P5(m):
    got = m.mrope_components(64, (11, 11, 10))
    want = [i % 3 for i in range(30)] + [0, 1]
    assert list(got) == want
    got = m.mrope_components(128, (22, 21, 21))
    assert list(got) == [i % 3 for i in range(63)] + [0]
    got = m.mrope_components(128, (24, 20, 20))
    assert list(got) == [i % 3 for i in range(60)] + [0, 0, 0, 0]
    got = m.mrope_components(16, (4, 2, 2), interleaved=False)
    assert list(got) == [0, 0, 0, 0, 1, 1, 2, 2]
    # a position in one component turns exactly that component's pairs
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 64))
    rd = 64
    comps = m.mrope_components(rd, (11, 11, 10))
    for c in range(3):
        pos = np.zeros((3, 1), dtype=np.int64)
        pos[c, 0] = 321
        y = m.apply_rotary(x, m.rotary_angles(pos, rd, 1.0e6, comps), rd, False)
        moved = np.any(np.abs(y[0, :, :rd // 2] - x[0, :, :rd // 2]) > 1e-12, axis=0)
        assert np.array_equal(moved, comps == c)


# ------------------------------------------------------------------ P6 scalar formulation

def prologue_case(dtype="f16", D=64, rd=32, adjacent=False, interleaved=True, seed=6):
    rng = np.random.default_rng(seed)
    N, H, Hkv = 5, 4, 2
    normal = W.normal_bf16 if dtype == "bf16" else W.normal_f16
    Q, K = normal(rng, (N, H, D)), normal(rng, (N, Hkv, D))
    pos = np.stack([np.arange(N) + 90, rng.integers(0, 40, N), rng.integers(0, 40, N)]).astype(np.int64)
    half = rd // 2
    sections = (half - 2 * (half // 3), half // 3, half // 3)
    kw = dict(position_ids=pos, rotary_dim=rd, theta=1.0e6, sections=sections,
              interleaved=interleaved, adjacent=adjacent,
              q_norm_weight=(rng.standard_normal(D) * 0.2).astype(np.float32),
              k_norm_weight=(rng.standard_normal(D) * 0.2).astype(np.float32), eps=1e-6)
    return Q, K, kw


def check_P6(m):
    for dtype, adjacent, interleaved in (("f16", False, True), ("bf16", True, True), ("f16", False, False)):
        Q, K, kw = prologue_case(dtype, adjacent=adjacent, interleaved=interleaved)
        q64, k64 = m.qk_prologue(Q, K, rounded=False, **kw)
        qs, ks = scalar.qk_prologue_scalar(oracle.values(Q).tolist(), oracle.values(K).tolist(), Q.shape[-1], **kw)
        assert np.allclose(q64, np.array(qs), rtol=0, atol=1e-12)
        assert np.allclose(k64, np.array(ks), rtol=0, atol=1e-12)
        qr, kr = m.qk_prologue(Q, K, **kw)
        assert np.array_equal(qr.view(np.uint16), OP.to_dtype_bits(np.array(qs), dtype).view(np.uint16))
        assert np.array_equal(kr.view(np.uint16), OP.to_dtype_bits(np.array(ks), dtype).view(np.uint16))


# ------------------------------------------------------------------ P7 in the operator

def check_P7(m, operator=None):
    operator = operator or oracle.paged_attention
    b = W.make_batch([1, 5, 3], [9, 20, 0], num_heads=4, kv_num_heads=2, head_size=64, block_size=16,
                     seed=7, packed=True, slot_mode="drop", drop_count=1, name="prologue_op")
    Q, K, V, D, _ = oracle.resolve_call(b.query, None, None, 4, 2, 0.0)
    _, _, kw = prologue_case(D=64, rd=32)
    # text tokens: the three position rows are the token's logical position
    pos = np.concatenate([b.past[i] + np.arange(b.cum[i + 1] - b.cum[i]) for i in range(b.batch_size)])
    kw["position_ids"] = np.stack([pos] * 3).astype(np.int64)
    base = dict(num_heads=4, kv_num_heads=2)
    plain = operator(b.query, None, None, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                     b.slot_mapping, **base)
    none = operator(b.query, None, None, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                    b.slot_mapping, prologue=None, **base)
    assert np.array_equal(plain[0], none[0], equal_nan=True)
    got = operator(b.query, None, None, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                   b.slot_mapping, prologue=kw, **base)
    q2, k2 = m.qk_prologue(Q, K, **kw)
    N = b.num_tokens
    packed2 = np.concatenate([q2.reshape(N, -1), k2.reshape(N, -1), V.reshape(N, -1)], axis=1)
    want = operator(packed2, None, None, b.key_cache, b.value_cache, b.cum, b.past, b.block_table,
                    b.slot_mapping, **base)
    assert np.array_equal(got[0], want[0], equal_nan=True)
    assert np.array_equal(got[1].view(np.uint16), want[1].view(np.uint16))
    assert np.array_equal(got[2].view(np.uint16), want[2].view(np.uint16))


CHECKS = [check_P1, check_P2, check_P3, check_P4, check_P5, check_P6, check_P7]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_prologue_pin(check):
    check(impl())


# ------------------------------------------------------------------ planted mistakes

def _rot_sign_flipped(x, angles, rd, adjacent=False):
    return OP.apply_rotary(x, -angles, rd, adjacent)


def _rot_pairs_swapped(x, angles, rd, adjacent=False):
    return OP.apply_rotary(x, angles, rd, not adjacent)


def _norm_without_offset(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def _norm_eps_outside(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * (1.0 + np.asarray(w))


def _angles_head_size_exponent(position_ids, rd, theta, comps):
    half = rd // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / (2 * rd))  # as if the exponent used the head size
    pos = np.asarray(position_ids)[comps, :].T.astype(np.float64)
    return pos * inv[None, :]


def _angles_first_row_only(position_ids, rd, theta, comps):
    return OP.rotary_angles(position_ids, rd, theta, np.zeros_like(comps))


def _sections_contiguous(rd, sections, interleaved=True):
    return OP.mrope_components(rd, sections, interleaved=False)


def _round_through_f32(x, dtype):
    if dtype == "bf16":
        return W.round_bf16(np.asarray(x, dtype=np.float32))
    return OP.to_dtype_bits(x, dtype)


def _prologue_rope_before_norm(Q, K, **kw):
    kw = dict(kw)
    rounded = kw.pop("rounded", True)
    qn, kn = kw.pop("q_norm_weight", None), kw.pop("k_norm_weight", None)
    eps = kw.pop("eps", 1e-6)
    q, k = OP.qk_prologue(Q, K, rounded=False, **kw)
    if qn is not None:
        q = OP.offset_rms_norm(q, qn, eps)
    if kn is not None:
        k = OP.offset_rms_norm(k, kn, eps)
    if not rounded:
        return q, k
    dtype = "bf16" if np.asarray(Q).dtype == np.uint16 else "f16"
    return OP.to_dtype_bits(q, dtype), OP.to_dtype_bits(k, dtype)


def _prologue_k_untouched(Q, K, **kw):
    q, _ = OP.qk_prologue(Q, K, **kw)
    if kw.get("rounded", True):
        return q, np.asarray(K)
    return q, oracle.values(K)


MUTANTS = {
    "rotation sign": dict(apply_rotary=_rot_sign_flipped),
    "pairing swapped": dict(apply_rotary=_rot_pairs_swapped),
    "norm weight without the offset": dict(offset_rms_norm=_norm_without_offset),
    "eps outside the root": dict(offset_rms_norm=_norm_eps_outside),
    "frequency exponent over twice the rotary dim": dict(rotary_angles=_angles_head_size_exponent),
    "every pair on the first position row": dict(rotary_angles=_angles_first_row_only),
    "contiguous sections": dict(mrope_components=_sections_contiguous),
    "bf16 rounded through fp32": dict(to_dtype_bits=_round_through_f32),
    "RoPE before the norm": dict(qk_prologue=_prologue_rope_before_norm),
    "K not transformed": dict(qk_prologue=_prologue_k_untouched),
}


def _mutant_impl(patch):
    """A copy of the prologue whose pieces call the patched ones (the whole
    qk_prologue is rebuilt from the patched parts unless it is patched itself)."""
    m = impl(**patch)
    if "qk_prologue" not in patch:
        def qk(Q, K, *, position_ids=None, rotary_dim=0, theta=1.0e6, sections=None, interleaved=True,
               adjacent=False, q_norm_weight=None, k_norm_weight=None, eps=1e-6, rounded=True):
            dtype = "bf16" if np.asarray(Q).dtype == np.uint16 else "f16"
            q, k = oracle.values(Q), oracle.values(K)
            if q_norm_weight is not None:
                q = m.offset_rms_norm(q, q_norm_weight, eps)
            if k_norm_weight is not None:
                k = m.offset_rms_norm(k, k_norm_weight, eps)
            if rotary_dim:
                ang = m.rotary_angles(position_ids, rotary_dim, theta,
                                      m.mrope_components(rotary_dim, sections, interleaved))
                q = m.apply_rotary(q, ang, rotary_dim, adjacent)
                k = m.apply_rotary(k, ang, rotary_dim, adjacent)
            if not rounded:
                return q, k
            return m.to_dtype_bits(q, dtype), m.to_dtype_bits(k, dtype)
        m.qk_prologue = qk
    return m


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name):
    m = _mutant_impl(MUTANTS[name])
    caught = []
    for check in CHECKS:
        try:
            if check is check_P7:
                def op(*a, prologue=None, **kw):
                    return oracle.paged_attention(*a, **kw) if prologue is None else \
                        _operator_with(m, *a, prologue=prologue, **kw)
                check(m, op)
            else:
                check(m)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"planted mistake '{name}' passed every pin"


def _operator_with(m, query, key, value, kc, vc, cum, past, table, sm, *, prologue, num_heads, kv_num_heads,
                   **kw):
    """The operator with the mutant's prologue: transform, then the plain operator."""
    Q, K, V, D, _ = oracle.resolve_call(query, key, value, num_heads, kv_num_heads, 0.0)
    q2, k2 = m.qk_prologue(Q, K, **prologue)
    N = Q.shape[0]
    if key is None:
        packed = np.concatenate([q2.reshape(N, -1), k2.reshape(N, -1), V.reshape(N, -1)], axis=1)
        return oracle.paged_attention(packed, None, None, kc, vc, cum, past, table, sm,
                                      num_heads=num_heads, kv_num_heads=kv_num_heads, **kw)
    return oracle.paged_attention(q2.reshape(N, -1), k2.reshape(N, -1), value, kc, vc, cum, past, table, sm,
                                  num_heads=num_heads, kv_num_heads=kv_num_heads, **kw)
