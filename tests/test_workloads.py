"""Checks of the seeded input generators (CPU only).

Page tables must obey the KVCacheSpec rules of "WS2 CP-Aware Attention
Contract" (Mode-Specific Metadata): trailing padding, ceil(kv_len/page_size)
active pages, no page repeated inside a sequence, sharing only as a fully
populated read-only prefix with the same leading ids.  The named workloads
must have the shapes their descriptions state.
"""
import numpy as np
import pytest

import workloads as W


def check_table(b: W.Batch, shared_ok=False):
    bs = b.block_size
    owners = {}
    for i in range(b.batch_size):
        L = int(b.kv_lens[i])
        n = W.pages_needed(L, bs)
        row = b.block_table[i]
        active = row[:n]
        assert np.all((active >= 0) & (active < b.num_blocks))
        assert len(set(active.tolist())) == n, "page repeated inside a sequence"
        if b.name != "tiny":
            assert np.all(row[n:] == -1), "padding must be trailing -1"
        for j, pg in enumerate(active.tolist()):
            owners.setdefault(pg, []).append((i, j))
    p = b.past.astype(np.int64)
    for pg, users in owners.items():
        if len(users) == 1:
            continue
        assert shared_ok, "page shared without a declared prefix"
        js = {j for _, j in users}
        assert len(js) == 1, "shared page at different logical positions"
        j = js.pop()
        for i, _ in users:
            # fully populated and never written: lies entirely below past
            assert (j + 1) * bs <= p[i]
            # same leading ids as every other user
            for i2, _ in users:
                assert np.array_equal(b.block_table[i, :j + 1], b.block_table[i2, :j + 1])


def test_tiny_shape():
    b = W.tiny(0)
    assert b.cum.tolist() == [0, 3, 4] and b.past.tolist() == [5, 20]
    assert b.key_cache.shape == (8, 16, 2, 64) and b.query.shape == (4, 256)
    assert sorted(b.block_table.reshape(-1).tolist()) == list(range(8))
    check_table(b)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_shape(seed):
    b = W.pure_decode(seed)
    assert b.batch_size == 64 and b.num_tokens == 64
    assert b.past.min() >= 512 and b.past.max() <= 4096
    assert b.num_blocks == sum(W.pages_needed(L, 16) for L in b.kv_lens)
    check_table(b)


def test_mixed_shape():
    b = W.mixed(0)
    assert sorted(b.q_lens.tolist()) == [1] * 8 + [512] * 8
    assert b.num_tokens == 8 + 8 * 512 and b.block_size == 256
    check_table(b)


def test_long_prefill_shape():
    b = W.long_prefill(0)
    assert b.q_lens.tolist() == [2048] and b.past.tolist() == [2048]
    assert b.num_heads == 16 and b.kv_num_heads == 4 and b.num_blocks == 16
    check_table(b)


@pytest.mark.parametrize("seed", [0, 1])
def test_serving_shape(seed):
    b = W.serving(seed, meta_only=True)
    assert b.packed and b.query.shape == (4320, (32 + 16) * 128)
    assert b.num_blocks == 4096 and b.block_table.shape == (256, 65)
    sm = b.slot_mapping
    assert np.count_nonzero(sm == -1) == 216
    live = sm[sm >= 0]
    assert len(set(live.tolist())) == live.size, "two tokens share a slot"
    check_table(b, shared_ok=True)
    # every page a new token lands in is exclusive to its sequence
    users = {}
    for i in range(b.batch_size):
        for pg in b.block_table[i, :W.pages_needed(int(b.kv_lens[i]), 256)].tolist():
            users[pg] = users.get(pg, 0) + 1
    for s in live.tolist():
        assert users[s // 256] == 1


def test_allocator_slots_walk():
    # the allocator's enumeration agrees with placing tokens page by page
    b = W.make_batch([3, 0, 9], [14, 2, 0], num_heads=2, kv_num_heads=1, head_size=4,
                     block_size=4, seed=5, slot_mode="derived")
    expect = []
    for i in range(3):
        pages = b.block_table[i]
        for t in range(int(b.q_lens[i])):
            pos = int(b.past[i]) + t
            page, off = 0, pos
            while off >= 4:
                page, off = page + 1, off - 4
            expect.append(int(pages[page]) * 4 + off)
    assert b.slot_mapping.tolist() == expect


def test_seed_reproducible():
    a, b = W.mixed(3), W.mixed(3)
    assert np.array_equal(a.query.view(np.uint16), b.query.view(np.uint16))
    assert np.array_equal(a.block_table, b.block_table)
