"""Pins for the integer cache model.

What fixes it: a crop keeps exactly the accepted prefix and the cache grows by
the accepted rows ("DFlash KV Injection Walkthrough" Step 7;
"DFlash源码导读二 ..." section 4); pages come from a fixed pool through a page
table and return to a free list ("KV Cache + Speculative Decoding 面试 Cheat
Sheet" 5.2, 6.2).  Independent checks: the paged and the contiguous layouts,
whose index arithmetic differs, must agree on every logical row; a plain list
of appended rows per sequence must agree with both; page accounting must obey
closed forms.
"""
import numpy as np
import pytest

from oracle.cache_model import CacheError, CacheModel, ERR_CAPACITY, ERR_RANGE


def _random_ops(seed, n_seqs, steps, max_rows):
    rng = np.random.default_rng(seed)
    ops = []
    for _ in range(steps):
        if rng.random() < 0.6:
            ops.append(("append", rng.integers(0, max_rows + 1, size=n_seqs)))
        else:
            ops.append(("crop", rng.random(n_seqs)))
    return ops


@pytest.mark.parametrize("seed", range(6))
def test_paged_contiguous_and_list_agree(seed):
    n_seqs, n_kv, d_h, ps = 3, 2, 4, 8
    paged = CacheModel(n_seqs, n_kv, d_h, ps, capacity=64, max_pages_per_seq=16)
    contig = CacheModel(n_seqs, n_kv, d_h, 0, capacity=128)
    lists = [[] for _ in range(n_seqs)]
    rng = np.random.default_rng(1000 + seed)
    for kind, arg in _random_ops(seed, n_seqs, 40, 11):
        if kind == "append":
            n = [int(a) for a in arg]
            if any(len(lists[s]) + n[s] > 128 for s in range(n_seqs)):
                continue
            cu = np.concatenate([[0], np.cumsum(n)])
            k = rng.integers(0, 2 ** 16, size=(cu[-1], n_kv, d_h), dtype=np.uint16)
            v = rng.integers(0, 2 ** 16, size=(cu[-1], n_kv, d_h), dtype=np.uint16)
            paged.append(cu, k, v)
            contig.append(cu, k, v)
            for s in range(n_seqs):
                lists[s] += [(k[j], v[j]) for j in range(cu[s], cu[s + 1])]
        else:
            new = [int(f * len(lists[s])) for s, f in enumerate(arg)]
            old_pages = paged.pages_in_use()
            old_len = list(paged.len)
            paged.crop(new)
            contig.crop(new)
            for s in range(n_seqs):
                del lists[s][new[s]:]
            freed = sum(-(-o // ps) - -(-nl // ps) for o, nl in zip(old_len, new))
            assert old_pages - paged.pages_in_use() == freed
        assert paged.pages_in_use() + len(paged.free) == paged.capacity
        for s in range(n_seqs):
            assert len(paged.pages[s]) == -(-paged.len[s] // ps)
            kp, vp = paged.rows(s)
            kc, vc = contig.rows(s)
            assert np.array_equal(kp, kc) and np.array_equal(vp, vc)
            if lists[s]:
                kl = np.stack([r[0] for r in lists[s]], axis=1)
                vl = np.stack([r[1] for r in lists[s]], axis=1)
                assert np.array_equal(kp, kl) and np.array_equal(vp, vl)
            else:
                assert kp.shape[1] == 0
        used = [pg for pl in paged.pages for pg in pl]
        assert len(used) == len(set(used))


def test_lowest_free_page_first_and_reuse_after_crop():
    m = CacheModel(2, 1, 2, 4, capacity=8, max_pages_per_seq=8)
    z = lambda n: np.zeros((n, 1, 2), dtype=np.uint16)  # noqa: E731
    m.append([0, 5, 9], z(9), z(9))       # seq0: 5 rows -> pages 0,1 ; seq1: 4 rows -> page 2
    assert m.block_table() == [[0, 1], [2]]
    m.crop([3, 4])                         # seq0 back to 1 page: page 1 freed
    assert m.block_table() == [[0], [2]] and m.free == {1, 3, 4, 5, 6, 7}
    m.append([0, 0, 1], z(1), z(1))        # seq1 grows to 5 rows: takes page 1 (lowest free)
    assert m.block_table() == [[0], [2, 1]]


def test_errors_change_nothing():
    m = CacheModel(2, 1, 2, 4, capacity=3, max_pages_per_seq=2)
    z = lambda n: np.ones((n, 1, 2), dtype=np.uint16)  # noqa: E731
    m.append([0, 4, 6], z(6), z(6))
    snap = (list(m.len), m.block_table(), set(m.free), m.K.copy(), m.V.copy())
    with pytest.raises(CacheError) as e:
        m.append([0, 5, 5], z(5), z(5))    # seq0 would need 3 pages > max 2
    assert e.value.code == ERR_CAPACITY
    with pytest.raises(CacheError) as e:
        m.append([0, 4, 8], z(8), z(8))    # needs 2 new pages, 1 free
    assert e.value.code == ERR_CAPACITY
    with pytest.raises(CacheError) as e:
        m.crop([5, 0])                     # beyond the current length
    assert e.value.code == ERR_RANGE
    assert (list(m.len), m.block_table(), set(m.free)) == snap[:3]
    assert np.array_equal(m.K, snap[3]) and np.array_equal(m.V, snap[4])
    c = CacheModel(1, 1, 2, 0, capacity=4)
    with pytest.raises(CacheError) as e:
        c.append([0, 5], z(5), z(5))
    assert e.value.code == ERR_CAPACITY and c.len == [0]


def test_walkthrough_growth():
    """Round 1 writes 3 context + 4 block rows, the crop keeps positions 0-2;
    round 2 writes 3 + 4 more and the crop keeps positions 0-5."""
    m = CacheModel(1, 8, 64, 0, capacity=64)
    for rnd, keep in ((1, 3), (2, 6)):
        rows = np.full((7, 8, 64), rnd, dtype=np.uint16)
        m.append([0, 7], rows, rows)
        m.crop([keep])
        assert m.len == [keep]
    k, _ = m.rows(0)
    assert list(k[0, :, 0]) == [1, 1, 1, 2, 2, 2]


@pytest.mark.parametrize("seed", range(4))
def test_ring_holds_the_last_rows(seed):
    """A ring keeps the rows of positions [max(0, hw - capacity), len): they
    must equal the plain per-sequence list of appended rows there (the list
    has no slots, so a wrong slot or a stale overwrite shows up)."""
    n_seqs, n_kv, d_h, cap = 2, 2, 3, 16
    ring = CacheModel(n_seqs, n_kv, d_h, 0, capacity=cap, ring=True)
    lists = [[] for _ in range(n_seqs)]
    rng = np.random.default_rng(2000 + seed)
    for kind, arg in _random_ops(seed, n_seqs, 60, 9):
        if kind == "append":
            n = [int(a) for a in arg]
            cu = np.concatenate([[0], np.cumsum(n)])
            k = rng.integers(0, 2 ** 16, size=(cu[-1], n_kv, d_h), dtype=np.uint16)
            v = rng.integers(0, 2 ** 16, size=(cu[-1], n_kv, d_h), dtype=np.uint16)
            ring.append(cu, k, v)
            for s in range(n_seqs):
                lists[s] += [(k[j], v[j]) for j in range(cu[s], cu[s + 1])]
        else:
            new = [int(f * len(lists[s])) for s, f in enumerate(arg)]
            ring.crop(new)
            for s in range(n_seqs):
                del lists[s][new[s]:]
        for s in range(n_seqs):
            assert ring.len[s] == len(lists[s])
            lo, kr, vr = ring.held(s)
            assert lo == max(0, ring.hw[s] - cap)
            for pos in range(lo, ring.len[s]):
                assert np.array_equal(kr[:, pos - lo], lists[s][pos][0])
                assert np.array_equal(vr[:, pos - lo], lists[s][pos][1])


def test_ring_wider_than_every_length_is_the_contiguous_cache():
    rng = np.random.default_rng(7)
    ring = CacheModel(2, 1, 4, 0, capacity=64, ring=True)
    flat = CacheModel(2, 1, 4, 0, capacity=64)
    for _ in range(30):
        n = rng.integers(0, 6, size=2)
        if all(flat.len[s] + n[s] <= 64 for s in range(2)):
            cu = np.concatenate([[0], np.cumsum(n)])
            k = rng.integers(0, 2 ** 16, size=(cu[-1], 1, 4), dtype=np.uint16)
            for m in (ring, flat):
                m.append(cu, k, k)
        else:
            new = [x // 2 for x in flat.len]
            for m in (ring, flat):
                m.crop(new)
        assert np.array_equal(ring.K, flat.K) and np.array_equal(ring.V, flat.V)


def test_ring_round_cycle_and_errors():
    """Rounds that append n + B rows and crop the B block rows run forever on
    a ring of window + B - 1 slots; a crop far back makes the next window reach
    rows the ring no longer holds; the call-level limits."""
    W, B, cap = 12, 4, 16                      # cap >= W + B - 1 = 15
    m = CacheModel(1, 1, 2, 0, capacity=cap, ring=True)
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(0, 6))
        assert m.layer_call_status([n], B, W) == 0
        z = np.zeros((n + B, 1, 2), dtype=np.uint16)
        m.append([0, n + B], z, z)
        m.crop([m.len[0] - B])
    assert m.len[0] > 4 * cap
    assert m.layer_call_status([0], B, 0) == -2          # full attention on a ring
    assert m.layer_call_status([0], B, cap) == ERR_CAPACITY
    assert m.layer_call_status([cap - B + 1], B, W) == ERR_CAPACITY
    m.crop([m.len[0] - 8])                                # the window now starts below hw - cap
    assert m.layer_call_status([0], B, W) == ERR_RANGE
    with pytest.raises(CacheError) as e:
        m.append([0, cap + 1], np.zeros((cap + 1, 1, 2), np.uint16), np.zeros((cap + 1, 1, 2), np.uint16))
    assert e.value.code == ERR_CAPACITY
