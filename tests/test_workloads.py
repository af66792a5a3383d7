"""The synthetic workloads have the structure the pages' decode shapes call for."""
import numpy as np

import oracle
import workloads as WL


def _sets(wl):
    return [set(int(t) for t in wl.sel[r] if 0 <= t < wl.seq_lens[r]) for r in range(wl.rows)]


def test_tiny_structure():
    wl = WL.make("tiny")
    assert wl.sel.shape == (2, 32) and wl.seq_lens.tolist() == [100, 173]
    assert sorted(wl.block_tables.ravel().tolist()) == list(range(32))
    for r in range(2):
        row = wl.sel[r]
        assert (row == -1).sum() == 6
        assert len(set(row[row >= 0].tolist())) == 23      # 3 repeats
        assert (row < wl.seq_lens[r]).all()


def test_glm_structure():
    wl = WL.make("glm", with_pool=False)
    assert wl.sel.shape == (32, 2048)
    for r in range(wl.rows):
        row = np.sort(wl.sel[r])
        assert len(set(row.tolist())) == 2048
        pools = row.reshape(-1, 4)
        assert (pools[:, 0] % 4 == 0).all() and (np.diff(pools, axis=1) == 1).all()
    assert sorted(wl.block_tables.ravel().tolist()) == list(range(4096))


def test_long_structure():
    wl = WL.make("long", with_pool=False)
    assert wl.sel.shape == (128, 2048) and wl.num_pages == 786432
    assert wl.pool_bytes == 24 * 2 ** 30
    assert len(np.unique(wl.block_tables)) == 128 * 2048     # no page shared
    row = wl.sel[0]
    assert len(set(row.tolist())) == 2048
    pool_ids, counts = np.unique(row // 4, return_counts=True)
    assert (counts == 4).sum() >= 358


def test_verify_overlap():
    wl = WL.make("verify", with_pool=False)
    sets = _sets(wl)
    for s in range(0, 64, 9):
        rows = sets[4 * s: 4 * s + 4]
        assert all(len(x) == 2048 for x in rows)
        inter = set.intersection(*rows)
        assert 0.58 <= len(inter) / 2048 <= 0.66
        base = wl.seq_lens[4 * s] - 1
        for j in range(4):
            assert wl.seq_lens[4 * s + j] == base + j + 1
            assert max(rows[j]) <= base + j
            assert np.array_equal(wl.block_tables[4 * s + j], wl.block_tables[4 * s])


def test_ragged_structure():
    wl = WL.make("ragged", with_pool=False)
    assert wl.seq_lens.min() >= 16 and wl.seq_lens.max() <= 65536
    for r in range(wl.rows):
        L = int(wl.seq_lens[r])
        row = wl.sel[r]
        uniq = oracle.select_row(row, L)
        if L < 2048:
            assert uniq.size == L and (row == -1).sum() == 2048 - L
        else:
            assert uniq.size == 1127 and (row == -1).sum() == 307


def test_pool_quantisation_saturates():
    rng = np.random.default_rng(0)
    pool = WL.host_pool(rng, 4, 64, 512, 2.0, 0.02)   # sigma/scale = 100: some |x| > 448
    assert not np.isin(pool, [0x7F, 0xFF]).any()      # never NaN
    assert np.isin(pool, [0x7E, 0xFE]).any()          # saturated to +-448


def test_generation_is_seeded():
    a = WL.make("tiny")
    b = WL.make("tiny")
    assert np.array_equal(a.sel, b.sel) and np.array_equal(a.pool, b.pool)
    c = WL.make("tiny", sel_seed=3)
    assert not np.array_equal(a.sel, c.sel)
    assert np.array_equal(a.q_bits, c.q_bits)
