"""The library's host block-table builder: bit-exact against the reference
builder in oracle/ and the invariants its definition fixes (CPU only)."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_20_amd as p
    return p


@pytest.mark.parametrize("lens,pool,seed,maxp", [
    ([5, 17, 33], 10, 7, 3),
    ([1], 1, 0, 1),
    ([16, 16, 16, 0], 40, 2 ** 63 + 12345, 4),
    (list(np.random.default_rng(1).integers(1, 300, 50)), 2000, 99, 19),
])
def test_builder_matches_reference(pa, orc, lens, pool, seed, maxp):
    ours, slots = pa.attn_block_table_build(lens, 16, pool, seed, maxp, want_slots=True)
    ref, ref_slots = orc.build_block_table(lens, 16, pool, seed, maxp, want_slots=True)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(slots, ref_slots)


def test_builder_invariants(pa):
    rng = np.random.default_rng(2)
    lens = rng.integers(1, 500, 64)
    need = (lens + 15) // 16
    pool = int(need.sum()) + 64
    t = pa.attn_block_table_build(lens, 16, pool, 5, int(need.max()) + 2)
    used = []
    for s, n in enumerate(need):
        assert (t[s, :n] >= 0).all() and (t[s, :n] < pool).all()
        assert (t[s, n:] == -1).all()
        used.extend(t[s, :n].tolist())
    assert len(used) == len(set(used))  # pairwise distinct across sequences
    t2 = pa.attn_block_table_build(lens, 16, pool, 5, int(need.max()) + 2)
    np.testing.assert_array_equal(t, t2)  # deterministic per seed
    t3 = pa.attn_block_table_build(lens, 16, pool, 6, int(need.max()) + 2)
    assert not np.array_equal(t, t3)


def test_builder_errors(pa):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_block_table_build([100], 16, 3, 0, 8)  # pool too small
    assert e.value.code == pa.ATTN_E_RANGE
    assert "pool has 3" in pa.attn_last_error()
    with pytest.raises(pa.AttnError) as e:
        pa.attn_block_table_build([100], 16, 30, 0, 2)  # row too short
    assert e.value.code == pa.ATTN_E_RANGE
    assert "needs 7 pages" in pa.attn_last_error()
    pa.attn_block_table_build([100], 16, 30, 0, 8)
    assert pa.attn_last_error() == ""
