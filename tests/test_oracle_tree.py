"""Pins of the oracle's tree-round view (CPU).

``oracle.tree_view`` lays row r's branch -- the context, then the round rows
its mask names -- out as a plain sequence.  What its definition fixes, and
what is checked here without calling it twice:
  * bf16, and fp8 rounds inside one page: the view is the byte gather of the
    branch positions (numpy fancy indexing), with each page's stored scale;
  * a chain mask gives the cache itself, byte for byte and scale for scale;
  * fp8 rows that move down into the page before theirs keep their value to
    within half an E4M3 step at the view page's scale (codes decoded with
    torch's float8_e4m3fn, a library routine), the other tokens keep their
    codes unless the scale grew, and a grown scale is the least power-of-two
    multiple of the stored one that holds the moved values.
"""
import numpy as np
import pytest
import torch

from test_oracle_pins import PAGE, bf16_round

KV_BF16, KV_FP8 = 0, 1


def e4m3_value(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def to_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_cache(orc, rng, lens, Hk, d, fp8, spare=2):
    need = [-(-c // PAGE) for c in lens]
    n_pages = sum(need) + spare
    max_pages = max(need) + 1
    perm = rng.permutation(n_pages)
    table = np.full((len(lens), max_pages), -1, np.int32)
    el = np.uint8 if fp8 else np.uint16
    kp = np.zeros((n_pages, Hk, PAGE, d), el)
    vp = np.zeros_like(kp)
    ks = np.ones((n_pages, Hk), np.float32) if fp8 else None
    vs = np.ones((n_pages, Hk), np.float32) if fp8 else None
    at = 0
    for s, (c, n) in enumerate(zip(lens, need)):
        table[s, :n] = perm[at:at + n]
        at += n
        k = to_bits(bf16_round(rng.standard_normal((c, Hk, d))))
        v = to_bits(bf16_round(rng.standard_normal((c, Hk, d))))
        t = np.arange(c)
        slots = (table[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32)
        orc.kv_append(k, v, slots, kp, vp, ks, vs, n_head_kv=Hk, head_dim=d, page_size=PAGE,
                      kv_dtype=KV_FP8 if fp8 else KV_BF16)
    return kp, vp, ks, vs, table


def random_masks(rng, R, chain=False):
    m = []
    for r in range(R):
        parent = r - 1 if chain else int(rng.integers(-1, r))
        m.append((1 << r) | (m[parent] if parent >= 0 else 0))
    return m


def branch(C, R, mask):
    C0 = C - R
    return list(range(C0)) + [C0 + j for j in range(R) if mask >> j & 1]


def view(orc, cache, table_row, C, R, mask, r, Hk, d, fp8):
    kp, vp, ks, vs, _ = cache
    return orc.tree_view(kp, vp, ks, vs, table_row, C, R, mask, r, n_head_kv=Hk, head_dim=d,
                         page_size=PAGE, kv_dtype=KV_FP8 if fp8 else KV_BF16)


@pytest.mark.parametrize("fp8", [False, True])
def test_view_is_the_gather_inside_one_page(orc, fp8):
    rng = np.random.default_rng(41)
    Hk, d, R = 2, 64, 8
    lens = [8, 40, 528, 1000, 333]  # C0 % 16 = 0, 0, 8, 0, 5
    cache = make_cache(orc, rng, lens, Hk, d, fp8)
    kp, vp, ks, vs, table = cache
    for s, C in enumerate(lens):
        assert (C - R) % PAGE + R <= PAGE
        for r, m in enumerate(random_masks(rng, R)):
            k2, v2, ks2, vs2, L = view(orc, cache, table[s], C, R, m, r, Hk, d, fp8)
            pos = np.array(branch(C, R, m))
            assert L == len(pos)
            sp, so = table[s, pos // PAGE], pos % PAGE
            i = np.arange(L)
            np.testing.assert_array_equal(k2[i // PAGE, :, i % PAGE], kp[sp, :, so])
            np.testing.assert_array_equal(v2[i // PAGE, :, i % PAGE], vp[sp, :, so])
            tail = np.arange(L, k2.shape[0] * PAGE)
            assert not k2[tail // PAGE, :, tail % PAGE].any()
            if fp8:
                first = sp[np.arange(0, L, PAGE)]
                np.testing.assert_array_equal(ks2, ks[first])
                np.testing.assert_array_equal(vs2, vs[first])


def test_chain_mask_gives_the_cache(orc):
    rng = np.random.default_rng(42)
    Hk, d, R = 2, 64, 8
    lens = [PAGE * 3 + 4, PAGE * 7 + 2, PAGE * 9 + 7]  # rounds across a page boundary
    cache = make_cache(orc, rng, lens, Hk, d, True)
    kp, vp, ks, vs, table = cache
    for s, C in enumerate(lens):
        assert (C - R) % PAGE + R > PAGE
        for r, m in enumerate(random_masks(rng, R, chain=True)):
            k2, v2, ks2, vs2, L = view(orc, cache, table[s], C, R, m, r, Hk, d, True)
            assert L == C - R + r + 1
            npg = k2.shape[0]
            pages = table[s, :npg]
            i = np.arange(L)
            np.testing.assert_array_equal(k2[i // PAGE, :, i % PAGE], kp[pages[i // PAGE], :, i % PAGE])
            np.testing.assert_array_equal(v2[i // PAGE, :, i % PAGE], vp[pages[i // PAGE], :, i % PAGE])
            np.testing.assert_array_equal(ks2, ks[pages])
            np.testing.assert_array_equal(vs2, vs[pages])


def check_cross_page_view(orc, cache, s, C, R, m, r, Hk, d):
    """The three properties of an fp8 view page that receives moved rows.
    Returns whether any scale grew."""
    kp, vp, ks, vs, table = cache
    k2, v2, ks2, vs2, L = view(orc, cache, table[s], C, R, m, r, Hk, d, True)
    pos = np.array(branch(C, R, m))
    C0 = C - R
    tp = C0 // PAGE
    grew = False
    for pool, sc, pool2, sc2 in ((kp, ks, k2, ks2), (vp, vs, v2, vs2)):
        t = np.arange(tp * PAGE, min(L, tp * PAGE + PAGE))
        sp, so = table[s, pos[t] // PAGE], pos[t] % PAGE
        home = table[s, tp]
        moved = sp != home
        for h in range(Hk):
            orig = e4m3_value(pool[sp, h, so]) * sc[sp, h][:, None]   # exact in fp64
            s_home, s_view = float(sc[home, h]), float(sc2[tp, h])
            a = float(np.max(np.abs(orig[moved]).astype(np.float32), initial=0.0))
            k = round(np.log2(s_view / s_home))
            assert s_view == np.float32(s_home * 2.0 ** k) and k >= 0
            if k == 0:
                assert np.float32(a) / np.float32(s_home) <= 448
                np.testing.assert_array_equal(pool2[tp, h, t[~moved] % PAGE], pool[sp[~moved], h, so[~moved]])
            else:
                grew = True
                assert np.float32(a) / np.float32(s_view) <= 448
                assert np.float32(a) / np.float32(s_view / 2) > 448
            got = e4m3_value(pool2[tp, h, t % PAGE]) * s_view
            bound = np.maximum(np.abs(orig) * 2.0 ** -4, s_view * 2.0 ** -10) * (1 + 1e-6)
            assert (np.abs(got - orig) <= bound).all()
        # the next view page holds rows of the next cache page only, bytes and scale unchanged
        if L > tp * PAGE + PAGE:
            t = np.arange(tp * PAGE + PAGE, L)
            assert (table[s, pos[t] // PAGE] == table[s, tp + 1]).all()
            np.testing.assert_array_equal(pool2[tp + 1, :, t % PAGE],
                                          pool[table[s, tp + 1], :, pos[t] % PAGE])
            np.testing.assert_array_equal(sc2[tp + 1], sc[table[s, tp + 1]])
    # pages below the round are the cache's
    np.testing.assert_array_equal(k2[:tp], kp[table[s, :tp]])
    np.testing.assert_array_equal(ks2[:tp], ks[table[s, :tp]])
    return grew


def test_moved_rows_keep_their_value(orc):
    rng = np.random.default_rng(43)
    Hk, d, R = 4, 64, 8
    lens = [PAGE * 3 + 5, PAGE * 6 + 7, PAGE * 11 + 1, PAGE * 2 + 6]
    cache = make_cache(orc, rng, lens, Hk, d, True)
    kp, vp, ks, vs, table = cache
    for s, C in enumerate(lens):
        # shrink the next page's values: moved rows must be re-encoded, not copied
        nxt = table[s, (C - R) // PAGE + 1]
        ks[nxt] *= 0.7
        vs[nxt] *= 0.7
    n_moved = 0
    for s, C in enumerate(lens):
        assert (C - R) % PAGE + R > PAGE
        for trial in range(6):
            for r, m in enumerate(random_masks(rng, R)):
                check_cross_page_view(orc, cache, s, C, R, m, r, Hk, d)
                C0 = C - R
                b = branch(C, R, m)[C0:]
                n_moved += sum(1 for i, p in enumerate(b) if p // PAGE > (C0 + i) // PAGE)
    assert n_moved > 20


def test_moved_rows_grow_the_scale(orc):
    rng = np.random.default_rng(44)
    Hk, d, R = 2, 64, 8
    lens = [PAGE * 4 + 3, PAGE * 8 + 6]
    cache = make_cache(orc, rng, lens, Hk, d, True)
    kp, vp, ks, vs, table = cache
    for s, C in enumerate(lens):
        nxt = table[s, (C - R) // PAGE + 1]
        ks[nxt] *= 64.0
        vs[nxt] *= 1.0 + 1.0 / 3.0  # not a power of two: moved V rows are re-rounded
    grew = 0
    for s, C in enumerate(lens):
        C0 = C - R
        # row R-1 with only itself and row 0: it moves into the page of C0
        m = 1 | (1 << (R - 1))
        assert (C0 + R - 1) // PAGE > C0 // PAGE
        grew += check_cross_page_view(orc, cache, s, C, R, m, R - 1, Hk, d)
    assert grew == len(lens)


def test_invalid_masks_are_refused(orc):
    rng = np.random.default_rng(45)
    cache = make_cache(orc, rng, [70], 2, 64, True)
    table = cache[4]
    for m, r in ((0b0101, 0), (0b0010, 2), (0, 0), (1 << 8, 7)):
        with pytest.raises(ValueError):
            view(orc, cache, table[0], 70, 8, m, r, 2, 64, True)
    with pytest.raises(ValueError):
        view(orc, cache, table[0], 7, 8, 1, 0, 2, 64, True)  # ctx_len < rows
