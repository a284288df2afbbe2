"""Pins of the oracle's e4m3 codec and of its append/quantise step (CPU).

The codec is pinned to torch's float8_e4m3fn conversions (a library routine
implementing the OCP E4M3 format) over all 256 codes and over values around
every rounding boundary; the append step to the properties its definition
fixes; the fp8 attention path to torch SDPA over the dequantised values.
"""
import numpy as np
import pytest
import torch

from test_oracle_pins import PAGE, bits_to_f64, bf16_round, sdpa, Case


def torch_e4m3_value(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(y):
    t = torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_table_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_value(codes)
    ref = torch_e4m3_value(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = torch_e4m3_value(finite)
    mags = np.unique(np.abs(vals))
    mids = (mags[1:] + mags[:-1]) / 2  # exact ties (representable in fp32)
    ys = np.concatenate([
        vals, mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        rng.uniform(-448, 448, 2000), rng.uniform(-0.02, 0.02, 2000),
        [0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 447.9],
    ]).astype(np.float32)
    ours = orc.e4m3_encode(ys)
    ref = torch_e4m3_encode(ys)
    np.testing.assert_array_equal(ours, ref)


def test_encode_saturates(orc):
    ys = np.array([448.0, 449.0, 464.0, 500.0, 1e30, np.inf, -449.0, -np.inf], np.float32)
    np.testing.assert_array_equal(orc.e4m3_encode(ys),
                                  np.array([0x7E] * 6 + [0xFE] * 2, np.uint8))


def test_encode_roundtrip_every_code(orc):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = orc.e4m3_value(finite).astype(np.float32)
    np.testing.assert_array_equal(orc.e4m3_encode(vals), finite)


def _pools(n_pages, Hk, d, fp8):
    shape = (n_pages, Hk, PAGE, d)
    if fp8:
        return (np.full(shape, 0x7F, np.uint8), np.full(shape, 0x7F, np.uint8),
                np.full((n_pages, Hk), np.nan, np.float32),
                np.full((n_pages, Hk), np.nan, np.float32))
    return np.full(shape, 0x7FC0, np.uint16), np.full(shape, 0x7FC0, np.uint16), None, None


def test_append_bf16_is_a_scatter(orc):
    rng = np.random.default_rng(4)
    k = bf16_round(rng.standard_normal((20, 2, 8)))
    v = bf16_round(rng.standard_normal((20, 2, 8)))
    slots = rng.permutation(6 * PAGE)[:20].astype(np.int32)
    slots[3] = -1
    kp, vp, _, _ = _pools(6, 2, 8, False)
    orc.kv_append(k, v, slots, kp, vp, n_head_kv=2, head_dim=8, page_size=PAGE)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        np.testing.assert_array_equal(kp[s // PAGE, :, s % PAGE], k[t])
        np.testing.assert_array_equal(vp[s // PAGE, :, s % PAGE], v[t])
    written = np.zeros((6, PAGE), bool)
    written[slots[slots >= 0] // PAGE, slots[slots >= 0] % PAGE] = True
    assert (kp.transpose(0, 2, 1, 3)[~written] == 0x7FC0).all()


def test_append_fp8_scale_and_codes(orc):
    rng = np.random.default_rng(5)
    Hk, d = 2, 16
    k = bf16_round(rng.standard_normal((16 + 7, Hk, d)) * 3)
    v = bf16_round(rng.standard_normal((16 + 7, Hk, d)))
    slots = np.concatenate([2 * PAGE + np.arange(16), 5 * PAGE + np.arange(7)]).astype(np.int32)
    kp, vp, ks, vs = _pools(8, Hk, d, True)
    orc.kv_append(k, v, slots, kp, vp, ks, vs, n_head_kv=Hk, head_dim=d, page_size=PAGE,
                  kv_dtype=orc.KV_FP8)
    for src, pool, sc in ((k, kp, ks), (v, vp, vs)):
        x = bits_to_f64(src).astype(np.float32)
        for page, rows in ((2, slice(0, 16)), (5, slice(16, 23))):
            for h in range(Hk):
                amax = np.float32(np.max(np.abs(x[rows, h])))
                assert sc[page, h] == np.float32(amax / np.float32(448.0))
                q = (x[rows, h] / sc[page, h]).astype(np.float32)
                n = rows.stop - rows.start
                codes = pool[page, h, :n]
                np.testing.assert_array_equal(codes, torch_e4m3_encode(q))
                # the absmax element lands on the largest code
                assert (np.abs(torch_e4m3_value(codes)) == 448.0).any()
                # dequantised values within half a code step of the input
                deq = orc.e4m3_value(codes) * float(sc[page, h])
                assert np.all(np.abs(deq - x[rows, h]) <= 2.0 ** -4 * np.abs(x[rows, h]) +
                              2.0 ** -10 * float(sc[page, h]))
        untouched = np.ones(8, bool)
        untouched[[2, 5]] = False
        assert np.isnan(sc[untouched]).all() and (pool[untouched] == 0x7F).all()


def test_append_fp8_later_call_keeps_or_doubles_scale(orc):
    rng = np.random.default_rng(6)
    Hk, d = 1, 16
    kp, vp, ks, vs = _pools(2, Hk, d, True)
    k1 = bf16_round(rng.standard_normal((5, Hk, d)))
    orc.kv_append(k1, k1, np.arange(5, dtype=np.int32) + PAGE, kp, vp, ks, vs, n_head_kv=Hk,
                  head_dim=d, page_size=PAGE, kv_dtype=orc.KV_FP8)
    s0 = np.float32(ks[1, 0])
    c0 = kp[1, 0, :5].copy()
    # rows that fit keep the scale and the earlier codes
    half = bf16_round(np.full((1, Hk, d), 0.5))
    orc.kv_append(half, half, np.array([PAGE + 5], np.int32), kp, vp, ks, vs, n_head_kv=Hk,
                  head_dim=d, page_size=PAGE, kv_dtype=orc.KV_FP8)
    assert ks[1, 0] == s0 and (kp[1, 0, :5] == c0).all()
    c5 = kp[1, 0, 5].copy()
    # rows that do not fit: the scale doubles until 100 / scale <= 448
    big = bf16_round(np.full((3, Hk, d), 100.0))
    orc.kv_append(big, big, np.arange(6, 9, dtype=np.int32) + PAGE, kp, vp, ks, vs,
                  n_head_kv=Hk, head_dim=d, page_size=PAGE, kv_dtype=orc.KV_FP8)
    s1 = np.float32(ks[1, 0])
    k = int(round(np.log2(s1 / s0)))
    assert k >= 1 and s1 == s0 * np.float32(2.0 ** k)
    assert np.float32(100.0) / s1 <= 448 < np.float32(100.0) / (s1 / np.float32(2))
    # earlier codes re-encoded at s1: torch's E4M3 conversion of
    # fp32(fp32(value * s0) / s1), and equal values wherever they stay normal
    old = np.concatenate([c0, c5[None]])
    y = (torch_e4m3_value(old).astype(np.float32) * s0) / s1
    np.testing.assert_array_equal(kp[1, 0, :6], torch_e4m3_encode(y))
    stays = np.abs(torch_e4m3_value(old)) * 2.0 ** -k >= 2.0 ** -6
    assert stays.any()
    np.testing.assert_array_equal((torch_e4m3_value(kp[1, 0, :6]) * float(s1))[stays],
                                  (torch_e4m3_value(old) * float(s0))[stays])
    # the new rows are codes of 100 / s1, not saturated
    np.testing.assert_array_equal(kp[1, 0, 6:9],
                                  torch_e4m3_encode(np.full((3, d), np.float32(100.0) / s1)))
    assert not (kp[1, 0, 6:9] == 0x7E).all()
    # a zero page gets scale 1
    z = np.zeros((1, Hk, d), np.uint16)
    orc.kv_append(z, z, np.array([0], np.int32), kp, vp, ks, vs, n_head_kv=Hk, head_dim=d,
                  page_size=PAGE, kv_dtype=orc.KV_FP8)
    assert ks[0, 0] == 1.0 and (kp[0, 0, 0] == 0).all()


def test_fp8_pages_filled_one_token_per_call_stay_accurate(orc):
    """Decode-style appends (one token per sequence per call) against the
    attention over the unquantised bf16 rows: within the fp8 tolerance."""
    rng = np.random.default_rng(8)
    S, C, H, Hk, d = 3, 300, 8, 2, 64
    n_pages = S * -(-C // PAGE)
    table = rng.permutation(n_pages).astype(np.int32).reshape(S, -1)
    k = bf16_round(rng.standard_normal((S, C, Hk, d)))
    v = bf16_round(rng.standard_normal((S, C, Hk, d)))
    q = bf16_round(rng.standard_normal((S, 1, H, d)))
    slot = lambda s, t: table[s, t // PAGE] * PAGE + t % PAGE
    kb, vb, _, _ = _pools(n_pages, Hk, d, False)
    kf, vf, ks, vs = _pools(n_pages, Hk, d, True)
    for t in range(C):
        sl = np.array([slot(s, t) for s in range(S)], np.int32)
        orc.kv_append(k[:, t], v[:, t], sl, kb, vb, n_head_kv=Hk, head_dim=d, page_size=PAGE)
        orc.kv_append(k[:, t], v[:, t], sl, kf, vf, ks, vs, n_head_kv=Hk, head_dim=d,
                      page_size=PAGE, kv_dtype=orc.KV_FP8)
    lens = np.full(S, C, np.int32)
    ref = orc.paged_attention(q, kb, vb, table, lens, n_head=H, n_head_kv=Hk, head_dim=d,
                              page_size=PAGE)
    got = orc.paged_attention(q, kf, vf, table, lens, n_head=H, n_head_kv=Hk, head_dim=d,
                              page_size=PAGE, kv_dtype=orc.KV_FP8, k_scale=ks, v_scale=vs)
    assert np.abs(got - ref).max() <= 2e-2


def test_fp8_attention_matches_sdpa_on_dequantised(orc):
    rng = np.random.default_rng(7)
    case = Case(rng, [40, 19], 8, 4, 2, 16)
    # quantise the logical cache with the oracle's own append
    kp, vp, ks, vs = _pools(case.n_pages, 2, 16, True)
    slots = np.concatenate([case.table[s, np.arange(c) // PAGE] * PAGE + np.arange(c) % PAGE
                            for s, c in enumerate(case.lens)]).astype(np.int32)
    K = np.concatenate(case.k)
    V = np.concatenate(case.v)
    orc.kv_append(K, V, slots, kp, vp, ks, vs, n_head_kv=2, head_dim=16, page_size=PAGE,
                  kv_dtype=orc.KV_FP8)
    got = orc.paged_attention(case.q, kp, vp, case.table, case.lens, n_head=4, n_head_kv=2,
                              head_dim=16, page_size=PAGE, kv_dtype=orc.KV_FP8, k_scale=ks,
                              v_scale=vs)
    # reference: dequantise each token with its page scale (fp64), then SDPA
    ref_case = Case(rng, [40, 19], 8, 4, 2, 16)
    ref_case.q, ref_case.lens, ref_case.table = case.q, case.lens, case.table
    deq_k, deq_v = [], []
    for s, c in enumerate(case.lens):
        t = np.arange(c)
        p = case.table[s, t // PAGE]
        o = t % PAGE
        dk = orc.e4m3_value(kp[p, :, o]) * ks[p][:, :, None].astype(np.float64)
        dv = orc.e4m3_value(vp[p, :, o]) * vs[p][:, :, None].astype(np.float64)
        deq_k.append(dk)
        deq_v.append(dv)
    g = 2
    for s, c in enumerate(case.lens):
        Kt = torch.from_numpy(deq_k[s]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
        Vt = torch.from_numpy(deq_v[s]).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
        Q = torch.from_numpy(bits_to_f64(case.q[s])).permute(1, 0, 2).contiguous()
        pos = torch.arange(8) + (int(c) - 8)
        mask = torch.arange(int(c))[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=mask)
        np.testing.assert_allclose(got[s], o.permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
