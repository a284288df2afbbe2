"""Pins of the CPU oracle against things other than itself (CPU only).

- brute force: pure-Python attention over *unpaged*, contiguous K/V with
  math.fsum / math.exp on tiny inputs;
- a library routine: torch's scaled_dot_product_attention in fp64 on the
  CPU, K/V repeated per GQA group, explicit bottom-right causal mask;
- closed forms: one-token context, constant V, zero query, two keys;
- invariants: page relabelling, key shift, V scaling, key order.

A dropped term, a wrong sign, an off-by-one in the causal limit, a swapped
GQA mapping or a transposed page layout in the oracle fails one of these.
"""
import math

import numpy as np
import pytest
import torch

PAGE = 16


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64/fp32 values to bf16 (returned as uint16 bits)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Case:
    """Tiny paged problem: logical K/V per sequence, a random table, pools."""

    def __init__(self, rng, lens, rows, n_head, n_head_kv, d, spare=3, kv_bits=None):
        self.lens = np.asarray(lens, np.int32)
        self.rows, self.H, self.Hk, self.d = rows, n_head, n_head_kv, d
        self.S = len(lens)
        self.max_pages = max(-(-c // PAGE) for c in lens) + 1
        need = [-(-c // PAGE) for c in lens]
        self.n_pages = sum(need) + spare
        perm = rng.permutation(self.n_pages)
        self.table = np.full((self.S, self.max_pages), -1, np.int32)
        pos = 0
        for s, n in enumerate(need):
            self.table[s, :n] = perm[pos:pos + n]
            pos += n
        self.k = [bf16_round(rng.standard_normal((c, n_head_kv, d))) for c in lens]
        self.v = [bf16_round(rng.standard_normal((c, n_head_kv, d))) for c in lens]
        self.q = bf16_round(rng.standard_normal((self.S, rows, n_head, d)))
        self.build_pools()

    def build_pools(self):
        kp = np.full((self.n_pages, self.Hk, PAGE, self.d), 0x7FC0, np.uint16)  # NaN poison
        vp = kp.copy()
        for s in range(self.S):
            for t in range(self.lens[s]):
                p = self.table[s, t // PAGE]
                kp[p, :, t % PAGE, :] = self.k[s][t]
                vp[p, :, t % PAGE, :] = self.v[s][t]
        self.kp, self.vp = kp, vp

    def oracle(self, orc, **kw):
        return orc.paged_attention(self.q, self.kp, self.vp, self.table, self.lens, n_head=self.H,
                                   n_head_kv=self.Hk, head_dim=self.d, page_size=PAGE, **kw)


def brute(case: Case) -> np.ndarray:
    """Unpaged pure-Python attention, straight from the definition."""
    g = case.H // case.Hk
    out = np.zeros((case.S, case.rows, case.H, case.d))
    for s in range(case.S):
        K = bits_to_f64(case.k[s])
        V = bits_to_f64(case.v[s])
        Q = bits_to_f64(case.q[s])
        C = int(case.lens[s])
        for r in range(case.rows):
            last = C - case.rows + r
            for h in range(case.H):
                kh = h // g
                q = Q[r, h].tolist()
                sc = [math.fsum(qi * ki for qi, ki in zip(q, K[t, kh].tolist())) /
                      math.sqrt(case.d) for t in range(last + 1)]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                for i in range(case.d):
                    out[s, r, h, i] = math.fsum(w[t] * V[t, kh, i] for t in range(last + 1)) / z
    return out


def sdpa(case: Case) -> np.ndarray:
    """torch SDPA in fp64 on the CPU, per sequence, with an explicit mask."""
    g = case.H // case.Hk
    out = np.zeros((case.S, case.rows, case.H, case.d))
    for s in range(case.S):
        C = int(case.lens[s])
        K = torch.from_numpy(bits_to_f64(case.k[s])).permute(1, 0, 2)  # [Hk, C, d]
        V = torch.from_numpy(bits_to_f64(case.v[s])).permute(1, 0, 2)
        K = K.repeat_interleave(g, dim=0).contiguous()
        V = V.repeat_interleave(g, dim=0).contiguous()
        Q = torch.from_numpy(bits_to_f64(case.q[s])).permute(1, 0, 2).contiguous()  # [H, R, d]
        pos = torch.arange(case.rows) + (C - case.rows)
        mask = torch.arange(C)[None, :] <= pos[:, None]  # [R, C] True = attend
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        out[s] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("lens,rows,H,Hk,d", [
    ([1, 5, 17], 1, 4, 2, 8),        # decode, one-token context, page tails
    ([9, 16, 33], 1, 6, 3, 16),      # GQA g = 2, exact page, ragged
    ([8, 20, 40], 8, 4, 1, 8),       # verify rows (causal within the round)
    ([12, 31], 12, 2, 2, 16),        # prefill chunk covering the whole context
    ([40], 5, 8, 2, 12),             # prefill chunk after cached rows
])
def test_oracle_matches_bruteforce(orc, lens, rows, H, Hk, d):
    rng = np.random.default_rng(1234 + sum(lens) + rows)
    case = Case(rng, lens, rows, H, Hk, d)
    got = case.oracle(orc)
    ref = brute(case)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("lens,rows,H,Hk,d", [
    ([3, 64, 100], 1, 8, 2, 32),
    ([50, 77], 8, 16, 4, 32),
    ([200], 64, 4, 4, 16),
])
def test_oracle_matches_torch_sdpa_fp64(orc, lens, rows, H, Hk, d):
    rng = np.random.default_rng(99 + sum(lens))
    case = Case(rng, lens, rows, H, Hk, d)
    got = case.oracle(orc)
    ref = sdpa(case)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_closed_form_one_token_context(orc):
    rng = np.random.default_rng(5)
    case = Case(rng, [1, 1], 1, 4, 2, 16)
    got = case.oracle(orc)
    for s in range(2):
        for h in range(4):
            np.testing.assert_array_equal(got[s, 0, h], bits_to_f64(case.v[s][0, h // 2]))


def test_closed_form_constant_v(orc):
    rng = np.random.default_rng(6)
    case = Case(rng, [37], 1, 4, 2, 8)
    c = bf16_round(rng.standard_normal((2, 8)))
    case.v = [np.broadcast_to(c, case.v[0].shape).copy()]
    case.build_pools()
    got = case.oracle(orc)
    for h in range(4):
        np.testing.assert_allclose(got[0, 0, h], bits_to_f64(c[h // 2]), rtol=0, atol=1e-13)


def test_closed_form_zero_query_is_prefix_mean(orc):
    rng = np.random.default_rng(7)
    case = Case(rng, [29], 4, 2, 1, 8)
    case.q[:] = 0
    got = case.oracle(orc)
    V = bits_to_f64(case.v[0])[:, 0, :]
    for r in range(4):
        last = 29 - 4 + r
        np.testing.assert_allclose(got[0, r, 0], V[:last + 1].mean(axis=0), atol=1e-13)


def test_closed_form_two_keys_sigmoid(orc):
    rng = np.random.default_rng(8)
    case = Case(rng, [2], 1, 1, 1, 16)
    got = case.oracle(orc)[0, 0, 0]
    Q = bits_to_f64(case.q[0, 0, 0])
    K = bits_to_f64(case.k[0])[:, 0]
    V = bits_to_f64(case.v[0])[:, 0]
    delta = (Q @ K[0] - Q @ K[1]) / 4.0
    sig = 1.0 / (1.0 + math.exp(-delta))
    np.testing.assert_allclose(got, sig * V[0] + (1 - sig) * V[1], atol=1e-13)


def test_invariant_page_relabelling_is_exact(orc):
    rng = np.random.default_rng(9)
    case = Case(rng, [45, 9, 70], 8, 4, 2, 16, spare=5)
    base = case.oracle(orc)
    perm = rng.permutation(case.n_pages)  # new id of old page p is perm[p]
    kp = np.empty_like(case.kp)
    vp = np.empty_like(case.vp)
    kp[perm] = case.kp
    vp[perm] = case.vp
    table = np.where(case.table >= 0, perm[np.maximum(case.table, 0)], -1).astype(np.int32)
    got = orc.paged_attention(case.q, kp, vp, table, case.lens, n_head=4, n_head_kv=2,
                              head_dim=16, page_size=PAGE)
    np.testing.assert_array_equal(got, base)


def test_invariant_key_shift_and_v_scale(orc):
    rng = np.random.default_rng(10)
    case = Case(rng, [33], 1, 2, 1, 8)
    # make column 3 of K a multiple of 1/16 so that adding 0.5 stays exact
    k0 = bits_to_f64(case.k[0])
    k0[..., 3] = np.round(k0[..., 3] * 16) / 16
    case.k = [bf16_round(k0)]
    case.build_pools()
    base = case.oracle(orc)
    # K_t -> K_t + u (u a power of two times a bf16 vector that keeps K exact):
    # the score moves by q.u for every key, so the softmax does not change.
    u = np.zeros(8)
    u[3] = 0.5
    k = bits_to_f64(case.k[0]) + u
    case2 = Case(rng, [33], 1, 2, 1, 8)
    case2.q, case2.table, case2.lens, case2.v = case.q, case.table, case.lens, case.v
    case2.k = [bf16_round(k)]
    assert np.array_equal(bits_to_f64(case2.k[0]), k)  # exact in bf16
    case2.build_pools()
    np.testing.assert_allclose(case2.oracle(orc), base, atol=1e-12)
    # V -> 2 V doubles the output exactly.
    case3 = Case(rng, [33], 1, 2, 1, 8)
    case3.q, case3.table, case3.lens, case3.k = case.q, case.table, case.lens, case.k
    case3.v = [bf16_round(2.0 * bits_to_f64(case.v[0]))]
    case3.build_pools()
    np.testing.assert_allclose(case3.oracle(orc), 2.0 * base, atol=1e-12)


def test_invariant_decode_key_order_irrelevant(orc):
    rng = np.random.default_rng(11)
    case = Case(rng, [50], 1, 4, 2, 8)
    base = case.oracle(orc)
    order = rng.permutation(50)
    case.k = [case.k[0][order]]
    case.v = [case.v[0][order]]
    case.build_pools()
    np.testing.assert_allclose(case.oracle(orc), base, atol=1e-12)


def test_causal_rows_equal_shorter_decodes(orc):
    """Row r of an R-row call equals a one-row call whose context ends at
    that row's position (the verify <-> decode relation, in the oracle)."""
    rng = np.random.default_rng(12)
    case = Case(rng, [40, 25], 8, 4, 2, 16)
    full = case.oracle(orc)
    for r in range(8):
        lens = case.lens - 8 + r + 1
        one = orc.paged_attention(case.q[:, r:r + 1], case.kp, case.vp, case.table, lens,
                                  n_head=4, n_head_kv=2, head_dim=16, page_size=PAGE)
        np.testing.assert_array_equal(one[:, 0], full[:, r])


def test_row_mask_and_range_errors(orc):
    rng = np.random.default_rng(13)
    case = Case(rng, [20], 3, 2, 1, 8)
    mask = np.array([[1, 0, 1]])
    got = case.oracle(orc, row_mask=mask)
    full = case.oracle(orc)
    assert np.isnan(got[0, 1]).all()
    np.testing.assert_array_equal(got[0, 0], full[0, 0])
    with pytest.raises(ValueError):
        orc.paged_attention(case.q, case.kp, case.vp, case.table, np.array([2], np.int32),
                            n_head=2, n_head_kv=1, head_dim=8, page_size=PAGE)
    bad = case.table.copy()
    bad[0, 0] = case.n_pages
    with pytest.raises(ValueError):
        orc.paged_attention(case.q, case.kp, case.vp, bad, case.lens, n_head=2, n_head_kv=1,
                            head_dim=8, page_size=PAGE)
