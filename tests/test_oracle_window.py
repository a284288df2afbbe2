"""Pins of the oracle's window / floor bound (CPU only).

The row at position p attends keys max(floor, p - window + 1) .. p
("Radiance Architecture Plugins -- declaring a model", section "Declare:
buffers and KV groups": a window-bounded KV group and a ring whose floor is
set at runtime).  Checked against a pure-Python brute force and torch's
fp64 SDPA with the explicit band mask, and the closed forms window = 1 and
floor = position (the row's own V); pages below the floor must not be read.
"""
import math

import numpy as np
import pytest
import torch

from test_oracle_pins import PAGE, Case, bits_to_f64


def lower(case, s, r, window, floor):
    p = int(case.lens[s]) - case.rows + r
    lo = int(floor[s]) if floor is not None else 0
    if window > 0:
        lo = max(lo, p - window + 1)
    return lo, p


def brute_window(case: Case, window, floor) -> np.ndarray:
    g = case.H // case.Hk
    out = np.zeros((case.S, case.rows, case.H, case.d))
    for s in range(case.S):
        K, V, Q = bits_to_f64(case.k[s]), bits_to_f64(case.v[s]), bits_to_f64(case.q[s])
        for r in range(case.rows):
            lo, p = lower(case, s, r, window, floor)
            for h in range(case.H):
                kh = h // g
                q = Q[r, h].tolist()
                sc = [math.fsum(qi * ki for qi, ki in zip(q, K[t, kh].tolist())) /
                      math.sqrt(case.d) for t in range(lo, p + 1)]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                for i in range(case.d):
                    out[s, r, h, i] = math.fsum(
                        w[t - lo] * V[t, kh, i] for t in range(lo, p + 1)) / z
    return out


def sdpa_window(case: Case, window, floor) -> np.ndarray:
    g = case.H // case.Hk
    out = np.zeros((case.S, case.rows, case.H, case.d))
    for s in range(case.S):
        C = int(case.lens[s])
        K = torch.from_numpy(bits_to_f64(case.k[s])).permute(1, 0, 2)
        V = torch.from_numpy(bits_to_f64(case.v[s])).permute(1, 0, 2)
        K = K.repeat_interleave(g, dim=0).contiguous()
        V = V.repeat_interleave(g, dim=0).contiguous()
        Q = torch.from_numpy(bits_to_f64(case.q[s])).permute(1, 0, 2).contiguous()
        lo = torch.tensor([lower(case, s, r, window, floor)[0] for r in range(case.rows)])
        pos = torch.arange(case.rows) + (C - case.rows)
        t = torch.arange(C)[None, :]
        mask = (t <= pos[:, None]) & (t >= lo[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        out[s] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("lens,rows,H,Hk,d,window,floor", [
    ([5, 17, 40], 1, 4, 2, 8, 3, None),           # decode, window inside a page
    ([33, 50], 1, 6, 3, 16, 16, [4, 20]),         # window and floor both bite
    ([20, 45], 8, 4, 1, 8, 5, None),              # verify rows, window < rows
    ([40], 12, 8, 2, 12, 17, [10]),               # prefill chunk after cached rows
    ([31], 31, 2, 2, 16, 0, [0]),                 # floor 0, no window: the plain call
])
def test_window_matches_bruteforce(orc, lens, rows, H, Hk, d, window, floor):
    rng = np.random.default_rng(777 + sum(lens) + rows + window)
    case = Case(rng, lens, rows, H, Hk, d)
    fl = None if floor is None else np.asarray(floor, np.int32)
    got = case.oracle(orc, window=window, kv_floor=fl)
    ref = brute_window(case, window, fl)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("lens,rows,H,Hk,d,window,floor", [
    ([64, 100], 1, 8, 2, 32, 37, [10, 70]),
    ([77], 8, 16, 4, 32, 20, None),
    ([200], 64, 4, 4, 16, 50, [30]),
])
def test_window_matches_torch_sdpa_fp64(orc, lens, rows, H, Hk, d, window, floor):
    rng = np.random.default_rng(4242 + sum(lens))
    case = Case(rng, lens, rows, H, Hk, d)
    fl = None if floor is None else np.asarray(floor, np.int32)
    got = case.oracle(orc, window=window, kv_floor=fl)
    ref = sdpa_window(case, window, fl)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_window_one_is_the_rows_own_value(orc):
    rng = np.random.default_rng(8)
    case = Case(rng, [9, 30], 4, 4, 2, 16)
    got = case.oracle(orc, window=1)
    for s in range(case.S):
        V = bits_to_f64(case.v[s])
        for r in range(case.rows):
            p = int(case.lens[s]) - case.rows + r
            for h in range(case.H):
                assert np.array_equal(got[s, r, h], V[p, h // 2])


def test_floor_at_first_row_gives_its_value(orc):
    rng = np.random.default_rng(9)
    case = Case(rng, [18, 40], 3, 2, 2, 8)
    fl = case.lens - case.rows
    got = case.oracle(orc, kv_floor=fl)
    for s in range(case.S):
        V = bits_to_f64(case.v[s])
        p0 = int(fl[s])
        g = case.H // case.Hk
        assert np.array_equal(got[s, 0], V[p0][np.arange(case.H) // g])


def test_pages_below_the_floor_are_not_read(orc):
    rng = np.random.default_rng(10)
    case = Case(rng, [70, 90], 2, 4, 2, 16)
    fl = np.array([40, 35], np.int32)
    ref = case.oracle(orc, kv_floor=fl, window=9)
    # release the pages wholly below each floor: entry -1, page poisoned
    for s in range(case.S):
        for e in range(int(fl[s]) // PAGE):
            case.kp[case.table[s, e]] = 0x7FC0
            case.vp[case.table[s, e]] = 0x7FC0
            case.table[s, e] = -1
    got = case.oracle(orc, kv_floor=fl, window=9)
    assert np.array_equal(got, ref)
    with pytest.raises(ValueError):
        case.oracle(orc)  # the plain call does read them


def test_wide_window_is_the_plain_call(orc):
    rng = np.random.default_rng(11)
    case = Case(rng, [25, 60], 8, 4, 2, 16)
    assert np.array_equal(case.oracle(orc, window=60), case.oracle(orc))


def test_floor_range_is_checked(orc):
    rng = np.random.default_rng(12)
    case = Case(rng, [20, 30], 4, 4, 2, 8)
    with pytest.raises(ValueError):
        case.oracle(orc, kv_floor=np.array([17, 0], np.int32))  # above 20 - 4
    with pytest.raises(ValueError):
        case.oracle(orc, kv_floor=np.array([-1, 0], np.int32))
