"""Pins of the oracle's query rounding for the fp8 prefill (CPU only).

Rule under test (the build context's `attn_prefill_fp8` bits, "Radiance
Architecture Plugins -- declaring a model", section "Declare: the metadata";
the rule itself is this oracle's reading): per query vector, the scale is the
smallest power of two 2^e with max|q| <= 448 * 2^e (e >= -117), and each
element becomes 2^e times the nearest E4M3 value of q / 2^e, ties to even.

Pinned against torch's float8_e4m3fn cast with the exponent found by a plain
search, the exponent's defining inequality, closed forms (representable
vectors are unchanged, zero stays zero), symmetry under sign and powers of
two, the half-ulp error bound, and the attention composition.
"""
import numpy as np
import pytest
import torch

from test_oracle_pins import PAGE, Case, bf16_round, bits_to_f64


def search_exp(amax: float) -> int:
    """Smallest e >= -117 with amax <= 448 * 2^e, by counting up."""
    e = -117
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return e


def torch_round(q_bits: np.ndarray) -> np.ndarray:
    """The rule through torch's own E4M3 cast (round to nearest even)."""
    q = bits_to_f64(q_bits)
    out = np.empty_like(q)
    flat, res = q.reshape(-1, q.shape[-1]), out.reshape(-1, q.shape[-1])
    for i, v in enumerate(flat):
        e = search_exp(float(np.max(np.abs(v))))
        y = torch.from_numpy(np.ldexp(v, -e).astype(np.float32))
        r = y.to(torch.float8_e4m3fn).to(torch.float64).numpy()
        res[i] = np.ldexp(r, e)
    return bf16_round(out)


def vectors(rng, n, d):
    """bf16 vectors over many magnitudes, with exact ties between E4M3
    neighbours planted after the scale is fixed by a 448 * 2^k element."""
    out = []
    for i in range(n):
        k = int(rng.integers(-30, 30))
        v = rng.standard_normal(d) * 2.0 ** k
        if i % 3 == 0:
            v[0] = 448.0 * 2.0 ** k  # fixes e = k
            j = rng.integers(1, d, size=d // 4)
            m = rng.integers(8, 15, size=j.size)  # mantissa 1.m/8 .. with a tie bit
            ex = rng.integers(-6, 8, size=j.size)
            v[j] = (1.0 + (2 * m + 1) / 16.0 - 1.0) * 2.0 ** (ex + k)  # halfway points
        out.append(v)
    return bf16_round(np.array(out))


def test_matches_torch_float8_cast(orc):
    rng = np.random.default_rng(1)
    for d in (8, 64, 256):
        q = vectors(rng, 60, d)
        got = orc.round_q_e4m3(q)
        np.testing.assert_array_equal(got, torch_round(q))


def test_exponent_is_the_smallest_power_of_two(orc):
    rng = np.random.default_rng(2)
    q = vectors(rng, 200, 32)
    _, exps = orc.round_q_e4m3(q, return_exps=True)
    amax = np.max(np.abs(bits_to_f64(q)), axis=-1)
    for a, e in zip(amax, exps):
        assert a <= 448.0 * 2.0 ** e
        assert e == -117 or a > 448.0 * 2.0 ** (e - 1)
        assert e == search_exp(float(a))


def test_closed_forms(orc):
    # representable at its own scale: unchanged
    vals = orc.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))
    rng = np.random.default_rng(3)
    for k in (-20, 0, 5):
        v = rng.choice(vals, size=64) * rng.choice([-1.0, 1.0], size=64)
        v[3] = 448.0
        q = bf16_round(v * 2.0 ** k)
        np.testing.assert_array_equal(orc.round_q_e4m3(q), q)
    # zero vector: zero, exponent -117
    z = np.zeros((1, 16), np.uint16)
    got, e = orc.round_q_e4m3(z, return_exps=True)
    np.testing.assert_array_equal(got, z)
    assert int(e[0, ]) == -117
    # one element: it sets the scale and lands on 448 * 2^e exactly... or
    # below it when |q| is not 448 times a power of two; a single 1.0 -> 1.0
    one = bf16_round(np.array([[1.0, 0, 0, 0]]))
    np.testing.assert_array_equal(orc.round_q_e4m3(one), one)
    # the 1.0625 tie (between 1 and 1.125) goes to the even code, 1.0
    tie = bf16_round(np.array([[448.0, 1.0625, 1.1875, -2.125]]))
    exp = bf16_round(np.array([[448.0, 1.0, 1.25, -2.0]]))
    np.testing.assert_array_equal(orc.round_q_e4m3(tie), exp)


def test_sign_and_power_of_two_symmetry(orc):
    rng = np.random.default_rng(4)
    q = vectors(rng, 50, 32)
    r = bits_to_f64(orc.round_q_e4m3(q))
    neg = bits_to_f64(orc.round_q_e4m3(q ^ np.uint16(0x8000)))
    np.testing.assert_array_equal(neg, -r)
    for j in (-3, 4):
        qs = bf16_round(bits_to_f64(q) * 2.0 ** j)
        np.testing.assert_array_equal(bits_to_f64(orc.round_q_e4m3(qs)), r * 2.0 ** j)


def test_half_ulp_error_bound(orc):
    rng = np.random.default_rng(5)
    q = vectors(rng, 120, 64)
    qv = bits_to_f64(q)
    r, exps = orc.round_q_e4m3(q, return_exps=True)
    rv = bits_to_f64(r)
    scale = 2.0 ** exps[:, None].astype(np.float64)
    # normal E4M3 range (|y| >= 2^-6): relative half-ulp 2^-4; below it the
    # spacing is 2^-9, so half of it, 2^-10, absolute (in units of the scale)
    y = np.abs(qv) / scale
    err = np.abs(rv - qv) / scale
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= y[normal] * 2.0 ** -4)
    assert np.all(err[~normal] <= 2.0 ** -10)


def test_attention_with_rounded_q(orc):
    rng = np.random.default_rng(6)
    case = Case(rng, [20, 45], 6, 4, 2, 16)
    got = case.oracle(orc, q_fp8=True)
    q0 = case.q
    case.q = orc.round_q_e4m3(q0)
    ref = case.oracle(orc)
    np.testing.assert_array_equal(got, ref)
    # a query already on the E4M3 grid at its scale: same result as plain
    assert np.array_equal(case.oracle(orc, q_fp8=True), ref)
    case.q = q0
    assert not np.array_equal(got, case.oracle(orc))  # rounding does change it


def test_non_finite_is_refused(orc):
    q = bf16_round(np.array([[1.0, np.inf, 0.0, 0.0]]))
    with pytest.raises(ValueError):
        orc.round_q_e4m3(q)
