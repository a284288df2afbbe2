"""GPU parity of the fp8 prefill (ATTN_PREFILL_FP8_QK: QK^T on the fp8
matrix unit, each query vector rounded to E4M3 at a power-of-two scale;
ATTN_PREFILL_FP8_PV: PV on the fp8 matrix unit, each tile's probabilities
with its V page scales folded in rounded to E4M3) against the CPU oracle
with the same query rounding, and the rule that prefill_fp8 = 0 is the
plain prefill bit for bit (MI355X only).

The PV rounding has no counterpart in the oracle: it gives each softmax
weight a relative error of at most 2^-4, so an output element may move by
up to 2^-4 times the softmax average of |v| over the same keys, which the
oracle computes as attention over the codes with their sign bits cleared.
PV cases pass when every element is within the larger of the fp8 tolerance
and that bound."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import (PAGE, TOL, GpuCache, OracleCache, bf16_to_f64, excess_err, max_err,
                      same_bits, say)

pytestmark = pytest.mark.gpu


def prefill_case(name, n_rows, ctx, H, Hk, d, seed):
    return synth.Workload(name, 1, n_rows, H, Hk, d, True, "fixed", ctx, ctx, seed,
                          kind="prefill")


CASES = [
    prefill_case("pq_d256_g4", 130, 1500, 16, 4, 256, 61),
    prefill_case("pq_d128_g4", 77, 900, 8, 2, 128, 62),
    prefill_case("pq_d256_g8", 300, 700, 32, 4, 256, 63),
    prefill_case("pq_d128_g1_whole", 64, 64, 4, 4, 128, 64),
    prefill_case("pq_d256_one_row", 1, 1, 8, 2, 256, 65),
    prefill_case("pq_d128_g16", 40, 333, 32, 2, 128, 66),
]


def run_fp8(gpu, inp, bits, q=None, table=None):
    w = inp.w
    q = (inp.q if q is None else q).view(w.rows, w.n_head, w.head_dim)
    table = inp.table if table is None else table
    out = torch.empty_like(q)
    pa.attn_paged_prefill_fp8(q, w.rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, table,
                              table.shape[1], int(inp.lengths[0]), w.n_head, w.n_head_kv,
                              w.head_dim, PAGE, gpu.kv, bits, out)
    return out


def oracle_fp8(oc, q, row_mask=None):
    w = oc.w
    return oracle.paged_attention(
        synth.bits(q), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head, n_head_kv=w.n_head_kv,
        head_dim=w.head_dim, page_size=PAGE, kv_dtype=oracle.KV_FP8, k_scale=oc.ks,
        v_scale=oc.vs, row_mask=row_mask, q_fp8=True)


@pytest.fixture(scope="module", params=CASES, ids=[w.name for w in CASES])
def case(request):
    w = request.param
    say("[gpu] fp8 prefill case", w.name, "rows", w.rows, "ctx", w.ctx_lo)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    return w, inp, gpu, OracleCache(inp)


def test_qk_fp8_parity(case):
    w, inp, gpu, oc = case
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK)
    torch.cuda.synchronize()
    ref = oracle_fp8(oc, inp.q)
    ex = excess_err(out, ref.reshape(out.shape), TOL[True])
    plain = oc.attend(inp.q)
    say("[gpu]", w.name, "excess vs rounded-q oracle", ex, "max err vs plain oracle",
        max_err(out, plain.reshape(out.shape)))
    assert ex <= 0


def test_qk_fp8_scaled_and_zero_queries(case):
    """Query vectors over a wide range of magnitudes (powers of two, exact in
    bf16) and all-zero vectors: the power-of-two scale follows each vector."""
    w, inp, gpu, oc = case
    q = inp.q.clone()
    f = torch.tensor([2.0 ** -8, 4.0, 2.0 ** -30, 1.0], device="cuda")
    q = q * f[torch.arange(w.n_head, device="cuda") % 4].view(1, 1, w.n_head, 1).to(q.dtype)
    q[..., 1::4, :] = 0  # zero vectors on every fourth head
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK, q=q)
    torch.cuda.synchronize()
    ref = oracle_fp8(oc, q)
    ex = excess_err(out, ref.reshape(out.shape), TOL[True])
    say("[gpu]", w.name, "scaled queries excess", ex)
    assert ex <= 0


def test_bits_zero_is_the_plain_prefill(case):
    w, inp, gpu, oc = case
    out = run_fp8(gpu, inp, 0)
    plain = gpu.run("prefill")
    torch.cuda.synchronize()
    assert same_bits(out, plain.view_as(out))


def test_qk_fp8_determinism(case):
    w, inp, gpu, oc = case
    a = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK)
    b = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK)
    torch.cuda.synchronize()
    assert same_bits(a, b)


def test_qk_fp8_bad_page_gives_nan():
    w = prefill_case("pq_bad", 50, 500, 8, 2, 128, 67)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    table = inp.table.clone()
    table[0, 5] = inp.n_pages + 3
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK, table=table)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


def test_qk_fp8_bf16_cache_is_refused():
    w = synth.Workload("pq_bf16", 1, 8, 8, 2, 128, False, "fixed", 40, 40, 68, kind="prefill")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    with pytest.raises(pa.AttnError) as e:
        run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK)
    assert e.value.code == pa.ATTN_E_UNSUPPORTED


def test_qk_fp8_full_chunk_sampled_rows():
    """The 4,096-row chunk over 28,672 cached rows with an fp8 cache, in the
    launch the benchmark times; sampled rows against the oracle."""
    w = synth.scaled(synth.WORKLOADS["prefill_4096_over_28672"], kv_fp8=True,
                     name="prefill_4096_over_28672_fp8kv")
    say("[gpu] full fp8 prefill chunk")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rows = sorted({0, 1, 31, 32, 4095} | set(range(0, 4096, 256)))
    mask = np.zeros((1, w.rows), bool)
    mask[0, rows] = True
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    ref = oracle_fp8(oc, inp.q, row_mask=mask)
    err = max_err(out.view(1, w.rows, w.n_head, w.head_dim), ref, row_mask=mask)
    say("[gpu] full fp8 prefill sampled rows", len(rows), "max abs err", err)
    assert err <= TOL[True]
    del gpu, inp
    torch.cuda.empty_cache()


def pv_bound(oc, q, qk, row_mask=None):
    """2^-4 times the softmax average of |v| of every output element."""
    w = oc.w
    return 2.0 ** -4 * oracle.paged_attention(
        synth.bits(q), oc.k, (oc.v & 0x7F).astype(np.uint8), oc.table, oc.lens,
        n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8, k_scale=oc.ks, v_scale=oc.vs, row_mask=row_mask, q_fp8=qk)


@pytest.mark.parametrize("qk", [False, True], ids=["pv", "qk_pv"])
def test_pv_fp8_parity(case, qk):
    w, inp, gpu, oc = case
    bits = pa.ATTN_PREFILL_FP8_PV | (pa.ATTN_PREFILL_FP8_QK if qk else 0)
    out = run_fp8(gpu, inp, bits)
    torch.cuda.synchronize()
    ref = oracle.paged_attention(
        synth.bits(inp.q), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head,
        n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE, kv_dtype=oracle.KV_FP8,
        k_scale=oc.ks, v_scale=oc.vs, q_fp8=qk)
    err = np.abs(bf16_to_f64(out).reshape(ref.shape) - ref)
    lim = np.maximum(TOL[True], pv_bound(oc, inp.q, qk))
    say("[gpu]", w.name, "pv bits", bits, "max err", err.max(), "max err / limit",
        (err / lim).max())
    assert (err <= lim).all()


def test_pv_fp8_determinism(case):
    w, inp, gpu, oc = case
    bits = pa.ATTN_PREFILL_FP8_QK | pa.ATTN_PREFILL_FP8_PV
    a = run_fp8(gpu, inp, bits)
    b = run_fp8(gpu, inp, bits)
    torch.cuda.synchronize()
    assert same_bits(a, b)


def test_pv_fp8_scaled_values():
    """V pages of very different magnitudes (scales spanning 2^-20 .. 2^6):
    each tile's P takes its pages' scales over the largest one's power of
    two, and the output still meets its bound."""
    w = prefill_case("pv_scaled", 90, 700, 8, 2, 128, 69)
    inp = synth.draw(w, "cuda")
    f = 2.0 ** torch.tensor([-20.0, -3.0, 0.0, 6.0, -9.0], device="cuda")
    tok = torch.arange(inp.v_src.shape[0], device="cuda")
    inp.v_src.copy_((inp.v_src.float() * f[(tok // PAGE) % 5].view(-1, 1, 1)).to(torch.bfloat16))
    gpu = GpuCache(inp)
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    bits = pa.ATTN_PREFILL_FP8_QK | pa.ATTN_PREFILL_FP8_PV
    out = run_fp8(gpu, inp, bits)
    torch.cuda.synchronize()
    ref = oracle_fp8(oc, inp.q)
    err = np.abs(bf16_to_f64(out).reshape(ref.shape) - ref)
    lim = np.maximum(TOL[True] * np.abs(ref).max(), pv_bound(oc, inp.q, True))
    say("[gpu] pv scaled values max err", err.max(), "max err / limit", (err / lim).max())
    assert (err <= lim).all()


def test_pv_fp8_bad_page_gives_nan():
    w = prefill_case("pv_bad", 50, 500, 8, 2, 128, 70)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    table = inp.table.clone()
    table[0, 7] = -5
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_PV, table=table)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


def test_qk_pv_fp8_full_chunk_sampled_rows():
    """The 4,096-row chunk over 28,672 cached rows with an fp8 cache and both
    bits, in the launch the benchmark times; sampled rows against the oracle
    at the fp8 tolerance."""
    w = synth.scaled(synth.WORKLOADS["prefill_4096_over_28672"], kv_fp8=True,
                     name="prefill_4096_over_28672_fp8kv")
    say("[gpu] full fp8 prefill chunk, QK and PV bits")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = run_fp8(gpu, inp, pa.ATTN_PREFILL_FP8_QK | pa.ATTN_PREFILL_FP8_PV)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rows = sorted({0, 1, 31, 32, 4095} | set(range(0, 4096, 256)))
    mask = np.zeros((1, w.rows), bool)
    mask[0, rows] = True
    oc = OracleCache(inp)
    ref = oracle_fp8(oc, inp.q, row_mask=mask)
    err = max_err(out.view(1, w.rows, w.n_head, w.head_dim), ref, row_mask=mask)
    say("[gpu] full fp8 chunk QK+PV sampled rows", len(rows), "max abs err", err)
    assert err <= TOL[True]
    del gpu, inp
    torch.cuda.empty_cache()

