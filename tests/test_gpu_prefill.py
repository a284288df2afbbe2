"""GPU parity of the prefill chunk against the CPU oracle (MI355X only).

Small cases cover ragged position blocks, chunks that are the whole context
and chunks after cached rows, GQA groups 1..8 and both KV dtypes, with the
elementwise bound tol + 1/2 ulp_bf16(|oracle|); the full 4096-row chunk over
28,672 cached rows is checked on 316 sampled rows (every head) with the plain bound.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_20_amd import synth
from gpu_util import TOL, GpuCache, OracleCache, excess_err, max_err, same_bits, say

pytestmark = pytest.mark.gpu


def prefill_case(name, n_rows, ctx, H, Hk, d, fp8, seed):
    return synth.Workload(name, 1, n_rows, H, Hk, d, fp8, "fixed", ctx, ctx, seed,
                          kind="prefill")


CASES = [
    prefill_case("pf_whole_ctx_g4", 40, 40, 8, 2, 128, False, 41),
    prefill_case("pf_over_cache_d256", 100, 1000, 16, 4, 256, False, 42),
    prefill_case("pf_g1_fp8", 77, 300, 8, 8, 128, True, 43),
    prefill_case("pf_g8", 130, 700, 32, 4, 128, False, 44),
    prefill_case("pf_fp8_d256", 64, 2000, 16, 4, 256, True, 45),
    prefill_case("pf_one_row", 1, 1, 8, 2, 128, False, 46),
    prefill_case("pf_g2_d256", 33, 1234, 4, 2, 256, False, 47),
    prefill_case("pf_long_chunk", 600, 650, 8, 2, 128, False, 48),
]


@pytest.fixture(scope="module", params=CASES, ids=[w.name for w in CASES])
def case(request):
    w = request.param
    say("[gpu] prefill case", w.name, "rows", w.rows, "ctx", w.ctx_lo)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("prefill")
    torch.cuda.synchronize()
    return w, inp, gpu, out


def test_prefill_parity(case):
    w, inp, gpu, out = case
    ref = OracleCache(inp).attend(inp.q)
    say("[gpu]", w.name, "max abs err", max_err(out, ref))
    assert excess_err(out, ref, TOL[w.kv_fp8]) <= 0


def test_prefill_determinism(case):
    w, inp, gpu, out = case
    again = gpu.run("prefill")
    torch.cuda.synchronize()
    assert same_bits(again, out)


def test_prefill_bad_page_gives_nan():
    w = prefill_case("pf_bad", 50, 500, 8, 2, 128, False, 49)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    table = inp.table.clone()
    table[0, 5] = -3
    out = gpu.run("prefill", table=table)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


def test_prefill_full_chunk_sampled_rows():
    w = synth.WORKLOADS["prefill_4096_over_28672"]
    say("[gpu] full prefill chunk")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("prefill")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # every 16th row, and every row of the first and last 32 positions (the
    # heads of a position block sit 32 rows apart in a workgroup)
    rows = sorted(set(range(0, 4096, 16)) | set(range(32)) | set(range(4064, 4096)))
    mask = np.zeros((1, w.rows), bool)
    mask[0, rows] = True
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    ref = oc.attend(inp.q, row_mask=mask)
    err = max_err(out, ref, row_mask=mask)
    say("[gpu] full prefill sampled rows", len(rows), "max abs err", err)
    assert err <= TOL[False]
    del gpu, inp
    torch.cuda.empty_cache()


def _score_jump_inputs(w, lo, hi):
    """Keys [lo, hi) score 11.3 (q = k = 1 at head_dim 128), every other key
    scores 0; V is +1 on the other keys and -1 on [lo, hi).  The row max
    jumps by more than 2^8 inside one key tile, so a tile's rescale must
    cover all of its scores."""
    inp = synth.draw(w, "cuda")
    k = torch.zeros_like(inp.k_src)
    v = torch.ones_like(inp.v_src)
    k[lo:hi] = 1.0
    v[lo:hi] = -1.0
    inp.k_src, inp.v_src = k, v
    inp.q = torch.ones_like(inp.q)
    return inp


@pytest.mark.parametrize("lo,hi", [(32, 64), (48, 64), (16, 32), (100, 130)])
def test_prefill_score_jump_inside_tile(lo, hi):
    w = prefill_case("pf_jump", 8, 160, 8, 2, 128, False, 50)
    inp = _score_jump_inputs(w, lo, hi)
    gpu = GpuCache(inp)
    out = gpu.run("prefill")
    torch.cuda.synchronize()
    ref = OracleCache(inp).attend(inp.q)
    say("[gpu] prefill score jump", lo, hi, "max abs err", max_err(out, ref))
    assert excess_err(out, ref, TOL[False]) <= 0
