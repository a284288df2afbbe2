"""GPU parity of speculative rounds of every width 1..8 (causal chains after
the cached context) against the CPU oracle, and the bitwise rule that each
round row equals the decode row at its position (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, GpuCache, OracleCache, excess_err, same_bits, say

pytestmark = pytest.mark.gpu

L = synth.listed
CONFIGS = [
    L("vw_bf16_d256_g4", [8, 300, 515, 1100], 8, 16, 4, 256, False, 71),
    L("vw_fp8_d128_g4", [9, 512, 1030], 8, 32, 8, 128, True, 72),
    L("vw_bf16_d128_g8", [40, 700], 8, 16, 2, 128, False, 73),
    L("vw_bf16_d128_g1", [20, 530], 8, 4, 4, 128, False, 74),
    L("vw_fp8_d256_g2", [17, 640], 8, 8, 4, 256, True, 75),
]


@pytest.fixture(scope="module", params=CONFIGS, ids=[w.name for w in CONFIGS])
def cfg(request):
    w = request.param
    say("[gpu] verify-width config", w.name, "lengths", w.ctx_list)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    return w, inp, gpu


def run_width(gpu, inp, q, width, lengths=None):
    w = inp.w
    lengths = inp.lengths if lengths is None else lengths
    n_seq = q.shape[0]
    wsb = pa.attn_paged_workspace_bytes(1, n_seq, inp.table.shape[1], w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    pa.attn_paged_verify_width(q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                               inp.table.shape[1], lengths, n_seq, width, w.n_head, w.n_head_kv,
                               w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    return out


@pytest.mark.parametrize("width", range(1, 9))
def test_width_parity_and_rows_equal_decode(cfg, width):
    w, inp, gpu = cfg
    q = inp.q[:, :width].contiguous()
    out = run_width(gpu, inp, q, width)
    torch.cuda.synchronize()
    oc = OracleCache(inp)
    ref = oracle.paged_attention(
        synth.bits(q), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head, n_head_kv=w.n_head_kv,
        head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=oc.ks, v_scale=oc.vs)
    ex = excess_err(out, ref, TOL[w.kv_fp8])
    say("[gpu]", w.name, "width", width, "excess", ex)
    assert ex <= 0
    for r in range(width):
        lens = inp.lengths - width + r + 1
        dec = gpu.run("decode", q=q[:, r:r + 1].contiguous(), lengths=lens)
        torch.cuda.synchronize()
        assert same_bits(dec[:, 0], out[:, r]), "row %d" % r


def test_width_8_is_verify(cfg):
    w, inp, gpu = cfg
    out = run_width(gpu, inp, inp.q, 8)
    ver = gpu.run("verify")
    torch.cuda.synchronize()
    assert same_bits(out, ver)


def test_width_1_is_decode(cfg):
    w, inp, gpu = cfg
    q = inp.q[:, :1].contiguous()
    out = run_width(gpu, inp, q, 1)
    dec = gpu.run("decode", q=q)
    torch.cuda.synchronize()
    assert same_bits(out, dec)
