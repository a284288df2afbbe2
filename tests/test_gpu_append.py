"""fp8 pages filled over many calls (MI355X only): one token per sequence
per call (the decode pattern) and runs of three tokens (verify-like).  A
page's first rows set its scale, so later rows often outgrow it and the call
must grow the scale and re-encode the page's earlier codes.  The GPU's codes
and scales equal the oracle's append of the same calls, byte for byte, and
attention over the result stays within the fp8 tolerance of attention over
the bf16 rows (contexts of 640 keys; at a few hundred keys quantising each
page even in one call costs about that much) and no further from it than
pages quantised in one call."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, bf16_to_f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,per_call", [(128, 1), (256, 1), (128, 3)])
def test_fp8_pages_built_over_many_calls_match_oracle(d, per_call):
    S, C, H, Hk = 3, 640, 8, 2
    w = synth.listed("app_calls_d%d_r%d" % (d, per_call), [C] * S, 1, H, Hk, d, True, 71)
    inp = synth.draw(w, "cuda")
    say("[gpu] fp8 append over calls", w.name)
    k_src, v_src = inp.k_src, inp.v_src
    gk, gv, gks, gvs = synth.poison_pools(inp.n_pages, w, "cuda")
    shape = (inp.n_pages, Hk, PAGE, d)
    ok, ov = np.full(shape, 0x7F, np.uint8), np.full(shape, 0x7F, np.uint8)
    oks = np.full((inp.n_pages, Hk), np.nan, np.float32)
    ovs = np.full((inp.n_pages, Hk), np.nan, np.float32)
    kb, vb = synth.bits(k_src), synth.bits(v_src)
    slots = inp.slots.cpu().numpy()
    grew = 0
    for t0 in range(0, C, per_call):
        rows = np.array([s * C + t for s in range(S) for t in range(t0, min(t0 + per_call, C))])
        rows_t = torch.from_numpy(rows).cuda()
        before = oks.copy()
        pa.attn_kv_append(k_src.index_select(0, rows_t), v_src.index_select(0, rows_t),
                          inp.slots.index_select(0, rows_t), len(rows), gk, gv, gks, gvs,
                          inp.n_pages, Hk, d, PAGE, pa.KV_FP8_E4M3)
        oracle.kv_append(kb[rows], vb[rows], slots[rows], ok, ov, oks, ovs, n_head_kv=Hk,
                         head_dim=d, page_size=PAGE, kv_dtype=oracle.KV_FP8)
        if t0 % PAGE:
            grew += int(np.sum(oks > before))
    torch.cuda.synchronize()
    assert grew > 0  # the case exercises scale growth
    np.testing.assert_array_equal(gk.cpu().numpy(), ok)
    np.testing.assert_array_equal(gv.cpu().numpy(), ov)
    np.testing.assert_array_equal(gks.cpu().numpy().view(np.uint32), oks.view(np.uint32))
    np.testing.assert_array_equal(gvs.cpu().numpy().view(np.uint32), ovs.view(np.uint32))
    # attention over the fp8 pages against attention over the bf16 rows
    wsb = pa.attn_paged_workspace_bytes(0, S, inp.table.shape[1], H, d)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp.q)
    pa.attn_paged_decode(inp.q, gk, gv, gks, gvs, inp.n_pages, inp.table, inp.table.shape[1],
                         inp.lengths, S, H, Hk, d, PAGE, pa.KV_FP8_E4M3, out, ws, wsb)
    torch.cuda.synchronize()
    bk, bv = np.full(shape, 0x7FC0, np.uint16), np.full(shape, 0x7FC0, np.uint16)
    oracle.kv_append(kb, vb, slots, bk, bv, n_head_kv=Hk, head_dim=d, page_size=PAGE)
    ref = oracle.paged_attention(synth.bits(inp.q), bk, bv, inp.table.cpu().numpy(),
                                 inp.lengths.cpu().numpy(), n_head=H, n_head_kv=Hk,
                                 head_dim=d, page_size=PAGE)
    err = np.abs(bf16_to_f64(out) - ref).max()
    # the same rows quantised with each page written in one call
    wk, wv = np.full(shape, 0x7F, np.uint8), np.full(shape, 0x7F, np.uint8)
    wks = np.full((inp.n_pages, Hk), np.nan, np.float32)
    wvs = np.full((inp.n_pages, Hk), np.nan, np.float32)
    oracle.kv_append(kb, vb, slots, wk, wv, wks, wvs, n_head_kv=Hk, head_dim=d,
                     page_size=PAGE, kv_dtype=oracle.KV_FP8)
    one = oracle.paged_attention(synth.bits(inp.q), wk, wv, inp.table.cpu().numpy(),
                                 inp.lengths.cpu().numpy(), n_head=H, n_head_kv=Hk,
                                 head_dim=d, page_size=PAGE, kv_dtype=oracle.KV_FP8,
                                 k_scale=wks, v_scale=wvs)
    err_one = np.abs(one - ref).max()
    say("[gpu]", w.name, "scale growths", grew, "max err vs bf16 rows", err,
        "(pages quantised in one call: %.4f)" % err_one)
    assert err <= TOL[True]
    assert err <= 1.25 * err_one
