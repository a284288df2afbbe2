"""Parity at the shapes and in the launches the benchmark's extended lines
time (MI355X only): the 256-sequence fp8 decode with a 4096-key window,
rounds of widths 1/2/4/8 and 8-row tree rounds over the 32-sequence verify
cache, and the mixed step of 256 decode rows and a 2048-row chunk.  Sampled
sequences and rows against the oracle (the full outputs are checked finite)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, GpuCache, OracleCache, max_err, say
from test_gpu_tree import oracle_view, oracle_view_attention, run_tree, scratch_for

pytestmark = pytest.mark.gpu


def spread(lens, k=5):
    """Sequences at the minimum, quartiles and maximum of the lengths."""
    order = np.argsort(np.asarray(lens), kind="stable")
    return sorted({int(order[int(round(q * (len(order) - 1)))]) for q in np.linspace(0, 1, k)})


def kv_of(w):
    return oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16


def test_window_4096_on_the_fp8_decode_workload():
    w = synth.WORKLOADS["decode_256seq_fp8"]
    say("[gpu] bench shape: decode_256seq_fp8, window 4096")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    wsb = pa.attn_paged_workspace_bytes(1, w.n_seq, w.max_pages, w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp.q)
    pa.attn_paged_decode_window(inp.q, 1, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                                w.max_pages, inp.lengths, w.n_seq, 4096, None, w.n_head,
                                w.n_head_kv, w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    seqs = spread(inp.lengths.cpu().tolist())
    oc = OracleCache(inp, seqs)
    ref = oracle.paged_attention(
        synth.bits(inp.q[seqs]), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head,
        n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE, kv_dtype=kv_of(w),
        k_scale=oc.ks, v_scale=oc.vs, window=4096)
    err = max_err(out, ref, seqs)
    say("[gpu] window 4096 sampled seqs", seqs, "max abs err", err)
    assert err <= TOL[True]
    del gpu, inp
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def verify_cache():
    w = synth.WORKLOADS["verify_32seq_8rows"]
    need = sum(-(-c // PAGE) for c in synth.draw_lengths(
        w, torch.Generator(device="cpu").manual_seed(w.seed)).tolist())
    w = synth.scaled(w, pool_pages=need + w.n_seq + 2 * w.n_seq * 8)  # room for tree views
    say("[gpu] bench shape: verify_32seq_8rows")
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    yield w, inp, gpu
    del gpu, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("width", [1, 2, 4, 8])
def test_widths_on_the_verify_workload(verify_cache, width):
    w, inp, gpu = verify_cache
    q = inp.q[:, :width].contiguous()
    wsb = pa.attn_paged_workspace_bytes(1, w.n_seq, w.max_pages, w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    pa.attn_paged_verify_width(q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                               w.max_pages, inp.lengths, w.n_seq, width, w.n_head, w.n_head_kv,
                               w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    seqs = [0, 13, 31]
    oc = OracleCache(inp, seqs)
    ref = oracle.paged_attention(
        synth.bits(q[seqs]), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head,
        n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE, kv_dtype=kv_of(w))
    err = max_err(out, ref, seqs)
    say("[gpu] width", width, "sampled seqs", seqs, "max abs err", err)
    assert err <= TOL[False]


def test_tree8_on_the_verify_workload(verify_cache):
    w, inp, gpu = verify_cache
    masks = synth.tree_masks(w.n_seq, 8, 1008)  # the benchmark's trees
    out = run_tree(gpu, inp, masks, scratch_for(inp))
    assert torch.isfinite(out.float()).all()
    oc = OracleCache(inp)
    worst = 0.0
    for s in (0, 31):
        for r in range(8):
            ref = oracle_view_attention(inp, s, r, oracle_view(oc, inp, s, r, int(masks[s, r])))
            worst = max(worst, float(np.max(np.abs(out[s, r].float().cpu().double().numpy()
                                                   - ref))))
    say("[gpu] tree8 sampled seqs 0, 31 max abs err", worst)
    assert worst <= TOL[False]


def test_mixed_step_of_the_benchmark():
    w, inp, q, cu, lens = synth.mixed_step()
    say("[gpu] bench shape: mixed step")
    gpu = GpuCache(inp)
    mp = inp.table.shape[1]
    wsb = pa.attn_paged_workspace_bytes(3, 256, mp, w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    pa.attn_paged_mixed(q, int(q.shape[0]), cu, 257, 256, 2048, gpu.k, gpu.v, gpu.ks, gpu.vs,
                        inp.n_pages, inp.table, mp, inp.lengths, w.n_head, w.n_head_kv,
                        w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # decode rows of sampled sequences
    seqs = spread(lens[:256])
    oc = OracleCache(inp, seqs)
    qd = synth.bits(q[seqs]).reshape(len(seqs), 1, w.n_head, w.head_dim)
    ref = oracle.paged_attention(qd, oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head,
                                 n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
                                 kv_dtype=kv_of(w), k_scale=oc.ks, v_scale=oc.vs)
    err_d = float(np.max(np.abs(out[seqs].float().cpu().double().numpy() - ref[:, 0])))
    # sampled rows of the chunk (sequence 256)
    rows = sorted({0, 1, 1023, 2047} | set(range(0, 2048, 128)))
    mask = np.zeros((1, 2048), bool)
    mask[0, rows] = True
    oc2 = OracleCache(inp, [256])
    qc = synth.bits(q[256:]).reshape(1, 2048, w.n_head, w.head_dim)
    ref2 = oracle.paged_attention(qc, oc2.k, oc2.v, oc2.table, oc2.lens, n_head=w.n_head,
                                  n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
                                  kv_dtype=kv_of(w), k_scale=oc2.ks, v_scale=oc2.vs,
                                  row_mask=mask)
    got = out[256:].float().cpu().double().numpy()[rows]
    err_c = float(np.max(np.abs(got - ref2[0, rows])))
    say("[gpu] mixed step: decode seqs", seqs, "max abs err", err_d, "chunk rows", len(rows),
        "max abs err", err_c)
    assert err_d <= TOL[True] and err_c <= TOL[True]
    del gpu, inp
    torch.cuda.empty_cache()
