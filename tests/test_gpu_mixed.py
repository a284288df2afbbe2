"""GPU parity of the mixed step (decode rows beside prefill chunks in one
call) against the CPU oracle, and its row invariance: every decode row is
bit for bit the plain decode call's and every chunk row the plain prefill
call's (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, GpuCache, OracleCache, excess_err, max_err, same_bits, say

pytestmark = pytest.mark.gpu


def make_step(name, dec_lens, chunks, H, Hk, d, fp8, seed):
    """Sequences: decode ones (ctx each), then chunk ones ((ctx, rows) each).
    Returns the cache inputs, the token-major q, cu_seqlens and row counts."""
    lens = list(dec_lens) + [c for c, _ in chunks]
    w = synth.listed(name, lens, 1, H, Hk, d, fp8, seed)
    inp = synth.draw(w, "cuda")
    q_rows = [1] * len(dec_lens) + [r for _, r in chunks]
    n_tok = sum(q_rows)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 7)
    q = synth.normal_bf16((n_tok, H, d), gen)
    cu = np.concatenate([[0], np.cumsum(q_rows)]).astype(np.int32)
    return w, inp, q, cu, q_rows


def run_mixed(gpu, w, inp, q, cu, n_dec, max_q_len=None, lengths=None, out=None):
    n_seq = len(cu) - 1
    n_tok = int(cu[-1])
    max_q_len = max(int(np.max(np.diff(cu)[n_dec:])) if n_seq > n_dec else 1, 1) \
        if max_q_len is None else max_q_len
    lengths = inp.lengths if lengths is None else lengths
    out = torch.empty_like(q) if out is None else out
    wsb = pa.attn_paged_workspace_bytes(3, max(n_dec, 1), inp.table.shape[1], w.n_head,
                                        w.head_dim)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    pa.attn_paged_mixed(q, n_tok, cu_d, n_seq, n_dec, max_q_len, gpu.k, gpu.v, gpu.ks, gpu.vs,
                        inp.n_pages, inp.table, inp.table.shape[1], lengths, w.n_head,
                        w.n_head_kv, w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    return out


def oracle_rows(inp, s, q_rows_t):
    """fp64 attention of the given token rows of sequence s (its last rows)."""
    w = inp.w
    oc = OracleCache(inp, seqs=[s])
    qb = synth.bits(q_rows_t)[None]
    return oracle.paged_attention(
        qb, oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head, n_head_kv=w.n_head_kv,
        head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=oc.ks,
        v_scale=oc.vs)[0]


STEPS = [
    ("mx_bf16_g4", [700, 33, 1025, 512, 90], [(300, 300), (1000, 77), (513, 64)], 8, 2, 128,
     False),
    ("mx_fp8_d256", [2000, 17], [(1500, 130)], 16, 4, 256, True),
    # fp8 at head_dim 128: the chunk half in four-wave workgroups beside the decode
    ("mx_fp8_d128", [3000, 17, 1024, 700], [(2048, 200), (600, 64), (90, 90)], 32, 8, 128,
     True),
    ("mx_g8_chunks_only", [], [(40, 40), (900, 129)], 32, 4, 128, False),
    ("mx_decode_only", [100, 5000, 640], [], 8, 2, 128, False),
]


@pytest.fixture(scope="module", params=STEPS, ids=[s[0] for s in STEPS])
def step(request):
    name, dec, chunks, H, Hk, d, fp8 = request.param
    say("[gpu] mixed step", name, "decode", dec, "chunks", chunks)
    w, inp, q, cu, q_rows = make_step(name, dec, chunks, H, Hk, d, fp8, 60)
    gpu = GpuCache(inp)
    out = run_mixed(gpu, w, inp, q, cu, len(dec))
    torch.cuda.synchronize()
    return w, inp, q, cu, len(dec), gpu, out


def test_mixed_parity(step):
    w, inp, q, cu, n_dec, gpu, out = step
    worst = -1.0
    for s in range(len(cu) - 1):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        ref = oracle_rows(inp, s, q[rows])
        worst = max(worst, excess_err(out[rows], ref, TOL[w.kv_fp8]))
        assert excess_err(out[rows], ref, TOL[w.kv_fp8]) <= 0, s
    say("[gpu] mixed", w.name, "worst excess", worst)


def test_mixed_rows_equal_plain_calls(step):
    w, inp, q, cu, n_dec, gpu, out = step
    if n_dec:
        qd = q[:n_dec].reshape(n_dec, 1, w.n_head, w.head_dim)
        dec = gpu.run("decode", q=qd, lengths=inp.lengths[:n_dec], table=inp.table[:n_dec],
                      n_seq=n_dec)
        torch.cuda.synchronize()
        assert same_bits(dec.reshape(n_dec, w.n_head, w.head_dim), out[:n_dec])
    for s in range(n_dec, len(cu) - 1):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        n = rows.stop - rows.start
        pf = torch.empty_like(q[rows])
        pa.attn_paged_prefill(q[rows], n, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages,
                              inp.table[s], inp.table.shape[1], int(inp.lengths[s]), w.n_head,
                              w.n_head_kv, w.head_dim, PAGE, gpu.kv, pf)
        torch.cuda.synchronize()
        assert same_bits(pf, out[rows]), s


def test_mixed_skips_a_bad_chunk_and_keeps_the_rest():
    """A chunk whose device length is below its rows is skipped (its rows
    keep what out held); the other rows are unaffected."""
    w, inp, q, cu, q_rows = make_step("mx_bad", [300, 64], [(200, 50), (400, 20)], 8, 2, 128,
                                      False, 61)
    gpu = GpuCache(inp)
    good = run_mixed(gpu, w, inp, q, cu, 2)
    lengths = inp.lengths.clone()
    lengths[2] = 10  # below that chunk's 50 rows
    sentinel = torch.full_like(q, 7.0)
    out = run_mixed(gpu, w, inp, q, cu, 2, lengths=lengths, out=sentinel)
    torch.cuda.synchronize()
    bad = slice(int(cu[2]), int(cu[3]))
    assert bool((out[bad].float() == 7.0).all())
    keep = torch.ones(q.shape[0], dtype=torch.bool, device=q.device)
    keep[bad] = False
    assert same_bits(out[keep], good[keep])


def test_mixed_larger_max_q_len_changes_nothing(step):
    """max_q_len only sizes the grid: a looser bound gives the same bits."""
    w, inp, q, cu, n_dec, gpu, out = step
    if n_dec == len(cu) - 1:
        pytest.skip("no chunk half")
    loose = int(cu[-1]) - n_dec
    again = run_mixed(gpu, w, inp, q, cu, n_dec, max_q_len=loose)
    torch.cuda.synchronize()
    assert same_bits(again, out)
