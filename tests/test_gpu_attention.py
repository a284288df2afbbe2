"""GPU parity of decode / verify and the append step against the CPU oracle,
and the bitwise invariants the oracle cannot pin (MI355X only).

Tolerance: on the named workloads, max abs error vs the fp64 oracle
<= 5e-3 with bf16 KV and <= 2e-2 with fp8 KV (sampled sequences); on the
small unit cases, whose contexts go down to one token so that |out| reaches
2-4, each element may also differ by half a bf16 ulp of the oracle value
(the output's own rounding).  The cache the oracle reads is built by the oracle's own append
from the same bf16 source, and the GPU's pool bytes must equal it exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import TOL, GpuCache, OracleCache, excess_err, max_err, same_bits, say

pytestmark = pytest.mark.gpu

L = synth.listed
SMALL = [
    L("dec_bf16_d128_g4", [1, 17, 511, 513, 1500], 1, 8, 2, 128, False, 11),
    L("dec_bf16_d256_g4", [33, 600, 1024, 2100], 1, 16, 4, 256, False, 12),
    L("dec_fp8_d128_g4", [1, 16, 100, 512, 1025, 2048, 2049, 3000, 4097], 1, 32, 8, 128, True,
      13),
    L("dec_fp8_d256_g2", [40, 700, 1600], 1, 8, 4, 256, True, 14),
    L("dec_bf16_d128_g1", [20, 530], 1, 4, 4, 128, False, 15),
    L("dec_bf16_d128_g8", [300, 1100], 1, 16, 2, 128, False, 16),
    L("dec_bf16_d128_g16", [64, 777], 1, 16, 1, 128, False, 17),
    L("dec_bf16_d128_g3", [45, 600], 1, 6, 2, 128, False, 18),
    L("ver_bf16_d256_g4", [8, 520, 1300], 8, 16, 4, 256, False, 21, kind="verify"),
    # 2052 and 2056: rounds across and at the start of a 2048-key split
    L("ver_fp8_d128_g4", [9, 512, 515, 2000, 2052, 2056], 8, 32, 8, 128, True, 22,
      kind="verify"),
    L("ver_bf16_d128_g8", [100, 1030], 8, 16, 2, 128, False, 23, kind="verify"),
    L("ver_bf16_d128_g1", [600], 8, 2, 2, 128, False, 24, kind="verify"),
    L("ver_fp8_d256_g2", [17, 1111], 8, 4, 2, 256, True, 25, kind="verify"),
    # four and eight slot tiles per call: sibling items at head_dim 256 / 128
    L("ver_bf16_d256_g8", [600, 1030], 8, 16, 2, 256, False, 26, kind="verify"),
    L("ver_bf16_d128_g16", [300, 1500], 8, 16, 1, 128, False, 27, kind="verify"),
    L("ver_fp8_d128_g16", [90, 2100], 8, 16, 1, 128, True, 28, kind="verify"),
]


@pytest.fixture(scope="module", params=SMALL, ids=[w.name for w in SMALL])
def small(request):
    w = request.param
    say("[gpu] case", w.name, "lengths", w.ctx_list)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run(w.kind)
    torch.cuda.synchronize()
    return w, inp, gpu, out


def test_small_pool_bytes_match_oracle_append(small):
    w, inp, gpu, out = small
    OracleCache(inp).check_pools_equal(gpu)


def test_small_parity(small):
    """Elementwise |gpu - oracle| <= tol + 1/2 ulp_bf16(|oracle|): these cases
    include contexts of a few tokens, where |out| reaches 2-4."""
    w, inp, gpu, out = small
    ref = OracleCache(inp).attend(inp.q)
    say("[gpu]", w.name, "max abs err", max_err(out, ref))
    assert excess_err(out, ref, TOL[w.kv_fp8]) <= 0


def test_one_workgroup_walks_every_item_bitwise(small):
    """With the grid bound to one workgroup, each wave walks many work items
    (the ring runs across item boundaries); output must not change by a bit."""
    w, inp, gpu, out = small
    pa.attn_set_max_workgroups(1)
    try:
        one = gpu.run(w.kind)
        torch.cuda.synchronize()
    finally:
        pa.attn_set_max_workgroups(0)
    assert same_bits(one, out)


def test_small_determinism(small):
    w, inp, gpu, out = small
    again = gpu.run(w.kind)
    torch.cuda.synchronize()
    assert same_bits(again, out)


def test_verify_rows_equal_decode_rows_bitwise(small):
    w, inp, gpu, out = small
    if w.kind != "verify":
        pytest.skip("verify cases only")
    for r in range(8):
        lens = inp.lengths - 8 + r + 1
        q1 = inp.q[:, r:r + 1].contiguous()
        dec = gpu.run("decode", q=q1, lengths=lens)
        torch.cuda.synchronize()
        assert same_bits(dec[:, 0], out[:, r]), "row %d" % r


@pytest.mark.parametrize("g", [4, 8])
def test_head_dim_256_rounds_equal_decode_rows_random_lengths(g):
    """bf16 rounds at head_dim 256 (the split kernel's LDS-ring form: both
    slot tiles of a (sequence, split, kv head) in one item) over lengths that
    put the round on split, tile and page boundaries and near the start:
    every row is bit for bit the decode row at its position, and the rows
    meet the oracle."""
    rng = np.random.default_rng(600 + g)
    lens = [8, 9, 15, 16, 17, 23, 24, 31, 511, 512, 513, 519, 520, 1023, 1031, 1536, 1543]
    lens += [int(c) for c in rng.integers(8, 2600, size=23)]
    w = synth.listed("ring_rand_g%d" % g, lens, 8, 4 * g, 4, 256, False, 610 + g, kind="verify")
    say("[gpu] head_dim 256 rounds, g", g, "lengths", lens)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("verify")
    torch.cuda.synchronize()
    for r in range(8):
        dec = gpu.run("decode", q=inp.q[:, r:r + 1].contiguous(), lengths=inp.lengths - 8 + r + 1)
        torch.cuda.synchronize()
        assert same_bits(dec[:, 0], out[:, r]), "row %d" % r
    seqs = [0, 4, 8, 11, 16, 30]
    ref = OracleCache(inp, seqs).attend(inp.q)
    assert excess_err(out.index_select(0, torch.tensor(seqs, device="cuda")), ref, TOL[False]) <= 0
    del gpu, inp
    torch.cuda.empty_cache()


def test_batch_invariance(small):
    """Each sequence alone, and the batch reversed, give the same bits."""
    w, inp, gpu, out = small
    S = inp.q.shape[0]
    for s in range(S):
        one = gpu.run(w.kind, q=inp.q[s:s + 1], lengths=inp.lengths[s:s + 1],
                      table=inp.table[s:s + 1])
        torch.cuda.synchronize()
        assert same_bits(one[0], out[s]), "sequence %d alone" % s
    rev = torch.arange(S - 1, -1, -1, device="cuda")
    o2 = gpu.run(w.kind, q=inp.q[rev].contiguous(), lengths=inp.lengths[rev].contiguous(),
                 table=inp.table[rev].contiguous())
    torch.cuda.synchronize()
    assert same_bits(o2[rev], out)


def test_page_relabelling_bitwise(small):
    w, inp, gpu, out = small
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    perm = torch.randperm(inp.n_pages, generator=gen, device="cuda")
    k2 = torch.empty_like(gpu.k)
    v2 = torch.empty_like(gpu.v)
    k2[perm] = gpu.k
    v2[perm] = gpu.v
    table = torch.where(inp.table >= 0, perm[inp.table.clamp(min=0).long()].int(), inp.table)
    relab = GpuCache.__new__(GpuCache)
    relab.inp, relab.kv = inp, gpu.kv
    relab.k, relab.v = k2, v2
    relab.ks = relab.vs = None
    if w.kv_fp8:
        relab.ks = torch.empty_like(gpu.ks)
        relab.vs = torch.empty_like(gpu.vs)
        relab.ks[perm] = gpu.ks
        relab.vs[perm] = gpu.vs
    o2 = relab.run(w.kind, table=table.contiguous())
    torch.cuda.synchronize()
    assert same_bits(o2, out)


def test_isolation_from_other_pages(small):
    """Poisoning every page another sequence owns leaves a sequence's output
    unchanged (unused pages and page tails are NaN from the start)."""
    w, inp, gpu, out = small
    S = inp.q.shape[0]
    if S < 2:
        pytest.skip("needs two sequences")
    need = (inp.lengths[1].item() + 15) // 16
    pages = inp.table[1, :need].long()
    k_save, v_save = gpu.k[pages].clone(), gpu.v[pages].clone()
    try:
        if w.kv_fp8:
            gpu.k[pages] = 0x7F
            gpu.v[pages] = 0x7F
        else:
            gpu.k[pages] = float("nan")
            gpu.v[pages] = float("nan")
        o2 = gpu.run(w.kind)
        torch.cuda.synchronize()
        keep = [s for s in range(S) if s != 1]
        assert same_bits(o2[keep], out[keep])
        assert torch.isnan(o2[1].float()).all()
    finally:
        gpu.k[pages] = k_save
        gpu.v[pages] = v_save


def test_device_side_bad_lengths_give_nan_rows():
    w = L("bad_len", [100, 200, 300], 1, 8, 2, 128, False, 31)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    good = gpu.run("decode")
    lens = inp.lengths.clone()
    lens[1] = 0                      # below the call's one row
    lens[2] = w.max_pages * 16 + 1   # beyond the table row
    bad = gpu.run("decode", lengths=lens)
    torch.cuda.synchronize()
    assert same_bits(bad[0], good[0])
    assert torch.isnan(bad[1:].float()).all()


def test_device_side_bad_page_gives_nan_rows():
    w = L("bad_page", [100, 200], 1, 8, 2, 128, False, 32)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    good = gpu.run("decode")
    table = inp.table.clone()
    table[1, 3] = inp.n_pages + 7    # outside the pool
    bad = gpu.run("decode", table=table)
    torch.cuda.synchronize()
    assert same_bits(bad[0], good[0])
    assert torch.isnan(bad[1].float()).all()


def test_fp8_v_codes_exhaustive():
    """One-token context with V scale 1: the output is the V codes' values
    (bf16 holds every e4m3 value exactly), so all 256 codes of the in-register
    conversion are checked against the format table."""
    H, Hk, d = 2, 1, 256
    n_pages = 2
    k = torch.zeros((n_pages, Hk, 16, d), dtype=torch.uint8, device="cuda")
    v = torch.zeros((n_pages, Hk, 16, d), dtype=torch.uint8, device="cuda")
    v[1, 0, 0] = torch.arange(256, dtype=torch.int32, device="cuda").to(torch.uint8)
    ks = torch.ones((n_pages, Hk), device="cuda")
    vs = torch.ones((n_pages, Hk), device="cuda")
    table = torch.tensor([[1, -1]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([1], dtype=torch.int32, device="cuda")
    q = torch.randn((1, 1, H, d), device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    wsb = pa.attn_paged_workspace_bytes(0, 1, 2, H, d)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    pa.attn_paged_decode(q, k, v, ks, vs, n_pages, table, 2, lens, 1, H, Hk, d, 16,
                         pa.KV_FP8_E4M3, out, ws, wsb)
    torch.cuda.synchronize()
    want = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    got = out[0, 0].float().cpu().double().numpy()
    for h in range(H):
        nan = np.isnan(want)
        np.testing.assert_array_equal(np.isnan(got[h]), nan)
        np.testing.assert_array_equal(got[h][~nan], want[~nan])


def test_append_fp8_incremental_matches_oracle():
    """A page written by two calls keeps the first call's scale (the call
    that wrote offset 0) and saturates later rows; decode-style single-row
    appends reuse stored scales."""
    w = L("inc", [37, 16, 5], 1, 8, 2, 128, True, 33)
    inp = synth.draw(w, "cuda")
    gk, gv, gks, gvs = synth.poison_pools(inp.n_pages, w, "cuda")
    ok = oracle.KV_FP8
    shape = (inp.n_pages, w.n_head_kv, 16, w.head_dim)
    ok_k = np.full(shape, 0x7F, np.uint8)
    ok_v = np.full(shape, 0x7F, np.uint8)
    ok_ks = np.full((inp.n_pages, w.n_head_kv), np.nan, np.float32)
    ok_vs = ok_ks.copy()
    n = inp.slots.numel()
    ksrc = inp.k_src.clone()
    ksrc[n // 2:] *= 4  # later rows larger than the scale the first call set
    cuts = [0, 7, n // 2, n - 1, n]
    for a, b in zip(cuts[:-1], cuts[1:]):
        pa.attn_kv_append(ksrc[a:b], inp.v_src[a:b], inp.slots[a:b], b - a, gk, gv, gks, gvs,
                          inp.n_pages, w.n_head_kv, w.head_dim, 16, pa.KV_FP8_E4M3)
        oracle.kv_append(synth.bits(ksrc[a:b]), synth.bits(inp.v_src[a:b]),
                         synth.bits(inp.slots[a:b]), ok_k, ok_v, ok_ks, ok_vs,
                         n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=16, kv_dtype=ok)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(synth.bits(gk), ok_k)
    np.testing.assert_array_equal(synth.bits(gv), ok_v)
    np.testing.assert_array_equal(gks.cpu().numpy(), ok_ks)
    np.testing.assert_array_equal(gvs.cpu().numpy(), ok_vs)


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times.
# ---------------------------------------------------------------------------

def _sample_seqs(lengths: torch.Tensor, k: int):
    lens = lengths.cpu().numpy()
    order = np.argsort(lens, kind="stable")
    picks = {int(order[0]), int(order[-1])}
    for q in np.linspace(0, len(lens) - 1, k):
        picks.add(int(order[int(round(q))]))
    return sorted(picks)


@pytest.mark.parametrize("name,k", [("decode_1seq_ctx512", 1), ("decode_64seq_hd256", 8),
                                    ("verify_32seq_8rows", 4), ("decode_256seq_fp8", 16)])
def test_full_workload_sampled_parity(name, k):
    w = synth.WORKLOADS[name]
    say("[gpu] full workload", name)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run(w.kind)
    torch.cuda.synchronize()
    seqs = _sample_seqs(inp.lengths, k)
    oc = OracleCache(inp, seqs)
    oc.check_pools_equal(gpu)
    ref = oc.attend(inp.q)
    err = max_err(out, ref, seqs=seqs)
    say("[gpu]", name, "sampled seqs", seqs, "max abs err", err)
    assert err <= TOL[w.kv_fp8]
    assert torch.isfinite(out.float()).all()
    if w.kind == "verify":
        for r in (0, 3, 7):
            dec = gpu.run("decode", q=inp.q[:, r:r + 1].contiguous(),
                          lengths=inp.lengths - 8 + r + 1)
            torch.cuda.synchronize()
            assert same_bits(dec[:, 0], out[:, r])
    del gpu, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_64seq_hd256", "verify_32seq_8rows"])
def test_full_workload_every_element(name):
    """Every output element of a full-size bf16 workload against the oracle
    over every sequence.  (The fp8 workload's 2.7 million cached tokens would
    take the oracle's one-thread E4M3 append minutes; it is sampled above.)"""
    w = synth.WORKLOADS[name]
    say("[gpu] full workload, every element", name)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run(w.kind)
    torch.cuda.synchronize()
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    ref = oc.attend(inp.q)
    err = max_err(out, ref)
    say("[gpu]", name, "all", w.n_seq, "sequences, max abs err", err)
    assert err <= TOL[w.kv_fp8]
    del gpu, inp, oc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["decode", "verify"])
def test_score_jump_inside_tile(kind):
    """Keys [40, 56) score 11.3 (q = k = 1 at head_dim 128), the rest 0, with
    V = -1 there and +1 elsewhere: the row max jumps by more than 2^8 inside
    one key tile."""
    rows = 1 if kind == "decode" else 8
    w = synth.listed("jump_" + kind, [90, 300], rows, 8, 2, 128, False, 51, kind=kind)
    inp = synth.draw(w, "cuda")
    k = torch.zeros_like(inp.k_src)
    v = torch.ones_like(inp.v_src)
    for s0 in (0, 90):  # both sequences' tokens
        k[s0 + 40:s0 + 56] = 1.0
        v[s0 + 40:s0 + 56] = -1.0
    inp.k_src, inp.v_src = k, v
    inp.q = torch.ones_like(inp.q)
    gpu = GpuCache(inp)
    out = gpu.run(kind)
    torch.cuda.synchronize()
    ref = OracleCache(inp).attend(inp.q)
    say("[gpu] score jump", kind, "max abs err", max_err(out, ref))
    assert excess_err(out, ref, TOL[False]) <= 0
