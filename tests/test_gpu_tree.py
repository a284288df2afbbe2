"""GPU parity of tree-shaped speculative rounds (MI355X only).

Row r of a round attends the cached context plus the round rows its mask
names.  The oracle lays that branch out as a plain sequence (oracle.tree_view:
bytes copied; with fp8, rows moved down into the previous page re-encoded at
its scale).  Each tree row must equal, bit for bit, the GPU decode of the same
row over that view, and lie within tolerance of the CPU oracle over it; the
view pages the call builds must equal the oracle's byte for byte.  A chain
mask gives the width-R round.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, GpuCache, OracleCache, excess_err, same_bits, say

pytestmark = pytest.mark.gpu


def tree_workload(name, lens, R, H, Hk, d, fp8, seed):
    need = sum(-(-c // PAGE) for c in lens)
    return synth.Workload(name, len(lens), R, H, Hk, d, fp8, "list", min(lens), max(lens), seed,
                          pool_pages=need + len(lens) + 2 * len(lens) * R, kind="verify",
                          ctx_list=tuple(lens))


def random_masks(S, R, seed, chain=False):
    rng = np.random.default_rng(seed)
    masks = np.zeros((S, R), np.int32)
    for s in range(S):
        for r in range(R):
            parent = r - 1 if chain else int(rng.integers(-1, r))
            masks[s, r] = (1 << r) | (masks[s, parent] if parent >= 0 else 0)
    return masks


def scratch_for(inp):
    S, R = inp.q.shape[0], inp.q.shape[1]
    used = set(int(p) for p in inp.table.cpu().numpy().ravel() if p >= 0)
    free = [p for p in range(inp.n_pages) if p not in used]
    assert len(free) >= 2 * S * R
    return torch.tensor(free[:2 * S * R], dtype=torch.int32, device="cuda").view(S, R, 2)


def run_tree(gpu, inp, masks, scratch):
    w = inp.w
    S, R = inp.q.shape[0], inp.q.shape[1]
    wsb = pa.attn_paged_workspace_bytes(4, S, inp.table.shape[1], w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp.q)
    pa.attn_paged_verify_tree(inp.q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                              inp.table.shape[1], inp.lengths, S, R,
                              torch.from_numpy(masks).cuda(), scratch, w.n_head, w.n_head_kv,
                              w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    torch.cuda.synchronize()
    return out


def branch_positions(C, R, mask):
    C0 = C - R
    return list(range(C0)) + [C0 + j for j in range(R) if mask >> j & 1]


def oracle_view(oc, inp, s, r, mask):
    w = inp.w
    R = inp.q.shape[1]
    return oracle.tree_view(oc.k, oc.v, oc.ks, oc.vs, oc.table[s], int(oc.lens[s]), R, mask, r,
                            n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
                            kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16)


def gpu_view_decode(gpu, inp, s, r, view):
    """GPU decode of row (s, r) over the oracle's view of its branch."""
    w = inp.w
    k2, v2, ks2, vs2, n = view
    npg = k2.shape[0]
    k2 = torch.from_numpy(k2).cuda().view(gpu.k.dtype)
    v2 = torch.from_numpy(v2).cuda().view(gpu.v.dtype)
    if ks2 is not None:
        ks2, vs2 = torch.from_numpy(ks2).cuda(), torch.from_numpy(vs2).cuda()
    table = torch.arange(npg, dtype=torch.int32, device="cuda").view(1, npg)
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    q = inp.q[s, r].reshape(1, 1, w.n_head, w.head_dim).contiguous()
    out = torch.empty_like(q)
    wsb = pa.attn_paged_workspace_bytes(0, 1, npg, w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    pa.attn_paged_decode(q, k2, v2, ks2, vs2, npg, table, npg, lens, 1, w.n_head, w.n_head_kv,
                         w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    torch.cuda.synchronize()
    return out[0, 0]


def oracle_view_attention(inp, s, r, view):
    w = inp.w
    k2, v2, ks2, vs2, n = view
    npg = k2.shape[0]
    q = synth.bits(inp.q[s, r]).reshape(1, 1, w.n_head, w.head_dim)
    return oracle.paged_attention(
        q, k2, v2, np.arange(npg, dtype=np.int32).reshape(1, npg), np.array([n], np.int32),
        n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=ks2, v_scale=vs2)[0, 0]


def check_view_pages(gpu, inp, s, r, scratch, view):
    """The call's private pages hold the oracle's view pages of the round
    (rows below the view's length; scales with fp8)."""
    k2, v2, ks2, vs2, n = view
    R = inp.q.shape[1]
    tp = (int(inp.lengths[s]) - R) // PAGE
    for i, vp in enumerate(range(tp, k2.shape[0])):
        pg = int(scratch[s, r, i])
        rows = min(PAGE, n - vp * PAGE)
        for pool, ref in ((gpu.k, k2), (gpu.v, v2)):
            got = pool[pg, :, :rows].contiguous().view(torch.uint8).cpu().numpy()
            want = np.ascontiguousarray(ref[vp, :, :rows]).view(np.uint8)
            np.testing.assert_array_equal(got, want, err_msg=str((s, r, vp)))
        if ks2 is not None:
            np.testing.assert_array_equal(gpu.ks[pg].cpu().numpy(), ks2[vp])
            np.testing.assert_array_equal(gpu.vs[pg].cpu().numpy(), vs2[vp])


def moved_rows(C, R, mask):
    """Round rows of the branch that land in an earlier page than their own."""
    C0 = C - R
    js = [j for j in range(R) if mask >> j & 1]
    return sum(1 for i, j in enumerate(js) if (C0 + j) // PAGE > (C0 + i) // PAGE)


CASES = [
    # 1029 - 8 and 2051 - 8 put a round across a 512-key split boundary
    tree_workload("tr_bf16_d128_g4", [8, 300, 531, 1029, 1300, 2051], 8, 8, 2, 128, False, 111),
    tree_workload("tr_bf16_d256_g4_w5", [12, 700, 1029, 1538], 5, 16, 4, 256, False, 112),
    # 16 heads per kv head: the round's split kernel does not serve 3 rows at
    # head_dim 256 (or 8 at 128), so every view is decoded alone
    tree_workload("tr_bf16_d256_g16_w3", [5, 514, 900], 3, 32, 2, 256, False, 115),
    tree_workload("tr_bf16_d128_g16_w8", [9, 515, 1030], 8, 32, 2, 128, False, 116),
    # fp8: every round inside one page (C0 % 16 + R <= 16: 0, 3, 0, 0)
    tree_workload("tr_fp8_d128_g4", [8, 523, 1000, 4104], 8, 32, 8, 128, True, 113),
    # fp8 rounds across a page boundary (C0 % 16 = 4, 11, 5, 10): branches
    # that skip rows move later rows down into the page of C0
    tree_workload("tr_fp8_d128_cross", [60, 531, 1037, 2050], 8, 32, 8, 128, True, 114),
    tree_workload("tr_fp8_d256_cross_w5", [33, 707, 1298], 5, 16, 4, 256, True, 117),
]


@pytest.fixture(scope="module", params=CASES, ids=[w.name for w in CASES])
def case(request):
    w = request.param
    say("[gpu] tree case", w.name, "lengths", w.ctx_list, "width", w.rows)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    return w, inp, gpu


def test_tree_rows_equal_branch_decodes_and_oracle(case):
    w, inp, gpu = case
    S, R = inp.q.shape[0], inp.q.shape[1]
    masks = random_masks(S, R, 7)
    scratch = scratch_for(inp)
    out = run_tree(gpu, inp, masks, scratch)
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    lens = inp.lengths.cpu().numpy()
    sc = scratch.cpu().numpy()
    worst, moved = -1.0, 0
    for s in range(S):
        for r in range(R):
            view = oracle_view(oc, inp, s, r, int(masks[s, r]))
            assert view[4] == len(branch_positions(int(lens[s]), R, int(masks[s, r])))
            check_view_pages(gpu, inp, s, r, sc, view)
            dec = gpu_view_decode(gpu, inp, s, r, view)
            assert same_bits(dec, out[s, r]), (s, r)
            ref = oracle_view_attention(inp, s, r, view)
            ex = excess_err(out[s, r], ref, TOL[w.kv_fp8])
            worst = max(worst, ex)
            assert ex <= 0, (s, r)
            moved += moved_rows(int(lens[s]), R, int(masks[s, r]))
    if "cross" in w.name:
        assert moved > 0
    say("[gpu]", w.name, "worst excess", worst, "moved rows", moved)


def test_chain_tree_is_the_width_round(case):
    w, inp, gpu = case
    S, R = inp.q.shape[0], inp.q.shape[1]
    out = run_tree(gpu, inp, random_masks(S, R, 0, chain=True), scratch_for(inp))
    wsb = pa.attn_paged_workspace_bytes(1, S, inp.table.shape[1], w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(inp.q)
    try:
        pa.attn_paged_verify_width(inp.q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                                   inp.table.shape[1], inp.lengths, S, R, w.n_head, w.n_head_kv,
                                   w.head_dim, PAGE, gpu.kv, ref, ws, wsb)
    except pa.AttnError as e:
        # a width the round kernel does not serve: the chain rows are the
        # decode rows at their positions
        assert e.code == pa.ATTN_E_UNSUPPORTED
        for r in range(R):
            lens = inp.lengths - R + r + 1
            ref[:, r:r + 1] = gpu.run("decode", q=inp.q[:, r:r + 1].contiguous(), lengths=lens)
    torch.cuda.synchronize()
    assert same_bits(out, ref)


def test_bad_mask_gives_nan_row_only(case):
    w, inp, gpu = case
    S, R = inp.q.shape[0], inp.q.shape[1]
    masks = random_masks(S, R, 9)
    good = run_tree(gpu, inp, masks, scratch_for(inp))
    bad = masks.copy()
    bad[1, 0] |= 1 << (R - 1)        # names a later row
    bad[2, R - 1] &= ~(1 << (R - 1))  # does not name itself
    out = run_tree(gpu, inp, bad, scratch_for(inp))
    assert torch.isnan(out[1, 0].float()).all() and torch.isnan(out[2, R - 1].float()).all()
    keep = torch.ones(S, R, dtype=torch.bool)
    keep[1, 0] = keep[2, R - 1] = False
    assert same_bits(out[keep.cuda()], good[keep.cuda()])


def test_fp8_moved_rows_grow_the_view_scale():
    """Rows moved down from a page with a much larger scale grow the view
    page's scale (the page's other codes re-encoded); the view pages equal the
    oracle's, and each row the decode over that view."""
    w = tree_workload("tr_fp8_grow", [68, 531, 2050], 8, 16, 4, 128, True, 118)  # C0 % 16 = 12, 11, 10
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    oc = OracleCache(inp)
    S, R = 3, 8
    lens = inp.lengths.cpu().numpy()
    tab = inp.table.cpu().numpy()
    for s in range(S):
        tp = (int(lens[s]) - R) // PAGE
        # the same change to both caches: the next page's values 8x (K), 1.37x (V)
        gpu.ks[int(tab[s, tp + 1])] *= 8.0
        gpu.vs[int(tab[s, tp + 1])] *= 1.37
        oc.ks[oc.table[s, tp + 1]] *= np.float32(8.0)
        oc.vs[oc.table[s, tp + 1]] *= np.float32(1.37)
    oc.check_pools_equal(gpu)
    masks = np.zeros((S, R), np.int32)
    for s in range(S):
        for r in range(R):
            masks[s, r] = (1 << r) | (1 if r > 0 else 0)  # every row's parent is row 0
    scratch = scratch_for(inp)
    out = run_tree(gpu, inp, masks, scratch)
    sc = scratch.cpu().numpy()
    grown = 0
    for s in range(S):
        C0 = int(lens[s]) - R
        tp = C0 // PAGE
        for r in range(R):
            view = oracle_view(oc, inp, s, r, int(masks[s, r]))
            check_view_pages(gpu, inp, s, r, sc, view)
            assert same_bits(gpu_view_decode(gpu, inp, s, r, view), out[s, r]), (s, r)
            ex = excess_err(out[s, r], oracle_view_attention(inp, s, r, view), TOL[True])
            assert ex <= 0, (s, r)
            if (C0 + r) // PAGE > tp:  # row r moved next to row 0
                grown += int((view[2][tp] != oc.ks[oc.table[s, tp]]).any())
    assert grown > 0
