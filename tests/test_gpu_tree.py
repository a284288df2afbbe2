"""GPU parity of tree-shaped speculative rounds (MI355X only).

Row r of a round attends the cached context plus the round rows its mask
names.  Each tree row must equal, bit for bit, the GPU decode of the same
row over its branch laid out contiguously (the same stored bytes copied to
fresh pages), and lie within tolerance of the CPU oracle over the branch
built from the oracle's own cache.  A chain mask gives the width-R round.
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


def gpu_branch_decode(gpu, inp, s, r, pos):
    """Decode of row (s, r) over its branch copied byte for byte to new pages."""
    w = inp.w
    n = len(pos)
    npg = -(-n // PAGE)
    tab = inp.table[s].long()
    p = torch.tensor(pos, device="cuda")
    src_page, src_row = tab[p // PAGE], p % PAGE
    shape = (npg, w.n_head_kv, PAGE, w.head_dim)
    k2 = torch.zeros(shape, dtype=gpu.k.dtype, device="cuda")
    v2 = torch.zeros(shape, dtype=gpu.v.dtype, device="cuda")
    dst = torch.arange(n, device="cuda")
    k2[dst // PAGE, :, dst % PAGE, :] = gpu.k[src_page, :, src_row, :]
    v2[dst // PAGE, :, dst % PAGE, :] = gpu.v[src_page, :, src_row, :]
    ks2 = vs2 = None
    if gpu.ks is not None:
        first = src_page[torch.arange(npg, device="cuda") * PAGE]
        ks2 = gpu.ks[first].contiguous()
        vs2 = gpu.vs[first].contiguous()
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


def oracle_branch(oc, inp, s, r, pos):
    """The oracle over the branch copied from the oracle's own cache."""
    w = inp.w
    n = len(pos)
    npg = -(-n // PAGE)
    tab = oc.table[s]
    p = np.asarray(pos)
    sp, sr = tab[p // PAGE], p % PAGE
    k2 = np.zeros((npg, w.n_head_kv, PAGE, w.head_dim), oc.k.dtype)
    v2 = np.zeros_like(k2)
    i = np.arange(n)
    k2[i // PAGE, :, i % PAGE, :] = oc.k[sp, :, sr, :]
    v2[i // PAGE, :, i % PAGE, :] = oc.v[sp, :, sr, :]
    ks2 = vs2 = None
    if oc.ks is not None:
        first = sp[np.arange(npg) * PAGE]
        ks2, vs2 = oc.ks[first], oc.vs[first]
    q = synth.bits(inp.q[s, r]).reshape(1, 1, w.n_head, w.head_dim)
    return oracle.paged_attention(
        q, k2, v2, np.arange(npg, dtype=np.int32).reshape(1, npg), np.array([n], np.int32),
        n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=ks2, v_scale=vs2)[0, 0]


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
    out = run_tree(gpu, inp, masks, scratch_for(inp))
    oc = OracleCache(inp)
    oc.check_pools_equal(gpu)
    lens = inp.lengths.cpu().numpy()
    worst = -1.0
    for s in range(S):
        for r in range(R):
            pos = branch_positions(int(lens[s]), R, int(masks[s, r]))
            dec = gpu_branch_decode(gpu, inp, s, r, pos)
            assert same_bits(dec, out[s, r]), (s, r)
            ref = oracle_branch(oc, inp, s, r, pos)
            ex = excess_err(out[s, r], ref, TOL[w.kv_fp8])
            worst = max(worst, ex)
            assert ex <= 0, (s, r)
    say("[gpu]", w.name, "worst excess", worst)


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


def test_fp8_round_across_a_page_gives_nan():
    w = tree_workload("tr_fp8_cross", [60, 531], 8, 8, 2, 128, True, 114)  # C0 % 16 = 4, 11
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = run_tree(gpu, inp, random_masks(2, 8, 3), scratch_for(inp))
    assert torch.isnan(out[1].float()).all()       # 523 % 16 = 11: 11 + 8 > 16
    assert torch.isfinite(out[0].float()).all()    # 52 % 16 = 4: inside one page
