"""GPU parity of sliding-window / runtime-floor attention against the CPU
oracle, and its bitwise rules: each row equals the one-row call at its
position with the same window and floor, window 0 with floor 0 is the plain
call, and pages below the first key attended are never read (MI355X only)."""
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
    L("wd_bf16_d128_g4", [8, 40, 515, 1300, 2100], 8, 8, 2, 128, False, 81),
    L("wd_fp8_d128_g4", [9, 600, 1030, 3000], 8, 32, 8, 128, True, 82),
    L("wd_bf16_d256_g4", [20, 700, 1600], 8, 16, 4, 256, False, 83),
    L("wd_fp8_d256_g2", [17, 1111], 8, 8, 4, 256, True, 84),
]
WINDOWS = [1, 17, 513, 1000]


@pytest.fixture(scope="module", params=CONFIGS, ids=[w.name for w in CONFIGS])
def cfg(request):
    w = request.param
    say("[gpu] window config", w.name, "lengths", w.ctx_list)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    return w, inp, gpu, OracleCache(inp)


def floors_for(inp, rows, seed):
    """A floor per sequence in 0 .. C - rows (some 0, some near the row)."""
    rng = np.random.default_rng(seed)
    lens = inp.lengths.cpu().numpy()
    f = np.array([rng.integers(0, c - rows + 1) if i % 2 else 0 for i, c in enumerate(lens)],
                 np.int32)
    return f


def run_window(gpu, inp, q, window, floor_d, table=None, lengths=None):
    w = inp.w
    rows = q.shape[1]
    n_seq = q.shape[0]
    table = inp.table if table is None else table
    lengths = inp.lengths if lengths is None else lengths
    wsb = pa.attn_paged_workspace_bytes(1, n_seq, table.shape[1], w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    pa.attn_paged_decode_window(q, rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, table,
                                table.shape[1], lengths, n_seq, window, floor_d, w.n_head,
                                w.n_head_kv, w.head_dim, PAGE, gpu.kv, out, ws, wsb)
    return out


def oracle_window(oc, q, window, floor):
    w = oc.w
    return oracle.paged_attention(
        synth.bits(q), oc.k, oc.v, oc.table, oc.lens, n_head=w.n_head, n_head_kv=w.n_head_kv,
        head_dim=w.head_dim, page_size=PAGE,
        kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=oc.ks, v_scale=oc.vs,
        window=window, kv_floor=floor)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("rows", [1, 8])
def test_window_parity(cfg, window, rows):
    w, inp, gpu, oc = cfg
    q = inp.q[:, :rows].contiguous()
    floor = floors_for(inp, rows, window + rows)
    out = run_window(gpu, inp, q, window, torch.from_numpy(floor).cuda())
    torch.cuda.synchronize()
    ref = oracle_window(oc, q, window, floor)
    ex = excess_err(out, ref, TOL[w.kv_fp8])
    say("[gpu]", w.name, "rows", rows, "window", window, "excess", ex)
    assert ex <= 0


@pytest.mark.parametrize("window", [17, 513])
def test_window_rows_equal_one_row_calls(cfg, window):
    w, inp, gpu, oc = cfg
    floor = torch.from_numpy(floors_for(inp, 8, 5)).cuda()
    out = run_window(gpu, inp, inp.q, window, floor)
    for r in range(8):
        lens = inp.lengths - 8 + r + 1
        one = run_window(gpu, inp, inp.q[:, r:r + 1].contiguous(), window, floor, lengths=lens)
        torch.cuda.synchronize()
        assert same_bits(one[:, 0], out[:, r]), "row %d" % r


def test_no_window_no_floor_is_the_plain_call(cfg):
    w, inp, gpu, oc = cfg
    out = run_window(gpu, inp, inp.q, 0, None)
    ver = gpu.run("verify")
    q1 = inp.q[:, :1].contiguous()
    out1 = run_window(gpu, inp, q1, 0, None)
    dec = gpu.run("decode", q=q1)
    torch.cuda.synchronize()
    assert same_bits(out, ver)
    assert same_bits(out1, dec)


def test_released_pages_below_the_window_are_not_read(cfg):
    """Entries of pages wholly below every row's first key set to -1: same
    bits, no NaN."""
    w, inp, gpu, oc = cfg
    window = 300
    floor = torch.from_numpy(floors_for(inp, 8, 6)).cuda()
    ref = run_window(gpu, inp, inp.q, window, floor)
    table = inp.table.clone()
    lens = inp.lengths.cpu().numpy()
    fl = floor.cpu().numpy()
    for s, c in enumerate(lens):
        lo = max(int(fl[s]), int(c) - 8 - window + 1)
        table[s, :lo // PAGE] = -1
    out = run_window(gpu, inp, inp.q, window, floor, table=table)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert same_bits(out, ref)


def unused_page(inp):
    """A pool page no sequence uses (its codes, values and fp8 scales are
    NaN)."""
    lens = inp.lengths.cpu().numpy()
    table = inp.table.cpu().numpy()
    used = {int(p) for s, c in enumerate(lens) for p in table[s, :-(-int(c) // PAGE)]}
    free = [p for p in range(inp.n_pages) if p not in used]
    assert free
    return free[0]


def test_released_entries_naming_a_poisoned_page_change_nothing(cfg):
    """Entries below every row's first key that name an in-range page whose
    values and scales are NaN: same bits as with -1 entries (the page is
    neither read nor its scales used)."""
    w, inp, gpu, oc = cfg
    window = 300
    floor = torch.from_numpy(floors_for(inp, 8, 6)).cuda()
    table = inp.table.clone()
    lens = inp.lengths.cpu().numpy()
    fl = floor.cpu().numpy()
    poison = unused_page(inp)
    table_m1 = inp.table.clone()
    for s, c in enumerate(lens):
        lo = max(int(fl[s]), int(c) - 8 - window + 1)
        table[s, :lo // PAGE] = poison
        table_m1[s, :lo // PAGE] = -1
    ref = run_window(gpu, inp, inp.q, window, floor, table=table_m1)
    out = run_window(gpu, inp, inp.q, window, floor, table=table)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert same_bits(out, ref)


def test_bad_floor_gives_nan_rows_of_that_sequence_only(cfg):
    w, inp, gpu, oc = cfg
    floor = torch.zeros(inp.q.shape[0], dtype=torch.int32, device="cuda")
    ref = run_window(gpu, inp, inp.q, 100, floor)
    floor[0] = int(inp.lengths[0]) - 8 + 1  # above the first row's position
    out = run_window(gpu, inp, inp.q, 100, floor)
    torch.cuda.synchronize()
    assert torch.isnan(out[0].float()).all()
    assert same_bits(out[1:], ref[1:])


PF_CASES = [
    (synth.Workload("pfw_bf16_d128", 1, 130, 8, 2, 128, False, "fixed", 1500, 1500, 91,
                    kind="prefill"), [(64, 0), (1, 0), (200, 900), (0, 700), (5000, 37)]),
    (synth.Workload("pfw_fp8_d256", 1, 77, 16, 4, 256, True, "fixed", 900, 900, 92,
                    kind="prefill"), [(100, 0), (33, 500), (0, 823)]),
    (synth.Workload("pfw_bf16_g8", 1, 300, 32, 4, 128, False, "fixed", 700, 700, 93,
                    kind="prefill"), [(0, 0), (129, 0), (64, 333)]),
]


@pytest.mark.parametrize("w,windows", PF_CASES, ids=[c[0].name for c in PF_CASES])
def test_prefill_window_parity(w, windows):
    say("[gpu] prefill window", w.name)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    oc = OracleCache(inp)
    q = inp.q.view(w.rows, w.n_head, w.head_dim)
    C = int(inp.lengths[0])
    for window, floor in windows:
        out = torch.empty_like(q)
        pa.attn_paged_prefill_window(q, w.rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages,
                                     inp.table, inp.table.shape[1], C, window, floor, w.n_head,
                                     w.n_head_kv, w.head_dim, PAGE, gpu.kv, out)
        torch.cuda.synchronize()
        ref = oracle_window(oc, inp.q, window, np.array([floor], np.int32))[0]
        ex = excess_err(out, ref, TOL[w.kv_fp8])
        say("[gpu]", w.name, "window", window, "floor", floor, "excess", ex)
        assert ex <= 0
        if window == 0 and floor == 0:
            plain = gpu.run("prefill")
            torch.cuda.synchronize()
            assert same_bits(out, plain.view_as(out))
    # released pages below the first key of every row
    window, floor = windows[-1]
    lo = max(floor, C - w.rows - window + 1) if window > 0 else floor
    table = inp.table.clone()
    table[0, :lo // PAGE] = -1
    out2 = torch.empty_like(q)
    pa.attn_paged_prefill_window(q, w.rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, table,
                                 table.shape[1], C, window, floor, w.n_head, w.n_head_kv,
                                 w.head_dim, PAGE, gpu.kv, out2)
    out1 = torch.empty_like(q)
    pa.attn_paged_prefill_window(q, w.rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages,
                                 inp.table, inp.table.shape[1], C, window, floor, w.n_head,
                                 w.n_head_kv, w.head_dim, PAGE, gpu.kv, out1)
    # the same entries naming a page whose values are NaN
    used = {int(p) for p in inp.table[0, :-(-C // PAGE)].cpu().numpy()}
    poison = next(p for p in range(inp.n_pages) if p not in used)
    table_p = inp.table.clone()
    table_p[0, :lo // PAGE] = poison
    out3 = torch.empty_like(q)
    pa.attn_paged_prefill_window(q, w.rows, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, table_p,
                                 table_p.shape[1], C, window, floor, w.n_head, w.n_head_kv,
                                 w.head_dim, PAGE, gpu.kv, out3)
    torch.cuda.synchronize()
    assert same_bits(out2, out1)
    assert same_bits(out3, out1)
