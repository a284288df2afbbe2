"""GPU tests at the limits (MI355X only): the largest batch a call takes
(4,096 sequences), a context long enough for the combine to run over more
than four groups of 64 splits, and the one-key context, where the
attention's closed form (the value row itself) is met exactly."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth
from gpu_util import PAGE, TOL, GpuCache, OracleCache, excess_err, max_err, same_bits, say

pytestmark = pytest.mark.gpu

MAX_SEQ = 4096


def short_lengths(n, rows, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(rows, 120, size=n)
    lens[::997] = rng.integers(600, 1500, size=len(lens[::997]))  # a few longer ones
    return [int(c) for c in lens]


@pytest.mark.parametrize("rows,fp8", [(1, True), (1, False), (8, False)])
def test_largest_batch(rows, fp8):
    lens = short_lengths(MAX_SEQ, rows, 3 + rows)
    w = synth.listed("max_batch_r%d_%s" % (rows, "fp8" if fp8 else "bf16"), lens, rows, 8, 2,
                     128, fp8, 141 + rows, kind="decode" if rows == 1 else "verify")
    say("[gpu] largest batch", w.name)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("decode" if rows == 1 else "verify")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    seqs = [0, 1, 997, 2048, MAX_SEQ - 1]
    oc = OracleCache(inp, seqs)
    ref = oc.attend(inp.q)
    err = max_err(out, ref, seqs)
    say("[gpu]", w.name, "sampled", seqs, "max abs err", err)
    assert excess_err(out.index_select(0, torch.tensor(seqs, device="cuda")), ref, TOL[fp8]) <= 0
    # the same sequences in a batch of their own: the same bits
    sub = torch.tensor(seqs, device="cuda")
    q2 = inp.q.index_select(0, sub).contiguous()
    out2 = gpu.run("decode" if rows == 1 else "verify", q=q2,
                   lengths=inp.lengths.index_select(0, sub).contiguous(),
                   table=inp.table.index_select(0, sub).contiguous())
    torch.cuda.synchronize()
    assert same_bits(out2, out.index_select(0, sub))
    del gpu, inp
    torch.cuda.empty_cache()


def test_verify_d256_either_side_of_the_lds_ring_batch():
    """bf16 verify rounds at head_dim 256 run the split kernel's LDS-ring
    form for batches of at most 512 sequences and the register form (one
    slot tile per item) above: the same rows give the same bits either way."""
    n = 600
    lens = short_lengths(n, 8, 171)
    w = synth.listed("ring_edge_d256", lens, 8, 16, 4, 256, False, 172, kind="verify")
    say("[gpu] verify d256 batch", n)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("verify")  # register form
    torch.cuda.synchronize()
    seqs = [0, 3, 299, 597, n - 1]
    oc = OracleCache(inp, seqs)
    ref = oc.attend(inp.q)
    assert excess_err(out.index_select(0, torch.tensor(seqs, device="cuda")), ref, TOL[False]) <= 0
    for part in (torch.arange(0, 512, device="cuda"), torch.arange(88, n, device="cuda")):
        out2 = gpu.run("verify", q=inp.q.index_select(0, part).contiguous(),
                       lengths=inp.lengths.index_select(0, part).contiguous(),
                       table=inp.table.index_select(0, part).contiguous())  # LDS-ring form
        torch.cuda.synchronize()
        assert same_bits(out2, out.index_select(0, part))
    del gpu, inp
    torch.cuda.empty_cache()


def test_batch_above_the_limit_is_refused():
    lens = [4] * (MAX_SEQ + 1)
    w = synth.listed("too_many", lens, 1, 8, 2, 128, False, 150)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    with pytest.raises(pa.AttnError) as e:
        gpu.run("decode")
    assert e.value.code == pa.ATTN_E_UNSUPPORTED


@pytest.mark.parametrize("fp8", [True, False])
def test_long_context_many_split_groups(fp8):
    """131,109 keys: 129 splits of 1024 keys (fp8) or 257 of 512 (bf16), so
    the combine's max and sums run over three or five groups of 64 splits."""
    w = synth.listed("long_ctx_%s" % ("fp8" if fp8 else "bf16"), [131109, 70001], 1, 32, 8, 128,
                     fp8, 151)
    say("[gpu] long context", w.name)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("decode")
    torch.cuda.synchronize()
    oc = OracleCache(inp)
    ref = oc.attend(inp.q)
    err = max_err(out, ref)
    say("[gpu]", w.name, "max abs err", err)
    assert err <= TOL[fp8]
    del gpu, inp
    torch.cuda.empty_cache()


def test_one_key_is_the_value_row():
    """Context of one token: every head's output is its kv head's value row
    (exp2(0) = 1, one term), bit for bit, in decode and in a one-row
    prefill."""
    w = synth.listed("one_key", [1, 1, 1], 1, 16, 4, 256, False, 152)
    inp = synth.draw(w, "cuda")
    gpu = GpuCache(inp)
    out = gpu.run("decode")
    torch.cuda.synchronize()
    g = w.n_head // w.n_head_kv
    want = inp.v_src.repeat_interleave(g, dim=1)  # [3 tokens][H][d], one per sequence
    assert same_bits(out[:, 0], want)
    wp = synth.Workload("one_key_pf", 1, 1, 16, 4, 256, False, "fixed", 1, 1, 153,
                        kind="prefill")
    inp2 = synth.draw(wp, "cuda")
    gpu2 = GpuCache(inp2)
    outp = gpu2.run("prefill")
    torch.cuda.synchronize()
    assert same_bits(outp.view(1, 16, 256), inp2.v_src.repeat_interleave(g, dim=1))
