"""attn_paged_decode_noalloc on MI355X: the decode entry point whose split
partials live in the library's per-device scratch array instead of a caller
workspace.  Its output must be bit for bit attn_paged_decode's (same
kernels), on two calls in a row, the second with a smaller input (the array
keeps the first call's contents)."""
import pytest
import torch

from paged_kv_cache_20_amd import synth
from gpu_util import GpuCache, same_bits, say

pytestmark = pytest.mark.gpu


def decode_ws(pa, gpu, w, inp):
    wsb = pa.attn_paged_workspace_bytes(0, w.n_seq, w.max_pages, w.n_head, w.head_dim)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp.q)
    pa.attn_paged_decode(inp.q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                         w.max_pages, inp.lengths, w.n_seq, w.n_head, w.n_head_kv, w.head_dim,
                         16, gpu.kv, out, ws, wsb)
    return out


def decode_noalloc(pa, gpu, w, inp):
    out = torch.full_like(inp.q, float("nan"))
    pa.attn_paged_decode_noalloc(inp.q, gpu.k, gpu.v, gpu.ks, gpu.vs, inp.n_pages, inp.table,
                                 w.max_pages, inp.lengths, w.n_seq, w.n_head, w.n_head_kv,
                                 w.head_dim, 16, gpu.kv, out)
    return out


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_matches_workspace_decode_twice(fp8):
    import paged_kv_cache_20_amd as pa
    # a larger call, then a smaller one over fewer sequences and shorter contexts
    big = synth.listed("na_big_%d" % fp8, [3000, 517, 1, 2049, 8190, 1024, 77, 4097],
                       1, 32, 8, 128, fp8, 61)
    small = synth.listed("na_small_%d" % fp8, [600, 33, 1500], 1, 16, 4, 256, fp8, 62)
    for w in (big, small):
        say("[gpu] noalloc decode", w.name, "lengths", w.ctx_list)
        inp = synth.draw(w, "cuda")
        gpu = GpuCache(inp)
        ref = decode_ws(pa, gpu, w, inp)
        got = decode_noalloc(pa, gpu, w, inp)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert same_bits(got, ref), w.name
