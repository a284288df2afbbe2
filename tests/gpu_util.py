"""Helpers shared by the GPU tests: build a workload's cache on the GPU with
the library and the same cache on the CPU with the oracle, run the library's
attention, and compare.  Inputs come from paged_kv_cache_20_amd.synth only;
nothing the oracle sees comes from the library's kernels."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth

PAGE = 16
TOL = {False: 5e-3, True: 2e-2}  # max abs error vs the fp64 oracle: bf16 KV, fp8 KV


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


class GpuCache:
    """Pools on the GPU, filled by attn_kv_append from the workload's source."""

    def __init__(self, inp: synth.Inputs):
        w = inp.w
        self.inp = inp
        self.k, self.v, self.ks, self.vs = synth.poison_pools(inp.n_pages, w, "cuda")
        self.kv = pa.KV_FP8_E4M3 if w.kv_fp8 else pa.KV_BF16
        n_tok = inp.slots.numel()
        pa.attn_kv_append(inp.k_src, inp.v_src, inp.slots, n_tok, self.k, self.v, self.ks,
                          self.vs, inp.n_pages, w.n_head_kv, w.head_dim, PAGE, self.kv)

    def run(self, kind: str, q=None, lengths=None, table=None, n_seq=None, out=None):
        w, inp = self.inp.w, self.inp
        q = inp.q if q is None else q
        lengths = inp.lengths if lengths is None else lengths
        table = inp.table if table is None else table
        n_seq = q.shape[0] if n_seq is None else n_seq
        out = torch.empty_like(q) if out is None else out
        if kind == "prefill":
            pa.attn_paged_prefill(q.view(-1, w.n_head, w.head_dim), q.shape[1], self.k, self.v,
                                  self.ks, self.vs, inp.n_pages, table, table.shape[1],
                                  int(lengths[0]), w.n_head, w.n_head_kv, w.head_dim, PAGE,
                                  self.kv, out)
            return out
        op = 0 if kind == "decode" else 1
        wsb = pa.attn_paged_workspace_bytes(op, n_seq, table.shape[1], w.n_head, w.head_dim)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        fn = pa.attn_paged_decode if kind == "decode" else pa.attn_paged_verify
        fn(q, self.k, self.v, self.ks, self.vs, inp.n_pages, table, table.shape[1], lengths,
           n_seq, w.n_head, w.n_head_kv, w.head_dim, PAGE, self.kv, out, ws, wsb)
        return out


class OracleCache:
    """The same cache built on the CPU by the oracle's append, restricted to
    a subset of sequences (renumbered pages) so large workloads stay cheap."""

    def __init__(self, inp: synth.Inputs, seqs=None):
        w = inp.w
        lens = inp.lengths.cpu().numpy().astype(np.int64)
        seqs = np.arange(len(lens)) if seqs is None else np.asarray(seqs)
        self.seqs = seqs
        starts = np.concatenate([[0], np.cumsum(lens)])
        table = inp.table.cpu().numpy()
        need = (lens[seqs] + PAGE - 1) // PAGE
        self.old_pages = np.concatenate([table[s, :n] for s, n in zip(seqs, need)])
        self.n_pages = len(self.old_pages) + 1  # one spare, never used
        self.table = np.full((len(seqs), w.max_pages), -1, np.int32)
        pos = 0
        for i, n in enumerate(need):
            self.table[i, :n] = np.arange(pos, pos + n)
            pos += n
        self.lens = lens[seqs].astype(np.int32)
        rows = np.concatenate([np.arange(starts[s], starts[s + 1]) for s in seqs])
        rows_t = torch.from_numpy(rows).to(inp.k_src.device)
        k_bits = synth.bits(inp.k_src.index_select(0, rows_t))
        v_bits = synth.bits(inp.v_src.index_select(0, rows_t))
        slots = np.concatenate([self.table[i, np.arange(c) // PAGE] * PAGE + np.arange(c) % PAGE
                                for i, c in enumerate(self.lens)]).astype(np.int32)
        shape = (self.n_pages, w.n_head_kv, PAGE, w.head_dim)
        self.fp8 = w.kv_fp8
        if w.kv_fp8:
            self.k = np.full(shape, 0x7F, np.uint8)
            self.v = np.full(shape, 0x7F, np.uint8)
            self.ks = np.full((self.n_pages, w.n_head_kv), np.nan, np.float32)
            self.vs = np.full((self.n_pages, w.n_head_kv), np.nan, np.float32)
        else:
            self.k = np.full(shape, 0x7FC0, np.uint16)
            self.v = np.full(shape, 0x7FC0, np.uint16)
            self.ks = self.vs = None
        oracle.kv_append(k_bits, v_bits, slots, self.k, self.v, self.ks, self.vs,
                         n_head_kv=w.n_head_kv, head_dim=w.head_dim, page_size=PAGE,
                         kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16)
        self.w = w

    def check_pools_equal(self, gpu: GpuCache):
        """The GPU's pages for the subset equal the oracle's, byte for byte
        (token slots below each context; the rest of a page is poison in both
        and also compared)."""
        idx = torch.from_numpy(self.old_pages.astype(np.int64)).cuda()
        n = len(self.old_pages)
        gk = synth.bits(gpu.k.index_select(0, idx))
        gv = synth.bits(gpu.v.index_select(0, idx))
        np.testing.assert_array_equal(gk, self.k[:n])
        np.testing.assert_array_equal(gv, self.v[:n])
        if self.fp8:
            np.testing.assert_array_equal(gpu.ks.index_select(0, idx).cpu().numpy(), self.ks[:n])
            np.testing.assert_array_equal(gpu.vs.index_select(0, idx).cpu().numpy(), self.vs[:n])

    def attend(self, q: torch.Tensor, row_mask=None) -> np.ndarray:
        w = self.w
        qb = synth.bits(q.index_select(0, torch.from_numpy(self.seqs).to(q.device)))
        return oracle.paged_attention(
            qb, self.k, self.v, self.table, self.lens, n_head=w.n_head, n_head_kv=w.n_head_kv,
            head_dim=w.head_dim, page_size=PAGE,
            kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16, k_scale=self.ks,
            v_scale=self.vs, row_mask=row_mask)


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(int))


def excess_err(gpu_out: torch.Tensor, ref: np.ndarray, tol: float) -> float:
    """Largest amount by which |gpu - ref| exceeds tol + half a bf16 ulp of
    |ref| (<= 0 passes).  Used on short-context unit cases, where |out| can
    reach 2-4 and the bf16 rounding of the output alone exceeds the bound."""
    g = bf16_to_f64(gpu_out)
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float(np.max(np.abs(g - ref) - (tol + half_ulp_bf16(ref))))


def max_err(gpu_out: torch.Tensor, ref: np.ndarray, seqs=None, row_mask=None) -> float:
    g = bf16_to_f64(gpu_out if seqs is None else
                    gpu_out.index_select(0, torch.as_tensor(seqs, device=gpu_out.device)))
    if row_mask is not None:
        m = np.asarray(row_mask, bool)
        g, ref = g[m], ref[m]
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float(np.max(np.abs(g - ref)))


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality, treating +0 and -0 as equal."""
    ai = a.contiguous().view(torch.int16)
    bi = b.contiguous().view(torch.int16)
    za = (ai & 0x7FFF) == 0
    zb = (bi & 0x7FFF) == 0
    return bool(torch.all((ai == bi) | (za & zb)).item())
