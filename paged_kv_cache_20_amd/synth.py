"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs: context lengths, block tables, slot lists and
N(0, 1) values rounded to bf16.  It holds none of the attention or
quantisation arithmetic, so both the GPU path and the CPU oracle can take
its output.

Recipe (each workload, in draw order: lengths, block table, K, V, Q):
  - one torch.Generator on the target device, seeded with the workload seed;
  - lengths as the workload states (fixed, an explicit list, integer-uniform,
    or log-uniform: round(exp(U(ln lo, ln hi))) clipped to [lo, hi]);
  - a pool of sum_s ceil(C_s / 16) + n_seq spare pages (unless the workload
    fixes the pool), dealt to the sequences by one seeded permutation, so
    pages are non-overlapping and scattered; table columns past a sequence's
    pages are -1;
  - K and V: the logical cache, [sum_s C_s][n_head_kv][head_dim], one row per
    token of each sequence in order, N(0,1) in fp32 rounded to bf16 (round to
    nearest even); the slot list maps each row to its page and offset;
  - Q: [n_seq][rows][n_head][head_dim], N(0,1) rounded to bf16.
Unused pages and page tails start as NaN (bf16 0x7FC0, or e4m3 code 0x7F
with NaN scales), so any read of them shows in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    rows: int            # 1 decode, 8 verify, chunk length for prefill
    n_head: int
    n_head_kv: int
    head_dim: int
    kv_fp8: bool
    lengths: str         # "fixed", "uniform", "loguniform"
    ctx_lo: int
    ctx_hi: int
    seed: int
    pool_pages: Optional[int] = None   # fixed pool (else sum of needs + n_seq)
    kind: str = "decode"               # decode | verify | prefill
    ctx_list: tuple = ()               # lengths when lengths == "list"

    @property
    def max_pages(self) -> int:
        return -(-self.ctx_hi // PAGE)


# The five workloads of the study, named by what they are.
WORKLOADS: Dict[str, Workload] = {
    "decode_1seq_ctx512": Workload("decode_1seq_ctx512", 1, 1, 8, 2, 128, False, "fixed", 512,
                                   512, 1001, pool_pages=64),
    "decode_64seq_hd256": Workload("decode_64seq_hd256", 64, 1, 16, 4, 256, False, "uniform",
                                   1024, 8192, 1002),
    "verify_32seq_8rows": Workload("verify_32seq_8rows", 32, 8, 16, 4, 256, False, "fixed", 4104,
                                   4104, 1003, kind="verify"),
    "decode_256seq_fp8": Workload("decode_256seq_fp8", 256, 1, 32, 8, 128, True, "loguniform",
                                  2048, 32768, 1004),
    "prefill_4096_over_28672": Workload("prefill_4096_over_28672", 1, 4096, 16, 4, 256, False,
                                        "fixed", 32768, 32768, 1005, kind="prefill"),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def listed(name, lens, rows, n_head, n_head_kv, head_dim, kv_fp8, seed, kind="decode"):
    """A workload with an explicit list of context lengths."""
    lens = tuple(int(c) for c in lens)
    return Workload(name, len(lens), rows, n_head, n_head_kv, head_dim, kv_fp8, "list",
                    min(lens), max(lens), seed, kind=kind, ctx_list=lens)


def draw_lengths(w: Workload, gen: torch.Generator) -> torch.Tensor:
    dev = gen.device
    if w.lengths == "fixed":
        return torch.full((w.n_seq,), w.ctx_lo, dtype=torch.int32, device=dev)
    if w.lengths == "list":
        assert len(w.ctx_list) == w.n_seq
        return torch.tensor(w.ctx_list, dtype=torch.int32, device=dev)
    if w.lengths == "uniform":
        return torch.randint(w.ctx_lo, w.ctx_hi + 1, (w.n_seq,), generator=gen, device=dev,
                             dtype=torch.int64).to(torch.int32)
    if w.lengths == "loguniform":
        u = torch.rand((w.n_seq,), generator=gen, device=dev, dtype=torch.float64)
        x = torch.exp(math.log(w.ctx_lo) + u * (math.log(w.ctx_hi) - math.log(w.ctx_lo)))
        return torch.clamp(torch.round(x), w.ctx_lo, w.ctx_hi).to(torch.int32)
    raise ValueError(w.lengths)


def draw_block_table(lengths: torch.Tensor, max_pages: int, gen: torch.Generator,
                     pool_pages: Optional[int] = None):
    """Non-overlapping random pages from a shared pool: (table, n_pages)."""
    dev = gen.device
    lens = lengths.to("cpu", torch.int64)
    need = (lens + PAGE - 1) // PAGE
    total = int(need.sum())
    n_pages = pool_pages if pool_pages is not None else total + int(lens.numel())
    if n_pages < total:
        raise ValueError("pool too small")
    perm = torch.randperm(n_pages, generator=gen, device=dev).to(torch.int32)
    table = torch.full((lens.numel(), max_pages), -1, dtype=torch.int32, device=dev)
    pos = 0
    for s, n in enumerate(need.tolist()):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    return table, n_pages


def slot_list(table: torch.Tensor, lengths: torch.Tensor) -> torch.Tensor:
    """Token slot of every row of the logical cache (sequence-major)."""
    dev = table.device
    out = []
    for s, c in enumerate(lengths.to("cpu").tolist()):
        t = torch.arange(c, device=dev, dtype=torch.int64)
        out.append(table[s, t // PAGE].to(torch.int64) * PAGE + t % PAGE)
    return torch.cat(out).to(torch.int32)


def normal_bf16(shape, gen: torch.Generator, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to bf16, drawn in row chunks so the
    fp32 temporaries stay small."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=gen.device)
    flat = out.view(shape[0], -1)
    for i in range(0, shape[0], chunk_rows):
        j = min(shape[0], i + chunk_rows)
        flat[i:j] = torch.randn((j - i, flat.shape[1]), generator=gen, device=gen.device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def poison_pools(n_pages: int, w: Workload, device):
    """Empty K/V pools (and scales) filled with NaN patterns."""
    shape = (n_pages, w.n_head_kv, PAGE, w.head_dim)
    if w.kv_fp8:
        k = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
        v = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
        ks = torch.full((n_pages, w.n_head_kv), float("nan"), dtype=torch.float32, device=device)
        vs = torch.full((n_pages, w.n_head_kv), float("nan"), dtype=torch.float32, device=device)
        return k, v, ks, vs
    k = torch.full(shape, 0x7FC0, dtype=torch.int16, device=device).view(torch.bfloat16)
    v = torch.full(shape, 0x7FC0, dtype=torch.int16, device=device).view(torch.bfloat16)
    return k, v, None, None


@dataclass
class Inputs:
    w: Workload
    lengths: torch.Tensor      # int32 [n_seq]
    table: torch.Tensor        # int32 [n_seq][max_pages]
    n_pages: int
    k_src: torch.Tensor        # bf16 [sum C][n_head_kv][head_dim]
    v_src: torch.Tensor
    slots: torch.Tensor        # int32 [sum C]
    q: torch.Tensor            # bf16 [n_seq][rows][n_head][head_dim]
    extra: dict = field(default_factory=dict)


def draw(w: Workload, device="cpu", seed: Optional[int] = None) -> Inputs:
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    lengths = draw_lengths(w, gen)
    table, n_pages = draw_block_table(lengths, w.max_pages, gen, w.pool_pages)
    total = int(lengths.to(torch.int64).sum())
    k_src = normal_bf16((total, w.n_head_kv, w.head_dim), gen)
    v_src = normal_bf16((total, w.n_head_kv, w.head_dim), gen)
    q = normal_bf16((w.n_seq, w.rows, w.n_head, w.head_dim), gen)
    slots = slot_list(table, lengths)
    return Inputs(w, lengths, table, n_pages, k_src, v_src, slots, q)


def bits(t: torch.Tensor):
    """Storage bit pattern of a tensor as a numpy array (bf16 -> uint16)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.numpy()


def mixed_step(seed: int = 1006):
    """A continuous-batching step: 256 decode sequences of the fp8 decode
    workload's shape (H 32 / Hk 8, d 128, fp8 e4m3, lengths log-uniform in
    [2048, 32768], drawn with `seed` on the CPU) followed by one 2048-row
    prefill chunk after 6144 cached rows of the same layer.
    Returns (workload, inputs, q [256 + 2048][32][128], cu_seqlens, lengths)."""
    import itertools
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dec = scaled(WORKLOADS["decode_256seq_fp8"], seed=seed)
    lens = draw_lengths(dec, gen).tolist() + [8192]
    w = listed("mixed_256dec_fp8_plus_2048chunk", lens, 1, 32, 8, 128, True, seed)
    inp = draw(w, "cuda")
    q_rows = [1] * 256 + [2048]
    gq = torch.Generator(device="cuda")
    gq.manual_seed(seed + 1)
    q = normal_bf16((sum(q_rows), 32, 128), gq)
    cu = torch.tensor([0] + list(itertools.accumulate(q_rows)), dtype=torch.int32, device="cuda")
    return w, inp, q, cu, lens


def tree_masks(n_seq: int, rows: int, seed: int):
    """Random speculative trees: row r's parent is drawn uniformly among the
    earlier rows and "none" (numpy PCG64 with `seed`); its mask names r and
    its parent's mask.  int32 [n_seq][rows]."""
    import numpy as np
    rng = np.random.default_rng(seed)
    masks = np.zeros((n_seq, rows), np.int32)
    for s in range(n_seq):
        for r in range(rows):
            par = int(rng.integers(-1, r))
            masks[s, r] = (1 << r) | (masks[s, par] if par >= 0 else 0)
    return masks
