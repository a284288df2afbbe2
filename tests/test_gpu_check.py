"""Checked mode on the device: attn_check_device flags the first bad length or
block-table entry a call would read, and nothing else (MI355X only)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_20_amd as pa
from paged_kv_cache_20_amd import synth

pytestmark = pytest.mark.gpu

PAGE = 16


def run(table, lens, rows, n_pages, floor=None, window=0):
    err = torch.full((1,), 12345, dtype=torch.int64, device="cuda")
    pa.attn_check_device(table, lens, floor, window, lens.numel(), rows, table.shape[1], PAGE,
                         n_pages, err)
    torch.cuda.synchronize()
    return int(err.item())


@pytest.fixture(scope="module")
def inp():
    w = synth.listed("chk", [8, 40, 515, 1300, 33], 8, 8, 2, 128, False, 101)
    return synth.draw(w, "cuda")


def key(inp, s, e):
    return s * (inp.table.shape[1] + 1) + e + 1


def test_valid_inputs_give_minus_one(inp):
    assert run(inp.table, inp.lengths, 8, inp.n_pages) == -1
    assert run(inp.table, inp.lengths, 1, inp.n_pages) == -1


def test_first_bad_length_and_entry(inp):
    lens = inp.lengths.clone()
    lens[3] = 5  # below 8 rows
    assert run(inp.table, lens, 8, inp.n_pages) == key(inp, 3, -1)
    table = inp.table.clone()
    table[2, 7] = inp.n_pages          # outside the pool
    table[4, 1] = -2
    assert run(table, inp.lengths, 8, inp.n_pages) == key(inp, 2, 7)
    assert run(table, lens, 8, inp.n_pages) == key(inp, 2, 7)  # (2, 7) before (3, length)


def test_unread_entries_are_not_flagged(inp):
    table = inp.table.clone()
    need = (inp.lengths.cpu() + PAGE - 1) // PAGE
    table[1, int(need[1])] = -9        # past the sequence's last page
    assert run(table, inp.lengths, 8, inp.n_pages) == -1
    # below a floor / window: released pages may hold anything
    table[3, :10] = -1
    floor = torch.zeros_like(inp.lengths)
    floor[3] = 10 * PAGE
    assert run(table, inp.lengths, 1, inp.n_pages, floor=floor) == -1
    assert run(table, inp.lengths, 1, inp.n_pages) == key(inp, 3, 0)
    c = int(inp.lengths[3])
    assert run(table, inp.lengths, 1, inp.n_pages, window=c - 10 * PAGE) == -1
    assert run(table, inp.lengths, 1, inp.n_pages, window=c - 10 * PAGE + 1) == key(inp, 3, 9)
