"""The C-ABI boundary on the CPU: the library loads, exports every symbol
include/pagedattn.h declares, and every host-checkable argument error
returns its code and message without touching a device (no compute calls).
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_20_amd as p
    return p


def header_functions():
    src = open(os.path.join(ROOT, "include", "pagedattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(pa):
    names = header_functions()
    assert "attn_paged_decode" in names and "attn_kv_append" in names
    lib = pa.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pa.EXPORTS) == names


def test_caps(pa):
    for d in (128, 256):
        for kv in (pa.KV_BF16, pa.KV_FP8_E4M3):
            assert pa.attn_caps(d, 16, kv) == pa.ATTN_OK
    assert pa.attn_caps(96, 16, pa.KV_BF16) == pa.ATTN_E_UNSUPPORTED
    assert "head_dim 96" in pa.attn_last_error()
    assert pa.attn_caps(128, 32, pa.KV_BF16) == pa.ATTN_E_UNSUPPORTED
    assert pa.attn_caps(128, 16, 7) == pa.ATTN_E_UNSUPPORTED


def test_workspace_sizes(pa):
    a = pa.attn_paged_workspace_bytes(0, 256, 2048, 32, 128)
    b = pa.attn_paged_workspace_bytes(1, 256, 2048, 32, 128)
    # partials: one (o, m, l) record per (seq, split, row, head)
    splits = -(-2048 * 16 // 512)
    assert a >= 256 * splits * 32 * (128 + 2) * 4
    assert b >= 8 * 256 * splits * 32 * (128 + 2) * 4
    assert pa.attn_paged_workspace_bytes(0, 0, 2048, 32, 128) == 0
    assert pa.attn_paged_workspace_bytes(0, 4, 16, 32, 96) == 0
    assert pa.attn_paged_workspace_bytes(2, 1, 2048, 16, 256) == 0


FAKE = 1 << 40  # never dereferenced: every case fails its host check first


def decode_args(**over):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_scale=None, v_scale=None, n_pages=64,
             block_table=FAKE, max_pages_per_seq=32, ctx_lens=FAKE, n_seq=1, n_head=8,
             n_head_kv=2, head_dim=128, page_size=16, kv_dtype=0, out=FAKE, workspace=FAKE,
             workspace_bytes=1 << 30, stream=0)
    a.update(over)
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(q=None), -1, "q is NULL"),
    (dict(out=None), -1, "out is NULL"),
    (dict(block_table=None), -1, "block_table"),
    (dict(ctx_lens=None), -1, "ctx_lens"),
    (dict(kv_dtype=1), -1, "fp8 kv needs"),
    (dict(k_scale=FAKE), -1, "bf16 kv takes no scales"),
    (dict(kv_dtype=5), -1, "kv_dtype 5"),
    (dict(n_seq=0), -2, "zero sequences"),
    (dict(n_head=6, n_head_kv=4), -2, "not a multiple"),
    (dict(n_head=0), -2, "n_head"),
    (dict(head_dim=0), -2, "head_dim"),
    (dict(head_dim=96), -3, "head_dim 96"),
    (dict(page_size=32), -3, "page_size 32"),
    (dict(n_head=64, n_head_kv=2), -3, "query heads per kv head"),
    (dict(n_seq=5000), -3, "n_seq 5000"),
    (dict(n_pages=0), -2, "n_pages"),
    (dict(max_pages_per_seq=0), -2, "max_pages_per_seq"),
    (dict(workspace=None), -4, "workspace is NULL"),
    (dict(workspace=FAKE + 8), -4, "aligned"),
    (dict(workspace_bytes=100), -4, "workspace has 100 bytes"),
])
def test_decode_host_checks(pa, over, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_decode(**decode_args(**over))
    assert e.value.code == code
    assert needle in str(e.value)


@pytest.mark.parametrize("width,code,needle", [
    (0, -2, "zero rows"), (-3, -2, "zero rows"), (9, -3, "width 9"),
])
def test_verify_width_host_checks(pa, width, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_verify_width(**decode_args(width=width))
    assert e.value.code == code
    assert needle in str(e.value)


def test_verify_width_rejects_unserved_group(pa):
    # 32 query heads per kv head: more than one 16-slot tile per position
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_verify_width(**decode_args(width=5, n_head=32, n_head_kv=1,
                                                 head_dim=256))
    assert e.value.code == pa.ATTN_E_UNSUPPORTED
    assert "at most 16" in str(e.value)


def tree_args(**over):
    a = decode_args(width=8, tree_mask=FAKE, scratch_pages=FAKE)
    a.update(over)
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(width=0), -2, "zero rows"), (dict(width=9), -3, "width 9"),
    (dict(tree_mask=None), -1, "tree_mask"), (dict(scratch_pages=None), -1, "scratch_pages"),
    (dict(n_seq=0), -2, "zero sequences"), (dict(n_seq=600), -3, "n_seq * width 4800"),
    (dict(n_head=64, n_head_kv=2), -3, "query heads per kv head"),
    (dict(workspace_bytes=1000), -4, "workspace has 1000 bytes"),
    (dict(q=None), -1, "q is NULL"),
])
def test_verify_tree_host_checks(pa, over, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_verify_tree(**tree_args(**over))
    assert e.value.code == code
    assert needle in str(e.value)


def test_tree_workspace_covers_eight_one_row_sequences_per_sequence(pa):
    t = pa.attn_paged_workspace_bytes(4, 32, 257, 16, 256)
    d = pa.attn_paged_workspace_bytes(0, 32 * 8, 257, 16, 256)
    assert t >= d + 32 * 8 * (257 + 1) * 4


@pytest.mark.parametrize("over,code,needle", [
    (dict(rows=0), -2, "zero rows"), (dict(rows=9), -3, "rows 9"),
    (dict(window=-1), -5, "window -1"), (dict(q=None), -1, "q is NULL"),
])
def test_decode_window_host_checks(pa, over, code, needle):
    args = decode_args(rows=1, window=0, kv_floor=None)
    args.update(over)
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_decode_window(**args)
    assert e.value.code == code
    assert needle in str(e.value)


@pytest.mark.parametrize("over,code,needle", [
    (dict(window=-2), -5, "window -2"),
    (dict(kv_floor=-1), -5, "kv_floor -1"),
    (dict(kv_floor=28673), -5, "kv_floor 28673"),
    (dict(n_rows=0), -2, "zero rows"),
])
def test_prefill_window_host_checks(pa, over, code, needle):
    args = prefill_args(window=0, kv_floor=0)
    args.update(over)
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_prefill_window(**args)
    assert e.value.code == code
    assert needle in str(e.value)


@pytest.mark.parametrize("over,code,needle", [
    (dict(block_table=None), -1, "must not be NULL"),
    (dict(err_word=None), -1, "must not be NULL"),
    (dict(n_seq=0), -2, "zero sequences"),
    (dict(rows=0), -2, "zero sequences or rows"),
    (dict(n_pages=0), -2, "n_pages"),
    (dict(page_size=8), -3, "page_size 8"),
    (dict(window=-4), -5, "window -4"),
])
def test_check_device_host_checks(pa, over, code, needle):
    args = dict(block_table=FAKE, ctx_lens=FAKE, kv_floor=None, window=0, n_seq=4, rows=1,
                max_pages_per_seq=32, page_size=16, n_pages=64, err_word=FAKE, stream=0)
    args.update(over)
    with pytest.raises(pa.AttnError) as e:
        pa.attn_check_device(**args)
    assert e.value.code == code
    assert needle in str(e.value)


def test_verify_rejects_unserved_group(pa):
    # 32 query heads per kv head: more than one 16-slot tile per position
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_verify(**decode_args(n_head=32, n_head_kv=1, head_dim=256))
    assert e.value.code == pa.ATTN_E_UNSUPPORTED
    assert "at most 16" in str(e.value)


def prefill_args(**over):
    a = dict(q=FAKE, n_rows=4096, k_pool=FAKE, v_pool=FAKE, k_scale=None, v_scale=None,
             n_pages=4096, block_table=FAKE, max_pages_per_seq=2048, ctx_len=32768, n_head=16,
             n_head_kv=4, head_dim=256, page_size=16, kv_dtype=0, out=FAKE, workspace=None,
             workspace_bytes=0, stream=0)
    a.update(over)
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(n_rows=0), -2, "zero rows"),
    (dict(ctx_len=10, n_rows=20), -5, "below n_rows"),
    (dict(ctx_len=40000), -5, "exceeds"),
    (dict(head_dim=64), -3, "head_dim 64"),
    (dict(q=None), -1, "q is NULL"),
])
def test_prefill_host_checks(pa, over, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_prefill(**prefill_args(**over))
    assert e.value.code == code
    assert needle in str(e.value)


def mixed_args(**over):
    a = dict(q=FAKE, n_tok=4104, cu_seqlens=FAKE, n_seq=9, n_seq_decode=8, max_q_len=4096,
             k_pool=FAKE, v_pool=FAKE, k_scale=None, v_scale=None, n_pages=4096,
             block_table=FAKE, max_pages_per_seq=2048, ctx_lens=FAKE, n_head=16, n_head_kv=4,
             head_dim=256, page_size=16, kv_dtype=0, out=FAKE, workspace=FAKE,
             workspace_bytes=1 << 30, stream=0)
    a.update(over)
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(n_tok=0), -2, "zero rows"),
    (dict(n_seq=0), -2, "zero sequences"),
    (dict(n_seq_decode=10), -2, "n_seq_decode 10"),
    (dict(n_seq_decode=-1), -2, "n_seq_decode -1"),
    (dict(cu_seqlens=None), -1, "cu_seqlens is NULL"),
    (dict(ctx_lens=None), -1, "ctx_lens is NULL"),
    (dict(max_q_len=0), -2, "max_q_len 0"),
    (dict(max_q_len=4097), -2, "max_q_len 4097"),
    (dict(n_tok=8), -2, "cannot hold"),
    (dict(n_seq=8, n_tok=9), -2, "decode rows only"),
    (dict(n_head=6, n_head_kv=4), -2, "not a multiple"),
    (dict(n_head=12, n_head_kv=4), -3, "query heads per kv head"),
    (dict(head_dim=64), -3, "head_dim 64"),
    (dict(workspace_bytes=100), -4, "workspace has 100 bytes"),
    (dict(q=None), -1, "q is NULL"),
])
def test_mixed_host_checks(pa, over, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_mixed(**mixed_args(**over))
    assert e.value.code == code
    assert needle in str(e.value)


def test_mixed_workspace_is_the_decode_halfs(pa):
    assert pa.attn_paged_workspace_bytes(3, 8, 2048, 16, 256) == \
        pa.attn_paged_workspace_bytes(0, 8, 2048, 16, 256)


@pytest.mark.parametrize("over,code,needle", [
    (dict(n_tok=0), -2, "zero rows"),
    (dict(k_new=None), -1, "k_new"),
    (dict(slot_mapping=None), -1, "slot_mapping"),
    (dict(head_dim=512), -3, "head_dim 512"),
    (dict(kv_dtype=1), -1, "fp8 kv needs"),
])
def test_append_host_checks(pa, over, code, needle):
    a = dict(k_new=FAKE, v_new=FAKE, slot_mapping=FAKE, n_tok=4, k_pool=FAKE, v_pool=FAKE,
             k_scale=None, v_scale=None, n_pages=8, n_head_kv=2, head_dim=128, page_size=16,
             kv_dtype=0, stream=0)
    a.update(over)
    with pytest.raises(pa.AttnError) as e:
        pa.attn_kv_append(**a)
    assert e.value.code == code
    assert needle in str(e.value)


def test_host_checkers(pa):
    assert pa.attn_check_lengths_host([5, 9], 1, 1, 16) == 0
    with pytest.raises(pa.AttnError) as e:
        pa.attn_check_lengths_host([5, 20], 1, 1, 16)
    assert e.value.code == pa.ATTN_E_RANGE and "ctx_lens[1]" in str(e.value)
    with pytest.raises(pa.AttnError):
        pa.attn_check_lengths_host([5, 7], 8, 4, 16)
    bt = np.array([[0, 1], [2, -1]], np.int32)
    assert pa.attn_check_block_table_host(bt, [20, 3], 2, 16, 3) == 0
    with pytest.raises(pa.AttnError) as e:
        pa.attn_check_block_table_host(bt, [20, 20], 2, 16, 3)
    assert "block_table[1][1]" in str(e.value)


@pytest.mark.parametrize("over,code,needle", [
    (dict(prefill_fp8=4), -3, "prefill_fp8 bits 0x4"),
    (dict(prefill_fp8=1), -3, "need an fp8 cache"),
    (dict(prefill_fp8=2), -3, "need an fp8 cache"),
    (dict(prefill_fp8=1, kv_dtype=1, k_scale=FAKE, v_scale=FAKE, n_rows=0), -2, "zero rows"),
    (dict(prefill_fp8=1, kv_dtype=1, k_scale=None, v_scale=None), -1, "fp8 kv needs"),
    (dict(prefill_fp8=0, ctx_len=40000), -5, "exceeds"),
])
def test_prefill_fp8_host_checks(pa, over, code, needle):
    args = prefill_args(prefill_fp8=0)
    args.update(over)
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_prefill_fp8(**args)
    assert e.value.code == code
    assert needle in str(e.value)


def noalloc_args(**over):
    a = decode_args(**over)
    del a["workspace"], a["workspace_bytes"]
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(q=None), -1, "q is NULL"),
    (dict(n_seq=0), -2, "zero sequences"),
    (dict(head_dim=96), -3, "head_dim 96"),
    # 4096 sequences x 64 splits x 8 heads x 130 floats: beyond the 64 MiB array
    (dict(n_seq=4096, max_pages_per_seq=2048), -4, "scratch array holds"),
])
def test_decode_noalloc_host_checks(pa, over, code, needle):
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_decode_noalloc(**noalloc_args(**over))
    assert e.value.code == code
    assert needle in str(e.value)
    assert "attn_paged_decode_noalloc" in str(e.value)
