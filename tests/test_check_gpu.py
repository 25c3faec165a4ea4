"""Validation of device data (sparse_attn_validate and the SPARSE_ATTN_CHECK=1 mode) on planted
bad inputs: an out-of-range page-table entry among the used pages (one beyond a sequence's pages
is not counted), list entries past the query's position or negative, entries out of order, and a
sequence length of 0. The attention calls skip such entries (nothing faults); the report counts
them and locates the first of each kind."""
import os

import pytest
import torch

import flash_attention_int8_amd as fa
from dsa_harness import make_kv
from synthetic import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
INT32_MAX = 2 ** 31 - 1


def _w(**kw):
    base = dict(name="check", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_len=300,
                q_len=1, idx_dim=64, top_k=64, prefix_len=0, page_size=64, shuffled_pages=True,
                qkv_source="bf16")
    base.update(kw)
    return Workload(**base)


def _planted():
    w = _w()
    inp = make_inputs(w, seed=61, device="cpu", seq_lens=[300, 250], spare_pages=2).to(DEV)
    kv = make_kv(inp)
    lists = fa.index_topk(kv, inp.q_idx, 1, 1, w.top_k)
    torch.cuda.synchronize()
    bad_table = inp.page_table.clone()
    bad_table[0, 1] = inp.num_pages + 5     # a page sequence 0 uses (tokens 64..127)
    bad_table[1, 4] = -3                    # sequence 1 (250 tokens) uses pages 0..3 only
    bad = lists.clone()
    bad[0, 0, 0, 63] = 301                  # past pos 299: out of range (last entry: order kept)
    bad[0, 0, 1, 20] = -7                   # negative: out of range, and below the entry before
    a, b = bad[1, 0, 1, 10].item(), bad[1, 0, 1, 11].item()
    bad[1, 0, 1, 10], bad[1, 0, 1, 11] = b, a  # out of order once
    return w, inp, lists, bad_table, bad


def _kv_with(inp, table):
    kv = make_kv(inp)
    return fa.PagedKV(k_pool=inp.k_pool, v_pool=inp.v_pool, kidx_pool=inp.kidx_pool, page_table=table,
                      seq_lens=inp.seq_lens, max_seq_len=max(inp.seq_lens_host), prefix_len=0,
                      num_kv_heads=2, head_dim=128, idx_dim=64, num_idx_heads=2, page_size=64,
                      num_pages=inp.num_pages) if table is not None else kv


def test_validate_clean_and_planted():
    w, inp, lists, bad_table, bad = _planted()
    width = w.index_width
    rep = torch.full((8,), 123, dtype=torch.int32, device=DEV)
    fa.sparse_attn_validate(make_kv(inp), lists[:, 0].contiguous(), width, 1, 1, rep)
    torch.cuda.synchronize()
    assert rep.tolist() == [0, 0, 0, 0, INT32_MAX, INT32_MAX, 1, 0]
    fa.sparse_attn_validate(_kv_with(inp, bad_table), bad[:, 0].contiguous(), width, 1, 1, rep)
    torch.cuda.synchronize()
    max_pages = inp.page_table.shape[1]
    # rows are (b * q_len + i) * H_idx + g: row 0 = (0, 0), row 1 = (0, 1)
    assert rep.tolist() == [0, 1, 2, 2, 0 * max_pages + 1, 63, 1, 0]
    # a sequence length of 0 (and its pages then unused)
    lens = inp.seq_lens.clone()
    lens[1] = 0
    kv0 = fa.PagedKV(k_pool=inp.k_pool, v_pool=inp.v_pool, kidx_pool=inp.kidx_pool,
                     page_table=inp.page_table, seq_lens=lens, max_seq_len=300, prefix_len=0,
                     num_kv_heads=2, head_dim=128, idx_dim=64, num_idx_heads=2, page_size=64,
                     num_pages=inp.num_pages)
    fa.sparse_attn_validate(kv0, None, 0, 1, 1, rep)
    torch.cuda.synchronize()
    assert rep.tolist() == [1, 0, 0, 0, INT32_MAX, INT32_MAX, 1, 0]


def test_check_mode_reports_what_calls_read():
    w, inp, lists, bad_table, bad = _planted()
    kv_bad = _kv_with(inp, bad_table)
    rep = torch.zeros(8, dtype=torch.int32, device=DEV)
    q = inp.q[:, 0].contiguous()
    os.environ["SPARSE_ATTN_CHECK"] = "1"
    try:
        fa.sparse_attn_check_report(rep)    # clears what earlier calls left
        out, lse = fa.decode(kv_bad, q, bad[:, 0].contiguous())
        fa.sparse_attn_check_report(rep)
        torch.cuda.synchronize()
        assert rep.tolist() == [0, 1, 2, 2, 1, 63, 1, 0]
        assert torch.isfinite(out.float()).all()
        # a clean call adds nothing but its count
        fa.decode(make_kv(inp), q, lists[:, 0].contiguous())
        fa.sparse_attn_check_report(rep)
        torch.cuda.synchronize()
        assert rep.tolist() == [0, 0, 0, 0, INT32_MAX, INT32_MAX, 1, 0]
    finally:
        del os.environ["SPARSE_ATTN_CHECK"]
    # without the variable nothing is checked
    fa.decode(kv_bad, q, bad[:, 0].contiguous())
    fa.sparse_attn_check_report(rep)
    torch.cuda.synchronize()
    assert rep.tolist() == [0, 0, 0, 0, INT32_MAX, INT32_MAX, 0, 0]
