"""sparse_attn_fwd_decode_noalloc (split partials in the library's static device buffer)
against sparse_attn_fwd_decode (caller workspace): two calls in a row, the second smaller,
each bit-identical to the workspace entry point (same kernels and split choice) and within
the bar of the oracle. Both are called through the C ABI (ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import flash_attention_int8_amd as fa
from dsa_harness import GpuRun, OracleView, assert_close, compare_rows, make_kv
from synthetic import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _w(**kw) -> Workload:
    base = dict(name="noalloc", batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
                seq_len=6000, q_len=1, idx_dim=64, top_k=1024, prefix_len=5, page_size=64,
                shuffled_pages=True, qkv_source="bf16")
    base.update(kw)
    return Workload(**base)


def _both(inp, num_splits):
    w = inp.workload
    kv = make_kv(inp)
    idx = fa.index_topk(kv, inp.q_idx, 1, 1, w.top_k)[:, 0].contiguous()
    q = inp.q[:, 0].contiguous()
    B, Hq, D = q.shape
    width = int(idx.shape[-1])
    scale = 1.0 / math.sqrt(D)
    out_ws, lse_ws = fa.decode(kv, q, idx, num_splits=num_splits)
    out_na = torch.full_like(q, 7)
    lse_na = torch.full((B, Hq), 7.0, dtype=torch.float32, device=q.device)
    fa.sparse_attn_fwd_decode_noalloc(kv, q, Hq, idx, width, scale, num_splits, out_na, lse_na)
    torch.cuda.synchronize()
    return idx, (out_ws, lse_ws), (out_na, lse_na)


@pytest.mark.parametrize("num_splits", [0, 5])
def test_noalloc_decode_matches_workspace_entry(num_splits):
    first = make_inputs(_w(), seed=51, device="cpu", seq_lens=[6000, 4100, 5333], spare_pages=2).to(DEV)
    second = make_inputs(_w(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=3000, top_k=300,
                            prefix_len=0),
                         seed=52, device="cpu", seq_lens=[3000, 2222]).to(DEV)
    for inp in (first, second):
        w = inp.workload
        print(f"\n[noalloc] batch={w.batch} heads={w.num_q_heads}/{w.num_kv_heads} "
              f"T={w.seq_len} K={w.top_k} splits={num_splits}", flush=True)
        idx, (o_ws, l_ws), (o_na, l_na) = _both(inp, num_splits)
        assert torch.equal(o_na, o_ws)
        assert torch.equal(l_na, l_ws)
        ov = OracleView(inp)
        g = GpuRun()
        g.indices = idx.unsqueeze(1)
        g.out = o_na.unsqueeze(1)
        g.lse = l_na.unsqueeze(1)
        rows = [(b, 0, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
        assert_close(compare_rows(g, ov, rows))


def test_noalloc_rejects_more_than_its_buffer():
    """A call whose partials exceed the static buffer returns SA_ERR_SCRATCH before launching."""
    cap = fa.sparse_attn_decode_noalloc_max_bytes()
    assert cap == 16 << 20
    w = _w(batch=64, num_q_heads=64, num_kv_heads=8, seq_len=200, top_k=256, prefix_len=0)
    inp = make_inputs(w, seed=53, device=DEV, with_q=True)
    kv = make_kv(inp)
    q = inp.q[:, 0].contiguous()
    idx = torch.zeros((64, 8, 256), dtype=torch.int32, device=DEV)
    need = fa.sparse_attn_decode_workspace_size(kv, 64, 256, 256)
    assert need > cap
    out = torch.empty_like(q)
    with pytest.raises(fa.SparseAttnError) as e:
        fa.sparse_attn_fwd_decode_noalloc(kv, q, 64, idx, 256, 0.1, 256, out)
    assert e.value.status == fa.SA_ERR_SCRATCH
