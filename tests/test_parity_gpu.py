"""Parity of the HIP path with the fp64 oracle on seeded inputs (needs an MI355X).

Bars: selected index lists and indexer scores bit-exact; bf16 outputs within max-abs 2e-2
and mean-abs 2e-3 of the fp64 oracle; fp32 LSE within 1e-3 on the decode and gathered-row
prefill paths (fp32 row sums) and within 4e-3 on the dense and masked-tile paths (bf16-rounded
P in the row sum).
Small cases check every row and cover ragged lengths, shuffled pages with spare pages,
a forced prefix longer than some sequences, shared indexer heads, every group size, both
head dims, all indexer widths, split counts and heavy score ties.
"""
import math

import numpy as np
import pytest
import torch

import flash_attention_int8_amd as fa
import oracle
from synthetic import CONFIGS, Workload, make_inputs
from dsa_harness import (LSE_ABS_FP32_SUM, OracleView, assert_close, bits, compare_block,
                         compare_rows, make_kv, merge_stats, run_gpu, f64, sampled_positions)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def all_rows(inp):
    w = inp.workload
    return [(b, i, g) for b in range(w.batch) for i in range(w.q_len) for g in range(w.num_kv_heads)]


def W(**kw) -> Workload:
    base = dict(name="case", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_len=256,
                q_len=256, idx_dim=64, top_k=32, prefix_len=0, page_size=64, shuffled_pages=True,
                qkv_source="bf16")
    base.update(kw)
    return Workload(**base)


def _banner(msg):
    print(f"\n[parity] {msg}", flush=True)


# ------------------------------------------------------------------ small cases, every row

SMALL = {
    "tiny_sparse_prefill": (CONFIGS["tiny_sparse_prefill"], {}),
    "tiny_dense": (CONFIGS["tiny_sparse_prefill"].with_(top_k=0, idx_dim=0), {}),
    "ragged_prefill_prefix": (W(batch=2, seq_len=300, q_len=250, top_k=40, prefix_len=5),
                              dict(seq_lens=[300, 250], spare_pages=3)),
    "prefill_g1_d64_didx32": (W(num_q_heads=2, num_kv_heads=2, head_dim=64, idx_dim=32, seq_len=200,
                                q_len=200, top_k=16), {}),
    "prefill_g8_didx128": (W(num_q_heads=16, num_kv_heads=2, idx_dim=128, seq_len=192, q_len=130,
                             top_k=24, prefix_len=3), dict(seq_lens=[192])),
    "prefill_shared_indexer": (W(batch=2, seq_len=160, q_len=160, top_k=20), dict(num_idx_heads=1)),
    "prefill_ties": (W(seq_len=320, q_len=320, top_k=50, prefix_len=7), dict(idx_values=(-1, 0, 1))),
    "dense_ragged_paged": (W(batch=2, seq_len=300, q_len=300, idx_dim=0, top_k=0),
                           dict(seq_lens=[300, 301], spare_pages=2)),
    "dense_d64_g2": (W(num_q_heads=4, head_dim=64, idx_dim=0, top_k=0, seq_len=257, q_len=257,
                       page_size=128), {}),
    "dense_contiguous_g4": (W(idx_dim=0, top_k=0, seq_len=512, q_len=512, page_size=512,
                              shuffled_pages=False), {}),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_every_row(name):
    w, kw = SMALL[name]
    _banner(f"small case {name}: {w}")
    inp = make_inputs(w, seed=11, device="cpu", **kw).to(DEV)
    gpu = run_gpu(inp, q_chunk=96 if w.q_len > 200 else None)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    assert_close(compare_rows(gpu, ov, all_rows(inp)))


MASKED_CASES = [n for n, (w, _) in SMALL.items() if not w.dense]


@pytest.mark.parametrize("name", MASKED_CASES)
def test_masked_prefill_every_row(name):
    """Sparse prefill on masked dense tiles: the oracle's result on every row, and the same
    lists as the gathered path (the lists come from the same top-K call)."""
    w, kw = SMALL[name]
    _banner(f"masked prefill {name}: {w}")
    inp = make_inputs(w, seed=11, device="cpu", **kw).to(DEV)
    chunk = 96 if w.q_len > 200 else None
    gpu = run_gpu(inp, q_chunk=chunk, masked=True)
    gat = run_gpu(inp, q_chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(gpu.indices, gat.indices)
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


def test_masked_prefill_irregular_lists():
    """Hand-made lists: -1 holes, ids past the query position or the sequence, negative ids,
    repeated ids (counted once) and an empty list (out = 0, lse = -inf); several 64-key tiles
    and a ragged 256-query block."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=700, q_len=300, top_k=64, idx_dim=64)
    _banner("masked prefill, irregular lists")
    inp = make_inputs(w, seed=21, device="cpu", seq_lens=[700, 650], spare_pages=2)
    rng = np.random.default_rng(5)
    B, S, H, Wd = w.batch, w.q_len, w.num_kv_heads, 80
    lists = np.full((B, S, H, Wd), -1, dtype=np.int32)
    for b in range(B):
        for i in range(S):
            pos = oracle.query_position(inp.seq_lens_host[b], S, i)
            for g in range(H):
                n = int(rng.integers(1, 60))
                ids = rng.integers(0, pos + 1, size=n)
                junk = np.array([pos + 1, pos + 50, inp.seq_lens_host[b] + 3, -7, ids[0]])
                row = np.concatenate([ids, junk[: int(rng.integers(0, 6))]])
                rng.shuffle(row)
                lists[b, i, g, :len(row)] = row
    lists[1, 17, 1, :] = -1        # empty list
    lists[0, 0, 0, :] = 0          # the only visible key, repeated
    inp = inp.to(DEV)
    kv = make_kv(inp)
    idx = torch.from_numpy(lists).to(DEV)
    out, lse = fa.prefill_masked(kv, inp.q, q_tail=S, indices=idx)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    G = w.group
    errs, lse_errs = [], []
    for b in range(B):
        for i in range(S):
            pos = oracle.query_position(inp.seq_lens_host[b], S, i)
            for g in range(H):
                keys = np.unique(lists[b, i, g])
                keys = keys[(keys >= 0) & (keys <= pos)]
                got = f64(out[b, i, g * G:(g + 1) * G])
                got_lse = lse[b, i, g * G:(g + 1) * G].double().cpu().numpy()
                if len(keys) == 0:
                    assert np.all(got == 0) and np.all(np.isneginf(got_lse)), (b, i, g)
                    continue
                kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, ov.table[b], w.page_size, g, keys))
                vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, ov.table[b], w.page_size, g, keys))
                qb = oracle.bf16_to_f64(bits(inp.q[b, i, g * G:(g + 1) * G]))
                o, l = oracle.attend(qb, kr, vr, 1.0 / math.sqrt(w.head_dim))
                errs.append(np.abs(got - o).ravel())
                lse_errs.append(np.abs(got_lse - l))
    e = np.concatenate(errs)
    assert_close((float(e.max()), float(e.mean()), float(np.concatenate(lse_errs).max())))


@pytest.mark.parametrize("n_new,shared_idx,hole", [(1, False, False), (70, False, True),
                                                   (1, True, True), (130, True, False)])
def test_kv_append_matches_oracle(n_new, shared_idx, hole):
    """New tokens written through the page table: every pool element equals the oracle's
    append (bit-exact), tokens of a page missing from the table are skipped, and a decode step
    over the updated cache matches the oracle."""
    w = W(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_len=300, q_len=1, top_k=40,
          idx_dim=64, prefix_len=2)
    _banner(f"kv append n_new={n_new} shared_idx={shared_idx} hole={hole}")
    lens = [300, 200, 177]
    inp = make_inputs(w, seed=31, device="cpu", seq_lens=lens, spare_pages=3,
                      num_idx_heads=1 if shared_idx else None)
    if hole:  # the page of sequence 1's last token is missing
        inp.page_table[1, (lens[1] - 1) // w.page_size] = -1
    g = torch.Generator().manual_seed(32)
    Hi = inp.num_idx_heads
    k_new = torch.randn((w.batch, n_new, w.num_kv_heads, w.head_dim), generator=g).to(torch.bfloat16)
    v_new = torch.randn((w.batch, n_new, w.num_kv_heads, w.head_dim), generator=g).to(torch.bfloat16)
    i_new = torch.randint(-127, 128, (w.batch, n_new, Hi, w.idx_dim), generator=g).to(torch.int8)
    # oracle: the same rows written into host copies of the pools
    kp, vp, ip = bits(inp.k_pool), bits(inp.v_pool), inp.kidx_pool.numpy().copy()
    table = inp.page_table.numpy()
    for b in range(w.batch):
        t = np.arange(lens[b] - n_new, lens[b])
        for h in range(w.num_kv_heads):
            oracle.append_rows(kp, table[b], w.page_size, h, t, bits(k_new[b, :, h]))
            oracle.append_rows(vp, table[b], w.page_size, h, t, bits(v_new[b, :, h]))
        for h in range(Hi):
            oracle.append_rows(ip, table[b], w.page_size, h, t, i_new[b, :, h].numpy())
    inp = inp.to(DEV)
    kv = make_kv(inp)
    fa.kv_append(kv, k_new.to(DEV), v_new.to(DEV), i_new.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits(inp.k_pool), kp)
    assert np.array_equal(bits(inp.v_pool), vp)
    assert np.array_equal(inp.kidx_pool.cpu().numpy(), ip)
    if not hole:
        gpu = run_gpu(inp, fused=True)
        torch.cuda.synchronize()
        assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


WINDOW_CASES = {
    # (workload, inputs, window)
    "decode_window_ragged": (W(batch=4, num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=128,
                               seq_len=3000, q_len=1, top_k=100, prefix_len=13),
                             dict(seq_lens=[3000, 64, 777, 10], spare_pages=5), 200),
    "decode_window_long": (W(batch=2, seq_len=40000, q_len=1, top_k=2048, prefix_len=5),
                           dict(seq_lens=[40000, 20000]), 512),
    "prefill_window_ragged": (W(batch=2, seq_len=300, q_len=250, top_k=40, prefix_len=5),
                              dict(seq_lens=[300, 250], spare_pages=3), 64),
    "prefill_window_ties_shared": (W(seq_len=320, q_len=320, top_k=50, prefix_len=7),
                                   dict(idx_values=(-1, 0, 1), num_idx_heads=1), 33),
}


@pytest.mark.parametrize("name", list(WINDOW_CASES))
def test_index_topk_window_matches_oracle(name):
    """Hybrid lists (the last `window` keys and the prefix forced, the top-K over the rest):
    bit-exact against the oracle, and attention over them (gathered, masked dense, decode)
    within the bar."""
    w, kw, win = WINDOW_CASES[name]
    _banner(f"hybrid lists {name} window={win}")
    inp = make_inputs(w, seed=41, device="cpu", **kw).to(DEV)
    kv = make_kv(inp)
    B, S, G, Hi = w.batch, w.q_len, w.group, inp.num_idx_heads
    width = w.prefix_len + w.top_k + win
    lists = torch.empty((B, S, Hi, width), dtype=torch.int32, device=DEV)
    chunk = 96 if S > 200 else S
    for q0 in range(0, S, chunk):
        c = min(chunk, S - q0)
        lists[:, q0:q0 + c] = fa.index_topk_window(kv, inp.q_idx[:, q0:q0 + c].contiguous(), c, S - q0,
                                                   w.top_k, win)
    outs = []
    if S == 1:
        o, l = fa.decode(kv, inp.q[:, 0].contiguous(), lists[:, 0].contiguous())
        outs.append((o.unsqueeze(1), l.unsqueeze(1)))
    else:
        outs.append(fa.prefill(kv, inp.q, q_tail=S, indices=lists))
        outs.append(fa.prefill_masked(kv, inp.q, q_tail=S, indices=lists))
    torch.cuda.synchronize()
    ov = OracleView(inp)
    got_lists = lists.cpu().numpy()
    rows = all_rows(inp)
    if len(rows) > 300:
        rows = rows[:: len(rows) // 300]
    scale = 1.0 / math.sqrt(w.head_dim)
    errs = [[] for _ in outs]
    lerrs = [[] for _ in outs]
    for (b, i, g) in rows:
        gi = 0 if Hi == 1 else g
        pos = oracle.query_position(inp.seq_lens_host[b], S, i)
        qi = inp.q_idx[b, i, gi].cpu().numpy()
        fn = lambda t: oracle.index_scores(qi, oracle.page_rows(ov.kidx, ov.table[b], w.page_size, gi, t))
        want = oracle.hybrid_index_list(pos, w.prefix_len, win, w.top_k, width, fn)
        assert np.array_equal(got_lists[b, i, gi], want), (name, b, i, g)
        keys = want[want >= 0]
        kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, ov.table[b], w.page_size, g, keys))
        vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, ov.table[b], w.page_size, g, keys))
        qb = oracle.bf16_to_f64(bits(inp.q[b, i, g * G:(g + 1) * G]))
        o_ref, l_ref = oracle.attend(qb, kr, vr, scale)
        for k, (o, l) in enumerate(outs):
            errs[k].append(np.abs(f64(o[b, i, g * G:(g + 1) * G]) - o_ref).ravel())
            lerrs[k].append(np.abs(l[b, i, g * G:(g + 1) * G].double().cpu().numpy() - l_ref))
    for e, le in zip(errs, lerrs):
        e = np.concatenate(e)
        assert_close((float(e.max()), float(e.mean()), float(np.concatenate(le).max())))


DECODE = {
    "decode_ragged_prefix": (W(batch=4, num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=128,
                               seq_len=1000, q_len=1, top_k=100, prefix_len=13),
                             dict(seq_lens=[1000, 64, 777, 10], spare_pages=5)),
    "decode_g4_d128": (W(batch=3, num_q_heads=16, num_kv_heads=4, seq_len=5000, q_len=1, top_k=256),
                       dict(seq_lens=[5000, 4097, 300])),
    "decode_g2_shared_indexer": (W(batch=2, num_q_heads=4, seq_len=3000, q_len=1, top_k=64,
                                   idx_dim=32), dict(num_idx_heads=1)),
    "decode_ties": (W(batch=2, seq_len=4000, q_len=1, top_k=300, prefix_len=2),
                    dict(idx_values=(-1, 0, 1))),
    "decode_g1": (W(batch=2, num_q_heads=2, num_kv_heads=2, seq_len=2000, q_len=1, top_k=128), {}),
    # rows of >= 16384 candidates take the multi-workgroup selection
    "decode_long_ragged_prefix": (W(batch=3, seq_len=70000, q_len=1, top_k=500, prefix_len=100),
                                  dict(seq_lens=[70000, 16500, 40000])),
    "decode_long_ties": (W(batch=2, seq_len=33000, q_len=1, top_k=700, prefix_len=3),
                         dict(idx_values=(-1, 0, 1))),
    "decode_long_shared_indexer": (W(batch=2, num_q_heads=8, seq_len=24576, q_len=1, top_k=2048,
                                     idx_dim=32), dict(num_idx_heads=1)),
    # the first tokens of sequences (1 and 2 cached tokens, a page boundary at 64 / 65) beside a
    # row long enough for the fused selection; the prefix covers the short rows entirely
    "decode_first_tokens": (W(batch=5, num_q_heads=8, num_kv_heads=2, seq_len=20000, q_len=1,
                              top_k=64, prefix_len=3),
                            dict(seq_lens=[20000, 1, 2, 64, 65])),
    # a large K: the fused final pass holds more candidates than its registers (general path),
    # and a row with barely more candidates than K
    "decode_large_k": (W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=40000, q_len=1,
                         top_k=12000, prefix_len=1), dict(seq_lens=[40000, 12100])),
    # the fused selection at d_idx = 128 (two waves per SIMD in its main pass), ragged rows
    "decode_long_didx128": (W(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, idx_dim=128,
                              seq_len=45000, q_len=1, top_k=1000, prefix_len=5),
                            dict(seq_lens=[45000, 17000, 30001])),
    # long rows on pages of 128 and 256 tokens (two and four 64-token blocks per page)
    "decode_long_page128": (W(batch=2, seq_len=36000, q_len=1, top_k=1500, prefix_len=7, page_size=128),
                            dict(seq_lens=[36000, 20000], spare_pages=3)),
    "decode_long_page256_g8": (W(batch=2, num_q_heads=16, num_kv_heads=2, seq_len=50000, q_len=1,
                                 top_k=2048, page_size=256), dict(seq_lens=[50000, 33333])),
}


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
@pytest.mark.parametrize("name", list(DECODE))
def test_decode_every_row(name, splits):
    w, kw = DECODE[name]
    _banner(f"decode case {name} splits={splits}")
    inp = make_inputs(w, seed=5, device="cpu", **kw).to(DEV)
    gpu = run_gpu(inp, num_splits=splits)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("name", ["decode_long_ragged_prefix", "decode_long_ties",
                                  "decode_long_shared_indexer", "decode_long_didx128",
                                  "decode_first_tokens", "decode_large_k",
                                  "decode_ragged_prefix", "decode_long_page128",
                                  "decode_long_page256_g8"])
def test_fused_index_topk_matches(name):
    """The fused indexer + top-K gives the oracle's lists, identical to the two-step path."""
    w, kw = DECODE[name]
    _banner(f"fused index+topk {name}")
    inp = make_inputs(w, seed=6, device="cpu", **kw).to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


FUSED_PREFILL = {
    **{n: SMALL[n] for n in MASKED_CASES},
    # rows of > 6144 candidates whose keys fall in a handful of 16-bit keys: the lists overflow
    # and the exact radix select runs on recomputed scores
    "prefill_long_ties": (W(seq_len=8000, q_len=32, top_k=300, prefix_len=2),
                          dict(idx_values=(-1, 0, 1))),
    "prefill_long_random": (W(batch=2, seq_len=20000, q_len=40, top_k=1000, prefix_len=5),
                            dict(seq_lens=[20000, 9000])),
    # K near the row length (more places than one wave's list holds, rows of 4000-6000
    # candidates) and rows shorter than K at the block's start
    "prefill_large_k": (W(seq_len=6000, q_len=3000, top_k=3000, prefix_len=4), {}),
}


@pytest.mark.parametrize("name", list(FUSED_PREFILL))
def test_fused_index_topk_prefill_matches(name):
    """Prefill blocks through sparse_attn_index_topk (16-bit keys, exact scores recomputed for
    the keys that tie in the K-th largest key): the same lists as index then topk, and the
    oracle's lists and outputs."""
    w, kw = FUSED_PREFILL[name]
    _banner(f"fused index+topk prefill {name}")
    inp = make_inputs(w, seed=17, device="cpu", **kw).to(DEV)
    chunk = 96 if w.q_len > 200 else None
    fused = run_gpu(inp, q_chunk=chunk, fused=True)
    two = run_gpu(inp, q_chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    rows = all_rows(inp)
    if len(rows) > 400:
        rows = rows[:: max(1, len(rows) // 400)]
    assert_close(compare_rows(fused, OracleView(inp), rows))


def test_fused_index_topk_concentrated_chunk_rescore():
    """One 8192-token chunk holds most of the top: its first 1024 tokens get maximal keys
    (so the chunk's threshold lands in their bin) and its next 1536 tokens keys one bin lower,
    part of which belong to the top-K. The chunk drops those, the candidates' K-th largest bin
    falls below its threshold, and the final pass must rescore the row exactly."""
    w = W(batch=2, seq_len=65536, q_len=1, top_k=2048)
    inp = make_inputs(w, seed=9, device="cpu")
    inp.q_idx.fill_(2)
    k = inp.kidx_pool
    k.copy_(torch.randint(-20, 21, k.shape, generator=torch.Generator().manual_seed(1)).to(torch.int8))
    table = inp.page_table
    for b in range(w.batch):
        for p in range(256, 272):       # chunk 2, first slab: score 2*127*64 = 16256
            k[table[b, p]] = 127
        for p in range(272, 296):       # next 24 blocks: score 2*64*64 = 8192, one bin lower
            k[table[b, p]] = 64
    inp = inp.to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("case", ["all_equal", "equal_with_some_higher", "narrow"])
def test_fused_index_topk_packed_scores(case):
    """Scores packed into one or two histogram bins, where a chunk's threshold is refined to a
    single key and keys equal to it stop being kept once the chunk holds K candidates:
      all_equal               every indexer key zero, so the top-K is the first K tokens
      equal_with_some_higher  zero keys except scattered blocks of small positive keys, so the
                              top holds those blocks plus the earliest ties
      narrow                  small random keys (values in [-20, 20]) under a constant query"""
    w = W(batch=2, seq_len=65536, q_len=1, top_k=2048, prefix_len=3)
    _banner(f"fused index+topk, packed scores: {case}")
    inp = make_inputs(w, seed=21, device="cpu", seq_lens=[65536, 40001])
    k = inp.kidx_pool
    if case == "narrow":
        inp.q_idx.fill_(2)
        k.copy_(torch.randint(-20, 21, k.shape, generator=torch.Generator().manual_seed(5)).to(torch.int8))
    else:
        inp.q_idx.fill_(1)
        k.zero_()
        if case == "equal_with_some_higher":
            table = inp.page_table
            for b in range(w.batch):
                for j in range(9):       # 9 blocks of 64 keys spread over the first 40000 tokens
                    k[table[b, 3 + 67 * j]] = 1 + j % 3
    inp = inp.to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


def test_fused_index_topk_spread_maximal_blocks():
    """24 blocks of maximal keys spread over the row (every 4th block pattern) among small
    random keys: the lists must still equal the two-step path and the oracle."""
    w = W(batch=2, seq_len=65536, q_len=1, top_k=2048)
    inp = make_inputs(w, seed=9, device="cpu")
    inp.q_idx.fill_(1)
    k = inp.kidx_pool
    k.copy_(torch.randint(-20, 21, k.shape, generator=torch.Generator().manual_seed(1)).to(torch.int8))
    table = inp.page_table
    for b in range(w.batch):
        for j in range(24):
            k[table[b, 4 * ((7 * j) % 256)]] = 127
    inp = inp.to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


def test_fused_index_topk_many_chunks_ragged():
    """Rows of more 8192-token chunks than the final pass has waves (each wave holds several
    chunks' candidates), ragged lengths so some waves hold none, and a forced prefix."""
    w = W(batch=3, head_dim=64, seq_len=300000, q_len=1, top_k=2048, prefix_len=7)
    _banner("fused index+topk 300K rows, ragged")
    inp = make_inputs(w, seed=12, device="cpu", seq_lens=[300000, 140000, 20000]).to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


def test_fused_index_topk_top_far_above_thresholds():
    """The top of each row lies far above every chunk's threshold (blocks of maximal keys
    outside the chunks' first 4096 tokens, the sample that sets a chunk's threshold, hundreds
    of coarse bins above the bulk), so the K-th largest falls beyond the final pass's fine
    histogram; 2560 tied maximal keys also make the tie order decide which 2048 are kept."""
    w = W(batch=2, seq_len=131072, q_len=1, top_k=2048)
    _banner("fused index+topk, top far above the chunk thresholds")
    inp = make_inputs(w, seed=13, device="cpu")
    inp.q_idx.fill_(127)
    k = inp.kidx_pool
    k.copy_(torch.randint(-127, 128, k.shape, generator=torch.Generator().manual_seed(3)).to(torch.int8))
    table = inp.page_table
    for b in range(w.batch):
        for c in range(8):              # 5 blocks in each of chunks 2, 4, .., 16, past the sample
            for j in range(5):
                k[table[b, 128 * (2 * c + 1) + 64 + 13 * j]] = 127
    inp = inp.to(DEV)
    fused = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("seq_len,q_len,prefix,vals", [
    (16000, 40, 3, 100000),     # rows of <= 32768 candidates, streamed: sampled lists
    (30000, 24, 0, 3),          # <= 32768, every key in one bin: the lists overflow, so the
                                # streamed two-digit radix select decides
    (30000, 24, 1, -1),         # <= 32768, keys 4096*k + {0,1,2}: short lists, ties at tau
    (33005, 2050, 5, 40000),    # > 32768 candidates and > 2048 rows: three passes over HBM
    (30000, 24, 2, -2),         # <= 32768, the top far above the sampled threshold: the lists
                                # hold it, but beyond the fine bins, so the radix select decides
])
def test_topk_row_paths(seq_len, q_len, prefix, vals):
    """Stand-alone top-K on score rows written directly (random ints in [-vals, vals); for
    vals == -1 multiples of 4096 in [-20, 20) plus 0..2; for vals == -2 ints in [-2000, 2000)
    with 1500 tokens per row raised to 600000 plus 0..49), for each single-row selection path
    and every outcome of the sampled short list; sampled rows must equal the oracle's lists."""
    top_k = 1000
    _banner(f"topk rows seq_len={seq_len} q_len={q_len} P={prefix} vals={vals}")
    w = W(num_q_heads=1, num_kv_heads=1, head_dim=64, idx_dim=32, seq_len=seq_len, q_len=q_len,
          top_k=top_k, prefix_len=prefix)
    inp = make_inputs(w, seed=21, device=DEV)
    kv = make_kv(inp)
    gen = torch.Generator().manual_seed(22)
    stride = (seq_len + 3) & ~3  # the ABI takes row strides in multiples of 4 scores
    if vals > 0:
        scores = torch.randint(-vals, vals, (1, q_len, 1, stride), generator=gen, dtype=torch.int32)
    elif vals == -2:
        scores = torch.randint(-2000, 2000, (1, q_len, 1, stride), generator=gen, dtype=torch.int32)
        for i in range(q_len):
            hot = torch.randperm(seq_len - 3 * q_len, generator=gen)[:1500]
            scores[0, i, 0, hot] = 600000 + torch.randint(0, 50, (1500,), generator=gen, dtype=torch.int32)
    else:
        scores = (4096 * torch.randint(-20, 20, (1, q_len, 1, stride), generator=gen, dtype=torch.int32)
                  + torch.randint(0, 3, (1, q_len, 1, stride), generator=gen, dtype=torch.int32))
    got = fa.topk(kv, scores.to(DEV), q_len, q_len, top_k).cpu().numpy()
    rows = range(q_len) if q_len <= 64 else np.linspace(0, q_len - 1, 48).astype(int)
    host = scores.numpy()
    for i in rows:
        pos = oracle.query_position(seq_len, q_len, int(i))
        want = oracle.index_list(pos, prefix, top_k, prefix + top_k, lambda t: host[0, i, 0, t])
        assert np.array_equal(got[0, i, 0], want), (i, got[0, i, 0][:8], want[:8])


def test_scores_exact_prefill_and_decode():
    for w, kw in [SMALL["ragged_prefill_prefix"], DECODE["decode_ragged_prefix"],
                  SMALL["prefill_g8_didx128"]]:
        _banner(f"scores {w}")
        inp = make_inputs(w, seed=3, device="cpu", **kw).to(DEV)
        gpu = run_gpu(inp, keep_scores=True, q_chunk=64)
        torch.cuda.synchronize()
        ov = OracleView(inp)
        for q0, sc in gpu.scores:
            sc = sc.cpu().numpy()
            for b in range(w.batch):
                for ic in range(sc.shape[1]):
                    for gi in range(inp.num_idx_heads):
                        c, want = ov.scores_row(b, q0 + ic, gi)
                        assert np.array_equal(sc[b, ic, gi, c], want), (b, q0 + ic, gi)


# ------------------------------------------------------------------ invariances

def _repack(inp, seed):
    """Same logical K/V/indexer content under a different page permutation."""
    w = inp.workload
    n = inp.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(seed)).to(DEV)
    new = make_inputs(w, seed=0, device="cpu", seq_lens=inp.seq_lens_host,
                      num_idx_heads=inp.num_idx_heads, spare_pages=n - sum(
                          -(-t // w.page_size) for t in inp.seq_lens_host)).to(DEV)
    new.q, new.q_idx = inp.q, inp.q_idx
    new.k_pool = torch.empty_like(inp.k_pool)
    new.v_pool = torch.empty_like(inp.v_pool)
    new.k_pool[perm] = inp.k_pool
    new.v_pool[perm] = inp.v_pool
    if inp.kidx_pool is not None:
        new.kidx_pool = torch.empty_like(inp.kidx_pool)
        new.kidx_pool[perm] = inp.kidx_pool
    tbl = inp.page_table.long()
    new.page_table = torch.where(tbl >= 0, perm[tbl.clamp(min=0)], tbl).to(torch.int32)
    return new


@pytest.mark.parametrize("name", ["ragged_prefill_prefix", "dense_ragged_paged"])
def test_page_permutation_is_bit_identical(name):
    w, kw = SMALL[name]
    inp = make_inputs(w, seed=2, device="cpu", **kw).to(DEV)
    a = run_gpu(inp)
    b = run_gpu(_repack(inp, 99))
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.lse, b.lse)
    if a.indices is not None:
        assert torch.equal(a.indices, b.indices)


def test_decode_permutation_and_determinism():
    w, kw = DECODE["decode_g4_d128"]
    inp = make_inputs(w, seed=8, device="cpu", **kw).to(DEV)
    a = run_gpu(inp, num_splits=4)
    a2 = run_gpu(inp, num_splits=4)
    b = run_gpu(_repack(inp, 5), num_splits=4)
    torch.cuda.synchronize()
    for x in (a2, b):
        assert torch.equal(a.indices, x.indices)
        assert torch.equal(a.out, x.out)
        assert torch.equal(a.lse, x.lse)


def test_decode_matches_last_prefill_row():
    """Decode at position T-1 equals row T-1 of a prefill over the same cache."""
    w = W(batch=2, seq_len=700, q_len=700, top_k=64, prefix_len=4)
    inp = make_inputs(w, seed=4, device="cpu").to(DEV)
    pre = run_gpu(inp, q_chunk=128)
    dec_inp = make_inputs(w.with_(q_len=1), seed=4, device="cpu").to(DEV)
    dec_inp.q = inp.q[:, -1:].contiguous()
    dec_inp.q_idx = inp.q_idx[:, -1:].contiguous()
    for splits in (1, 5):
        dec = run_gpu(dec_inp, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(dec.indices[:, 0], pre.indices[:, -1])
        d = (f64(dec.out[:, 0]) - f64(pre.out[:, -1]))
        assert np.abs(d).max() <= 1e-2


def test_top_k_covering_context_equals_dense():
    """K >= every row's candidate count: each list is 0..pos, and the gathered, masked-dense and
    dense causal kernels give the same attention (each within the bar of the oracle)."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=300, q_len=300, top_k=400, prefix_len=3)
    _banner("top-K covering the context vs dense")
    inp = make_inputs(w, seed=23, device="cpu", seq_lens=[300, 300], spare_pages=2).to(DEV)
    gat = run_gpu(inp, q_chunk=128)
    msk = run_gpu(inp, q_chunk=128, masked=True, fused=True)
    kv = make_kv(inp)
    den_out, den_lse = fa.prefill(kv, inp.q, q_tail=w.q_len)
    torch.cuda.synchronize()
    for b in range(w.batch):
        for i in (0, 1, 63, 64, 150, 299):
            want = np.full(w.index_width, -1, dtype=np.int32)
            want[: i + 1] = np.arange(i + 1)
            for g in range(w.num_kv_heads):
                assert np.array_equal(gat.indices[b, i, g].cpu().numpy(), want)
                assert np.array_equal(msk.indices[b, i, g].cpu().numpy(), want)
    ref = f64(den_out)
    for got in (gat.out, msk.out):
        d = np.abs(f64(got) - ref)
        assert d.max() <= 1e-2 and d.mean() <= 1e-3, (d.max(), d.mean())
    assert_close(compare_rows(gat, OracleView(inp), all_rows(inp)[::7]))


def test_lse_matches_definition_dense():
    """Dense LSE equals log-sum-exp of the scaled logits computed by the oracle."""
    w = SMALL["dense_contiguous_g4"][0]
    inp = make_inputs(w, seed=1, device="cpu").to(DEV)
    gpu = run_gpu(inp)
    torch.cuda.synchronize()
    rows = [(0, i, g) for i in (0, 1, 63, 64, 200, 511) for g in range(w.num_kv_heads)]
    assert_close(compare_rows(gpu, OracleView(inp), rows))


# ------------------------------------------------------------------ fused prefill (thresholds, dispatch)

SPARSE_SMALL = [n for n, (w, _) in SMALL.items() if not w.dense]


@pytest.mark.parametrize("name", SPARSE_SMALL)
def test_thresholds_and_fused_masked_every_row(name):
    """sparse_attn_select_thresholds equals the oracle's (tau, t_cut) on every row, bit for bit,
    and sparse_attn_prefill_fused on the masked path (no lists: masks from recomputed scores)
    matches the oracle on every row."""
    w, kw = SMALL[name]
    _banner(f"thresholds + fused masked prefill {name}: {w}")
    inp = make_inputs(w, seed=11, device="cpu", **kw).to(DEV)
    chunk = 96 if w.q_len > 200 else None
    gpu = run_gpu(inp, q_chunk=chunk, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("path", [fa.SA_PREFILL_GATHER, fa.SA_PREFILL_AUTO])
@pytest.mark.parametrize("name", SPARSE_SMALL)
def test_fused_prefill_other_paths_every_row(name, path):
    w, kw = SMALL[name]
    _banner(f"fused prefill path={path} {name}")
    inp = make_inputs(w, seed=11, device="cpu", **kw).to(DEV)
    gpu = run_gpu(inp, q_chunk=96 if w.q_len > 200 else None, prefill_path=path)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("top_k,want", [(64, fa.SA_PREFILL_GATHER), (384, fa.SA_PREFILL_GATHER),
                                         (420, fa.SA_PREFILL_MASKED), (2048, fa.SA_PREFILL_MASKED)])
def test_fused_prefill_dispatch_both_sides(top_k, want):
    """A 256-query block at the end of an 8192-token sequence with a 4-token prefix (mean
    8060.5 candidates, so the masked share 1/20 is 403 keys): top-64 and top-384 below it,
    top-420 and top-2048 above it. AUTO takes the expected path, and both paths match the
    oracle on sampled rows and every KV group (the masked path with key splits: 16 workgroups
    for 128 tiles); thresholds bit-exact."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=8192, q_len=256, top_k=top_k, prefix_len=4)
    _banner(f"fused prefill dispatch top_k={top_k}")
    inp = make_inputs(w, seed=41, device=DEV, seq_lens=[8192, 7000])
    kv = make_kv(inp)
    assert fa.sparse_attn_prefill_fused_choice(kv, w.num_q_heads, w.q_len, w.q_len, top_k) == want
    rows = [(b, i, g) for b in range(2) for i in (0, 1, 77, 128, 200, 254, 255) for g in range(2)]
    ov = OracleView(inp)
    for path in (fa.SA_PREFILL_AUTO, fa.SA_PREFILL_GATHER, fa.SA_PREFILL_MASKED):
        gpu = run_gpu(inp, prefill_path=path, thresholds=True)
        torch.cuda.synchronize()
        assert_close(compare_rows(gpu, ov, rows))


@pytest.mark.parametrize("values,seq_len", [((0,), 1500), ((-1, 1), 1500), ((-2, 0, 3), 700)])
def test_thresholds_many_equal_scores(values, seq_len):
    """Indexer values from tiny sets: every score equal (all keys of a row share one histogram
    bin, more than the selection's LDS lists hold, so it takes its histogram passes), or a few
    distinct scores with long runs of ties. Thresholds bit-exact and the masked fused prefill
    within the bar on every row."""
    w = W(batch=1, num_q_heads=8, num_kv_heads=2, seq_len=seq_len, q_len=96, top_k=100, prefix_len=3)
    _banner(f"thresholds, indexer values {values}, T={seq_len}")
    inp = make_inputs(w, seed=43, device="cpu", idx_values=values).to(DEV)
    gpu = run_gpu(inp, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("tiles,top_k", [((0, 8), 40), ((3, 11, 19), 150), ((5,), 70)])
def test_thresholds_boundary_keys_in_one_wave(tiles, top_k):
    """The keys of the boundary bin all lie in 64-key tiles that one wave of the selection
    takes (tiles 8 apart), tied at the top score, so one wave feeds every query's list and the
    last tie taken decides t_cut. Thresholds bit-exact, outputs within the bar."""
    w = W(batch=1, num_q_heads=8, num_kv_heads=2, seq_len=2048, q_len=64, top_k=top_k)
    _banner(f"thresholds, boundary keys in tiles {tiles}, K={top_k}")
    inp = make_inputs(w, seed=44, device="cpu", idx_values=(-1, 0))
    inp.q_idx.fill_(1)
    table = inp.page_table
    for t in tiles:  # 64-token pages: tile t is page t
        inp.kidx_pool[table[0, t]] = 1
    inp = inp.to(DEV)
    gpu = run_gpu(inp, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


@pytest.mark.parametrize("seq_len,q_len", [(70000, 40), (65600, 100)])
def test_thresholds_rows_over_65535_candidates(seq_len, q_len):
    """Rows of more than 65535 candidates through the threshold pass (counts past 16 bits);
    the second case's block straddles that count. Thresholds bit-exact and outputs within the
    bar."""
    w = W(batch=1, num_q_heads=8, num_kv_heads=2, seq_len=seq_len, q_len=q_len, top_k=700, prefix_len=5)
    _banner(f"thresholds, rows of {seq_len} tokens")
    inp = make_inputs(w, seed=45, device="cpu").to(DEV)
    gpu = run_gpu(inp, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


def _random_case(seed):
    """A small random workload and its input options, drawn from `seed`: batch 1-3, 1-2 KV
    heads, group 1/2/4/8, d 64/128, d_idx 32/64/128, pages of 64-256 tokens, ragged lengths,
    a forced prefix, a shared indexer head or tied indexer values now and then."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 4))
    hkv = int(rng.integers(1, 3))
    group = int(rng.choice([1, 2, 4, 8]))
    decode = rng.random() < 0.3
    q_len = 1 if decode else int(rng.integers(1, 300))
    t_max = int(rng.integers(max(q_len, 2), 1500))
    lens = [int(rng.integers(q_len, t_max + 1)) for _ in range(B)]
    lens[int(rng.integers(0, B))] = t_max
    dense = (not decode) and rng.random() < 0.15
    w = W(batch=B, num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=int(rng.choice([64, 128])),
          seq_len=t_max, q_len=q_len, idx_dim=0 if dense else int(rng.choice([32, 64, 128])),
          top_k=0 if dense else int(rng.integers(1, 600)),
          prefix_len=0 if dense or rng.random() < 0.5 else int(rng.integers(1, 11)),
          page_size=int(rng.choice([64, 128, 256])))
    kw = dict(seq_lens=lens, spare_pages=int(rng.integers(0, 4)))
    if not dense and rng.random() < 0.3:
        kw["num_idx_heads"] = 1
    if not dense and rng.random() < 0.25:
        kw["idx_values"] = (-1, 0, 1)
    return w, kw


@pytest.mark.parametrize("seed", range(48))
def test_random_small_configs_every_row(seed):
    """Random small workloads (see _random_case) through every path that applies, each against
    the oracle on every row: decode (two-step and fused selection), or prefill with the two-step
    lists on gathered rows and on masked tiles, and the fused prefill (automatic and masked
    paths, with its thresholds), or dense prefill."""
    w, kw = _random_case(seed)
    _banner(f"random case {seed}: {w} {kw}")
    inp = make_inputs(w, seed=500 + seed, device="cpu", **kw).to(DEV)
    ov = OracleView(inp)
    rows = all_rows(inp)
    runs = []
    if w.dense:
        runs.append(run_gpu(inp))
    elif w.q_len == 1:
        runs += [run_gpu(inp), run_gpu(inp, fused=True)]
    else:
        chunk = [None, 64, 96][seed % 3]
        runs += [run_gpu(inp, q_chunk=chunk), run_gpu(inp, q_chunk=chunk, masked=True),
                 run_gpu(inp, q_chunk=chunk, prefill_path=fa.SA_PREFILL_AUTO, thresholds=True),
                 run_gpu(inp, q_chunk=chunk, prefill_path=fa.SA_PREFILL_MASKED)]
    torch.cuda.synchronize()
    for r in runs:
        assert_close(compare_rows(r, ov, rows))


@pytest.mark.parametrize("top_k", [1, 2])
@pytest.mark.parametrize("tied", [False, True])
def test_degenerate_top_k_every_path(top_k, tied):
    """Top-1 and top-2 (with every indexer score tied, the lowest candidate tokens win):
    prefill blocks through the two-step and fused list selections on gathered rows and masked
    tiles and through the fused prefill (thresholds, masked and automatic paths), and long
    decode rows through the two-step and fused selections; every row against the oracle."""
    kw = dict(idx_values=(0,)) if tied else {}
    _banner(f"top_k={top_k} tied={tied}")
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=300, q_len=200, top_k=top_k, prefix_len=2)
    inp = make_inputs(w, seed=46, device="cpu", seq_lens=[300, 260], **kw).to(DEV)
    ov = OracleView(inp)
    rows = all_rows(inp)
    runs = [run_gpu(inp, q_chunk=64), run_gpu(inp, q_chunk=64, fused=True),
            run_gpu(inp, q_chunk=64, masked=True),
            run_gpu(inp, q_chunk=64, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True),
            run_gpu(inp, q_chunk=64, prefill_path=fa.SA_PREFILL_AUTO)]
    torch.cuda.synchronize()
    for r in runs:
        assert_close(compare_rows(r, ov, rows))
    wd = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=20000, q_len=1, top_k=top_k, prefix_len=0)
    inp = make_inputs(wd, seed=47, device="cpu", seq_lens=[20000, 17000], **kw).to(DEV)
    ov = OracleView(inp, host_copy=False)
    runs = [run_gpu(inp), run_gpu(inp, fused=True)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0].indices, runs[1].indices)
    for r in runs:
        assert_close(compare_rows(r, ov, all_rows(inp)))


def test_fused_prefill_middle_blocks_ragged():
    """Blocks of 160 queries in the middle of sequences of different lengths, with a prefix and
    spare pages: every block through the masked path and the gathered path, every row."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=900, q_len=800, top_k=96, prefix_len=9)
    _banner("fused prefill, middle blocks")
    inp = make_inputs(w, seed=42, device="cpu", seq_lens=[900, 820], spare_pages=4).to(DEV)
    ov = OracleView(inp)
    for path in (fa.SA_PREFILL_MASKED, fa.SA_PREFILL_GATHER):
        gpu = run_gpu(inp, q_chunk=160, prefill_path=path, thresholds=True)
        torch.cuda.synchronize()
        assert_close(compare_rows(gpu, ov, all_rows(inp)))


SPLIT_CASES = {
    # one 128-query block at the end: 16 workgroups, 64 key tiles -> 8 key splits of 8 tiles;
    # the shorter sequence leaves its last two splits empty
    "g4_d128_ragged": (W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=4096, q_len=128, top_k=256,
                         prefix_len=4), dict(seq_lens=[4096, 3000], spare_pages=4), None),
    # group size 1, head_dim 64: 2 workgroups, 47 tiles -> 5 splits of 10 (the last one 7)
    "g1_d64": (W(num_q_heads=2, num_kv_heads=2, head_dim=64, idx_dim=32, seq_len=3000, q_len=100,
                 top_k=200), {}, None),
    # group size 8, 96-query blocks at four positions (the last block 12 queries)
    "g8_blocks": (W(num_q_heads=16, num_kv_heads=2, seq_len=2500, q_len=300, top_k=400, prefix_len=3),
                  {}, 96),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_fused_masked_key_splits_every_row(name):
    """Short blocks on the masked path split their causal key tiles among several workgroups
    (too few query blocks to fill the CUs) and merge the split results: every row within the
    bar, thresholds bit-exact."""
    w, kw, chunk = SPLIT_CASES[name]
    _banner(f"fused masked prefill with key splits {name}: {w}")
    inp = make_inputs(w, seed=43, device="cpu", **kw).to(DEV)
    gpu = run_gpu(inp, q_chunk=chunk, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert_close(compare_rows(gpu, OracleView(inp), all_rows(inp)))


def test_fused_masked_missing_pages_every_row():
    """Pages missing from the table (entry -1) on the masked path: their keys are not
    candidates of the selection and take no part in the attention, forced prefix keys
    included. The expected values come from the oracle's selection and attention over the
    keys whose pages are present: thresholds bit-exact and every row within the bar, for a
    block that splits its key tiles (16 workgroups, 64 tiles)."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=4096, q_len=128, top_k=256, prefix_len=4)
    _banner("fused masked prefill, missing pages")
    inp = make_inputs(w, seed=44, device="cpu", seq_lens=[4096, 3000], spare_pages=4)
    inp.page_table[0, 0] = -1    # tokens 0..63 of sequence 0, the forced prefix among them
    inp.page_table[0, 17] = -1
    inp.page_table[1, 40] = -1
    inp.page_table[1, 46] = -1   # the last page of sequence 1, holding the block's last queries
    inp = inp.to(DEV)
    gpu = run_gpu(inp, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    G, scale, ps = w.group, 1.0 / math.sqrt(w.head_dim), w.page_size
    q_idx = inp.q_idx.cpu().numpy()
    errs, lerrs = [], []
    for b in range(w.batch):
        T = inp.seq_lens_host[b]
        table = np.asarray(ov.table[b])
        t_all = np.arange(T, dtype=np.int64)
        present = table[t_all // ps] >= 0
        for i in range(w.q_len):
            pos = oracle.query_position(T, w.q_len, i)
            c = oracle.candidate_keys(pos, w.prefix_len)
            c = c[present[c]]
            f = oracle.forced_keys(pos, w.prefix_len)
            f = f[present[f]]
            for g in range(w.num_kv_heads):
                sc = oracle.index_scores(q_idx[b, i, g], oracle.page_rows(ov.kidx, table, ps, g, c))
                want = oracle.selection_thresholds(sc, c, w.top_k)
                got = tuple(int(x) for x in gpu.thresholds[b, i, g].cpu())
                assert got == want, (b, i, g, got, want)
                keys = np.sort(np.concatenate([f, oracle.topk_select(sc, c, w.top_k)]))
                sl = slice(g * G, (g + 1) * G)
                qb = oracle.bf16_to_f64(bits(inp.q[b, i, sl]))
                kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, table, ps, g, keys))
                vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, table, ps, g, keys))
                o_ref, l_ref = oracle.attend(qb, kr, vr, scale)
                errs.append(np.abs(f64(gpu.out[b, i, sl]) - o_ref).ravel())
                lerrs.append(np.abs(gpu.lse[b, i, sl].double().cpu().numpy() - l_ref))
    e = np.concatenate(errs)
    assert_close((float(e.max()), float(e.mean()), float(np.concatenate(lerrs).max())))


def test_fused_decode_missing_pages():
    """Pages missing from the table in the fused decode selection: keys on them are not
    candidates (the forced prefix is listed whatever its page) and the decode attention leaves
    every key on a missing page out. Lists bit-exact against the oracle's selection over the
    candidates whose pages are present; outputs against the oracle's attention over the listed
    keys with present pages."""
    w = W(batch=3, num_q_heads=8, num_kv_heads=2, seq_len=40000, q_len=1, top_k=500, prefix_len=3)
    _banner("fused decode selection, missing pages")
    inp = make_inputs(w, seed=45, device="cpu", seq_lens=[40000, 33000, 20000], spare_pages=8)
    inp.page_table[0, 0] = -1      # the forced prefix's page
    inp.page_table[0, 130] = -1    # a page inside the second 8192-token chunk
    inp.page_table[1, 515] = -1    # the page holding the query of sequence 1 (tokens 32960..33023)
    for p in range(200, 260):      # most of a chunk of sequence 2
        inp.page_table[2, p] = -1
    inp = inp.to(DEV)
    gpu = run_gpu(inp, fused=True)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    G, scale, ps = w.group, 1.0 / math.sqrt(w.head_dim), w.page_size
    q_idx = inp.q_idx.cpu().numpy()
    errs, lerrs = [], []
    for b in range(w.batch):
        T = inp.seq_lens_host[b]
        table = np.asarray(ov.table[b])
        present = table[np.arange(T, dtype=np.int64) // ps] >= 0
        pos = oracle.query_position(T, 1, 0)
        c = oracle.candidate_keys(pos, w.prefix_len)
        c = c[present[c]]
        f = oracle.forced_keys(pos, w.prefix_len)
        for g in range(w.num_kv_heads):
            sc = oracle.index_scores(q_idx[b, 0, g], oracle.page_rows(ov.kidx, table, ps, g, c))
            keys = np.sort(np.concatenate([f, oracle.topk_select(sc, c, w.top_k)]))
            want = np.full(w.index_width, -1, dtype=np.int64)
            want[:keys.size] = keys
            got = gpu.indices[b, 0, g].cpu().numpy()
            assert np.array_equal(got, want), (b, g, got[:16], want[:16])
            keys = keys[present[keys]]
            sl = slice(g * G, (g + 1) * G)
            qb = oracle.bf16_to_f64(bits(inp.q[b, 0, sl]))
            kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, table, ps, g, keys))
            vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, table, ps, g, keys))
            o_ref, l_ref = oracle.attend(qb, kr, vr, scale)
            errs.append(np.abs(f64(gpu.out[b, 0, sl]) - o_ref).ravel())
            lerrs.append(np.abs(gpu.lse[b, 0, sl].double().cpu().numpy() - l_ref))
    e = np.concatenate(errs)
    assert_close((float(e.max()), float(e.mean()), float(np.concatenate(lerrs).max()),
                  LSE_ABS_FP32_SUM))


# ------------------------------------------------------------------ int8 minimum, missing pages

def _saturate(inp, rng, q_frac, key_frac):
    """Writes -128 into every entry of a fraction of the indexer queries and keys: such a
    query scores such a key at d_idx * 2^14, the largest score int8 values can make (the
    value at which the 16-bit prefill keys saturate at 65535). A few keys get one entry -127
    (one step below) and a few all +127 (the most negative scores)."""
    q, k = inp.q_idx, inp.kidx_pool
    nq = q.shape[0] * q.shape[1] * q.shape[2]
    qf = q.view(nq, -1)
    qf[torch.from_numpy(rng.random(nq) < q_frac)] = -128
    nk = k.shape[0] * k.shape[1] * k.shape[2]
    kf = k.view(nk, -1)
    r = rng.random(nk)
    kf[torch.from_numpy(r < key_frac)] = -128
    near = torch.from_numpy((r >= key_frac) & (r < key_frac * 1.5))
    kf[near] = -128
    kf[near, 0] = -127
    kf[torch.from_numpy((r >= key_frac * 1.5) & (r < key_frac * 1.8))] = 127


@pytest.mark.parametrize("d_idx", [32, 64, 128])
def test_int8_minimum_ties_at_largest_score(d_idx):
    """Queries and keys of all -128 reach the largest score (d_idx * 2^14) on more keys than K
    takes, so the lower-index rule decides among them. The two-step path, the fused 16-bit
    prefill selection and the fused decode selection all give the oracle's lists bit for bit;
    attention through both prefill kernels and the decode within the bar."""
    rng = np.random.default_rng(d_idx)
    # prefill block (q_len >= 16, rows <= 32K: the 16-bit key path)
    w = W(batch=1, num_q_heads=8, num_kv_heads=2, seq_len=1100, q_len=300, idx_dim=d_idx, top_k=48,
          prefix_len=2)
    _banner(f"int8 minimum, prefill, d_idx={d_idx}")
    inp = make_inputs(w, seed=31, device="cpu")
    _saturate(inp, rng, q_frac=0.5, key_frac=0.15)
    inp = inp.to(DEV)
    two = run_gpu(inp)
    fused = run_gpu(inp, fused=True, masked=True)
    thr = run_gpu(inp, prefill_path=fa.SA_PREFILL_MASKED, thresholds=True)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    ov = OracleView(inp)
    assert_close(compare_rows(two, ov, all_rows(inp)))
    assert_close(compare_rows(fused, ov, all_rows(inp)))
    assert_close(compare_rows(thr, ov, all_rows(inp)))
    # decode rows of >= 16384 candidates (the fused decode path), ties at the top spread over
    # every chunk
    wd = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=20000, q_len=1, idx_dim=d_idx, top_k=256)
    _banner(f"int8 minimum, decode, d_idx={d_idx}")
    inp = make_inputs(wd, seed=32, device="cpu")
    _saturate(inp, rng, q_frac=0.75, key_frac=0.03)
    inp = inp.to(DEV)
    two = run_gpu(inp)
    fused = run_gpu(inp, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fused.indices, two.indices)
    assert_close(compare_rows(fused, OracleView(inp), all_rows(inp)))


def test_missing_page_keys_are_left_out():
    """A page missing from the table (entry -1): its keys take no part in the softmax of the
    dense kernel, the masked-dense kernel and the gathered kernel alike (lists of every
    causal key), matching the oracle over the present keys."""
    w = W(batch=2, num_q_heads=8, num_kv_heads=2, seq_len=330, q_len=300, idx_dim=64, top_k=330)
    _banner("missing page: dense, masked and gathered prefill")
    inp = make_inputs(w, seed=33, device="cpu", seq_lens=[330, 300], spare_pages=1)
    inp.page_table[0, 2] = -1       # tokens 128..191 of sequence 0
    inp.page_table[1, 0] = -1       # tokens 0..63 of sequence 1: its first queries see nothing
    inp = inp.to(DEV)
    kv = make_kv(inp)
    S, H, width = w.q_len, w.num_kv_heads, 330
    lists = torch.full((w.batch, S, H, width), -1, dtype=torch.int32)
    for b in range(w.batch):
        for i in range(S):
            pos = oracle.query_position(inp.seq_lens_host[b], S, i)
            if pos >= 0:
                lists[b, i, :, :pos + 1] = torch.arange(pos + 1, dtype=torch.int32)
    lists = lists.to(DEV)
    out_d, lse_d = fa.prefill(kv, inp.q, q_tail=S)
    out_m, lse_m = fa.prefill_masked(kv, inp.q, q_tail=S, indices=lists)
    out_g, lse_g = fa.prefill(kv, inp.q, q_tail=S, indices=lists)
    torch.cuda.synchronize()
    ov = OracleView(inp)
    G, scale = w.group, 1.0 / math.sqrt(w.head_dim)
    errs, lerrs = [], []
    for b in range(w.batch):
        T = inp.seq_lens_host[b]
        for i in range(S):
            pos = oracle.query_position(T, S, i)
            keys = np.array([t for t in range(pos + 1) if ov.table[b][t // w.page_size] >= 0])
            for g in range(H):
                sl = slice(g * G, (g + 1) * G)
                outs = [(out_d, lse_d), (out_m, lse_m), (out_g, lse_g)]
                if keys.size == 0:      # nothing to attend: out 0, lse -inf (all three kernels)
                    for o, l in outs:
                        assert torch.all(o[b, i, sl] == 0) and torch.all(torch.isneginf(l[b, i, sl]))
                    continue
                qb = oracle.bf16_to_f64(bits(inp.q[b, i, sl]))
                kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, ov.table[b], w.page_size, g, keys))
                vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, ov.table[b], w.page_size, g, keys))
                o_ref, l_ref = oracle.attend(qb, kr, vr, scale)
                for o, l in outs:
                    errs.append(np.abs(f64(o[b, i, sl]) - o_ref).ravel())
                    lerrs.append(np.abs(l[b, i, sl].double().cpu().numpy() - l_ref))
    e = np.concatenate(errs)
    assert_close((float(e.max()), float(e.mean()), float(np.concatenate(lerrs).max())))


# ------------------------------------------------------------------ full-size workloads

# Oracle results of the full-size prefill blocks, shared by the tests that run the same seeded
# inputs through different GPU paths (the inputs are a pure function of workload and seed).
_ORACLE_CACHE = {}


def _check_full_prefill(name, seed, gpu, inp, rows_of_b):
    """Every KV group of the sampled rows of every sequence against the oracle (index lists
    bit-exact, outputs within the bar); returns the number of (row, group) pairs checked."""
    w = inp.workload
    ov = OracleView(inp, host_copy=True)
    stats, n = [], 0
    for b in range(w.batch):
        rows = rows_of_b(b)
        for g in range(w.num_kv_heads):
            key = (name, seed, b, g)
            mx, mean, le, want = compare_block(gpu, ov, b, rows, g, _ORACLE_CACHE.get(key))
            _ORACLE_CACHE[key] = want
            stats.append((mx, mean, le))
            n += len(rows)
    assert_close(merge_stats(stats))
    return n


def test_full_dense_prefill_8k():
    """Dense causal 8K, B=4: per sequence the first and last 64 queries and 256 seeded others
    (1024 random rows in all), every KV group (all 32 query heads)."""
    w = CONFIGS["dense_prefill_8k"]
    _banner(f"full {w.name}")
    inp = make_inputs(w, seed=2, device=DEV)
    gpu = run_gpu(inp)
    torch.cuda.synchronize()
    n = _check_full_prefill(w.name, 2, gpu, inp,
                            lambda b: sampled_positions(w.q_len, 256, edge=64, seed=20 + b))
    assert n == 4 * 384 * 8


def test_full_sparse_decode_128k():
    w = CONFIGS["sparse_decode_128k"]
    _banner(f"full {w.name}")
    inp = make_inputs(w, seed=3, device=DEV)
    gpu = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(gpu.indices, two.indices)
    ov = OracleView(inp, host_copy=False)
    assert_close(compare_rows(gpu, ov, all_rows(inp)))


_ROWS_32K = None


def _rows_32k():
    global _ROWS_32K
    if _ROWS_32K is None:
        _ROWS_32K = sampled_positions(CONFIGS["sparse_prefill_32k"].q_len, 1024, edge=64, seed=40)
    return _ROWS_32K


def test_full_sparse_prefill_32k():
    """Two-step selection and gathered-row attention over the 32K prefill in 2048-query
    blocks: the first and last 64 queries and 1024 seeded others, all 8 KV groups, lists
    bit-exact and outputs within the bar."""
    w = CONFIGS["sparse_prefill_32k"]
    _banner(f"full {w.name}")
    inp = make_inputs(w, seed=4, device=DEV)
    gpu = run_gpu(inp, q_chunk=2048)
    torch.cuda.synchronize()
    n = _check_full_prefill(w.name, 4, gpu, inp, lambda b: _rows_32k())
    assert n == 1152 * 8


def test_full_sparse_prefill_32k_masked():
    """The 32K sparse prefill as the benchmark runs it: fused selection (16-bit keys) and the
    attention on masked dense tiles, in 2048-query blocks; lists equal the two-step path's on
    every row, and the sampled rows (as above) match the oracle."""
    w = CONFIGS["sparse_prefill_32k"]
    _banner(f"full {w.name}, fused selection, masked dense tiles")
    inp = make_inputs(w, seed=4, device=DEV)
    gpu = run_gpu(inp, q_chunk=2048, masked=True, fused=True)
    two = run_gpu(inp, q_chunk=2048)
    torch.cuda.synchronize()
    assert torch.equal(gpu.indices, two.indices)
    del two
    torch.cuda.synchronize()
    n = _check_full_prefill(w.name, 4, gpu, inp, lambda b: _rows_32k())
    assert n == 1152 * 8


def test_full_sparse_prefill_32k_fused():
    """The 32K sparse prefill through sparse_attn_prefill_fused (AUTO: every 2048-query block
    takes the masked path, no lists), with the thresholds of every block: sampled rows as above,
    (tau, t_cut) bit-exact and outputs within the bar."""
    w = CONFIGS["sparse_prefill_32k"]
    _banner(f"full {w.name}, fused prefill (thresholds, masks from recomputed scores)")
    inp = make_inputs(w, seed=4, device=DEV)
    kv = make_kv(inp)
    for q0 in range(0, w.q_len, 2048):
        assert fa.sparse_attn_prefill_fused_choice(kv, w.num_q_heads, 2048, w.q_len - q0,
                                                   w.top_k) == fa.SA_PREFILL_MASKED
    gpu = run_gpu(inp, q_chunk=2048, prefill_path=fa.SA_PREFILL_AUTO, thresholds=True)
    torch.cuda.synchronize()
    n = _check_full_prefill(w.name, 4, gpu, inp, lambda b: _rows_32k())
    assert n == 1152 * 8


def test_full_sparse_decode_1m_prefix():
    w = CONFIGS["sparse_decode_1m_prefix"]
    _banner(f"full {w.name}")
    inp = make_inputs(w, seed=5, device=DEV)
    gpu = run_gpu(inp, fused=True)
    two = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.equal(gpu.indices, two.indices)
    ov = OracleView(inp, host_copy=False)
    assert_close(compare_rows(gpu, ov, all_rows(inp)))   # all 32 (sequence, group) rows
    # every list starts with the forced prefix 0..195
    idx = gpu.indices[:, 0].cpu().numpy()
    assert np.all(idx[..., :196] == np.arange(196))


def test_full_sparse_decode_128k_window():
    """The 128K decode step with hybrid lists as the benchmark runs it (the last 512 keys forced
    beside the top-2048; fused selection at window-shortened positions, then split-K decode):
    sampled rows' lists bit-exact against the oracle, their attention within the bar."""
    w = CONFIGS["sparse_decode_128k"]
    win = 512
    _banner(f"full {w.name}, hybrid lists window={win}")
    inp = make_inputs(w, seed=3, device=DEV)
    kv = make_kv(inp)
    width = w.prefix_len + w.top_k + win
    lists = fa.index_topk_window(kv, inp.q_idx, 1, 1, w.top_k, win)
    o, lse = fa.decode(kv, inp.q[:, 0].contiguous(), lists[:, 0].contiguous())
    torch.cuda.synchronize()
    ov = OracleView(inp, host_copy=False)
    got = lists.cpu().numpy()
    G, scale = w.group, 1.0 / math.sqrt(w.head_dim)
    errs, lerrs = [], []
    for b in range(w.batch):
        for g in ((b % 8), (b + 5) % 8):
            pos = oracle.query_position(inp.seq_lens_host[b], 1, 0)
            qi = inp.q_idx[b, 0, g].cpu().numpy()
            fn = lambda t: oracle.index_scores(qi, oracle.page_rows(ov.kidx, ov.table[b], w.page_size, g, t))
            want = oracle.hybrid_index_list(pos, w.prefix_len, win, w.top_k, width, fn)
            assert np.array_equal(got[b, 0, g], want), (b, g)
            keys = want[want >= 0]
            assert keys.size == w.top_k + win and keys[-1] == pos
            kr = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, ov.table[b], w.page_size, g, keys))
            vr = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, ov.table[b], w.page_size, g, keys))
            qb = oracle.bf16_to_f64(bits(inp.q[b, 0, g * G:(g + 1) * G]))
            o_ref, l_ref = oracle.attend(qb, kr, vr, scale)
            errs.append(np.abs(f64(o[b, g * G:(g + 1) * G]) - o_ref).ravel())
            lerrs.append(np.abs(lse[b, g * G:(g + 1) * G].double().cpu().numpy() - l_ref))
    e = np.concatenate(errs)
    assert_close((float(e.max()), float(e.mean()), float(np.concatenate(lerrs).max())))
