"""Test plumbing: run the HIP path through the binding, and feed the same inputs to the oracle.

The oracle reads device pools through DevicePool, which fancy-indexes the torch tensor drawn
by the `synthetic` generator and copies the requested rows to host memory. No oracle input
comes from the HIP library.
"""
import math
from typing import Optional

import numpy as np
import torch

import flash_attention_int8_amd as fa
import oracle
from synthetic import Inputs

MAX_ABS = 2e-2     # bf16 output vs fp64 oracle, max over elements
MEAN_ABS = 2e-3    # ... mean over elements
# fp32 log-sum-exp vs fp64. The kernels round each P to bf16 before P.V and add those rounded
# values into the row sum (so O is an exact convex combination of the weights P.V saw); a
# rounded P is off by at most 2^-8 of itself, so the sum, and exp(LSE), by at most 2^-8:
# |LSE error| <= ln(1 + 2^-8) = 3.9e-3, reached when one key dominates a short list.
LSE_ABS = 4e-3
# The decode and gathered-row prefill attention add the fp32 P (before its bf16 rounding) into
# the row sum, so their LSE carries only fp32 rounding; the bound there is the planned 1e-3.
LSE_ABS_FP32_SUM = 1e-3


class DevicePool:
    """pool[phys, head, slot] -> numpy rows (bf16 bits as uint16, int8 as int8)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, key):
        phys, head, slot = key
        dev = self.t.device
        p = torch.as_tensor(np.asarray(phys), device=dev, dtype=torch.long)
        s = torch.as_tensor(np.asarray(slot), device=dev, dtype=torch.long)
        rows = self.t[p, int(head), s]
        if rows.dtype == torch.bfloat16:
            return rows.view(torch.int16).cpu().numpy().view(np.uint16)
        return rows.cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_kv(inp: Inputs) -> fa.PagedKV:
    w = inp.workload
    return fa.PagedKV(k_pool=inp.k_pool, v_pool=inp.v_pool, kidx_pool=inp.kidx_pool,
                      page_table=inp.page_table, seq_lens=inp.seq_lens,
                      max_seq_len=max(inp.seq_lens_host), prefix_len=w.prefix_len,
                      num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                      idx_dim=w.idx_dim if not w.dense else 0, num_idx_heads=inp.num_idx_heads,
                      page_size=w.page_size, num_pages=inp.num_pages)


class GpuRun:
    def __init__(self):
        self.scores = []       # list of (q0, scores chunk)
        self.indices = None
        self.thresholds = None
        self.out = None
        self.lse = None
        self.lse_fp32_sum = False  # the row sum of this run's attention adds fp32 P


def run_gpu(inp: Inputs, *, num_splits: int = 0, q_chunk: Optional[int] = None,
            keep_scores: bool = False, fused: bool = False, masked: bool = False,
            prefill_path: Optional[int] = None, thresholds: bool = False) -> GpuRun:
    """The whole path on the device: index -> top-K -> attention (or dense attention).
    fused=True selects with sparse_attn_index_topk instead of index then topk; masked=True
    runs the prefill attention on masked dense tiles (sparse_attn_fwd_prefill_masked);
    prefill_path runs each prefill block through sparse_attn_prefill_fused on that path (no
    lists come back); thresholds=True also keeps sparse_attn_select_thresholds' (tau, t_cut)."""
    w = inp.workload
    kv = make_kv(inp)
    r = GpuRun()
    B, S = w.batch, w.q_len
    if w.dense:
        r.out, r.lse = fa.prefill(kv, inp.q, q_tail=S)
        return r
    if S == 1:
        if fused:
            idx = fa.index_topk(kv, inp.q_idx, 1, 1, w.top_k)
        else:
            scores = fa.index(kv, inp.q_idx, 1, 1)
            idx = fa.topk(kv, scores, 1, 1, w.top_k)
            if keep_scores:
                r.scores.append((0, scores))
        r.indices = idx
        r.out, r.lse = fa.decode(kv, inp.q[:, 0].contiguous(), idx[:, 0].contiguous(),
                                 num_splits=num_splits)
        r.lse_fp32_sum = True
        r.out = r.out.unsqueeze(1)
        r.lse = r.lse.unsqueeze(1)
        return r
    q_chunk = q_chunk or S
    T = max(inp.seq_lens_host)
    if prefill_path is None:
        r.indices = torch.empty((B, S, inp.num_idx_heads, w.index_width), dtype=torch.int32,
                                device=inp.q.device)
    if thresholds:
        r.thresholds = torch.empty((B, S, inp.num_idx_heads, 2), dtype=torch.int32, device=inp.q.device)
    r.out = torch.empty_like(inp.q)
    r.lse = torch.empty((B, S, w.num_q_heads), dtype=torch.float32, device=inp.q.device)
    for q0 in range(0, S, q_chunk):
        c = min(q_chunk, S - q0)
        tail = S - q0
        qi = inp.q_idx[:, q0:q0 + c].contiguous()
        if thresholds:
            r.thresholds[:, q0:q0 + c] = fa.select_thresholds(kv, qi, c, tail, w.top_k)
        if prefill_path is not None:
            qc = inp.q[:, q0:q0 + c].contiguous()
            out, lse = fa.prefill_fused(kv, qc, qi, tail, w.top_k, path=prefill_path)
            r.out[:, q0:q0 + c] = out
            r.lse[:, q0:q0 + c] = lse
            continue
        if fused:
            idx = fa.index_topk(kv, qi, c, tail, w.top_k)
        else:
            scores = fa.index(kv, qi, c, tail)
            idx = fa.topk(kv, scores, c, tail, w.top_k)
            if keep_scores:
                r.scores.append((q0, scores))
        qc = inp.q[:, q0:q0 + c].contiguous()
        if masked:
            out, lse = fa.prefill_masked(kv, qc, q_tail=tail, indices=idx)
        else:
            out, lse = fa.prefill(kv, qc, q_tail=tail, indices=idx)
        r.indices[:, q0:q0 + c] = idx
        r.out[:, q0:q0 + c] = out
        r.lse[:, q0:q0 + c] = lse
    # the gathered-row kernel's row sum adds fp32 P; the masked-tile kernel's adds the rounded P
    r.lse_fp32_sum = (prefill_path is None and not masked) or prefill_path == fa.SA_PREFILL_GATHER
    del T
    return r


class OracleView:
    """Host-side views of one workload's inputs for the oracle."""

    def __init__(self, inp: Inputs, host_copy: bool = True):
        self.inp = inp
        self.w = inp.workload
        if host_copy:
            self.k_pool = bits(inp.k_pool)
            self.v_pool = bits(inp.v_pool)
            self.kidx = None if inp.kidx_pool is None else inp.kidx_pool.cpu().numpy()
        else:
            self.k_pool = DevicePool(inp.k_pool)
            self.v_pool = DevicePool(inp.v_pool)
            self.kidx = None if inp.kidx_pool is None else DevicePool(inp.kidx_pool)
        self.table = inp.page_table.cpu().numpy()
        self._q = inp.q
        self._q_idx = inp.q_idx

    def query(self, b: int, i: int, g: int):
        """(index list or None, O [G][d], LSE [G]) of query token i of sequence b, KV group g."""
        w = self.w
        heads = list(oracle.group_query_heads(g, w.num_q_heads, w.num_kv_heads))
        qb = bits(self._q[b, i, heads[0]:heads[-1] + 1])
        pos = oracle.query_position(self.inp.seq_lens_host[b], w.q_len, i)
        scale = 1.0 / math.sqrt(w.head_dim)
        if w.dense:
            o, lse = oracle.dense_query(q_bits=qb, k_pool=self.k_pool, v_pool=self.v_pool,
                                        page_table_row=self.table[b], page_size=w.page_size,
                                        kv_head=g, pos=pos, sm_scale=scale)
            return None, o, lse
        gi = 0 if self.inp.num_idx_heads == 1 else g
        qi = self._q_idx[b, i, gi].cpu().numpy()
        return oracle.dsa_query(q_bits=qb, q_idx_vec=qi, kidx_pool=self.kidx, k_pool=self.k_pool,
                                v_pool=self.v_pool, page_table_row=self.table[b],
                                page_size=w.page_size, kv_head=g, idx_head=gi, pos=pos,
                                prefix_len=w.prefix_len, top_k=w.top_k, sm_scale=scale)

    def thresholds(self, b: int, i: int, gi: int):
        """Oracle (tau, t_cut) of the selection of (b, i, gi)."""
        c, sc = self.scores_row(b, i, gi)
        return oracle.selection_thresholds(sc, c, self.w.top_k)

    def scores_row(self, b: int, i: int, gi: int) -> np.ndarray:
        """Oracle indexer scores of every candidate key of (b, i, gi), with their tokens."""
        w = self.w
        pos = oracle.query_position(self.inp.seq_lens_host[b], w.q_len, i)
        c = oracle.candidate_keys(pos, w.prefix_len)
        k = oracle.page_rows(self.kidx, self.table[b], w.page_size, gi, c)
        return c, oracle.index_scores(self._q_idx[b, i, gi].cpu().numpy(), k)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def compare_rows(gpu: GpuRun, ov: OracleView, rows, check_lse: bool = True):
    """Checks the given (b, i, g) rows; returns (max_abs, mean_abs, max_lse, lse_bound) over
    them, lse_bound being the LSE bar of the run's attention path."""
    w = ov.w
    G = w.group
    errs, lse_errs = [], []
    for (b, i, g) in rows:
        idx, o, lse = ov.query(b, i, g)
        if idx is not None and getattr(gpu, "indices", None) is not None:
            gi = 0 if ov.inp.num_idx_heads == 1 else g
            got = gpu.indices[b, i, gi].cpu().numpy()
            assert np.array_equal(got, idx), (b, i, g, got[:16], idx[:16])
        if idx is not None and getattr(gpu, "thresholds", None) is not None:
            gi = 0 if ov.inp.num_idx_heads == 1 else g
            want = ov.thresholds(b, i, gi)
            got = tuple(int(x) for x in gpu.thresholds[b, i, gi].cpu())
            assert got == want, (b, i, g, got, want)
        og = f64(gpu.out[b, i, g * G:(g + 1) * G])
        errs.append(np.abs(og - o).ravel())
        if check_lse and gpu.lse is not None:
            lg = gpu.lse[b, i, g * G:(g + 1) * G].double().cpu().numpy()
            lse_errs.append(np.abs(lg - lse))
    e = np.concatenate(errs)
    le = float(np.concatenate(lse_errs).max()) if lse_errs else 0.0
    bound = LSE_ABS_FP32_SUM if getattr(gpu, "lse_fp32_sum", False) else LSE_ABS
    return float(e.max()), float(e.mean()), le, bound


def assert_close(stats):
    """stats = (max_abs, mean_abs, max_lse[, lse_bound]); the bound defaults to LSE_ABS."""
    mx, mean, lse = stats[:3]
    bound = stats[3] if len(stats) > 3 else LSE_ABS
    assert mx <= MAX_ABS, f"max abs error {mx}"
    assert mean <= MEAN_ABS, f"mean abs error {mean}"
    assert lse <= bound, f"lse error {lse} (bound {bound})"


def sampled_positions(S: int, n_random: int, edge: int = 64, seed: int = 0) -> list:
    """The first and last `edge` query rows of a block of S plus `n_random` seeded others."""
    ends = set(range(min(S, edge))) | set(range(max(0, S - edge), S))
    mid = np.array([i for i in range(S) if i not in ends], dtype=np.int64)
    rng = np.random.default_rng(seed)
    pick = rng.choice(mid.size, size=min(n_random, mid.size), replace=False) if mid.size else []
    return sorted(ends | set(int(mid[j]) for j in pick))


def oracle_block(ov: OracleView, b: int, rows, g: int):
    """Oracle results of query tokens `rows` of sequence b, KV group g, from host copies of
    the pools: (index lists [n][P+K] or None for dense, O [n][G][d], LSE [n][G]). Scores of
    all rows come from one exact float64 product (oracle.index_scores_many), dense rows from
    oracle.attend_causal_many."""
    w, inp = ov.w, ov.inp
    T = inp.seq_lens_host[b]
    G = w.group
    rows = [int(i) for i in rows]
    pos = np.array([oracle.query_position(T, w.q_len, i) for i in rows], dtype=np.int64)
    t = np.arange(T, dtype=np.int64)
    scale = 1.0 / math.sqrt(w.head_dim)
    sel = torch.as_tensor(rows, device=inp.q.device, dtype=torch.long)
    qd = oracle.bf16_to_f64(bits(inp.q[b].index_select(0, sel)[:, g * G:(g + 1) * G]))
    kd = oracle.bf16_to_f64(oracle.page_rows(ov.k_pool, ov.table[b], w.page_size, g, t))
    vd = oracle.bf16_to_f64(oracle.page_rows(ov.v_pool, ov.table[b], w.page_size, g, t))
    if w.dense:
        o, lse = oracle.attend_causal_many(qd, kd, vd, pos, scale)
        return None, o, lse
    gi = 0 if inp.num_idx_heads == 1 else g
    kidx = oracle.page_rows(ov.kidx, ov.table[b], w.page_size, gi, t)
    qi = inp.q_idx[b].index_select(0, sel)[:, gi].cpu().numpy()
    sc = oracle.index_scores_many(qi, kidx)
    width = w.prefix_len + w.top_k
    lists = np.empty((len(rows), width), dtype=np.int64)
    thr = np.empty((len(rows), 2), dtype=np.int64)
    o = np.empty((len(rows), G, w.head_dim))
    lse = np.empty((len(rows), G))
    for n, p in enumerate(pos):
        lists[n] = oracle.index_list(int(p), w.prefix_len, w.top_k, width, lambda c, n=n: sc[n, c])
        c = oracle.candidate_keys(int(p), w.prefix_len)
        thr[n] = oracle.selection_thresholds(sc[n, c], c, w.top_k)
        keys = lists[n][lists[n] >= 0]
        o[n], lse[n] = oracle.attend(qd[n], kd[keys], vd[keys], scale)
    return (lists, thr), o, lse


def compare_block(gpu: GpuRun, ov: OracleView, b: int, rows, g: int, want=None):
    """compare_rows for many rows of one (sequence, group) through oracle_block (or a
    precomputed result `want`); returns (max_abs, mean_abs, max_lse, oracle result)."""
    w = ov.w
    G = w.group
    want = want if want is not None else oracle_block(ov, b, rows, g)
    sel_ref, o, lse = want
    sel = torch.as_tensor([int(i) for i in rows], device=gpu.out.device, dtype=torch.long)
    gi = 0 if ov.inp.num_idx_heads == 1 else g
    if sel_ref is not None and gpu.indices is not None:
        lists = sel_ref[0]
        got = gpu.indices[b].index_select(0, sel)[:, gi].cpu().numpy()
        bad = np.nonzero(np.any(got != lists, axis=1))[0]
        assert bad.size == 0, (b, g, [int(rows[k]) for k in bad[:8]], got[bad[0]][:16], lists[bad[0]][:16])
    if sel_ref is not None and gpu.thresholds is not None:
        thr = sel_ref[1]
        got = gpu.thresholds[b].index_select(0, sel)[:, gi].cpu().numpy().astype(np.int64)
        bad = np.nonzero(np.any(got != thr, axis=1))[0]
        assert bad.size == 0, (b, g, [int(rows[k]) for k in bad[:8]], got[bad[:4]], thr[bad[:4]])
    og = f64(gpu.out[b].index_select(0, sel)[:, g * G:(g + 1) * G])
    e = np.abs(og - o)
    le = 0.0
    if gpu.lse is not None:
        lg = gpu.lse[b].index_select(0, sel)[:, g * G:(g + 1) * G].double().cpu().numpy()
        le = float(np.abs(lg - lse).max())
    return float(e.max()), float(e.mean()), le, want


def merge_stats(stats):
    """Worst max-abs, mean of mean-abs (equal row counts per item), worst LSE error."""
    return (max(s[0] for s in stats), float(np.mean([s[1] for s in stats])), max(s[2] for s in stats),
            min(s[3] if len(s) > 3 else LSE_ABS for s in stats))
