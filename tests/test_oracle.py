"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself: a brute-force
enumeration, a closed form, a library routine, or a hand-worked example. A plausible slip
in the oracle (lowest instead of highest scores, ties to the higher index, a dropped
softmax scale, a transposed operand, a wrong page lookup, the prefix counted inside K)
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    """float -> bf16 bits for values that are exactly representable (tests only)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not bf16-exact"
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- conversions / positions

def test_bf16_bits_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3FC0], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 1.5]
    got = oracle.bf16_to_f64(bits)
    assert got.dtype == np.float64
    assert list(got) == want


def test_query_position_prefill_and_decode():
    assert [oracle.query_position(10, 10, i) for i in range(3)] == [0, 1, 2]
    assert oracle.query_position(131072, 1, 0) == 131071
    # a block of 4 queries that ends the sequence
    assert [oracle.query_position(20, 4, i) for i in range(4)] == [16, 17, 18, 19]


def test_group_heads_are_contiguous():
    assert list(oracle.group_query_heads(0, 32, 8)) == [0, 1, 2, 3]
    assert list(oracle.group_query_heads(7, 32, 8)) == [28, 29, 30, 31]
    assert list(oracle.group_query_heads(0, 4, 1)) == [0, 1, 2, 3]


# ---------------------------------------------------------------- indexer scores

@pytest.mark.parametrize("d_idx", [1, 32, 64, 128])
def test_index_scores_brute_force(d_idx):
    rng = np.random.default_rng(d_idx)
    q = rng.integers(-128, 128, size=d_idx).astype(np.int8)
    k = rng.integers(-128, 128, size=(37, d_idx)).astype(np.int8)
    got = oracle.index_scores(q, k)
    want = [sum(int(q[j]) * int(k[t, j]) for j in range(d_idx)) for t in range(k.shape[0])]
    assert got.dtype == np.int64
    assert list(got) == want


def test_index_scores_int8_extremes():
    q = np.full(64, -128, dtype=np.int8)
    assert list(oracle.index_scores(q, np.full((1, 64), -128, np.int8))) == [2 ** 20]
    assert list(oracle.index_scores(q, np.full((1, 64), 127, np.int8))) == [-64 * 128 * 127]
    q2 = np.full(128, -128, dtype=np.int8)
    assert list(oracle.index_scores(q2, np.full((1, 128), -128, np.int8))) == [2 ** 21]


@pytest.mark.parametrize("d_idx", [1, 32, 64, 128])
def test_index_scores_many_brute_force(d_idx):
    """The batched scores (a float64 matrix product) equal pure-Python integer loops, with
    the int8 minimum -128 mixed in, and equal index_scores row by row."""
    rng = np.random.default_rng(100 + d_idx)
    q = rng.integers(-128, 128, size=(5, d_idx)).astype(np.int8)
    k = rng.integers(-128, 128, size=(29, d_idx)).astype(np.int8)
    q[0] = -128
    k[3] = -128
    k[4] = 127
    got = oracle.index_scores_many(q, k)
    assert got.dtype == np.int64 and got.shape == (5, 29)
    want = [[sum(int(q[n, j]) * int(k[t, j]) for j in range(d_idx)) for t in range(29)] for n in range(5)]
    assert got.tolist() == want
    assert got[0, 3] == d_idx * 2 ** 14 and got[0, 4] == -d_idx * 128 * 127
    for n in range(5):
        assert np.array_equal(got[n], oracle.index_scores(q[n], k))


def test_index_scores_many_extremes_exact():
    """At the largest magnitudes (+-2^21 at d_idx = 128, one unit apart from neighbours) the
    float64 product is still exact."""
    q = np.full((2, 128), -128, dtype=np.int8)
    q[1, 0] = -127
    k = np.full((3, 128), -128, dtype=np.int8)
    k[1, :] = 127
    k[2, 5] = 127
    got = oracle.index_scores_many(q, k)
    assert got.tolist() == [[2 ** 21, -128 * 128 * 127, 2 ** 21 - 128 * 128 - 128 * 127],
                            [2 ** 21 - 128, -127 * 127 - 127 * 128 * 127,
                             2 ** 21 - 128 - 128 * 128 - 128 * 127]]


# ---------------------------------------------------------------- top-K

def _brute_topk(scores, t, k):
    order = sorted(range(len(t)), key=lambda j: (-int(scores[j]), int(t[j])))
    return sorted(int(t[j]) for j in order[:k])


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_full_sort(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 60))
    k = int(rng.integers(1, 70))
    span = int(rng.choice([2, 3, 5, 100, 10 ** 6]))  # small spans force many ties
    scores = rng.integers(-span, span + 1, size=n)
    t = np.sort(rng.choice(10 ** 4, size=n, replace=False)) if n else np.zeros(0, np.int64)
    got = oracle.topk_select(scores, t, k)
    assert list(got) == _brute_topk(scores, t, k)


def test_topk_invariants_large():
    rng = np.random.default_rng(7)
    n, k = 50_000, 2048
    scores = rng.integers(-40, 41, size=n)          # ~1200 copies of each value
    t = np.arange(100, 100 + n)
    sel = oracle.topk_select(scores, t, k)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    chosen = np.isin(t, sel)
    tau = scores[chosen].min()
    assert scores[~chosen].max() <= tau
    # among scores equal to tau, every chosen index is below every unchosen one
    eq = scores == tau
    assert t[eq & chosen].max() < t[eq & ~chosen].min()


def _kept_by_thresholds(scores, t, tau, t_cut):
    scores, t = np.asarray(scores), np.asarray(t)
    return t[(scores > tau) | ((scores == tau) & (t <= t_cut))]


@pytest.mark.parametrize("seed", range(30))
def test_selection_thresholds_rebuild_the_brute_force_top_k(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 60))
    t = np.sort(rng.choice(1000, size=n, replace=False))
    scores = rng.integers(-3, 4, size=n) * int(rng.choice([1, 1000]))   # heavy ties
    k = int(rng.integers(1, 70))
    tau, t_cut = oracle.selection_thresholds(scores, t, k)
    assert list(_kept_by_thresholds(scores, t, tau, t_cut)) == list(_brute_topk(scores, t, k))


def test_selection_thresholds_hand_worked():
    t = np.array([3, 5, 8, 9, 12, 20])
    s = np.array([7, 4, 4, 9, 4, 1])
    # K = 3: 9 (t9), 7 (t3), then the lowest token of the three 4s (t5): tau 4, cut at 5
    assert oracle.selection_thresholds(s, t, 3) == (4, 5)
    # K = 5: all three 4s are kept: no cut
    assert oracle.selection_thresholds(s, t, 5) == (4, oracle.INT32_MAX)
    # K = 4: two of the three 4s, cut at 8
    assert oracle.selection_thresholds(s, t, 4) == (4, 8)
    # K >= candidates: everything
    assert oracle.selection_thresholds(s, t, 6) == (oracle.INT32_MIN, oracle.INT32_MAX)
    assert oracle.selection_thresholds(s[:0], t[:0], 1) == (oracle.INT32_MIN, oracle.INT32_MAX)


def test_topk_all_equal_takes_lowest_indices():
    t = np.arange(5, 105)
    assert list(oracle.topk_select(np.zeros(100, np.int64), t, 7)) == list(range(5, 12))


def test_topk_few_candidates_keeps_all():
    t = np.array([3, 9, 11])
    assert list(oracle.topk_select([5, -1, 2], t, 3)) == [3, 9, 11]
    assert list(oracle.topk_select([5, -1, 2], t, 8)) == [3, 9, 11]
    assert list(oracle.topk_select([5, -1, 2], t, 2)) == [3, 11]


# ---------------------------------------------------------------- index lists / prefix

@pytest.mark.parametrize("prefix_len", [0, 1, 5, 196])
def test_index_list_prefix_always_present(prefix_len):
    rng = np.random.default_rng(prefix_len)
    top_k = 16
    width = prefix_len + top_k
    for pos in [0, 1, 3, prefix_len - 1, prefix_len, prefix_len + 3, prefix_len + 40, 500]:
        if pos < 0:
            continue
        scores = rng.integers(-5, 6, size=pos + 1)

        def score_fn(c):
            assert c.size == 0 or c.min() >= prefix_len  # prefix keys are never scored
            return scores[c]
        lst = oracle.index_list(pos, prefix_len, top_k, width, score_fn)
        assert lst.shape == (width,)
        keys = lst[lst >= 0]
        assert np.all(lst[keys.size:] == -1)
        assert np.all(np.diff(keys) > 0)
        visible_prefix = list(range(min(prefix_len, pos + 1)))
        assert list(keys[:len(visible_prefix)]) == visible_prefix
        n_cand = max(0, pos + 1 - prefix_len)
        assert keys.size == len(visible_prefix) + min(top_k, n_cand)  # prefix is outside K
        assert keys.max() <= pos


def test_index_list_ignores_prefix_scores():
    # Even if prefix keys would outscore everything, they occupy no top-K place.
    scores = np.array([10 ** 6] * 4 + list(range(20)))

    def score_fn(c):
        return scores[c]
    lst = oracle.index_list(23, 4, 3, 7, score_fn)
    assert list(lst) == [0, 1, 2, 3, 21, 22, 23]


# ---------------------------------------------------------------- paging

@pytest.mark.parametrize("seed", range(12))
def test_hybrid_list_matches_brute_force(seed):
    """Window + prefix forced, the top-K of the rest by (score desc, token asc): checked
    against a full sort of every key with the forced ones marked, on tied small scores."""
    rng = np.random.default_rng(100 + seed)
    pos = int(rng.integers(0, 90))
    P, W, K = int(rng.integers(0, 6)), int(rng.integers(0, 40)), int(rng.integers(1, 30))
    scores = rng.integers(-3, 4, size=pos + 1)
    got = oracle.hybrid_index_list(pos, P, W, K, P + K + W, lambda t: scores[t])
    forced = [t for t in range(pos + 1) if t < P or t > pos - W]
    rest = sorted((t for t in range(pos + 1) if t not in forced), key=lambda t: (-scores[t], t))
    want = sorted(forced + rest[:K])
    assert list(got[:len(want)]) == want
    assert np.all(got[len(want):] == -1) and len(got) == P + K + W


def test_hybrid_list_special_cases():
    rng = np.random.default_rng(7)
    scores = rng.integers(-50, 50, size=400)
    fn = lambda t: scores[t]
    for pos in (0, 5, 63, 200, 399):
        for P in (0, 3):
            # no window: the plain selection
            assert np.array_equal(oracle.hybrid_index_list(pos, P, 0, 20, P + 20, fn),
                                  oracle.index_list(pos, P, 20, P + 20, fn))
            # a window reaching the first key: every key, nothing screened
            got = oracle.hybrid_index_list(pos, P, pos + 1, 20, P + 20 + pos + 1, fn)
            assert np.array_equal(got[:pos + 1], np.arange(pos + 1))
            assert np.all(got[pos + 1:] == -1)
    # maximal scores inside the window take no place of the top-K
    s2 = scores.copy()
    s2[380:] = 10 ** 6
    got = oracle.hybrid_index_list(399, 2, 20, 10, 32, lambda t: s2[t])
    assert np.array_equal(got[-20:], np.arange(380, 400))
    top = got[(got >= 2) & (got < 380)]
    assert len(top) == 10 and np.array_equal(top, np.sort(oracle.topk_select(s2[2:380], np.arange(2, 380), 10)))


def test_page_rows_follow_the_page_table():
    rng = np.random.default_rng(3)
    T, ps, H, D = 200, 16, 3, 5
    pages = -(-T // ps)
    logical = rng.standard_normal((pages * ps, H, D))
    perm = rng.permutation(pages + 4)[:pages]          # spare physical pages too
    pool = np.zeros((pages + 4, H, ps, D))
    for p in range(pages):
        pool[perm[p]] = logical[p * ps:(p + 1) * ps].transpose(1, 0, 2)
    t = rng.integers(0, T, size=50)
    for h in range(H):
        assert np.array_equal(oracle.page_rows(pool, perm, ps, h, t), logical[t, h])


# ---------------------------------------------------------------- attention closed forms

def test_append_rows_round_trip_and_unpaged_equivalent():
    """Writing tokens through the page table lands them where page_rows reads them, touches
    nothing else, equals a plain write into the unpaged (logical-order) array, and skips
    tokens whose block is missing from the table."""
    rng = np.random.default_rng(3)
    page_size, n_pages, heads, d = 4, 6, 2, 3
    table = rng.permutation(n_pages + 2)[:n_pages]          # spare physical pages
    pool = rng.integers(-9, 9, size=(n_pages + 2, heads, page_size, d))
    before = pool.copy()
    t = np.array([0, 5, 6, 7, 13, 23])
    rows = rng.integers(100, 200, size=(len(t), d))
    oracle.append_rows(pool, table, page_size, 1, t, rows)
    assert np.array_equal(oracle.page_rows(pool, table, page_size, 1, t), rows)
    # unpaged: logical array [token][head][d] built from the table, written directly
    def unpaged(p):  # [page][head][slot][d] -> [token][head][d] in logical order
        return p[table].transpose(0, 2, 1, 3).reshape(n_pages * page_size, heads, d)
    logical = unpaged(before).copy()
    logical[t, 1] = rows
    assert np.array_equal(unpaged(pool), logical)
    spare = np.setdiff1d(np.arange(n_pages + 2), table)
    assert np.array_equal(pool[spare], before[spare])       # pages outside the table untouched
    # a missing block: its tokens are skipped, the others still written
    table2 = table.copy()
    table2[1] = -1                                           # tokens 4..7
    pool2 = before.copy()
    oracle.append_rows(pool2, table2, page_size, 0, t, rows)
    ok = (t // page_size) != 1
    assert np.array_equal(oracle.page_rows(pool2, table, page_size, 0, t[ok]), rows[ok])
    assert np.array_equal(pool2[table[1]], before[table[1]])


def test_attend_single_key():
    q = np.array([[0.5, -1.0, 2.0], [1.0, 1.0, 1.0]])
    k = np.array([[2.0, 1.0, 0.25]])
    v = np.array([[3.0, -4.0, 5.0]])
    o, lse = oracle.attend(q, k, v, 0.75)
    assert np.array_equal(o, np.repeat(v, 2, axis=0))
    assert np.allclose(lse, 0.75 * (q @ k[0]), rtol=0, atol=1e-15)


def test_attend_constant_v_and_identical_keys():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((9, 8))
    v_const = np.tile(rng.standard_normal(8), (9, 1))
    o, _ = oracle.attend(q, k, v_const, 0.3)
    assert np.allclose(o, v_const[:4], rtol=0, atol=1e-14)
    k_same = np.tile(k[0], (9, 1))
    v = rng.standard_normal((9, 8))
    o, lse = oracle.attend(q, k_same, v, 0.3)
    assert np.allclose(o, np.tile(v.mean(axis=0), (4, 1)), rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.3 * (q @ k[0]) + math.log(9), rtol=0, atol=1e-13)


def test_attend_probabilities_sum_to_one_and_match_logsumexp():
    rng = np.random.default_rng(1)
    n, d = 33, 16
    q = rng.standard_normal((3, d)) * 4
    k = rng.standard_normal((n, d))
    scale = 1 / math.sqrt(d)
    p, lse = oracle.attend(q, k, np.eye(n), scale)   # one-hot V rows expose the weights
    z = scale * (q @ k.T)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=0, atol=1e-12)
    assert np.allclose(p, np.exp(z - lse[:, None]), rtol=0, atol=1e-12)
    assert np.allclose(p, scipy.special.softmax(z, axis=1), rtol=0, atol=1e-12)


def test_dense_is_top_k_of_everything_and_masked_softmax():
    """K >= context reproduces dense causal attention, computed here as one full masked
    softmax(QK^T)V over the whole sequence."""
    rng = np.random.default_rng(5)
    T, d, ps, G = 70, 16, 16, 2
    pages = -(-T // ps)
    qf = rng.standard_normal((T, G, d)).astype(np.float32)
    kf = rng.standard_normal((pages * ps, d)).astype(np.float32)
    vf = rng.standard_normal((pages * ps, d)).astype(np.float32)
    qb = (qf.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 values do
    kb = (kf.view(np.uint32) >> 16).astype(np.uint16)
    vb = (vf.view(np.uint32) >> 16).astype(np.uint16)
    table = np.arange(pages)
    k_pool = kb.reshape(pages, 1, ps, d)
    v_pool = vb.reshape(pages, 1, ps, d)
    kidx = rng.integers(-127, 128, size=(pages, 1, ps, 8)).astype(np.int8)
    qidx = rng.integers(-127, 128, size=(T, 8)).astype(np.int8)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = (oracle.bf16_to_f64(x) for x in (qb, kb[:T], vb[:T]))
    z = scale * np.einsum("igd,td->git", qd, kd)
    z = np.where(np.arange(T)[None, None, :] <= np.arange(T)[None, :, None], z, -np.inf)
    want = np.einsum("git,td->igd", scipy.special.softmax(z, axis=2), vd)
    for i in [0, 1, 15, 16, 17, 40, 69]:
        idx, o, lse = oracle.dsa_query(q_bits=qb[i], q_idx_vec=qidx[i], kidx_pool=kidx, k_pool=k_pool,
                                       v_pool=v_pool, page_table_row=table, page_size=ps, kv_head=0,
                                       idx_head=0, pos=i, prefix_len=0, top_k=T, sm_scale=scale)
        assert list(idx[idx >= 0]) == list(range(i + 1))
        assert np.allclose(o, want[i], rtol=0, atol=1e-12)
        od, lsed = oracle.dense_query(q_bits=qb[i], k_pool=k_pool, v_pool=v_pool, page_table_row=table,
                                      page_size=ps, kv_head=0, pos=i, sm_scale=scale)
        assert np.allclose(od, want[i], rtol=0, atol=1e-12)
        assert np.allclose(lsed, lse, rtol=0, atol=1e-12)


def test_attend_causal_many_matches_masked_softmax_and_dense_query():
    """Many tokens at once: equals one full masked softmax(QK^T)V built with scipy, and
    dense_query token by token through a shuffled page table."""
    rng = np.random.default_rng(9)
    T, d, ps, G = 90, 16, 16, 4
    pages = -(-T // ps)
    q = rng.standard_normal((T, G, d)) * 2
    kf = rng.standard_normal((pages * ps, d)).astype(np.float32)
    vf = rng.standard_normal((pages * ps, d)).astype(np.float32)
    kb = (kf.view(np.uint32) >> 16).astype(np.uint16)
    vb = (vf.view(np.uint32) >> 16).astype(np.uint16)
    kd, vd = oracle.bf16_to_f64(kb[:T]), oracle.bf16_to_f64(vb[:T])
    scale = 1 / math.sqrt(d)
    pos = np.array([0, 1, 5, 15, 16, 17, 44, 63, 64, 89])
    o, lse = oracle.attend_causal_many(q[pos], kd, vd, pos, scale, chunk=3)
    z = scale * np.einsum("igd,td->igt", q[pos], kd)
    z = np.where(np.arange(T)[None, None, :] <= pos[:, None, None], z, -np.inf)
    want = np.einsum("igt,td->igd", scipy.special.softmax(z, axis=2), vd)
    assert np.allclose(o, want, rtol=0, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(z, axis=2), rtol=0, atol=1e-12)
    perm = rng.permutation(pages)
    k_pool = np.zeros((pages, 1, ps, d), np.uint16)
    v_pool = np.zeros((pages, 1, ps, d), np.uint16)
    k_pool[perm, 0] = kb.reshape(pages, ps, d)
    v_pool[perm, 0] = vb.reshape(pages, ps, d)
    q_bits = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o2, lse2 = oracle.attend_causal_many(oracle.bf16_to_f64(q_bits[pos]), kd, vd, pos, scale)
    for n, p in enumerate(pos):
        od, ld = oracle.dense_query(q_bits=q_bits[p], k_pool=k_pool, v_pool=v_pool, page_table_row=perm,
                                    page_size=ps, kv_head=0, pos=int(p), sm_scale=scale)
        assert np.allclose(o2[n], od, rtol=0, atol=1e-12)
        assert np.allclose(lse2[n], ld, rtol=0, atol=1e-12)


def test_attend_causal_many_closed_forms():
    """Position 0 sees only key 0 (O = V[0], LSE = its logit); constant V gives V."""
    rng = np.random.default_rng(10)
    T, d, G = 20, 8, 2
    q = rng.standard_normal((3, G, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    o, lse = oracle.attend_causal_many(q, k, v, [0, 0, 0], 0.5)
    assert np.allclose(o, np.broadcast_to(v[0], o.shape), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.5 * (q @ k[0]), rtol=0, atol=1e-14)
    vc = np.tile(v[7], (T, 1))
    o, _ = oracle.attend_causal_many(q, k, vc, [3, 11, 19], 0.5)
    assert np.allclose(o, np.broadcast_to(v[7], o.shape), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- hand-worked golden case

def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_dsa_8tok.json")))
    ps = g["page_size"]
    table = np.array(g["page_table"])
    n_pages = len(table)

    def paged(rows, dtype):
        rows = np.asarray(rows)
        pool = np.zeros((n_pages, 1, ps, rows.shape[1]), dtype=dtype)
        for t in range(rows.shape[0]):
            pool[table[t // ps], 0, t % ps] = rows[t]
        return pool
    kidx = paged(np.array(g["k_idx_logical"], dtype=np.int8), np.int8)
    k_pool = paged(_bits(g["k_logical"]), np.uint16)
    v_pool = paged(_bits(g["v_logical"]), np.uint16)
    env = {"e": math.e, "log": math.log}
    for case in g["cases"]:
        idx, o, lse = oracle.dsa_query(
            q_bits=_bits([g["q"]]), q_idx_vec=np.array(g["q_idx"], np.int8), kidx_pool=kidx,
            k_pool=k_pool, v_pool=v_pool, page_table_row=table, page_size=ps, kv_head=0, idx_head=0,
            pos=case["pos"], prefix_len=g["prefix_len"], top_k=g["top_k"], sm_scale=g["sm_scale"])
        assert list(idx) == case["index_list"], case["pos"]
        assert abs(o[0, 0] - eval(case["o0"], env)) < 1e-12, case["pos"]
        assert abs(o[0, 1] - eval(case["o1"], env)) < 1e-12, case["pos"]
        assert abs(lse[0] - eval(case["lse"], env)) < 1e-12, case["pos"]


# ----------------------------------------------------------------- KV block allocator pins

def _first_fit_one_at_a_time(in_use, table, old_lens, new_lens, page_size):
    """Independent restatement: walk the sequences, and for each missing logical block scan
    the map from block 0 for the first free block (no precomputed free list)."""
    in_use = [bool(x) for x in in_use]
    table = [list(map(int, row)) for row in table]
    max_pages = len(table[0])
    wanted = []
    for b in range(len(old_lens)):
        if old_lens[b] < 0 or new_lens[b] < 0 or (new_lens[b] + page_size - 1) // page_size > max_pages:
            return in_use, table, -1
        lo = (old_lens[b] + page_size - 1) // page_size
        hi = (new_lens[b] + page_size - 1) // page_size
        wanted += [(b, lp) for lp in range(lo, hi)]
    if sum(not x for x in in_use) < len(wanted):
        return in_use, table, len(wanted) - sum(not x for x in in_use)
    for b, lp in wanted:
        page = 0
        while in_use[page]:
            page += 1
        in_use[page] = True
        table[b][lp] = page
    return in_use, table, 0


def test_allocate_blocks_hand_example():
    """[DSA-page] §2.4 allocator, worked by hand: blocks 0, 2, 5 taken, 4-token blocks.
    Sequence 0 grows 3 -> 9 tokens (needs logical blocks 1, 2), sequence 1 grows 0 -> 5
    (blocks 0, 1); the free blocks 1, 3, 4, 6 go to them in that order."""
    in_use = np.array([1, 0, 1, 0, 0, 1, 0, 0], dtype=bool)
    table = np.full((2, 4), -1)
    table[0, 0] = 0
    u, t, st = oracle.allocate_blocks(in_use, table, [3, 0], [9, 5], 4)
    assert st == 0
    assert t.tolist() == [[0, 1, 3, -1], [4, 6, -1, -1]]
    assert u.tolist() == [True] * 7 + [False]
    # one block short: nothing changes, the status is the shortfall
    u2, t2, st2 = oracle.allocate_blocks(np.array([1, 0, 1, 1, 0, 1, 1, 0], bool), table, [3, 0], [9, 5], 4)
    assert st2 == 1 and t2.tolist() == table.tolist() and u2.sum() == 5
    # a length beyond the table, or a negative one: status -1, nothing changes
    for old, new in (([3, 0], [9, 17]), ([-1, 0], [9, 5]), ([3, 0], [9, -2])):
        u3, t3, st3 = oracle.allocate_blocks(in_use, table, old, new, 4)
        assert st3 == -1 and t3.tolist() == table.tolist() and u3.tolist() == in_use.tolist()
    # a shrinking or unchanged sequence needs nothing
    u4, t4, st4 = oracle.allocate_blocks(in_use, table, [9, 5], [4, 5], 4)
    assert st4 == 0 and t4.tolist() == table.tolist() and u4.tolist() == in_use.tolist()


def test_allocate_blocks_matches_one_at_a_time_first_fit():
    rng = np.random.default_rng(21)
    for trial in range(200):
        n_pages = int(rng.integers(1, 90))
        in_use = rng.random(n_pages) < rng.random()
        B = int(rng.integers(1, 6))
        ps = int(rng.choice([1, 2, 4, 8]))
        max_pages = int(rng.integers(1, 8))
        table = rng.integers(-1, n_pages, (B, max_pages))
        old = rng.integers(-1 if trial % 17 == 0 else 0, max_pages * ps + 1, B)
        new = old + rng.integers(-2, 2 * ps + 3, B)
        got = oracle.allocate_blocks(in_use, table, old, new, ps)
        want = _first_fit_one_at_a_time(in_use, table, old.tolist(), new.tolist(), ps)
        assert got[2] == want[2]
        assert got[0].tolist() == want[0] and got[1].tolist() == want[1]


def test_release_blocks_undoes_allocation():
    rng = np.random.default_rng(22)
    for trial in range(50):
        n_pages, B, ps, max_pages = 200, 4, 8, 6
        in_use = rng.random(n_pages) < 0.5
        table = np.full((B, max_pages), -1)
        new = rng.integers(0, max_pages * ps + 1, B)
        u, t, st = oracle.allocate_blocks(in_use, table, np.zeros(B, int), new, ps)
        assert st == 0
        taken = t[t >= 0]
        assert len(set(taken.tolist())) == taken.size          # distinct blocks
        assert not in_use[taken].any()                          # all were free before
        assert u.sum() == in_use.sum() + taken.size
        rel = rng.integers(0, 2, B)
        u2, t2 = oracle.release_blocks(u, t, new, rel, ps)
        for b in range(B):
            n = -(-int(new[b]) // ps)
            if rel[b]:
                assert (t2[b] == -1).all() and not u2[t[b, :n]].any()
            else:
                assert t2[b].tolist() == t[b].tolist() and u2[t[b, :n]].all()
        u3, t3 = oracle.release_blocks(u, t, new, np.ones(B, int), ps)
        assert u3.tolist() == in_use.tolist() and (t3 == -1).all()
