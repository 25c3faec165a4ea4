"""Reference semantics of the dynamic-sparse attention path, written as plain definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check and
the benchmark's CPU-baseline leg may use it.

[DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" (ruibaoantu.com).
[MTT-page] = "…在摩尔线程MTT S5000上的原生推理优化实践" (blog.csdn.net): §2.3 describes a hybrid of
global sparse and local sliding-window attention.
[DSA-page] §2.4 also describes the KV dynamic allocator (per-layer, per-head block maps),
modelled by allocate_blocks / release_blocks.

Readings taken where the page leaves a step open (each is also listed with its reason in
the design notes):
  * the indexer score is a plain int8 x int8 dot product accumulated exactly, with no scale,
    activation or per-head weight (§2.1 names only a "preliminary Q-K similarity");
  * one selection per (sequence, query token, KV-head group); the query heads of a group
    share it (§2.4 keeps selection state per head);
  * ties in score go to the lower token index; the selected list is returned in ascending
    token order and padded with -1 (the page states neither);
  * the forced prefix of §2.4 does not count toward K, and its keys are not scored;
  * query i of a block sits at position seq_len - q_tail + i and may attend to every cached
    key at or before its own position (the decode token is already in the cache);
  * query head h reads KV head h // (H_q / H_kv).

Parity pins (tests/test_oracle.py): index_scores against a pure-Python integer loop and
the int8 extreme closed form; index_scores_many against the same loop and extremes (the
-128 corner included) and row by row against index_scores; attend_causal_many against
closed forms (constant V, a query at position 0 seeing only key 0) and per token against
dense_query; selection_thresholds by rebuilding the kept set from (tau, t_cut) and comparing it
with a brute-force full sort, and a hand-worked case; topk_select against a brute-force full sort and the order
invariants; index_list against the prefix rule and a hand-worked golden case; attend
against closed forms (single key, constant V, identical keys, one-hot V rows giving the
probabilities), scipy's logsumexp, and a full-matrix masked softmax for the dense case;
page_rows against an unpaged copy under a random page permutation; append_rows against
page_rows (round trip) and an unpaged array write, untouched rows kept; hybrid_index_list
against a brute-force full sort with the window and prefix marked, index_list at window 0, and
every key at window >= pos + 1; allocate_blocks against a one-block-at-a-time first-fit
scan, the shortfall and bad-length cases leaving the map unchanged, and release_blocks
restoring the map after an allocation. No function is "parity unpinned".
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: a bf16 is the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def query_position(seq_len: int, q_tail: int, i: int) -> int:
    """Position of query i of a block whose first query sits q_tail tokens before the end.

    A full prefill has q_tail = T (so pos = i); a decode step has q_tail = 1 (pos = T - 1).
    """
    return int(seq_len) - int(q_tail) + int(i)


def group_query_heads(kv_head: int, num_q_heads: int, num_kv_heads: int) -> range:
    """Query heads sharing KV head `kv_head`: contiguous groups of H_q / H_kv heads."""
    g = int(num_q_heads) // int(num_kv_heads)
    return range(int(kv_head) * g, (int(kv_head) + 1) * g)


def forced_keys(pos: int, prefix_len: int) -> np.ndarray:
    """[DSA-page] §2.4: the prefix tokens the query can see are always attended."""
    return np.arange(0, min(int(prefix_len), int(pos) + 1), dtype=np.int64)


def candidate_keys(pos: int, prefix_len: int) -> np.ndarray:
    """[DSA-page] §2.1/§2.4: causal keys outside the forced prefix enter the screening."""
    return np.arange(int(prefix_len), int(pos) + 1, dtype=np.int64)


def page_rows(pool, page_table_row, page_size: int, head: int, t) -> np.ndarray:
    """[DSA-page] §2.2: token t of a sequence lives in block page_table[t // page_size] at slot
    t % page_size. `pool` is indexed [page][head][slot] -> row (any object with numpy-style
    fancy indexing that returns arrays)."""
    t = np.asarray(t, dtype=np.int64)
    table = np.asarray(page_table_row, dtype=np.int64)
    phys = table[t // page_size]
    slot = t % page_size
    return np.asarray(pool[phys, head, slot])


def append_rows(pool, page_table_row, page_size: int, head: int, t, rows) -> None:
    """[DSA-page] §2.2 / §2.3: a new token t of a sequence is stored in block
    page_table[t // page_size] at slot t % page_size (the write counterpart of page_rows).
    `pool` is a numpy array [page][head][slot][...], modified in place; `rows` holds one row
    per token of `t`. Tokens whose block is missing from the table (entry < 0) are skipped."""
    t = np.asarray(t, dtype=np.int64)
    table = np.asarray(page_table_row, dtype=np.int64)
    phys = table[t // page_size]
    ok = phys >= 0
    pool[phys[ok], head, (t % page_size)[ok]] = np.asarray(rows)[ok]


def allocate_blocks(in_use, table, old_lens, new_lens, page_size: int):
    """[DSA-page] §2.4: a KV dynamic allocator hands out and takes back cache blocks, with an
    independent block map per layer and head so that heads never write into each other's
    blocks. This is one such map: `in_use` (bool [num_pages]) marks the blocks taken and
    `table` (int [batch][max_pages]) is the block table of the sequences that use the map.

    A sequence growing from old_lens[b] to new_lens[b] tokens needs its logical blocks
    ceil(old / page_size) .. ceil(new / page_size) - 1. Reading taken where the page leaves
    the order open: the needs are served in (sequence, logical block) order by the free
    blocks in ascending block number (first fit). All or nothing: when fewer blocks are
    free than needed, nothing changes and the status is the shortfall; a negative length or
    a need beyond max_pages also changes nothing (status -1). Returns (in_use, table,
    status) as new arrays; status 0 on success.
    """
    in_use = np.array(in_use, dtype=bool)
    table = np.array(table, dtype=np.int64)
    max_pages = table.shape[1]
    needs = []
    for b, (old, new) in enumerate(zip(old_lens, new_lens)):
        old, new = int(old), int(new)
        last = -(-new // page_size)
        if old < 0 or new < 0 or last > max_pages:
            return in_use, table, -1
        needs += [(b, lp) for lp in range(-(-old // page_size), last)]
    free = np.flatnonzero(~in_use)
    if free.size < len(needs):
        return in_use, table, len(needs) - int(free.size)
    for (b, lp), page in zip(needs, free):
        table[b, lp] = page
        in_use[page] = True
    return in_use, table, 0


def release_blocks(in_use, table, seq_lens, release, page_size: int):
    """[DSA-page] §2.4, the other half of the allocator: the blocks of every sequence b with
    release[b] != 0 (its logical blocks 0 .. ceil(seq_lens[b] / page_size) - 1, at most
    max_pages) go back to the map and their table entries become -1. An entry outside
    [0, num_pages) frees nothing. Returns (in_use, table) as new arrays."""
    in_use = np.array(in_use, dtype=bool)
    table = np.array(table, dtype=np.int64)
    max_pages = table.shape[1]
    for b, (n, rel) in enumerate(zip(seq_lens, release)):
        if not rel:
            continue
        for lp in range(min(max(-(-int(n) // page_size), 0), max_pages)):
            page = table[b, lp]
            if 0 <= page < in_use.size:
                in_use[page] = False
            table[b, lp] = -1
    return in_use, table


def index_scores(q_idx_vec, k_rows) -> np.ndarray:
    """[DSA-page] §2.1: similarity of one indexer query with each candidate key.

    Exact integer dot products (int64), sigma(t) = sum_j q[j] * k[t, j].
    """
    q = np.asarray(q_idx_vec, dtype=np.int64)
    k = np.asarray(k_rows, dtype=np.int64)
    return k @ q


def index_scores_many(q_idx_rows, k_rows) -> np.ndarray:
    """[DSA-page] §2.1 for many indexer queries at once: sigma[n, t] = sum_j q[n, j] * k[t, j].

    Every product of two int8 values is an integer of magnitude at most 2^14, so each partial
    sum of a row is an integer far below 2^53 and a float64 matrix product is exact in any
    summation order (this is what lets BLAS do the work). Returned as int64 [n][T].
    """
    q = np.asarray(q_idx_rows, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    assert q.shape[-1] == k.shape[-1] and q.shape[-1] <= (1 << 30)
    return (q @ k.T).astype(np.int64)


def topk_select(scores, t, k: int) -> np.ndarray:
    """[DSA-page] §2.1: keep the K best-scoring candidates.

    `t` lists the candidate token indices in ascending order and `scores` their scores.
    The K largest by (score descending, index ascending) are kept; with K or fewer candidates
    all are kept. Returned in ascending token order.

    Steps: tau = the K-th largest score; every candidate scoring above tau is kept; the
    remaining places go to candidates scoring exactly tau, lowest index first.
    """
    scores = np.asarray(scores, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    n = scores.shape[0]
    if n <= k:
        return t.copy()
    tau = np.partition(scores, n - k)[n - k]
    above = scores > tau
    need = k - int(above.sum())
    at_tau = np.nonzero(scores == tau)[0][:need]
    keep = np.zeros(n, dtype=bool)
    keep[above] = True
    keep[at_tau] = True
    return t[keep]


INT32_MIN, INT32_MAX = -(1 << 31), (1 << 31) - 1


def selection_thresholds(scores, t, k: int):
    """The selection of topk_select written as two numbers (tau, t_cut): tau is the smallest
    kept score (the K-th largest) and t_cut the largest kept token scoring tau, so that a
    candidate is kept exactly when its score exceeds tau, or equals tau at a token <= t_cut.
    With K or fewer candidates every one is kept: (INT32_MIN, INT32_MAX). t_cut is INT32_MAX
    as well when every candidate scoring tau is kept."""
    scores = np.asarray(scores, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    if scores.shape[0] <= k:
        return INT32_MIN, INT32_MAX
    kept = np.isin(t, topk_select(scores, t, k))
    tau = int(scores[kept].min())
    at_tau = scores == tau
    if np.all(kept[at_tau]):
        return tau, INT32_MAX
    return tau, int(t[kept & at_tau].max())


def index_list(pos: int, prefix_len: int, top_k: int, width: int, score_fn) -> np.ndarray:
    """The key list one (query, KV-head group) attends to: the forced prefix followed by the
    top-K candidates, ascending, padded with -1 to `width` (= prefix_len + top_k).

    `score_fn(t)` returns the indexer scores of candidate tokens t.
    """
    f = forced_keys(pos, prefix_len)
    c = candidate_keys(pos, prefix_len)
    sel = topk_select(score_fn(c), c, top_k) if c.size else c
    keys = np.sort(np.concatenate([f, sel]))
    out = np.full(width, -1, dtype=np.int64)
    out[:keys.size] = keys
    return out


def hybrid_index_list(pos: int, prefix_len: int, window: int, top_k: int, width: int,
                      score_fn) -> np.ndarray:
    """[MTT-page] §2.3: hybrid attention = global sparse attention plus local sliding-window
    attention. Read here as one key list per (query, KV-head group): the last `window` keys up
    to the query (pos - window + 1 .. pos) are always attended, like the forced prefix of
    [DSA-page] §2.4, and are not screened; the top-K is taken over the remaining causal keys
    outside the prefix. Ascending, padded with -1 to `width` (= prefix_len + top_k + window).
    window = 0 gives index_list.
    """
    pos = int(pos)
    lo = max(0, pos - int(window) + 1)  # first window key (window empty when lo > pos)
    f = np.union1d(forced_keys(pos, prefix_len), np.arange(lo, pos + 1, dtype=np.int64))
    c = np.arange(int(prefix_len), lo, dtype=np.int64)  # screened: outside prefix and window
    sel = topk_select(score_fn(c), c, top_k) if c.size else c
    keys = np.sort(np.concatenate([f, sel]))
    out = np.full(width, -1, dtype=np.int64)
    out[:keys.size] = keys
    return out


def attend(q_heads, k_rows, v_rows, sm_scale: float):
    """Softmax attention of each query head over the given key/value rows, in float64.

    z_t = sm_scale * q . k_t;  O = sum_t softmax(z)_t v_t;  LSE = log sum_t exp(z_t).
    Returns (O [heads][d], LSE [heads]).
    """
    q = np.asarray(q_heads, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    z = float(sm_scale) * (q @ k.T)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    s = e.sum(axis=1)
    o = (e @ v) / s[:, None]
    return o, m + np.log(s)


def attend_causal_many(q_rows, k_rows, v_rows, positions, sm_scale: float, chunk: int = 64):
    """Dense causal attention of many query tokens of one KV group, in float64.

    q_rows [n][G][d] are the group's query heads of n tokens; k_rows, v_rows [T][d] the
    group's keys and values in token order; token n attends to keys 0..positions[n]. The
    logits form one full matrix with every non-causal entry at -inf; softmax per row, times V
    (the same definition as `attend` over keys 0..pos). Rows are processed `chunk` tokens at
    a time to bound memory. Returns (O [n][G][d], LSE [n][G]).
    """
    q = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    n, G, d = q.shape
    o = np.empty((n, G, v.shape[1]), dtype=np.float64)
    lse = np.empty((n, G), dtype=np.float64)
    t = np.arange(k.shape[0], dtype=np.int64)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = float(sm_scale) * (q[s:e].reshape(-1, d) @ k.T)            # [(e-s)*G][T]
        causal = t[None, :] <= np.repeat(pos[s:e], G)[:, None]
        z = np.where(causal, z, -np.inf)
        m = z.max(axis=1)
        w = np.exp(z - m[:, None])
        tot = w.sum(axis=1)
        o[s:e] = ((w @ v) / tot[:, None]).reshape(e - s, G, -1)
        lse[s:e] = (m + np.log(tot)).reshape(e - s, G)
    return o, lse


def dsa_query(*, q_bits, q_idx_vec, kidx_pool, k_pool, v_pool, page_table_row, page_size,
              kv_head, idx_head, pos, prefix_len, top_k, sm_scale):
    """One (query token, KV-head group) through the whole path of [DSA-page] §2.

    q_bits      bf16 bits of the group's query heads, [G][d]
    q_idx_vec   int8 indexer query of this token and indexer head, [d_idx]
    *_pool      [page][head][slot][...] pools (K/V as bf16 bits, indexer keys as int8)
    Returns (index list [P+K] int64 with -1 padding, O [G][d] f64, LSE [G] f64).
    """
    def score_fn(c):
        return index_scores(q_idx_vec, page_rows(kidx_pool, page_table_row, page_size, idx_head, c))

    idx = index_list(pos, prefix_len, top_k, prefix_len + top_k, score_fn)
    keys = idx[idx >= 0]
    k_rows = bf16_to_f64(page_rows(k_pool, page_table_row, page_size, kv_head, keys))
    v_rows = bf16_to_f64(page_rows(v_pool, page_table_row, page_size, kv_head, keys))
    o, lse = attend(bf16_to_f64(q_bits), k_rows, v_rows, sm_scale)
    return idx, o, lse


def dense_query(*, q_bits, k_pool, v_pool, page_table_row, page_size, kv_head, pos, sm_scale):
    """Dense causal attention of one query token's group: every key 0..pos is attended."""
    keys = np.arange(0, int(pos) + 1, dtype=np.int64)
    k_rows = bf16_to_f64(page_rows(k_pool, page_table_row, page_size, kv_head, keys))
    v_rows = bf16_to_f64(page_rows(v_pool, page_table_row, page_size, kv_head, keys))
    return attend(bf16_to_f64(q_bits), k_rows, v_rows, sm_scale)
