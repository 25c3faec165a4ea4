"""KV-cache block allocator on the GPU against the oracle ([DSA-page] §2.4: a KV dynamic
allocator with an independent block map per layer and head). Allocation is first fit in
(sequence, logical block) order, so maps, tables and status must match bit for bit."""
import numpy as np
import pytest
import torch

import flash_attention_int8_amd as fa
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(msg):
    print(f"\n[kv blocks] {msg}", flush=True)


def pack(in_use, tail_bits=None):
    """bool [M][num_pages] -> int32 [M][words] of uint32 bit words (bit p % 32 of word p / 32)."""
    M, n = in_use.shape
    words = -(-n // 32)
    full = np.zeros((M, words * 32), dtype=bool)
    full[:, :n] = in_use
    if tail_bits is not None:
        full[:, n:] = tail_bits
    packed = np.packbits(full.reshape(M, words, 32), axis=2, bitorder="little")
    return packed.view("<u4").reshape(M, words).view(np.int32).copy()


def unpack(words, n):
    w = np.ascontiguousarray(words).view("<u4")
    b = np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1, 4), axis=2, bitorder="little")
    full = b.reshape(w.shape[0], -1).astype(bool)
    return full[:, :n], full[:, n:]


def run_alloc(in_use, tables, old, new, ps, tail_bits=None):
    M, n = in_use.shape
    bm = torch.from_numpy(pack(in_use, tail_bits)).to(DEV)
    tab = torch.from_numpy(np.asarray(tables, dtype=np.int32)).to(DEV)
    st = fa.kv_alloc(bm, tab, torch.tensor(old, dtype=torch.int32, device=DEV),
                     torch.tensor(new, dtype=torch.int32, device=DEV), ps, n)
    torch.cuda.synchronize()
    u, tail = unpack(bm.cpu().numpy(), n)
    return u, tab.cpu().numpy(), st.cpu().numpy(), tail


def check_against_oracle(in_use, tables, old, new, ps, tail_bits=None):
    u, tab, st, tail = run_alloc(in_use, tables, old, new, ps, tail_bits)
    for m in range(in_use.shape[0]):
        ou, ot, ost = oracle.allocate_blocks(in_use[m], tables[m], old, new, ps)
        assert int(st[m]) == ost, f"map {m}: status {st[m]} vs {ost}"
        assert np.array_equal(u[m], ou), f"map {m}: block map differs"
        assert np.array_equal(tab[m], ot), f"map {m}: block table differs"
    if tail_bits is not None:
        assert np.array_equal(tail, np.broadcast_to(tail_bits, tail.shape))
    return u, tab, st


CASES = {
    # 4 layers x 8 heads, decode growth of a few blocks, 5000 blocks (not a multiple of 32)
    "decode_32_maps": dict(M=32, pages=5000, B=16, ps=64, max_pages=64, fill=0.5, grow=(0, 200)),
    # prefill-sized requests: the scan crosses several 1024-word steps (100000 blocks, 70% taken)
    "prefill_many_words": dict(M=3, pages=100000, B=4, ps=64, max_pages=1024, fill=0.7, grow=(20000, 32768)),
    # one-token blocks, every sequence grows, odd sizes
    "page_size_1": dict(M=5, pages=777, B=9, ps=1, max_pages=40, fill=0.3, grow=(0, 12)),
    # a batch larger than one workgroup's 1024 threads (two steps of the request prefix sum)
    "batch_3000": dict(M=2, pages=20000, B=3000, ps=16, max_pages=8, fill=0.6, grow=(0, 20)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kv_alloc_matches_oracle(name):
    c = CASES[name]
    _banner(name)
    rng = np.random.default_rng(sum(map(ord, name)))
    M, n, B, ps, mp = c["M"], c["pages"], c["B"], c["ps"], c["max_pages"]
    in_use = rng.random((M, n)) < c["fill"]
    # some maps almost full: fewer free blocks than needed, so they must stay unchanged
    in_use[M - 1, : n - 3] = True
    old = rng.integers(0, mp * ps // 2 + 1, B)
    new = np.minimum(old + rng.integers(c["grow"][0], c["grow"][1] + 1, B), mp * ps)
    tables = rng.integers(-1, n, (M, B, mp))
    tail = rng.random(32) < 0.5
    u, tab, st = check_against_oracle(in_use, tables, old.tolist(), new.tolist(), ps, tail[: (-n) % 32])
    assert (st[: M - 1] == 0).all() or name == "prefill_many_words"
    assert st[M - 1] > 0


def test_kv_alloc_bad_lengths_and_empty_need():
    _banner("bad lengths, empty need")
    rng = np.random.default_rng(5)
    M, n, B, ps, mp = 4, 300, 3, 8, 5
    in_use = rng.random((M, n)) < 0.4
    tables = rng.integers(-1, n, (M, B, mp))
    for old, new in (([0, 0, 0], [8, 41, 0]),      # 41 tokens need 6 > 5 blocks
                     ([-1, 0, 0], [8, 8, 8]),       # a negative length
                     ([0, 0, 0], [8, -3, 0]),
                     ([16, 9, 40], [16, 9, 40]),    # nothing to grow
                     ([30, 20, 10], [3, 2, 1])):    # shrinking: nothing to allocate
        u, tab, st = check_against_oracle(in_use, tables, old, new, ps)


def test_kv_alloc_then_release_decode_loop():
    """Two allocation steps in a row (a decode loop), then the release of some sequences, then
    an allocation that reuses the freed blocks: each step against the oracle."""
    _banner("alloc, alloc, release, alloc")
    rng = np.random.default_rng(11)
    M, n, B, ps, mp = 6, 2000, 12, 16, 32
    in_use = rng.random((M, n)) < 0.3
    tables = np.full((M, B, mp), -1)
    lens0 = rng.integers(0, 200, B)
    lens1 = lens0 + rng.integers(0, 40, B)
    u1, t1, st1 = check_against_oracle(in_use, tables, np.zeros(B, int).tolist(), lens0.tolist(), ps)
    u2, t2, st2 = check_against_oracle(u1, t1, lens0.tolist(), lens1.tolist(), ps)
    assert (st1 == 0).all() and (st2 == 0).all()
    rel = rng.integers(0, 2, B).astype(np.int32)
    bm = torch.from_numpy(pack(u2)).to(DEV)
    tab = torch.from_numpy(t2.astype(np.int32)).to(DEV)
    fa.kv_release(bm, tab, torch.tensor(lens1, dtype=torch.int32, device=DEV),
                  torch.from_numpy(rel).to(DEV), ps, n)
    torch.cuda.synchronize()
    u3, _ = unpack(bm.cpu().numpy(), n)
    t3 = tab.cpu().numpy()
    for m in range(M):
        ou, ot = oracle.release_blocks(u2[m], t2[m], lens1, rel, ps)
        assert np.array_equal(u3[m], ou) and np.array_equal(t3[m], ot)
    lens2 = np.where(rel != 0, rng.integers(0, 300, B), lens1)
    old2 = np.where(rel != 0, 0, lens1)
    check_against_oracle(u3, t3, old2.tolist(), lens2.tolist(), ps)


def _bf16(rng, shape):
    t = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
    return t, t.view(torch.int16).numpy().view(np.uint16)


def test_decode_loop_allocate_append_select_attend():
    """A decode loop over the cache upkeep and the hot path together ([DSA-page] §2.2-§2.4):
    blocks allocated from a partly taken map, the prompt's rows appended, then three steps of
    (allocate, append the new token, select, attend). Expected values come only from the
    oracle: its allocation of the same requests, pools filled by its append from the host-side
    token arrays, and its selection and attention over them."""
    _banner("decode loop: alloc, append, select, attend")
    rng = np.random.default_rng(31)
    B, H, G, d, di, ps, mp, npages, P, K = 3, 2, 4, 64, 32, 64, 12, 40, 2, 64
    Hq, steps = H * G, 3
    lens = np.array([300, 130, 1])
    tmax = int(lens.max()) + steps
    k_tok, k_bits = _bf16(rng, (B, tmax, H, d))
    v_tok, v_bits = _bf16(rng, (B, tmax, H, d))
    i_tok = rng.integers(-127, 128, (B, tmax, H, di)).astype(np.int8)
    q_step, q_bits = _bf16(rng, (steps, B, Hq, d))
    qi_step = rng.integers(-127, 128, (steps, B, H, di)).astype(np.int8)

    in_use = rng.random(npages) < 0.3
    bm = torch.from_numpy(pack(in_use[None])).to(DEV)
    tab = torch.full((1, B, mp), -1, dtype=torch.int32, device=DEV)
    o_use, o_tab = in_use.copy(), np.full((B, mp), -1)
    k_pool = torch.zeros((npages, H, ps, d), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    i_pool = torch.zeros((npages, H, ps, di), dtype=torch.int8, device=DEV)
    ok_pool = np.zeros((npages, H, ps, d), np.uint16)
    ov_pool = np.zeros_like(ok_pool)
    oi_pool = np.zeros((npages, H, ps, di), np.int8)
    seq_lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    kv = fa.PagedKV(k_pool=k_pool, v_pool=v_pool, kidx_pool=i_pool, page_table=tab[0],
                    seq_lens=seq_lens, max_seq_len=mp * ps, prefix_len=P)

    def grow(old, new):
        st = fa.kv_alloc(bm, tab, torch.tensor(old, dtype=torch.int32, device=DEV),
                         torch.tensor(new, dtype=torch.int32, device=DEV), ps, npages)
        nonlocal o_use, o_tab
        o_use, o_tab, o_st = oracle.allocate_blocks(o_use, o_tab, old, new, ps)
        torch.cuda.synchronize()
        assert int(st[0]) == o_st == 0
        assert np.array_equal(tab[0].cpu().numpy(), o_tab)
        seq_lens.copy_(torch.tensor(new, dtype=torch.int32))
        # append tokens old .. new - 1 of every sequence (n = the largest growth; positions
        # before a sequence's own new tokens are rewritten with their existing values)
        n = int(max(np.asarray(new) - np.asarray(old)))
        idx = np.asarray(new)[:, None] - n + np.arange(n)[None, :]
        src = np.clip(idx, 0, tmax - 1)
        take = lambda a: torch.from_numpy(np.take_along_axis(a, src[:, :, None, None], axis=1)) if isinstance(a, np.ndarray) \
            else torch.stack([a[b, src[b]] for b in range(B)])
        fa.kv_append(kv, take(k_tok).to(DEV), take(v_tok).to(DEV), take(i_tok).to(DEV))
        for b in range(B):
            t = np.arange(old[b], new[b])
            for h in range(H):
                oracle.append_rows(ok_pool, o_tab[b], ps, h, t, k_bits[b, t, h])
                oracle.append_rows(ov_pool, o_tab[b], ps, h, t, v_bits[b, t, h])
                oracle.append_rows(oi_pool, o_tab[b], ps, h, t, i_tok[b, t, h])

    grow([0] * B, lens.tolist())
    errs, lerrs = [], []
    for s in range(steps):
        grow(lens.tolist(), (lens + 1).tolist())
        lens = lens + 1
        lists = fa.index_topk(kv, torch.from_numpy(qi_step[s][:, None]).to(DEV), 1, 1, K)
        out, lse = fa.decode(kv, q_step[s].to(DEV), lists[:, 0].contiguous())
        torch.cuda.synchronize()
        got = lists[:, 0].cpu().numpy()
        for b in range(B):
            for g in range(H):
                idx, o_ref, l_ref = oracle.dsa_query(
                    q_bits=q_bits[s, b, g * G:(g + 1) * G], q_idx_vec=qi_step[s, b, g], kidx_pool=oi_pool,
                    k_pool=ok_pool, v_pool=ov_pool, page_table_row=o_tab[b], page_size=ps, kv_head=g,
                    idx_head=g, pos=int(lens[b]) - 1, prefix_len=P, top_k=K, sm_scale=d ** -0.5)
                assert np.array_equal(got[b, g], idx), (s, b, g)
                errs.append(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).ravel())
                lerrs.append(np.abs(lse[b, g * G:(g + 1) * G].double().cpu().numpy() - l_ref))
    e = np.concatenate(errs)
    assert e.max() <= 2e-2 and e.mean() <= 2e-3 and np.concatenate(lerrs).max() <= 4e-3
