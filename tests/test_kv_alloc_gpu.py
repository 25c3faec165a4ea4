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
