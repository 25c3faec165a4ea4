"""Seeded generation of queries, paged KV pools, indexer tensors and page tables.

Values: normals are drawn in fp32 and rounded to bf16 (round-to-nearest-even, torch's cast);
indexer entries are uniform integers in [-127, 127]. Every tensor has its own generator
stream, seeded from (seed, tensor id), so a tensor does not change when another one's size
does. Large pools are drawn in slices to bound the fp32 temporary.

Layouts (all row-major):
  q          bf16  [B][S][H_q][d]
  k_pool     bf16  [num_pages][H_kv][page_size][d]
  v_pool     bf16  [num_pages][H_kv][page_size][d]
  q_idx      int8  [B][S][H_idx][d_idx]
  kidx_pool  int8  [num_pages][H_idx][page_size][d_idx]
  page_table int32 [B][max_pages_per_seq]   (-1 past a sequence's last page)
  seq_lens   int32 [B]
"""
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import Workload

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "q_idx": 3, "k_idx": 4, "perm": 5}

_SLICE_ELEMS = 1 << 25  # fp32 temporaries of at most 128 MiB


@dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    q_idx: Optional[torch.Tensor]
    kidx_pool: Optional[torch.Tensor]
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    seq_lens_host: list
    num_idx_heads: int

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    def to(self, device) -> "Inputs":
        def mv(t):
            return None if t is None else t.to(device)
        return Inputs(self.workload, mv(self.q), mv(self.k_pool), mv(self.v_pool), mv(self.q_idx),
                      mv(self.kidx_pool), mv(self.page_table), mv(self.seq_lens),
                      list(self.seq_lens_host), self.num_idx_heads)


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + TENSOR_IDS[name])
    return g


def _normal_bf16(shape, gen, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _SLICE_ELEMS):
        e = min(n, s + _SLICE_ELEMS)
        flat[s:e] = torch.randn(e - s, generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)
    return out


def _int8_values(shape, gen, device, values: Optional[Sequence[int]]) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.int8, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _SLICE_ELEMS):
        e = min(n, s + _SLICE_ELEMS)
        if values is None:
            flat[s:e] = torch.randint(-127, 128, (e - s,), generator=gen, dtype=torch.int16,
                                      device=device).to(torch.int8)
        else:
            table = torch.tensor(list(values), dtype=torch.int8, device=device)
            pick = torch.randint(0, len(values), (e - s,), generator=gen, device=device)
            flat[s:e] = table[pick]
    return out


def make_inputs(w: Workload, seed: int = 0, device="cpu", *,
                seq_lens: Optional[Sequence[int]] = None,
                num_idx_heads: Optional[int] = None,
                idx_values: Optional[Sequence[int]] = None,
                spare_pages: int = 0,
                with_q: bool = True) -> Inputs:
    """Draw one workload's inputs on `device`.

    seq_lens      per-sequence cached lengths (default: all equal to w.seq_len); each must be
                  at least w.q_len because queries are the last q_len positions.
    num_idx_heads indexer heads, H_kv (default) or 1 (one indexer key shared by all KV heads).
    idx_values    draw indexer entries from this finite set instead of [-127, 127]
                  (a small set such as {-1, 0, 1} makes equal scores common).
    spare_pages   extra pool pages no sequence maps to (they still hold random data).
    """
    device = torch.device(device)
    B, S, Hq, Hkv, d = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    ps = w.page_size
    lens = [w.seq_len] * B if seq_lens is None else [int(x) for x in seq_lens]
    assert len(lens) == B and all(t >= S for t in lens), (lens, S)
    pages_per = [-(-t // ps) for t in lens]
    max_pages = max(pages_per)
    num_pages = sum(pages_per) + spare_pages
    h_idx = Hkv if num_idx_heads is None else int(num_idx_heads)

    if w.shuffled_pages:
        perm = torch.randperm(num_pages, generator=_gen(seed, "perm", "cpu"))
    else:
        perm = torch.arange(num_pages)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    base = 0
    for b in range(B):
        table[b, :pages_per[b]] = perm[base:base + pages_per[b]].to(torch.int32)
        base += pages_per[b]

    q = _normal_bf16((B, S, Hq, d), _gen(seed, "q", device), device) if with_q else None
    k_pool = _normal_bf16((num_pages, Hkv, ps, d), _gen(seed, "k", device), device)
    v_pool = _normal_bf16((num_pages, Hkv, ps, d), _gen(seed, "v", device), device)
    if w.dense:
        q_idx = kidx = None
    else:
        q_idx = _int8_values((B, S, h_idx, w.idx_dim), _gen(seed, "q_idx", device), device, idx_values)
        kidx = _int8_values((num_pages, h_idx, ps, w.idx_dim), _gen(seed, "k_idx", device), device,
                            idx_values)
    return Inputs(w, q, k_pool, v_pool, q_idx, kidx, table.to(device),
                  torch.tensor(lens, dtype=torch.int32, device=device), lens, h_idx)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw bf16 bit patterns of a tensor, as a host numpy uint16 array (a pure copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
