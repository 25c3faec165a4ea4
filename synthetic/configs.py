"""The workload shapes the library is measured and checked on.

Each workload names its sizes directly. Notation: B sequences, H_q query heads sharing
H_kv KV heads in contiguous groups, head dimension d, T cached tokens per sequence, S query
tokens per sequence (S = T for a prefill, S = 1 for a decode step), indexer width d_idx,
top-K per (query, KV-head group), always-attended prefix P, and page_size tokens per KV page.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int          # T, cached tokens per sequence (including the newest)
    q_len: int            # S, query tokens per sequence, the last S positions
    idx_dim: int          # d_idx; 0 for dense attention (no indexer)
    top_k: int            # K; 0 for dense attention
    prefix_len: int       # P, forced-attention prefix (0 when absent)
    page_size: int        # tokens per KV page
    shuffled_pages: bool  # page table is a seeded permutation of the pool
    qkv_source: str       # "f32" (drawn fp32, stored bf16) or "bf16"
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def dense(self) -> bool:
        return self.top_k == 0

    @property
    def pages_per_seq(self) -> int:
        return -(-self.seq_len // self.page_size)

    @property
    def index_width(self) -> int:
        return self.prefix_len + self.top_k

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = {
    "tiny_sparse_prefill": Workload(
        name="tiny_sparse_prefill", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
        seq_len=512, q_len=512, idx_dim=32, top_k=64, prefix_len=0, page_size=512,
        shuffled_pages=False, qkv_source="f32",
        description="B=1, 4/1 heads, S=T=512, d=64, int8 indexer d_idx=32, top-K=64 causal"),
    "dense_prefill_8k": Workload(
        name="dense_prefill_8k", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_len=8192, q_len=8192, idx_dim=0, top_k=0, prefix_len=0, page_size=8192,
        shuffled_pages=False, qkv_source="bf16",
        description="dense causal FlashAttention, B=4, 32/8 GQA, S=8192, d=128, contiguous KV"),
    "sparse_decode_128k": Workload(
        name="sparse_decode_128k", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_len=131072, q_len=1, idx_dim=64, top_k=2048, prefix_len=0, page_size=64,
        shuffled_pages=True, qkv_source="bf16",
        description="sparse decode, B=8, 32/8 GQA, d=128, 128K context, 64-token pages, "
                    "d_idx=64, top-K=2048"),
    "sparse_prefill_32k": Workload(
        name="sparse_prefill_32k", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_len=32768, q_len=32768, idx_dim=64, top_k=2048, prefix_len=0, page_size=64,
        shuffled_pages=True, qkv_source="bf16",
        description="sparse causal prefill, B=1, S=32768, 32/8 GQA, d=128, d_idx=64, "
                    "top-K=2048, 64-token pages"),
    "sparse_decode_1m_prefix": Workload(
        name="sparse_decode_1m_prefix", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
        seq_len=1048576, q_len=1, idx_dim=64, top_k=2048, prefix_len=196, page_size=64,
        shuffled_pages=True, qkv_source="bf16",
        description="million-token sparse decode, B=4, 32/8 GQA, d=128, 196-token forced "
                    "prefix, d_idx=64, top-K=2048, 64-token pages"),
}

ORDER = ["tiny_sparse_prefill", "dense_prefill_8k", "sparse_decode_128k",
         "sparse_prefill_32k", "sparse_decode_1m_prefix"]


def get_config(name: str) -> Workload:
    return CONFIGS[name]
