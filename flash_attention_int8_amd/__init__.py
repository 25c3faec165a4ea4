"""Python binding of the sparse-attention C ABI (include/sparse_attn.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libsparse_attn.so. PyTorch supplies device memory (tensor.data_ptr()) and the stream
(torch.cuda.current_stream()). The functions named sparse_attn_* mirror the C entry points
one-to-one and take caller-allocated outputs; the short helpers below them (index, topk,
prefill, decode) only allocate the outputs with torch and call those.

There is no fallback: if the shared library is missing, load() raises.
"""
import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_attn.so")
SA_ABI_VERSION = 1

STATUS = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_UNSUPPORTED",
          4: "SA_ERR_WORKSPACE", 5: "SA_ERR_HIP", 6: "SA_ERR_ABI", 7: "SA_ERR_ALIGN",
          8: "SA_ERR_SCRATCH"}
SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP, SA_ERR_ABI, \
    SA_ERR_ALIGN, SA_ERR_SCRATCH = range(9)

EXPORTS = ["sparse_attn_abi_version", "sparse_attn_status_string", "sparse_attn_index",
           "sparse_attn_topk_workspace_size", "sparse_attn_topk",
           "sparse_attn_index_topk_workspace_size", "sparse_attn_index_topk",
           "sparse_attn_index_topk_window_workspace_size", "sparse_attn_index_topk_window",
           "sparse_attn_fwd_prefill", "sparse_attn_prefill_masked_workspace_size",
           "sparse_attn_fwd_prefill_masked", "sparse_attn_kv_append", "sparse_attn_kv_alloc",
           "sparse_attn_kv_release", "sparse_attn_decode_workspace_size", "sparse_attn_fwd_decode",
           "sparse_attn_decode_noalloc_max_bytes", "sparse_attn_fwd_decode_noalloc",
           "sparse_attn_select_thresholds", "sparse_attn_prefill_fused_workspace_size",
           "sparse_attn_prefill_fused_choice", "sparse_attn_prefill_fused",
           "sparse_attn_calib_read", "sparse_attn_calib_gather", "sparse_attn_calib_mfma",
           "sparse_attn_validate", "sparse_attn_check_report", "sparse_attn_workspace_size"]
SA_OP_TOPK, SA_OP_INDEX_TOPK, SA_OP_INDEX_TOPK_WINDOW, SA_OP_PREFILL_MASKED, SA_OP_PREFILL_FUSED, \
    SA_OP_DECODE = range(1, 7)
SA_PREFILL_AUTO, SA_PREFILL_GATHER, SA_PREFILL_MASKED = 0, 1, 2


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)} "
                         f"({_lib.sparse_attn_status_string(status).decode() if _lib else '?'})")


class sa_paged_kv(ctypes.Structure):
    """Mirror of `struct sa_paged_kv` (field order and types must match the header)."""
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("max_seq_len", ctypes.c_int32),
        ("prefix_len", ctypes.c_int32),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("kidx_pool", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsparse_attn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m flash_attention_int8_amd._build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    KV = ctypes.POINTER(sa_paged_kv)
    sig = {
        "sparse_attn_abi_version": (I32, []),
        "sparse_attn_status_string": (ctypes.c_char_p, [I32]),
        "sparse_attn_index": (I32, [KV, P, I32, I32, P, I64, P]),
        "sparse_attn_topk_workspace_size": (SZ, [KV, I32, I32]),
        "sparse_attn_topk": (I32, [KV, P, I64, I32, I32, I32, P, P, SZ, P]),
        "sparse_attn_index_topk_workspace_size": (SZ, [KV, I32, I32]),
        "sparse_attn_index_topk": (I32, [KV, P, I32, I32, I32, P, P, SZ, P]),
        "sparse_attn_index_topk_window_workspace_size": (SZ, [KV, I32, I32, I32]),
        "sparse_attn_index_topk_window": (I32, [KV, P, I32, I32, I32, I32, P, P, SZ, P]),
        "sparse_attn_fwd_prefill": (I32, [KV, P, I32, I32, I32, P, I32, F32, P, P, P]),
        "sparse_attn_prefill_masked_workspace_size": (SZ, [KV, I32]),
        "sparse_attn_fwd_prefill_masked": (I32, [KV, P, I32, I32, I32, P, I32, F32, P, SZ, P, P, P]),
        "sparse_attn_kv_append": (I32, [KV, P, P, P, I32, P]),
        "sparse_attn_kv_alloc": (I32, [I32, I32, P, I32, I32, I32, P, P, P, P, P]),
        "sparse_attn_kv_release": (I32, [I32, I32, P, I32, I32, I32, P, P, P, P]),
        "sparse_attn_decode_workspace_size": (SZ, [KV, I32, I32, I32]),
        "sparse_attn_fwd_decode": (I32, [KV, P, I32, P, I32, F32, I32, P, SZ, P, P, P]),
        "sparse_attn_decode_noalloc_max_bytes": (SZ, []),
        "sparse_attn_fwd_decode_noalloc": (I32, [KV, P, I32, P, I32, F32, I32, P, P, P]),
        "sparse_attn_select_thresholds": (I32, [KV, P, I32, I32, I32, P, P]),
        "sparse_attn_prefill_fused_workspace_size": (SZ, [KV, I32, I32, I32, I32, I32]),
        "sparse_attn_prefill_fused_choice": (I32, [KV, I32, I32, I32, I32]),
        "sparse_attn_prefill_fused": (I32, [KV, P, P, I32, I32, I32, I32, F32, I32, P, SZ, P, P, P]),
        "sparse_attn_calib_read": (I32, [P, SZ, P, I32, P]),
        "sparse_attn_calib_gather": (I32, [P, SZ, P, I64, P, I32, P]),
        "sparse_attn_calib_mfma": (I32, [I32, I32, I32, P, P]),
        "sparse_attn_validate": (I32, [KV, P, I32, I32, I32, P, P]),
        "sparse_attn_check_report": (I32, [P, P]),
        "sparse_attn_workspace_size": (SZ, [I32, KV, I32, I32, I32, I32, I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.sparse_attn_abi_version() != SA_ABI_VERSION:
        raise RuntimeError("libsparse_attn.so ABI version mismatch")
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int):
    if status != SA_OK:
        raise SparseAttnError(fn, status)


class PagedKV:
    """Owns the ctypes descriptor for a set of device tensors (the tensors stay caller-owned)."""

    def __init__(self, *, k_pool=None, v_pool=None, kidx_pool=None, page_table, seq_lens,
                 max_seq_len: int, prefix_len: int = 0, num_kv_heads: Optional[int] = None,
                 page_size: Optional[int] = None, head_dim: Optional[int] = None,
                 idx_dim: Optional[int] = None, num_idx_heads: Optional[int] = None,
                 num_pages: Optional[int] = None):
        ref = k_pool if k_pool is not None else kidx_pool
        d = sa_paged_kv()
        d.abi_version = SA_ABI_VERSION
        d.batch = int(page_table.shape[0])
        d.num_kv_heads = int(num_kv_heads if num_kv_heads is not None else k_pool.shape[1])
        d.head_dim = int(head_dim if head_dim is not None else (k_pool.shape[3] if k_pool is not None else 0))
        d.num_idx_heads = int(num_idx_heads if num_idx_heads is not None else
                              (kidx_pool.shape[1] if kidx_pool is not None else d.num_kv_heads))
        d.idx_dim = int(idx_dim if idx_dim is not None else (kidx_pool.shape[3] if kidx_pool is not None else 0))
        d.page_size = int(page_size if page_size is not None else ref.shape[2])
        d.max_pages_per_seq = int(page_table.shape[1])
        d.num_pages = int(num_pages if num_pages is not None else ref.shape[0])
        d.max_seq_len = int(max_seq_len)
        d.prefix_len = int(prefix_len)
        d.k_pool = _ptr(k_pool, torch.bfloat16, "k_pool")
        d.v_pool = _ptr(v_pool, torch.bfloat16, "v_pool")
        d.kidx_pool = _ptr(kidx_pool, torch.int8, "kidx_pool")
        d.page_table = _ptr(page_table, torch.int32, "page_table")
        d.seq_lens = _ptr(seq_lens, torch.int32, "seq_lens")
        self.desc = d
        self._keep = (k_pool, v_pool, kidx_pool, page_table, seq_lens)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


# ------------------------------------------------------------------ 1:1 C entry points

def sparse_attn_index(kv: PagedKV, q_idx, q_len, q_tail, scores, score_row_stride, stream=None):
    lib = load()
    _check("sparse_attn_index", lib.sparse_attn_index(
        kv.ref, _ptr(q_idx, torch.int8, "q_idx"), q_len, q_tail, _ptr(scores, torch.int32, "scores"),
        score_row_stride, _stream(stream)))


def sparse_attn_topk_workspace_size(kv: PagedKV, q_len, top_k) -> int:
    return int(load().sparse_attn_topk_workspace_size(kv.ref, q_len, top_k))


def sparse_attn_topk(kv: PagedKV, scores, score_row_stride, q_len, q_tail, top_k, indices,
                     workspace=None, workspace_bytes=0, stream=None):
    lib = load()
    _check("sparse_attn_topk", lib.sparse_attn_topk(
        kv.ref, _ptr(scores, torch.int32, "scores"), score_row_stride, q_len, q_tail, top_k,
        _ptr(indices, torch.int32, "indices"), _ptr(workspace, None, "workspace"), workspace_bytes,
        _stream(stream)))


def sparse_attn_index_topk_workspace_size(kv: PagedKV, q_len, top_k) -> int:
    return int(load().sparse_attn_index_topk_workspace_size(kv.ref, q_len, top_k))


def sparse_attn_index_topk(kv: PagedKV, q_idx, q_len, q_tail, top_k, indices, workspace,
                           workspace_bytes, stream=None):
    lib = load()
    _check("sparse_attn_index_topk", lib.sparse_attn_index_topk(
        kv.ref, _ptr(q_idx, torch.int8, "q_idx"), q_len, q_tail, top_k,
        _ptr(indices, torch.int32, "indices"), _ptr(workspace, None, "workspace"), workspace_bytes,
        _stream(stream)))


def sparse_attn_index_topk_window_workspace_size(kv: PagedKV, q_len, top_k, window) -> int:
    return int(load().sparse_attn_index_topk_window_workspace_size(kv.ref, q_len, top_k, window))


def sparse_attn_index_topk_window(kv: PagedKV, q_idx, q_len, q_tail, top_k, window, indices,
                                  workspace, workspace_bytes, stream=None):
    lib = load()
    _check("sparse_attn_index_topk_window", lib.sparse_attn_index_topk_window(
        kv.ref, _ptr(q_idx, torch.int8, "q_idx"), q_len, q_tail, top_k, window,
        _ptr(indices, torch.int32, "indices"), _ptr(workspace, None, "workspace"), workspace_bytes,
        _stream(stream)))


def sparse_attn_fwd_prefill(kv: PagedKV, q, num_q_heads, q_len, q_tail, indices, index_width,
                            sm_scale, out, lse=None, stream=None):
    lib = load()
    _check("sparse_attn_fwd_prefill", lib.sparse_attn_fwd_prefill(
        kv.ref, _ptr(q, torch.bfloat16, "q"), num_q_heads, q_len, q_tail,
        _ptr(indices, torch.int32, "indices"), index_width, float(sm_scale),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_attn_prefill_masked_workspace_size(kv: PagedKV, q_len) -> int:
    return int(load().sparse_attn_prefill_masked_workspace_size(kv.ref, q_len))


def sparse_attn_fwd_prefill_masked(kv: PagedKV, q, num_q_heads, q_len, q_tail, indices, index_width,
                                   sm_scale, workspace, workspace_bytes, out, lse=None, stream=None):
    lib = load()
    _check("sparse_attn_fwd_prefill_masked", lib.sparse_attn_fwd_prefill_masked(
        kv.ref, _ptr(q, torch.bfloat16, "q"), num_q_heads, q_len, q_tail,
        _ptr(indices, torch.int32, "indices"), index_width, float(sm_scale),
        _ptr(workspace, None, "workspace"), workspace_bytes,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_attn_kv_append(kv: PagedKV, k_new, v_new, kidx_new, n_new, stream=None):
    lib = load()
    _check("sparse_attn_kv_append", lib.sparse_attn_kv_append(
        kv.ref, _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
        _ptr(kidx_new, torch.int8, "kidx_new"), n_new, _stream(stream)))


def kv_append(kv: PagedKV, k_new=None, v_new=None, kidx_new=None, stream=None):
    """Write new tokens into the paged pools: k_new/v_new [B][n][H_kv][d] bf16, kidx_new
    [B][n][H_idx][d_idx] int8 (either may be omitted); positions seq_lens[b] - n + i."""
    ref = k_new if k_new is not None else kidx_new
    n_new = int(ref.shape[1])
    sparse_attn_kv_append(kv, None if k_new is None else k_new.contiguous(),
                          None if v_new is None else v_new.contiguous(),
                          None if kidx_new is None else kidx_new.contiguous(), n_new, stream)


def sparse_attn_kv_alloc(num_maps, num_pages, block_maps, batch, page_size, max_pages_per_seq,
                         old_lens, new_lens, page_tables, status, stream=None):
    lib = load()
    _check("sparse_attn_kv_alloc", lib.sparse_attn_kv_alloc(
        num_maps, num_pages, _ptr(block_maps, torch.int32, "block_maps"), batch, page_size,
        max_pages_per_seq, _ptr(old_lens, torch.int32, "old_lens"),
        _ptr(new_lens, torch.int32, "new_lens"), _ptr(page_tables, torch.int32, "page_tables"),
        _ptr(status, torch.int32, "status"), _stream(stream)))


def sparse_attn_kv_release(num_maps, num_pages, block_maps, batch, page_size, max_pages_per_seq,
                           seq_lens, release, page_tables, stream=None):
    lib = load()
    _check("sparse_attn_kv_release", lib.sparse_attn_kv_release(
        num_maps, num_pages, _ptr(block_maps, torch.int32, "block_maps"), batch, page_size,
        max_pages_per_seq, _ptr(seq_lens, torch.int32, "seq_lens"),
        _ptr(release, torch.int32, "release"), _ptr(page_tables, torch.int32, "page_tables"),
        _stream(stream)))


def kv_alloc(block_maps, page_tables, old_lens, new_lens, page_size, num_pages, stream=None):
    """Grow the caches of every (layer, head) map: block_maps int32 [M][ceil(num_pages/32)]
    (the uint32 bit words, held as int32), page_tables int32 [M][B][max_pages], lengths int32
    [B]. Returns the int32 [M] status (0, the shortfall, or -1; see sparse_attn_kv_alloc)."""
    M, B, max_pages = page_tables.shape
    status = torch.empty(M, dtype=torch.int32, device=page_tables.device)
    sparse_attn_kv_alloc(M, num_pages, block_maps, B, page_size, max_pages, old_lens, new_lens,
                         page_tables, status, stream)
    return status


def kv_release(block_maps, page_tables, seq_lens, release, page_size, num_pages, stream=None):
    """Return the blocks of the sequences flagged in release (int32 [B]) to every map."""
    M, B, max_pages = page_tables.shape
    sparse_attn_kv_release(M, num_pages, block_maps, B, page_size, max_pages, seq_lens, release,
                           page_tables, stream)


def sparse_attn_decode_workspace_size(kv: PagedKV, num_q_heads, index_width, num_splits=0) -> int:
    return int(load().sparse_attn_decode_workspace_size(kv.ref, num_q_heads, index_width, num_splits))


def sparse_attn_fwd_decode(kv: PagedKV, q, num_q_heads, indices, index_width, sm_scale, num_splits,
                           workspace, workspace_bytes, out, lse=None, stream=None):
    lib = load()
    _check("sparse_attn_fwd_decode", lib.sparse_attn_fwd_decode(
        kv.ref, _ptr(q, torch.bfloat16, "q"), num_q_heads, _ptr(indices, torch.int32, "indices"),
        index_width, float(sm_scale), num_splits, _ptr(workspace, None, "workspace"), workspace_bytes,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_attn_decode_noalloc_max_bytes() -> int:
    return int(load().sparse_attn_decode_noalloc_max_bytes())


def sparse_attn_fwd_decode_noalloc(kv: PagedKV, q, num_q_heads, indices, index_width, sm_scale,
                                   num_splits, out, lse=None, stream=None):
    lib = load()
    _check("sparse_attn_fwd_decode_noalloc", lib.sparse_attn_fwd_decode_noalloc(
        kv.ref, _ptr(q, torch.bfloat16, "q"), num_q_heads, _ptr(indices, torch.int32, "indices"),
        index_width, float(sm_scale), num_splits, _ptr(out, torch.bfloat16, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_attn_select_thresholds(kv: PagedKV, q_idx, q_len, q_tail, top_k, thresholds, stream=None):
    lib = load()
    _check("sparse_attn_select_thresholds", lib.sparse_attn_select_thresholds(
        kv.ref, _ptr(q_idx, torch.int8, "q_idx"), q_len, q_tail, top_k,
        _ptr(thresholds, torch.int32, "thresholds"), _stream(stream)))


def sparse_attn_prefill_fused_workspace_size(kv: PagedKV, num_q_heads, q_len, q_tail, top_k,
                                             path=SA_PREFILL_AUTO) -> int:
    return int(load().sparse_attn_prefill_fused_workspace_size(kv.ref, num_q_heads, q_len, q_tail,
                                                               top_k, path))


def sparse_attn_prefill_fused_choice(kv: PagedKV, num_q_heads, q_len, q_tail, top_k) -> int:
    return int(load().sparse_attn_prefill_fused_choice(kv.ref, num_q_heads, q_len, q_tail, top_k))


def sparse_attn_prefill_fused(kv: PagedKV, q, q_idx, num_q_heads, q_len, q_tail, top_k, sm_scale,
                              path, workspace, workspace_bytes, out, lse=None, stream=None):
    lib = load()
    _check("sparse_attn_prefill_fused", lib.sparse_attn_prefill_fused(
        kv.ref, _ptr(q, torch.bfloat16, "q"), _ptr(q_idx, torch.int8, "q_idx"), num_q_heads, q_len,
        q_tail, top_k, float(sm_scale), path, _ptr(workspace, None, "workspace"), workspace_bytes,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream)))


def sparse_attn_validate(kv: PagedKV, indices, index_width, q_len, q_tail, report, stream=None):
    _check("sparse_attn_validate", load().sparse_attn_validate(
        kv.ref, _ptr(indices, torch.int32, "indices"), index_width, q_len, q_tail,
        _ptr(report, torch.int32, "report"), _stream(stream)))


def sparse_attn_check_report(report, stream=None):
    _check("sparse_attn_check_report", load().sparse_attn_check_report(
        _ptr(report, torch.int32, "report"), _stream(stream)))


def sparse_attn_calib_read(buf, sink, workgroups, stream=None):
    _check("sparse_attn_calib_read", load().sparse_attn_calib_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink, torch.int32, "sink"), workgroups,
        _stream(stream)))


def sparse_attn_calib_gather(pool, rows, sink, workgroups, stream=None):
    _check("sparse_attn_calib_gather", load().sparse_attn_calib_gather(
        _ptr(pool), pool.numel() * pool.element_size(), _ptr(rows, torch.int32, "rows"), rows.numel(),
        _ptr(sink, torch.int32, "sink"), workgroups, _stream(stream)))


def sparse_attn_calib_mfma(kind, iters, workgroups, sink, stream=None):
    _check("sparse_attn_calib_mfma", load().sparse_attn_calib_mfma(
        kind, iters, workgroups, _ptr(sink, torch.int32, "sink"), _stream(stream)))


# ------------------------------------------------------------------ allocating helpers

def _row_stride(max_seq_len: int) -> int:
    return (max_seq_len + 3) // 4 * 4


def index(kv: PagedKV, q_idx, q_len, q_tail, scores=None, stream=None):
    """Scores [B][q_len][H_idx][row_stride] int32 (only candidate columns are defined)."""
    d = kv.desc
    stride = _row_stride(d.max_seq_len)
    if scores is None:
        scores = torch.empty((d.batch, q_len, d.num_idx_heads, stride), dtype=torch.int32,
                             device=q_idx.device)
    sparse_attn_index(kv, q_idx, q_len, q_tail, scores, scores.shape[-1], stream)
    return scores


def topk(kv: PagedKV, scores, q_len, q_tail, top_k, indices=None, workspace=None, stream=None):
    d = kv.desc
    width = d.prefix_len + top_k
    if indices is None:
        indices = torch.empty((d.batch, q_len, d.num_idx_heads, width), dtype=torch.int32,
                              device=scores.device)
    need = sparse_attn_topk_workspace_size(kv, q_len, top_k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    sparse_attn_topk(kv, scores, scores.shape[-1], q_len, q_tail, top_k, indices, workspace,
                     0 if workspace is None else workspace.numel() * workspace.element_size(), stream)
    return indices


def index_topk(kv: PagedKV, q_idx, q_len, q_tail, top_k, indices=None, workspace=None,
               stream=None):
    """Fused indexer + top-K: the same lists as topk(index(...)) without score rows."""
    d = kv.desc
    width = d.prefix_len + top_k
    if indices is None:
        indices = torch.empty((d.batch, q_len, d.num_idx_heads, width), dtype=torch.int32,
                              device=q_idx.device)
    need = sparse_attn_index_topk_workspace_size(kv, q_len, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_idx.device)
    sparse_attn_index_topk(kv, q_idx, q_len, q_tail, top_k, indices, workspace,
                           workspace.numel() * workspace.element_size(), stream)
    return indices


def index_topk_window(kv: PagedKV, q_idx, q_len, q_tail, top_k, window, indices=None,
                      workspace=None, stream=None):
    """Hybrid lists: prefix + window forced, top-K over the rest; width P + top_k + window."""
    d = kv.desc
    width = d.prefix_len + top_k + window
    if indices is None:
        indices = torch.empty((d.batch, q_len, d.num_idx_heads, width), dtype=torch.int32,
                              device=q_idx.device)
    need = sparse_attn_index_topk_window_workspace_size(kv, q_len, top_k, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_idx.device)
    sparse_attn_index_topk_window(kv, q_idx, q_len, q_tail, top_k, window, indices, workspace,
                                  workspace.numel() * workspace.element_size(), stream)
    return indices


def prefill(kv: PagedKV, q, q_tail, indices=None, sm_scale=None, out=None, lse=None,
            want_lse=True, stream=None):
    """q [B][q_len][H_q][d] bf16 -> (out, lse). indices=None gives dense causal attention."""
    B, q_len, Hq, D = q.shape
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device=q.device)
    width = 0 if indices is None else int(indices.shape[-1])
    sparse_attn_fwd_prefill(kv, q, Hq, q_len, q_tail, indices, width, sm_scale, out, lse, stream)
    return out, lse


def select_thresholds(kv: PagedKV, q_idx, q_len, q_tail, top_k, thresholds=None, stream=None):
    """Per-row (tau, t_cut): int32 [B][q_len][H_idx][2]."""
    d = kv.desc
    if thresholds is None:
        thresholds = torch.empty((d.batch, q_len, d.num_idx_heads, 2), dtype=torch.int32,
                                 device=q_idx.device)
    sparse_attn_select_thresholds(kv, q_idx, q_len, q_tail, top_k, thresholds, stream)
    return thresholds


def prefill_fused(kv: PagedKV, q, q_idx, q_tail, top_k, sm_scale=None, path=SA_PREFILL_AUTO,
                  out=None, lse=None, workspace=None, want_lse=True, stream=None):
    """Indexer + top-K + attention of a prefill block in one call -> (out, lse)."""
    B, q_len, Hq, D = q.shape
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_prefill_fused_workspace_size(kv, Hq, q_len, q_tail, top_k, path)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    sparse_attn_prefill_fused(kv, q, q_idx, Hq, q_len, q_tail, top_k, sm_scale, path, workspace,
                              workspace.numel() * workspace.element_size(), out, lse, stream)
    return out, lse


def prefill_masked(kv: PagedKV, q, q_tail, indices, sm_scale=None, out=None, lse=None,
                   workspace=None, want_lse=True, stream=None):
    """Sparse prefill on dense matrix tiles: the same result as prefill(..., indices) (each
    listed key counted once), computed over every causal key with the unselected ones masked."""
    B, q_len, Hq, D = q.shape
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_prefill_masked_workspace_size(kv, q_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    sparse_attn_fwd_prefill_masked(kv, q, Hq, q_len, q_tail, indices, int(indices.shape[-1]), sm_scale,
                                   workspace, workspace.numel() * workspace.element_size(), out, lse,
                                   stream)
    return out, lse


def decode(kv: PagedKV, q, indices, sm_scale=None, num_splits=0, out=None, lse=None,
           workspace=None, want_lse=True, stream=None):
    """q [B][H_q][d] bf16, indices [B][H_idx][W] -> (out [B][H_q][d], lse [B][H_q])."""
    B, Hq, D = q.shape
    width = int(indices.shape[-1])
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_decode_workspace_size(kv, Hq, width, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sparse_attn_fwd_decode(kv, q, Hq, indices, width, sm_scale, num_splits, workspace, ws_bytes,
                           out, lse, stream)
    return out, lse
