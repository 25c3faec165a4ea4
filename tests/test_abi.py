"""The C ABI without a GPU: the library loads, exports every declared symbol, the ctypes
descriptor matches the C struct, and invalid arguments return their documented status
before anything is launched.

Every validation case below carries at least one invalid argument, so no call here ever
reaches a kernel launch (the fake device addresses are never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import pytest

import flash_attention_int8_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sparse_attn_\w+)", out))
    assert set(names) <= exported
    for n in names:
        assert hasattr(lib, n)


def test_abi_version_and_status_strings(lib):
    assert lib.sparse_attn_abi_version() == fa.SA_ABI_VERSION == 1
    for code in range(9):
        assert lib.sparse_attn_status_string(code) != b"unknown status"
    assert lib.sparse_attn_status_string(0) == b"ok"
    assert lib.sparse_attn_status_string(99) == b"unknown status"


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in fa.sa_paged_kv._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(sa_paged_kv, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sparse_attn.h"\n'
                   "int main(void) {\n" + body + '\n  printf("size %zu\\n", sizeof(sa_paged_kv));\n'
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(fa.sa_paged_kv, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(fa.sa_paged_kv)


# ----------------------------------------------------------------------------- validation

A = 0x7f0000000000  # a 16-byte aligned fake device address; never dereferenced


def desc(**over):
    d = fa.sa_paged_kv()
    vals = dict(abi_version=1, batch=2, num_kv_heads=8, head_dim=128, num_idx_heads=8, idx_dim=64,
                page_size=64, max_pages_per_seq=16, num_pages=32, max_seq_len=1024, prefix_len=0,
                k_pool=A, v_pool=A + 0x1000, kidx_pool=A + 0x2000, page_table=A + 0x3000,
                seq_lens=A + 0x4000)
    vals.update(over)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


def call_index(lib, d, q_idx=A, q_len=1, q_tail=1, scores=A, stride=1024):
    return lib.sparse_attn_index(ctypes.byref(d) if d is not None else None, q_idx, q_len, q_tail,
                                 scores, stride, None)


def call_topk(lib, d, scores=A, stride=1024, q_len=1, q_tail=1, k=64, idx=A, ws=None, ws_bytes=0):
    return lib.sparse_attn_topk(ctypes.byref(d), scores, stride, q_len, q_tail, k, idx, ws, ws_bytes, None)


def call_prefill(lib, d, q=A, hq=32, q_len=16, q_tail=16, idx=A, width=64, out=A, lse=None, scale=0.1):
    return lib.sparse_attn_fwd_prefill(ctypes.byref(d), q, hq, q_len, q_tail, idx, width, scale, out, lse, None)


def call_masked(lib, d, q=A, hq=32, q_len=16, q_tail=16, idx=A, width=64, ws=A, ws_bytes=1 << 30,
                out=A, lse=None, scale=0.1):
    return lib.sparse_attn_fwd_prefill_masked(ctypes.byref(d), q, hq, q_len, q_tail, idx, width, scale,
                                              ws, ws_bytes, out, lse, None)


@pytest.mark.parametrize("case,code", [
    (dict(q=None), fa.SA_ERR_NULL),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(out=None), fa.SA_ERR_NULL),
    (dict(d=desc(k_pool=None)), fa.SA_ERR_NULL),
    (dict(hq=12), fa.SA_ERR_SHAPE),                      # not a multiple of H_kv = 8
    (dict(width=0), fa.SA_ERR_SHAPE),
    (dict(scale=0.0), fa.SA_ERR_SHAPE),
    (dict(scale=float("nan")), fa.SA_ERR_SHAPE),
    (dict(q_len=17, q_tail=16), fa.SA_ERR_SHAPE),
    (dict(ws=None), fa.SA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), fa.SA_ERR_WORKSPACE),
    (dict(ws=A + 8), fa.SA_ERR_ALIGN),
    (dict(idx=A + 4), fa.SA_ERR_ALIGN),
    (dict(d=desc(head_dim=96)), fa.SA_ERR_UNSUPPORTED),
])
def test_prefill_masked_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_masked(lib, d, **case) == code


def test_prefill_masked_workspace_size(lib):
    d = desc()  # B=2, H_idx=8, max_seq_len=1024 -> 16 tiles
    for q_len, blocks in [(1, 1), (256, 1), (257, 2), (1000, 4)]:
        want = 2 * 8 * 8 * blocks * 16 * 256
        assert lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(d), q_len) == want
    assert lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(d), 0) == 0
    d1 = desc(num_idx_heads=1)
    assert lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(d1), 256) == 2 * 8 * 16 * 256


def call_window(lib, d, q_idx=A, q_len=1, q_tail=1, k=64, window=16, idx=A, ws=A, ws_bytes=1 << 30):
    return lib.sparse_attn_index_topk_window(ctypes.byref(d), q_idx, q_len, q_tail, k, window, idx,
                                             ws, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    (dict(window=-1), fa.SA_ERR_SHAPE),
    (dict(k=0), fa.SA_ERR_SHAPE),
    (dict(window=1 << 30), fa.SA_ERR_SHAPE),
    (dict(q_idx=None), fa.SA_ERR_NULL),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(ws=None), fa.SA_ERR_WORKSPACE),
    (dict(ws_bytes=64), fa.SA_ERR_WORKSPACE),
    (dict(ws=A + 4), fa.SA_ERR_ALIGN),
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),
    (dict(q_len=2, q_tail=1), fa.SA_ERR_SHAPE),
])
def test_index_topk_window_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_window(lib, d, **case) == code


def test_index_topk_window_workspace_grows_with_the_lists(lib):
    d = desc()
    plain = lib.sparse_attn_index_topk_workspace_size(ctypes.byref(d), 1, 64)
    w = lib.sparse_attn_index_topk_window_workspace_size(ctypes.byref(d), 1, 64, 16)
    assert w >= plain + 2 * 8 * 64 * 4  # the shortened lists (B=2, H_idx=8, P+K=64)
    assert lib.sparse_attn_index_topk_window_workspace_size(ctypes.byref(d), 1, 64, -1) == 0


def call_append(lib, d, k=A, v=A + 0x100, ki=A + 0x200, n=4):
    return lib.sparse_attn_kv_append(ctypes.byref(d), k, v, ki, n, None)


@pytest.mark.parametrize("case,code", [
    (dict(v=None), fa.SA_ERR_NULL),                       # K without V
    (dict(k=None), fa.SA_ERR_NULL),                       # V without K
    (dict(k=None, v=None, ki=None), fa.SA_ERR_NULL),      # nothing to write
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),       # indexer rows but no indexer pool
    (dict(d=desc(k_pool=None)), fa.SA_ERR_NULL),
    (dict(n=0), fa.SA_ERR_SHAPE),
    (dict(n=1025), fa.SA_ERR_SHAPE),                      # more than max_seq_len
    (dict(k=A + 2), fa.SA_ERR_ALIGN),
    (dict(ki=A + 8), fa.SA_ERR_ALIGN),
    (dict(d=desc(head_dim=96)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(idx_dim=48)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(abi_version=3)), fa.SA_ERR_ABI),
])
def test_kv_append_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_append(lib, d, **case) == code


def call_alloc(lib, maps=8, pages=1000, bm=A, batch=4, ps=64, mp=16, old=A + 0x100, new=A + 0x200,
               tab=A + 0x300, st=A + 0x400):
    return lib.sparse_attn_kv_alloc(maps, pages, bm, batch, ps, mp, old, new, tab, st, None)


def call_release(lib, maps=8, pages=1000, bm=A, batch=4, ps=64, mp=16, lens=A + 0x100, rel=A + 0x200,
                 tab=A + 0x300):
    return lib.sparse_attn_kv_release(maps, pages, bm, batch, ps, mp, lens, rel, tab, None)


@pytest.mark.parametrize("case,code", [
    (dict(bm=None), fa.SA_ERR_NULL),
    (dict(old=None), fa.SA_ERR_NULL),
    (dict(new=None), fa.SA_ERR_NULL),
    (dict(tab=None), fa.SA_ERR_NULL),
    (dict(st=None), fa.SA_ERR_NULL),
    (dict(maps=0), fa.SA_ERR_SHAPE),
    (dict(maps=65536), fa.SA_ERR_SHAPE),
    (dict(pages=0), fa.SA_ERR_SHAPE),
    (dict(batch=0), fa.SA_ERR_SHAPE),
    (dict(batch=8193), fa.SA_ERR_SHAPE),
    (dict(ps=0), fa.SA_ERR_SHAPE),
    (dict(mp=0), fa.SA_ERR_SHAPE),
    (dict(batch=8192, mp=1 << 18), fa.SA_ERR_SHAPE),     # batch * max_pages reaches 2^31
    (dict(bm=A + 4), fa.SA_ERR_ALIGN),
    (dict(tab=A + 0x308), fa.SA_ERR_ALIGN),
    (dict(st=A + 0x404), fa.SA_ERR_ALIGN),
])
def test_kv_alloc_validation(lib, case, code):
    assert call_alloc(lib, **case) == code


@pytest.mark.parametrize("case,code", [
    (dict(bm=None), fa.SA_ERR_NULL),
    (dict(lens=None), fa.SA_ERR_NULL),
    (dict(rel=None), fa.SA_ERR_NULL),
    (dict(tab=None), fa.SA_ERR_NULL),
    (dict(maps=0), fa.SA_ERR_SHAPE),
    (dict(pages=-5), fa.SA_ERR_SHAPE),
    (dict(batch=9000), fa.SA_ERR_SHAPE),
    (dict(mp=-1), fa.SA_ERR_SHAPE),
    (dict(rel=A + 0x204), fa.SA_ERR_ALIGN),
])
def test_kv_release_validation(lib, case, code):
    assert call_release(lib, **case) == code


def call_decode(lib, d, q=A, hq=32, idx=A, width=2048, splits=4, ws=A, ws_bytes=1 << 30, out=A, lse=None,
                scale=0.1):
    return lib.sparse_attn_fwd_decode(ctypes.byref(d), q, hq, idx, width, scale, splits, ws, ws_bytes,
                                      out, lse, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=None), fa.SA_ERR_NULL),
    (dict(d=desc(abi_version=2)), fa.SA_ERR_ABI),
    (dict(d=desc(page_table=None)), fa.SA_ERR_NULL),
    (dict(d=desc(seq_lens=None)), fa.SA_ERR_NULL),
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),
    (dict(q_idx=None), fa.SA_ERR_NULL),
    (dict(scores=None), fa.SA_ERR_NULL),
    (dict(d=desc(idx_dim=48)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(page_size=96)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(page_size=32)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(num_idx_heads=3)), fa.SA_ERR_SHAPE),
    (dict(d=desc(batch=0)), fa.SA_ERR_SHAPE),
    (dict(d=desc(max_seq_len=1025)), fa.SA_ERR_SHAPE),    # more than 16 pages x 64
    (dict(d=desc(prefix_len=-1)), fa.SA_ERR_SHAPE),
    (dict(q_len=0), fa.SA_ERR_SHAPE),
    (dict(q_len=4, q_tail=3), fa.SA_ERR_SHAPE),
    (dict(q_tail=1025), fa.SA_ERR_SHAPE),
    (dict(stride=1000), fa.SA_ERR_SHAPE),
    (dict(stride=1026), fa.SA_ERR_SHAPE),                   # not a multiple of 4
    (dict(scores=A + 4), fa.SA_ERR_ALIGN),
    (dict(d=desc(kidx_pool=A + 8)), fa.SA_ERR_ALIGN),
    (dict(d=desc(page_table=A + 4)), fa.SA_ERR_ALIGN),
])
def test_index_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_index(lib, d, **case) == code


@pytest.mark.parametrize("case,code", [
    (dict(k=0), fa.SA_ERR_SHAPE),
    (dict(scores=None), fa.SA_ERR_NULL),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(idx=A + 4), fa.SA_ERR_ALIGN),
    (dict(stride=512), fa.SA_ERR_SHAPE),
    (dict(q_len=2, q_tail=1), fa.SA_ERR_SHAPE),
])
def test_topk_validation(lib, case, code):
    assert call_topk(lib, desc(), **case) == code


@pytest.mark.parametrize("case,code", [
    (dict(d=desc(head_dim=96)), fa.SA_ERR_UNSUPPORTED),
    (dict(d=desc(k_pool=None)), fa.SA_ERR_NULL),
    (dict(d=desc(v_pool=None)), fa.SA_ERR_NULL),
    (dict(q=None), fa.SA_ERR_NULL),
    (dict(out=None), fa.SA_ERR_NULL),
    (dict(hq=30), fa.SA_ERR_SHAPE),                          # not a multiple of H_kv
    (dict(hq=24), fa.SA_ERR_UNSUPPORTED),                    # group of 3, sparse path
    (dict(hq=128), fa.SA_ERR_UNSUPPORTED),                   # group of 16, sparse path
    (dict(width=0), fa.SA_ERR_SHAPE),
    (dict(q=A + 2), fa.SA_ERR_ALIGN),
    (dict(out=A + 8), fa.SA_ERR_ALIGN),
    (dict(lse=A + 4), fa.SA_ERR_ALIGN),
    (dict(q_len=16, q_tail=2000), fa.SA_ERR_SHAPE),
    (dict(scale=0.0), fa.SA_ERR_SHAPE),
    (dict(scale=-0.5), fa.SA_ERR_SHAPE),
    (dict(idx=None, scale=float("nan")), fa.SA_ERR_SHAPE),
])
def test_prefill_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_prefill(lib, d, **case) == code


@pytest.mark.parametrize("case,code", [
    (dict(splits=-1), fa.SA_ERR_SHAPE),
    (dict(splits=257), fa.SA_ERR_SHAPE),
    (dict(ws=None), fa.SA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.SA_ERR_WORKSPACE),
    (dict(ws=A + 4), fa.SA_ERR_ALIGN),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(hq=24), fa.SA_ERR_UNSUPPORTED),
    (dict(width=0), fa.SA_ERR_SHAPE),
    (dict(d=desc(head_dim=32)), fa.SA_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), fa.SA_ERR_SHAPE),
])
def test_decode_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_decode(lib, d, **case) == code


def test_decode_workspace_size(lib):
    d = desc()
    # explicit splits: units (B * H_kv) * splits * G * (d + 2) floats
    assert lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 32, 2048, 4) == 2 * 8 * 4 * 4 * 130 * 4
    assert lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 32, 2048, 1) == 0
    # more splits than list entries are clamped to one entry per split
    assert lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 32, 3, 16) == 2 * 8 * 3 * 4 * 130 * 4
    auto = lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 32, 2048, 0)
    assert auto > 0 and auto % (2 * 8 * 4 * 130 * 4) == 0
    assert lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 30, 2048, 0) == 0


def call_decode_noalloc(lib, d, q=A, hq=32, idx=A, width=2048, splits=4, out=A, lse=None, scale=0.1):
    return lib.sparse_attn_fwd_decode_noalloc(None if d is None else ctypes.byref(d), q, hq, idx, width,
                                              scale, splits, out, lse, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=None), fa.SA_ERR_NULL),
    (dict(d=desc(abi_version=2)), fa.SA_ERR_ABI),
    (dict(splits=-1), fa.SA_ERR_SHAPE),
    (dict(splits=257), fa.SA_ERR_SHAPE),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(out=A + 8), fa.SA_ERR_ALIGN),
    (dict(hq=24), fa.SA_ERR_UNSUPPORTED),
    (dict(width=0), fa.SA_ERR_SHAPE),
    (dict(scale=float("nan")), fa.SA_ERR_SHAPE),
    # partials beyond the 16 MiB static buffer: 32 units x 256 splits x 4 heads x 130 floats
    (dict(d=desc(batch=4), splits=256), fa.SA_ERR_SCRATCH),
    (dict(d=desc(batch=64), width=4096, splits=64), fa.SA_ERR_SCRATCH),
])
def test_decode_noalloc_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_decode_noalloc(lib, d, **case) == code


def test_decode_noalloc_buffer_size(lib):
    cap = lib.sparse_attn_decode_noalloc_max_bytes()
    assert cap == 16 << 20
    d = desc(batch=4)
    need = lib.sparse_attn_decode_workspace_size(ctypes.byref(d), 32, 2048, 256)
    assert need > cap   # the SA_ERR_SCRATCH cases above really are over the limit
    d64 = desc(batch=64)
    assert lib.sparse_attn_decode_workspace_size(ctypes.byref(d64), 32, 4096, 64) > cap


def call_thresholds(lib, d, q_idx=A, q_len=16, q_tail=16, k=64, thr=A):
    return lib.sparse_attn_select_thresholds(None if d is None else ctypes.byref(d), q_idx, q_len, q_tail,
                                             k, thr, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=None), fa.SA_ERR_NULL),
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),
    (dict(q_idx=None), fa.SA_ERR_NULL),
    (dict(thr=None), fa.SA_ERR_NULL),
    (dict(thr=A + 4), fa.SA_ERR_ALIGN),
    (dict(k=0), fa.SA_ERR_SHAPE),
    (dict(q_len=17, q_tail=16), fa.SA_ERR_SHAPE),
    (dict(d=desc(idx_dim=48)), fa.SA_ERR_UNSUPPORTED),
    # more than 131072 tokens: the per-tile tie counts would not fit the workgroup's LDS
    (dict(d=desc(max_pages_per_seq=4096, max_seq_len=131073, num_pages=8192)), fa.SA_ERR_UNSUPPORTED),
])
def test_select_thresholds_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_thresholds(lib, d, **case) == code


def call_fused(lib, d, q=A, q_idx=A + 0x100, hq=32, q_len=16, q_tail=16, k=64, scale=0.1, path=0,
               ws=A, ws_bytes=1 << 34, out=A, lse=None):
    return lib.sparse_attn_prefill_fused(None if d is None else ctypes.byref(d), q, q_idx, hq, q_len,
                                         q_tail, k, scale, path, ws, ws_bytes, out, lse, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=None), fa.SA_ERR_NULL),
    (dict(d=desc(k_pool=None)), fa.SA_ERR_NULL),
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),
    (dict(q=None), fa.SA_ERR_NULL),
    (dict(q_idx=None), fa.SA_ERR_NULL),
    (dict(out=None), fa.SA_ERR_NULL),
    (dict(q=A + 2), fa.SA_ERR_ALIGN),
    (dict(hq=30), fa.SA_ERR_SHAPE),
    (dict(k=0), fa.SA_ERR_SHAPE),
    (dict(scale=0.0), fa.SA_ERR_SHAPE),
    (dict(path=3), fa.SA_ERR_SHAPE),
    (dict(ws=None), fa.SA_ERR_WORKSPACE),
    (dict(ws_bytes=64), fa.SA_ERR_WORKSPACE),
    (dict(ws=A + 8), fa.SA_ERR_ALIGN),
    (dict(hq=24, path=fa.SA_PREFILL_GATHER), fa.SA_ERR_UNSUPPORTED),    # group of 3: no gathered kernel
    (dict(d=desc(max_pages_per_seq=4096, max_seq_len=131073, num_pages=8192), path=fa.SA_PREFILL_MASKED),
     fa.SA_ERR_UNSUPPORTED),
])
def test_prefill_fused_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_fused(lib, d, **case) == code


def test_prefill_fused_dispatch_and_workspace(lib):
    d = desc(max_pages_per_seq=512, max_seq_len=32768, num_pages=1024)
    ch = lambda q_len, q_tail, k, hq=32: lib.sparse_attn_prefill_fused_choice(ctypes.byref(d), hq, q_len, q_tail, k)
    # a 2048-query block of a 32K prefill with top-2048: masked tiles at the start and the end
    assert ch(2048, 32768, 2048) == fa.SA_PREFILL_MASKED
    assert ch(2048, 2048, 2048) == fa.SA_PREFILL_MASKED
    # a small top-K far into a long context, or a short block: gathered rows
    assert ch(2048, 2048, 256) == fa.SA_PREFILL_GATHER
    assert ch(16, 16, 2048) == fa.SA_PREFILL_GATHER
    # a group of 3 has no gathered kernel: masked whatever the density
    assert ch(16, 16, 64, hq=24) == fa.SA_PREFILL_MASKED
    # more than 131072 tokens: no masked path
    dl = desc(max_pages_per_seq=4096, max_seq_len=200000, num_pages=8192)
    assert lib.sparse_attn_prefill_fused_choice(ctypes.byref(dl), 32, 2048, 2048, 2048) == fa.SA_PREFILL_GATHER
    ws = lambda q_len, q_tail, k, path: lib.sparse_attn_prefill_fused_workspace_size(ctypes.byref(d), 32, q_len,
                                                                                     q_tail, k, path)
    rows = 2 * 2048 * 8
    masked = ws(2048, 2048, 2048, fa.SA_PREFILL_MASKED)
    assert masked >= rows * 8 + lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(d), 2048)
    assert ws(2048, 2048, 2048, fa.SA_PREFILL_GATHER) >= rows * 2048 * 4
    assert ws(2048, 2048, 2048, fa.SA_PREFILL_AUTO) == masked
    assert ws(2048, 2048, 2048, 9) == 0   # not a path


def _align256(n):
    return (n + 255) // 256 * 256


def test_prefill_fused_crossover_and_key_splits(lib):
    """The measured crossover: masked tiles from top_k = 1/20 of the block's mean candidate
    count (here the last 2048-query block of 32768 tokens: 31744.5 candidates, so 1587.2), for
    blocks of 64 queries and more. The masked path's workspace holds the thresholds, the
    selection records and, for a block whose workgroups (one per 256 queries and query head)
    would leave CUs idle, the partial results of its key splits: up to 256 / workgroups
    splits of at least 8 key tiles each, at most 64."""
    d = desc(max_pages_per_seq=512, max_seq_len=32768, num_pages=1024)
    ch = lambda q_len, q_tail, k: lib.sparse_attn_prefill_fused_choice(ctypes.byref(d), 32, q_len, q_tail, k)
    assert ch(2048, 2048, 1587) == fa.SA_PREFILL_GATHER
    assert ch(2048, 2048, 1588) == fa.SA_PREFILL_MASKED
    assert ch(64, 64, 32768) == fa.SA_PREFILL_MASKED
    assert ch(63, 63, 32768) == fa.SA_PREFILL_GATHER
    for q_len, splits in ((2048, 1), (1024, 1), (512, 2), (128, 4), (64, 4)):
        # workgroups: ceil(q_len / 256) query blocks x batch 2 x 32 query heads
        wgs = -(-q_len // 256) * 2 * 32
        assert splits == max(1, min(256 // wgs, 512 // 8, 64))
        got = lib.sparse_attn_prefill_fused_workspace_size(ctypes.byref(d), 32, q_len, q_len, 2048,
                                                           fa.SA_PREFILL_MASKED)
        want = (_align256(2 * q_len * 8 * 2 * 4)
                + _align256(lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(d), q_len)))
        if splits > 1:
            want += 2 * q_len * 32 * splits * (128 + 2) * 4
        assert got == want, (q_len, got, want)
    # a short context: 15 key tiles, too few for two splits of at least 8
    ds = desc(max_pages_per_seq=64, max_seq_len=960, num_pages=256)
    got = lib.sparse_attn_prefill_fused_workspace_size(ctypes.byref(ds), 32, 128, 128, 64, fa.SA_PREFILL_MASKED)
    assert got == (_align256(2 * 128 * 8 * 2 * 4)
                   + _align256(lib.sparse_attn_prefill_masked_workspace_size(ctypes.byref(ds), 128)))


def call_validate(lib, d, idx=A, width=64, q_len=1, q_tail=1, report=A + 0x500):
    return lib.sparse_attn_validate(None if d is None else ctypes.byref(d), idx, width, q_len, q_tail,
                                    report, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=None), fa.SA_ERR_NULL),
    (dict(d=desc(abi_version=3)), fa.SA_ERR_ABI),
    (dict(d=desc(page_table=None)), fa.SA_ERR_NULL),
    (dict(report=None), fa.SA_ERR_NULL),
    (dict(report=A + 4), fa.SA_ERR_ALIGN),
    (dict(idx=A + 4), fa.SA_ERR_ALIGN),
    (dict(width=0), fa.SA_ERR_SHAPE),
    (dict(q_len=3, q_tail=2), fa.SA_ERR_SHAPE),
    (dict(q_tail=1025), fa.SA_ERR_SHAPE),
])
def test_validate_arguments(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_validate(lib, d, **case) == code


def test_check_report_arguments(lib):
    assert lib.sparse_attn_check_report(None, None) == fa.SA_ERR_NULL
    assert lib.sparse_attn_check_report(A + 4, None) == fa.SA_ERR_ALIGN


def test_workspace_size_by_op_equals_the_per_call_functions(lib):
    d = desc(max_pages_per_seq=512, max_seq_len=32768, num_pages=1024)
    r = ctypes.byref(d)
    ws = lambda op, q_len, q_tail, k, hq, extra: lib.sparse_attn_workspace_size(op, r, q_len, q_tail, k, hq, extra)
    assert ws(fa.SA_OP_TOPK, 1, 1, 2048, 32, 0) == lib.sparse_attn_topk_workspace_size(r, 1, 2048)
    assert ws(fa.SA_OP_INDEX_TOPK, 2048, 2048, 2048, 32, 0) == lib.sparse_attn_index_topk_workspace_size(r, 2048, 2048)
    assert ws(fa.SA_OP_INDEX_TOPK_WINDOW, 1, 1, 2048, 32, 512) == \
        lib.sparse_attn_index_topk_window_workspace_size(r, 1, 2048, 512)
    assert ws(fa.SA_OP_PREFILL_MASKED, 2048, 2048, 0, 32, 0) == lib.sparse_attn_prefill_masked_workspace_size(r, 2048)
    for path in (0, 1, 2):
        assert ws(fa.SA_OP_PREFILL_FUSED, 2048, 4096, 2048, 32, path) == \
            lib.sparse_attn_prefill_fused_workspace_size(r, 32, 2048, 4096, 2048, path)
    assert ws(fa.SA_OP_DECODE, 1, 1, 2048, 32, 8) == lib.sparse_attn_decode_workspace_size(r, 32, 2048, 8)
    assert ws(fa.SA_OP_DECODE, 1, 1, 2048, 32, 8) > 0
    assert ws(99, 1, 1, 2048, 32, 0) == 0


def call_index_topk(lib, d, q_idx=A, q_len=1, q_tail=1, k=64, idx=A, ws=A, ws_bytes=1 << 34):
    return lib.sparse_attn_index_topk(ctypes.byref(d), q_idx, q_len, q_tail, k, idx, ws, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    (dict(d=desc(kidx_pool=None)), fa.SA_ERR_NULL),
    (dict(q_idx=None), fa.SA_ERR_NULL),
    (dict(idx=None), fa.SA_ERR_NULL),
    (dict(ws=None), fa.SA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), fa.SA_ERR_WORKSPACE),
    (dict(ws=A + 8), fa.SA_ERR_ALIGN),
    (dict(k=0), fa.SA_ERR_SHAPE),
    (dict(q_len=2, q_tail=1), fa.SA_ERR_SHAPE),
    (dict(d=desc(idx_dim=16)), fa.SA_ERR_UNSUPPORTED),
])
def test_index_topk_validation(lib, case, code):
    case = dict(case)
    d = case.pop("d", desc())
    assert call_index_topk(lib, d, **case) == code


def test_index_topk_workspace_size(lib):
    # short rows: two-step fallback holds the score rows (B * q_len * H_idx * stride ints)
    d = desc()
    assert lib.sparse_attn_index_topk_workspace_size(ctypes.byref(d), 1, 64) >= 2 * 8 * 1024 * 4
    # long decode rows: fused path, candidate slots for every (row, 8192-token chunk)
    d = desc(max_seq_len=131072, max_pages_per_seq=2048, num_pages=4096, batch=2)
    n = lib.sparse_attn_index_topk_workspace_size(ctypes.byref(d), 1, 2048)
    assert n >= 2 * 8 * 16 * 8192 * 8
    assert lib.sparse_attn_index_topk_workspace_size(ctypes.byref(d), 1, 0) == 0
