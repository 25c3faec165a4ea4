// Host side of the C ABI in include/sparse_attn.h: argument validation, then kernel launch.
// Every check runs before anything is enqueued, so an error return launches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "../../include/sparse_attn.h"
#include "sa_common.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

enum Need : unsigned { NEED_KV = 1u, NEED_IDX = 2u };

// Validates the descriptor for the pools a call uses and flattens it.
int32_t check_kv(const sa_paged_kv* kv, unsigned need, sa::KvView* v) {
  if (kv == nullptr) return SA_ERR_NULL;
  if (kv->abi_version != SA_ABI_VERSION) return SA_ERR_ABI;
  if (kv->page_table == nullptr || kv->seq_lens == nullptr) return SA_ERR_NULL;
  if ((need & NEED_KV) && (kv->k_pool == nullptr || kv->v_pool == nullptr)) return SA_ERR_NULL;
  if ((need & NEED_IDX) && kv->kidx_pool == nullptr) return SA_ERR_NULL;
  if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1 || kv->num_pages < 1 ||
      kv->max_seq_len < 1 || kv->prefix_len < 0)
    return SA_ERR_SHAPE;
  if (!pow2(kv->page_size) || kv->page_size < 64 || kv->page_size > (1 << 24))
    return SA_ERR_UNSUPPORTED;
  if ((int64_t)kv->max_seq_len > (int64_t)kv->max_pages_per_seq * kv->page_size) return SA_ERR_SHAPE;
  if (kv->num_pages * (int64_t)kv->page_size > INT32_MAX) return SA_ERR_UNSUPPORTED;  // row ids are int32
  if (kv->num_idx_heads != kv->num_kv_heads && kv->num_idx_heads != 1) return SA_ERR_SHAPE;
  if ((need & NEED_KV) && kv->head_dim != 64 && kv->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if ((need & NEED_IDX) && kv->idx_dim != 32 && kv->idx_dim != 64 && kv->idx_dim != 128)
    return SA_ERR_UNSUPPORTED;
  if (!aligned16(kv->page_table) || !aligned16(kv->seq_lens)) return SA_ERR_ALIGN;
  if ((need & NEED_KV) && (!aligned16(kv->k_pool) || !aligned16(kv->v_pool))) return SA_ERR_ALIGN;
  if ((need & NEED_IDX) && !aligned16(kv->kidx_pool)) return SA_ERR_ALIGN;
  v->k_pool = kv->k_pool;
  v->v_pool = kv->v_pool;
  v->kidx_pool = kv->kidx_pool;
  v->page_table = kv->page_table;
  v->seq_lens = kv->seq_lens;
  v->num_pages = kv->num_pages;
  v->batch = kv->batch;
  v->num_kv_heads = kv->num_kv_heads;
  v->head_dim = kv->head_dim;
  v->num_idx_heads = kv->num_idx_heads;
  v->idx_dim = kv->idx_dim;
  v->page_size = kv->page_size;
  v->page_shift = log2i(kv->page_size);
  v->max_pages_per_seq = kv->max_pages_per_seq;
  v->max_seq_len = kv->max_seq_len;
  v->prefix_len = kv->prefix_len;
  return SA_OK;
}

int32_t check_block(const sa::KvView& v, int32_t q_len, int32_t q_tail) {
  if (q_len < 1 || q_tail < q_len || q_tail > v.max_seq_len) return SA_ERR_SHAPE;
  return SA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

// SPARSE_ATTN_CHECK=1 in the environment: every call first validates the device data it reads
// (sequence lengths, page-table entries, the index lists it takes) into the library's report,
// read back with sparse_attn_check_report.
bool check_mode() {
  const char* e = std::getenv("SPARSE_ATTN_CHECK");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

int32_t checked(const sa::KvView& v, const int32_t* lists, int width, int q_len, int q_tail,
                hipStream_t s) {
  if (!check_mode()) return SA_OK;
  int32_t* report = nullptr;
  if (sa::check_report_ptr(&report, s) != hipSuccess) return SA_ERR_HIP;
  return hip_status(sa::launch_check(v, lists, width, q_len, q_tail, report, s));
}

}  // namespace

extern "C" {

int32_t sparse_attn_abi_version(void) { return SA_ABI_VERSION; }

const char* sparse_attn_status_string(int32_t status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "a required pointer is NULL";
    case SA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case SA_ERR_UNSUPPORTED: return "size not supported by the kernels";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP runtime rejected a launch";
    case SA_ERR_ABI: return "descriptor ABI version mismatch";
    case SA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SA_ERR_SCRATCH: return "call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int32_t sparse_attn_index(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                          int32_t q_tail, int32_t* scores, int64_t score_row_stride,
                          void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, NEED_IDX, &v);
  if (st != SA_OK) return st;
  if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
  if (q_idx == nullptr || scores == nullptr) return SA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(scores)) return SA_ERR_ALIGN;
  if (score_row_stride < v.max_seq_len || (score_row_stride & 3) != 0) return SA_ERR_SHAPE;
  if ((st = checked(v, nullptr, 0, q_len, q_tail, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_index(v, q_idx, q_len, q_tail, scores, score_row_stride,
                                     static_cast<hipStream_t>(stream)));
}

size_t sparse_attn_topk_workspace_size(const sa_paged_kv* kv, int32_t q_len, int32_t top_k) {
  sa::KvView v;
  if (check_kv(kv, 0, &v) != SA_OK || q_len < 1 || top_k < 1) return 0;
  return sa::topk_workspace_bytes(v, q_len, top_k);
}

int32_t sparse_attn_topk(const sa_paged_kv* kv, const int32_t* scores, int64_t score_row_stride,
                         int32_t q_len, int32_t q_tail, int32_t top_k, int32_t* indices,
                         void* workspace, size_t workspace_bytes, void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, 0, &v);
  if (st != SA_OK) return st;
  if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
  if (scores == nullptr || indices == nullptr) return SA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(indices)) return SA_ERR_ALIGN;
  if (top_k < 1 || (int64_t)top_k + v.prefix_len > (1 << 30)) return SA_ERR_SHAPE;
  if (score_row_stride < v.max_seq_len || (score_row_stride & 3) != 0) return SA_ERR_SHAPE;
  const size_t need = sa::topk_workspace_bytes(v, q_len, top_k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return SA_ERR_ALIGN;
  if ((st = checked(v, nullptr, 0, q_len, q_tail, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_topk(v, scores, score_row_stride, q_len, q_tail, top_k, indices,
                                    workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

namespace {

int64_t score_stride(const sa::KvView& v) { return ((int64_t)v.max_seq_len + 3) & ~(int64_t)3; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the two-step fallback: score rows, then the selection workspace.
size_t composite_bytes(const sa::KvView& v, int32_t q_len, int32_t top_k) {
  const size_t scores = (size_t)v.batch * q_len * v.num_idx_heads * score_stride(v) * sizeof(int32_t);
  return align256(scores) + sa::topk_workspace_bytes(v, q_len, top_k);
}

}  // namespace

namespace {

size_t index_topk_bytes(const sa::KvView& v, int32_t q_len, int32_t top_k) {
  if (sa::fused_applies(v, q_len)) return sa::fused_workspace_bytes(v);
  return composite_bytes(v, q_len, top_k);
}

// The selection of sparse_attn_index_topk on a validated descriptor and workspace.
int32_t index_topk_run(const sa::KvView& v, const int8_t* q_idx, int32_t q_len, int32_t q_tail,
                       int32_t top_k, int32_t* indices, void* workspace, hipStream_t s) {
  if (sa::fused_applies(v, q_len))
    return hip_status(sa::launch_index_topk_fused(v, q_idx, q_tail, top_k, indices, workspace, s));
  if (sa::topk_coarse_applies(v, q_len)) {
    // many-query blocks of rows up to 32K: 16-bit keys (half the traffic of int32 scores) in the
    // score space of the workspace, row stride a multiple of 8 keys
    uint16_t* keys = static_cast<uint16_t*>(workspace);
    const int64_t kstride = ((int64_t)v.max_seq_len + 7) & ~(int64_t)7;
    hipError_t e = sa::launch_index_coarse(v, q_idx, q_len, q_tail, keys, kstride, s);
    if (e != hipSuccess) return SA_ERR_HIP;
    return hip_status(sa::launch_topk_coarse(v, keys, kstride, q_len, q_tail, top_k, q_idx, indices, s));
  }
  int32_t* scores = static_cast<int32_t*>(workspace);
  const int64_t stride = score_stride(v);
  void* tk_ws = static_cast<char*>(workspace) +
                align256((size_t)v.batch * q_len * v.num_idx_heads * stride * sizeof(int32_t));
  hipError_t e = sa::launch_index(v, q_idx, q_len, q_tail, scores, stride, s);
  if (e != hipSuccess) return SA_ERR_HIP;
  return hip_status(sa::launch_topk(v, scores, stride, q_len, q_tail, top_k, indices, tk_ws,
                                    sa::topk_workspace_bytes(v, q_len, top_k), s));
}

// Checks shared by the selection entry points; on success *need is the workspace size.
int32_t check_index_topk(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len, int32_t q_tail,
                         int32_t top_k, int64_t extra_width, const int32_t* indices, sa::KvView* v) {
  int32_t st = check_kv(kv, NEED_IDX, v);
  if (st != SA_OK) return st;
  if ((st = check_block(*v, q_len, q_tail)) != SA_OK) return st;
  if (q_idx == nullptr || indices == nullptr) return SA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(indices)) return SA_ERR_ALIGN;
  if (top_k < 1 || (int64_t)top_k + v->prefix_len + extra_width > (1 << 30)) return SA_ERR_SHAPE;
  return SA_OK;
}

}  // namespace

size_t sparse_attn_index_topk_workspace_size(const sa_paged_kv* kv, int32_t q_len, int32_t top_k) {
  sa::KvView v;
  if (check_kv(kv, NEED_IDX, &v) != SA_OK || q_len < 1 || top_k < 1) return 0;
  return index_topk_bytes(v, q_len, top_k);
}

int32_t sparse_attn_index_topk(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                               int32_t q_tail, int32_t top_k, int32_t* indices, void* workspace,
                               size_t workspace_bytes, void* stream) {
  sa::KvView v;
  int32_t st = check_index_topk(kv, q_idx, q_len, q_tail, top_k, 0, indices, &v);
  if (st != SA_OK) return st;
  const size_t need = index_topk_bytes(v, q_len, top_k);
  if (workspace == nullptr || workspace_bytes < need) return SA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SA_ERR_ALIGN;
  if ((st = checked(v, nullptr, 0, q_len, q_tail, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return index_topk_run(v, q_idx, q_len, q_tail, top_k, indices, workspace,
                        static_cast<hipStream_t>(stream));
}

namespace {

// Workspace of the hybrid selection: shortened lengths, the shortened lists, the selection's own.
size_t window_bytes(const sa::KvView& v, int32_t q_len, int32_t top_k) {
  const size_t rows = (size_t)v.batch * q_len * v.num_idx_heads;
  return align256((size_t)v.batch * sizeof(int32_t)) +
         align256(rows * ((size_t)v.prefix_len + top_k) * sizeof(int32_t)) +
         index_topk_bytes(v, q_len, top_k);
}

}  // namespace

size_t sparse_attn_index_topk_window_workspace_size(const sa_paged_kv* kv, int32_t q_len,
                                                    int32_t top_k, int32_t window) {
  sa::KvView v;
  if (check_kv(kv, NEED_IDX, &v) != SA_OK || q_len < 1 || top_k < 1 || window < 0) return 0;
  return window_bytes(v, q_len, top_k);
}

int32_t sparse_attn_index_topk_window(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                                      int32_t q_tail, int32_t top_k, int32_t window,
                                      int32_t* indices, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  sa::KvView v;
  if (window < 0) return SA_ERR_SHAPE;
  int32_t st = check_index_topk(kv, q_idx, q_len, q_tail, top_k, window, indices, &v);
  if (st != SA_OK) return st;
  const size_t need = window_bytes(v, q_len, top_k);
  if (workspace == nullptr || workspace_bytes < need) return SA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SA_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = checked(v, nullptr, 0, q_len, q_tail, s)) != SA_OK) return st;
  const size_t rows = (size_t)v.batch * q_len * v.num_idx_heads;
  char* base = static_cast<char*>(workspace);
  int32_t* short_lens = reinterpret_cast<int32_t*>(base);
  int32_t* lists = reinterpret_cast<int32_t*>(base + align256((size_t)v.batch * sizeof(int32_t)));
  void* inner = base + align256((size_t)v.batch * sizeof(int32_t)) +
                align256(rows * ((size_t)v.prefix_len + top_k) * sizeof(int32_t));
  if (sa::launch_window_lens(v, window, short_lens, s) != hipSuccess) return SA_ERR_HIP;
  sa::KvView vs = v;
  vs.seq_lens = short_lens;
  if ((st = index_topk_run(vs, q_idx, q_len, q_tail, top_k, lists, inner, s)) != SA_OK) return st;
  return hip_status(sa::launch_window_finish(v, short_lens, q_len, q_tail, top_k, window, lists,
                                             indices, s));
}

int32_t sparse_attn_fwd_prefill(const sa_paged_kv* kv, const uint16_t* q, int32_t num_q_heads,
                                int32_t q_len, int32_t q_tail, const int32_t* indices,
                                int32_t index_width, float sm_scale, uint16_t* out, float* lse,
                                void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, NEED_KV, &v);
  if (st != SA_OK) return st;
  if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
  if (q == nullptr || out == nullptr) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (lse != nullptr && !aligned16(lse))) return SA_ERR_ALIGN;
  if (num_q_heads < 1 || num_q_heads % v.num_kv_heads != 0) return SA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f) return SA_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (indices == nullptr) {
    if ((st = checked(v, nullptr, 0, q_len, q_tail, s)) != SA_OK) return st;
    return hip_status(sa::launch_attn_dense(v, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, s));
  }
  const int group = num_q_heads / v.num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return SA_ERR_UNSUPPORTED;
  if (index_width < 1) return SA_ERR_SHAPE;
  if (!aligned16(indices)) return SA_ERR_ALIGN;
  if ((st = checked(v, indices, index_width, q_len, q_tail, s)) != SA_OK) return st;
  return hip_status(sa::launch_attn_sparse_mfma(v, q, num_q_heads, q_len, q_tail, indices,
                                                index_width, sm_scale, out, lse, s));
}

int32_t sparse_attn_select_thresholds(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                                      int32_t q_tail, int32_t top_k, int32_t* thresholds,
                                      void* stream) {
  sa::KvView v;
  int32_t st = check_index_topk(kv, q_idx, q_len, q_tail, top_k, 0, thresholds, &v);
  if (st != SA_OK) return st;
  if (!sa::sel_thresh_applies(v)) return SA_ERR_UNSUPPORTED;
  if ((st = checked(v, nullptr, 0, q_len, q_tail, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_sel_thresh(v, q_idx, q_len, q_tail, top_k, thresholds, nullptr,
                                          static_cast<hipStream_t>(stream)));
}

namespace {

// Average number of candidate keys of a query of the block, from the host-side length bound.
double mean_candidates(const sa::KvView& v, int32_t q_len, int32_t q_tail) {
  const double first = (double)v.max_seq_len - q_tail;  // position of the block's first query
  return first + (q_len - 1) * 0.5 + 1.0 - v.prefix_len;
}

// Path of sparse_attn_prefill_fused: masked-dense tiles when top_k is a large enough share of
// the block's mean candidate count, else gathered rows. Measured on MI355X (32K context, blocks
// of 128, 512 and 2048 queries at five positions, top-K 32..2048, short blocks with key splits):
// the two paths cost the same at a share of about 1/20 for every block size (between 0.042 and
// 0.056 for 2048 queries, about 0.06 for 512 and 128); blocks under 64 queries would leave most
// of a 256-query tile empty and stay on gathered rows.
constexpr double kMaskedMinShare = 1.0 / 20.0;

int32_t fused_path(const sa::KvView& v, int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                   int32_t top_k, int32_t path) {
  const int group = num_q_heads / v.num_kv_heads;
  const bool gather_ok = group == 1 || group == 2 || group == 4 || group == 8;
  const bool masked_ok = sa::sel_thresh_applies(v);
  if (path == SA_PREFILL_GATHER) return gather_ok ? SA_PREFILL_GATHER : -1;
  if (path == SA_PREFILL_MASKED) return masked_ok ? SA_PREFILL_MASKED : -1;
  if (!masked_ok) return gather_ok ? SA_PREFILL_GATHER : -1;
  if (!gather_ok) return SA_PREFILL_MASKED;
  const bool dense_enough = (double)top_k >= kMaskedMinShare * mean_candidates(v, q_len, q_tail);
  return (dense_enough && q_len >= 64) ? SA_PREFILL_MASKED : SA_PREFILL_GATHER;
}

// Masked path: thresholds, selection records, then (short blocks) the key-split partials.
size_t fused_bytes(const sa::KvView& v, int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                   int32_t top_k, int32_t chosen) {
  const size_t rows = (size_t)v.batch * q_len * v.num_idx_heads;
  if (chosen == SA_PREFILL_MASKED)
    return align256(rows * 2 * sizeof(int32_t)) + align256(sa::sel_workspace_bytes(v, q_len)) +
           sa::dense_split_bytes(v, num_q_heads, q_len, sa::dense_splits(v, num_q_heads, q_len, q_tail));
  return align256(rows * ((size_t)v.prefix_len + top_k) * sizeof(int32_t)) + index_topk_bytes(v, q_len, top_k);
}

}  // namespace

size_t sparse_attn_prefill_fused_workspace_size(const sa_paged_kv* kv, int32_t num_q_heads,
                                                int32_t q_len, int32_t q_tail, int32_t top_k,
                                                int32_t path) {
  sa::KvView v;
  if (check_kv(kv, NEED_KV | NEED_IDX, &v) != SA_OK || q_len < 1 || top_k < 1) return 0;
  if (num_q_heads < 1 || num_q_heads % v.num_kv_heads != 0 || q_tail < q_len) return 0;
  if (path != SA_PREFILL_AUTO && path != SA_PREFILL_GATHER && path != SA_PREFILL_MASKED) return 0;
  const int32_t chosen = fused_path(v, num_q_heads, q_len, q_tail, top_k, path);
  return chosen < 0 ? 0 : fused_bytes(v, num_q_heads, q_len, q_tail, top_k, chosen);
}

int32_t sparse_attn_prefill_fused_choice(const sa_paged_kv* kv, int32_t num_q_heads, int32_t q_len,
                                         int32_t q_tail, int32_t top_k) {
  sa::KvView v;
  if (check_kv(kv, NEED_KV | NEED_IDX, &v) != SA_OK || q_len < 1 || top_k < 1) return -1;
  if (num_q_heads < 1 || num_q_heads % v.num_kv_heads != 0 || q_tail < q_len) return -1;
  return fused_path(v, num_q_heads, q_len, q_tail, top_k, SA_PREFILL_AUTO);
}

int32_t sparse_attn_prefill_fused(const sa_paged_kv* kv, const uint16_t* q, const int8_t* q_idx,
                                  int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                                  int32_t top_k, float sm_scale, int32_t path, void* workspace,
                                  size_t workspace_bytes, uint16_t* out, float* lse, void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, NEED_KV | NEED_IDX, &v);
  if (st != SA_OK) return st;
  if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
  if (q == nullptr || q_idx == nullptr || out == nullptr) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(q_idx) || !aligned16(out) || (lse != nullptr && !aligned16(lse)))
    return SA_ERR_ALIGN;
  if (num_q_heads < 1 || num_q_heads % v.num_kv_heads != 0) return SA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f) return SA_ERR_SHAPE;
  if (top_k < 1 || (int64_t)top_k + v.prefix_len > (1 << 30)) return SA_ERR_SHAPE;
  if (path != SA_PREFILL_AUTO && path != SA_PREFILL_GATHER && path != SA_PREFILL_MASKED)
    return SA_ERR_SHAPE;
  const int32_t chosen = fused_path(v, num_q_heads, q_len, q_tail, top_k, path);
  if (chosen < 0) return SA_ERR_UNSUPPORTED;
  const size_t need = fused_bytes(v, num_q_heads, q_len, q_tail, top_k, chosen);
  if (workspace == nullptr || workspace_bytes < need) return SA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SA_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = checked(v, nullptr, 0, q_len, q_tail, s)) != SA_OK) return st;
  char* base = static_cast<char*>(workspace);
  const size_t rows = (size_t)v.batch * q_len * v.num_idx_heads;
  if (chosen == SA_PREFILL_MASKED) {
    int32_t* thr = reinterpret_cast<int32_t*>(base);
    const size_t sel_off = align256(rows * 2 * sizeof(int32_t));
    uint64_t* sel = reinterpret_cast<uint64_t*>(base + sel_off);
    float* part = reinterpret_cast<float*>(base + sel_off + align256(sa::sel_workspace_bytes(v, q_len)));
    const int splits = sa::dense_splits(v, num_q_heads, q_len, q_tail);
    if (sa::launch_sel_thresh(v, q_idx, q_len, q_tail, top_k, thr, sel, s) != hipSuccess) return SA_ERR_HIP;
    return hip_status(sa::launch_attn_masked_records(v, q, num_q_heads, q_len, q_tail, sm_scale, sel,
                                                     splits, part, out, lse, s));
  }
  const int32_t width = v.prefix_len + top_k;
  int32_t* lists = reinterpret_cast<int32_t*>(base);
  void* inner = base + align256(rows * (size_t)width * sizeof(int32_t));
  if ((st = index_topk_run(v, q_idx, q_len, q_tail, top_k, lists, inner, s)) != SA_OK) return st;
  return hip_status(sa::launch_attn_sparse_mfma(v, q, num_q_heads, q_len, q_tail, lists, width,
                                                sm_scale, out, lse, s));
}

size_t sparse_attn_prefill_masked_workspace_size(const sa_paged_kv* kv, int32_t q_len) {
  sa::KvView v;
  if (check_kv(kv, 0, &v) != SA_OK || q_len < 1) return 0;
  return sa::sel_workspace_bytes(v, q_len);
}

int32_t sparse_attn_fwd_prefill_masked(const sa_paged_kv* kv, const uint16_t* q,
                                       int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                                       const int32_t* indices, int32_t index_width, float sm_scale,
                                       void* workspace, size_t workspace_bytes, uint16_t* out,
                                       float* lse, void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, NEED_KV, &v);
  if (st != SA_OK) return st;
  if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
  if (q == nullptr || out == nullptr || indices == nullptr) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(indices) || (lse != nullptr && !aligned16(lse)))
    return SA_ERR_ALIGN;
  if (num_q_heads < 1 || num_q_heads % v.num_kv_heads != 0) return SA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f) return SA_ERR_SHAPE;
  if (index_width < 1) return SA_ERR_SHAPE;
  const size_t need = sa::sel_workspace_bytes(v, q_len);
  if (workspace == nullptr || workspace_bytes < need) return SA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SA_ERR_ALIGN;
  if ((st = checked(v, indices, index_width, q_len, q_tail, static_cast<hipStream_t>(stream))) != SA_OK)
    return st;
  return hip_status(sa::launch_attn_masked(v, q, num_q_heads, q_len, q_tail, indices, index_width,
                                           sm_scale, workspace, out, lse,
                                           static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_kv_append(const sa_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new,
                              const int8_t* kidx_new, int32_t n_new, void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return SA_ERR_NULL;
  if (k_new == nullptr && kidx_new == nullptr) return SA_ERR_NULL;
  sa::KvView v;
  const unsigned need = (k_new != nullptr ? NEED_KV : 0u) | (kidx_new != nullptr ? NEED_IDX : 0u);
  int32_t st = check_kv(kv, need, &v);
  if (st != SA_OK) return st;
  if (n_new < 1 || n_new > v.max_seq_len) return SA_ERR_SHAPE;
  if ((k_new != nullptr && (!aligned16(k_new) || !aligned16(v_new))) ||
      (kidx_new != nullptr && !aligned16(kidx_new)))
    return SA_ERR_ALIGN;
  if ((st = checked(v, nullptr, 0, 1, 1, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_kv_append(v, k_new, v_new, kidx_new, n_new,
                                         static_cast<hipStream_t>(stream)));
}

namespace {

int32_t check_block_maps(int32_t num_maps, int32_t num_pages, int32_t batch, int32_t page_size,
                         int32_t max_pages_per_seq) {
  if (num_maps < 1 || num_maps > 65535 || num_pages < 1 || batch < 1 ||
      batch > sa::kAllocMaxBatch || page_size < 1 || max_pages_per_seq < 1)
    return SA_ERR_SHAPE;
  if ((int64_t)batch * max_pages_per_seq > INT32_MAX) return SA_ERR_SHAPE;
  return SA_OK;
}

}  // namespace

int32_t sparse_attn_kv_alloc(int32_t num_maps, int32_t num_pages, uint32_t* block_maps,
                             int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                             const int32_t* old_lens, const int32_t* new_lens,
                             int32_t* page_tables, int32_t* status, void* stream) {
  if (!block_maps || !old_lens || !new_lens || !page_tables || !status) return SA_ERR_NULL;
  const int32_t st = check_block_maps(num_maps, num_pages, batch, page_size, max_pages_per_seq);
  if (st != SA_OK) return st;
  if (!aligned16(block_maps) || !aligned16(old_lens) || !aligned16(new_lens) ||
      !aligned16(page_tables) || !aligned16(status))
    return SA_ERR_ALIGN;
  return hip_status(sa::launch_kv_alloc(num_maps, num_pages, block_maps, batch, page_size,
                                        max_pages_per_seq, old_lens, new_lens, page_tables, status,
                                        static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_kv_release(int32_t num_maps, int32_t num_pages, uint32_t* block_maps,
                               int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, const int32_t* release,
                               int32_t* page_tables, void* stream) {
  if (!block_maps || !seq_lens || !release || !page_tables) return SA_ERR_NULL;
  const int32_t st = check_block_maps(num_maps, num_pages, batch, page_size, max_pages_per_seq);
  if (st != SA_OK) return st;
  if (!aligned16(block_maps) || !aligned16(seq_lens) || !aligned16(release) ||
      !aligned16(page_tables))
    return SA_ERR_ALIGN;
  return hip_status(sa::launch_kv_release(num_maps, num_pages, block_maps, batch, page_size,
                                          max_pages_per_seq, seq_lens, release, page_tables,
                                          static_cast<hipStream_t>(stream)));
}

size_t sparse_attn_decode_workspace_size(const sa_paged_kv* kv, int32_t num_q_heads,
                                         int32_t index_width, int32_t num_splits) {
  sa::KvView v;
  if (check_kv(kv, 0, &v) != SA_OK || num_q_heads < 1 || index_width < 1) return 0;
  if (num_q_heads % v.num_kv_heads != 0 || (v.head_dim != 64 && v.head_dim != 128)) return 0;
  if (num_splits < 0 || num_splits > 256) return 0;
  const int64_t units = (int64_t)v.batch * v.num_kv_heads;
  int splits = num_splits > 0 ? num_splits
                             : sa::auto_splits(units, index_width, v.head_dim, num_q_heads / v.num_kv_heads);
  if (splits > index_width) splits = index_width;
  return sa::gather_workspace_bytes(units, num_q_heads / v.num_kv_heads, v.head_dim, splits);
}

namespace {

// Checks shared by the decode entry points; on success *splits and *need are the split count
// and the partials' size in bytes.
int32_t check_decode(const sa_paged_kv* kv, const uint16_t* q, int32_t num_q_heads,
                     const int32_t* indices, int32_t index_width, float sm_scale,
                     int32_t num_splits, const uint16_t* out, const float* lse, sa::KvView* v,
                     int* splits, size_t* need) {
  int32_t st = check_kv(kv, NEED_KV, v);
  if (st != SA_OK) return st;
  if (q == nullptr || out == nullptr || indices == nullptr) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(indices) || (lse != nullptr && !aligned16(lse)))
    return SA_ERR_ALIGN;
  if (num_q_heads < 1 || num_q_heads % v->num_kv_heads != 0) return SA_ERR_SHAPE;
  const int group = num_q_heads / v->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return SA_ERR_UNSUPPORTED;
  if (index_width < 1 || num_splits < 0 || num_splits > 256) return SA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f) return SA_ERR_SHAPE;
  const int64_t units = (int64_t)v->batch * v->num_kv_heads;
  int sp = num_splits > 0 ? num_splits : sa::auto_splits(units, index_width, v->head_dim, group);
  if (sp > index_width) sp = index_width;
  *splits = sp;
  *need = sa::gather_workspace_bytes(units, group, v->head_dim, sp);
  return SA_OK;
}

}  // namespace

int32_t sparse_attn_fwd_decode(const sa_paged_kv* kv, const uint16_t* q, int32_t num_q_heads,
                               const int32_t* indices, int32_t index_width, float sm_scale,
                               int32_t num_splits, void* workspace, size_t workspace_bytes,
                               uint16_t* out, float* lse, void* stream) {
  sa::KvView v;
  int splits = 0;
  size_t need = 0;
  int32_t st = check_decode(kv, q, num_q_heads, indices, index_width, sm_scale, num_splits, out,
                            lse, &v, &splits, &need);
  if (st != SA_OK) return st;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return SA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SA_ERR_ALIGN;
  }
  if ((st = checked(v, indices, index_width, 1, 1, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_attn_gather(v, q, num_q_heads, 1, 1, indices, index_width, sm_scale,
                                           splits, static_cast<float*>(workspace), out, lse,
                                           static_cast<hipStream_t>(stream)));
}

size_t sparse_attn_decode_noalloc_max_bytes(void) { return sa::kDecodeScratchBytes; }

int32_t sparse_attn_fwd_decode_noalloc(const sa_paged_kv* kv, const uint16_t* q,
                                       int32_t num_q_heads, const int32_t* indices,
                                       int32_t index_width, float sm_scale, int32_t num_splits,
                                       uint16_t* out, float* lse, void* stream) {
  sa::KvView v;
  int splits = 0;
  size_t need = 0;
  int32_t st = check_decode(kv, q, num_q_heads, indices, index_width, sm_scale, num_splits, out,
                            lse, &v, &splits, &need);
  if (st != SA_OK) return st;
  if (need > sa::kDecodeScratchBytes) return SA_ERR_SCRATCH;
  float* scratch = nullptr;
  if (need > 0 && sa::decode_scratch(&scratch) != hipSuccess) return SA_ERR_HIP;
  if ((st = checked(v, indices, index_width, 1, 1, static_cast<hipStream_t>(stream))) != SA_OK) return st;
  return hip_status(sa::launch_attn_gather(v, q, num_q_heads, 1, 1, indices, index_width, sm_scale,
                                           splits, scratch, out, lse,
                                           static_cast<hipStream_t>(stream)));
}

size_t sparse_attn_workspace_size(int32_t op, const sa_paged_kv* kv, int32_t q_len, int32_t q_tail,
                                  int32_t top_k, int32_t num_q_heads, int32_t extra) {
  switch (op) {
    case SA_OP_TOPK: return sparse_attn_topk_workspace_size(kv, q_len, top_k);
    case SA_OP_INDEX_TOPK: return sparse_attn_index_topk_workspace_size(kv, q_len, top_k);
    case SA_OP_INDEX_TOPK_WINDOW: return sparse_attn_index_topk_window_workspace_size(kv, q_len, top_k, extra);
    case SA_OP_PREFILL_MASKED: return sparse_attn_prefill_masked_workspace_size(kv, q_len);
    case SA_OP_PREFILL_FUSED:
      return sparse_attn_prefill_fused_workspace_size(kv, num_q_heads, q_len, q_tail, top_k, extra);
    case SA_OP_DECODE: return sparse_attn_decode_workspace_size(kv, num_q_heads, top_k, extra);
    default: return 0;
  }
}

int32_t sparse_attn_validate(const sa_paged_kv* kv, const int32_t* indices, int32_t index_width,
                             int32_t q_len, int32_t q_tail, int32_t* report, void* stream) {
  sa::KvView v;
  int32_t st = check_kv(kv, 0, &v);
  if (st != SA_OK) return st;
  if (report == nullptr) return SA_ERR_NULL;
  if (!aligned16(report)) return SA_ERR_ALIGN;
  if (indices != nullptr) {
    if ((st = check_block(v, q_len, q_tail)) != SA_OK) return st;
    if (index_width < 1) return SA_ERR_SHAPE;
    if (!aligned16(indices)) return SA_ERR_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (sa::launch_check_reset(report, s) != hipSuccess) return SA_ERR_HIP;
  return hip_status(sa::launch_check(v, indices, indices != nullptr ? index_width : 0, q_len, q_tail,
                                     report, s));
}

int32_t sparse_attn_check_report(int32_t* report, void* stream) {
  if (report == nullptr) return SA_ERR_NULL;
  if (!aligned16(report)) return SA_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* lib_report = nullptr;
  if (sa::check_report_ptr(&lib_report, s) != hipSuccess) return SA_ERR_HIP;
  return hip_status(sa::launch_check_copy_reset(lib_report, report, s));
}

int32_t sparse_attn_calib_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                               void* stream) {
  if (buf == nullptr || sink == nullptr) return SA_ERR_NULL;
  if (!aligned16(buf) || (bytes & 15) != 0) return SA_ERR_ALIGN;
  if (bytes < 16 || workgroups < 1 || workgroups > 65536) return SA_ERR_SHAPE;
  return hip_status(sa::launch_calib_read(buf, bytes, sink, workgroups, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_calib_gather(const void* pool, size_t pool_bytes, const int32_t* rows,
                                 int64_t n_rows, uint32_t* sink, int32_t workgroups, void* stream) {
  if (pool == nullptr || rows == nullptr || sink == nullptr) return SA_ERR_NULL;
  if (!aligned16(pool) || !aligned16(rows) || (pool_bytes & 255) != 0) return SA_ERR_ALIGN;
  if (pool_bytes < 256 || n_rows < 1 || workgroups < 1 || workgroups > 65536) return SA_ERR_SHAPE;
  return hip_status(sa::launch_calib_gather(pool, pool_bytes, rows, n_rows, sink, workgroups,
                                            static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_calib_mfma(int32_t kind, int32_t iters, int32_t workgroups, uint32_t* sink,
                               void* stream) {
  if (sink == nullptr) return SA_ERR_NULL;
  if ((kind != 0 && kind != 1) || iters < 1 || workgroups < 1 || workgroups > 65536) return SA_ERR_SHAPE;
  return hip_status(sa::launch_calib_mfma(kind, iters, workgroups, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
