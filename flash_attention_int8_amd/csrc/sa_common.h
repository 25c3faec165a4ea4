// Internal helpers shared by the gfx950 kernels and the host layer of the sparse-attention
// library. Not part of the public ABI (include/sparse_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// The descriptor after host-side validation, flattened into kernel arguments.
struct KvView {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int8_t* kidx_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int64_t num_pages;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_idx_heads;
  int32_t idx_dim;
  int32_t page_size;
  int32_t page_shift;  // log2(page_size)
  int32_t max_pages_per_seq;
  int32_t max_seq_len;
  int32_t prefix_len;
};

// Physical page of token t of sequence b, or -1 when the table entry is out of range.
__device__ __forceinline__ int64_t phys_page(const KvView& kv, int b, int t) {
  const int lp = t >> kv.page_shift;
  if (lp < 0 || lp >= kv.max_pages_per_seq) return -1;
  const int64_t p = kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
  return (p >= 0 && p < kv.num_pages) ? p : -1;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two bf16 packed in a 32-bit word -> floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;

// fp32 -> bf16 bits, round to nearest even (the compiler emits v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_v v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// DPP lane moves (within rows of 16 lanes).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16); every lane of a group gets the sum.
template <int N>
__device__ __forceinline__ int group_sum_i(int v) {
  if constexpr (N >= 2) v += dpp_i<DPP_QUAD_XOR1>(v);
  if constexpr (N >= 4) v += dpp_i<DPP_QUAD_XOR2>(v);
  if constexpr (N >= 8) v += dpp_i<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_i<DPP_ROW_MIRROR>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum_f(float v) {
  if constexpr (N >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
  if constexpr (N >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
  if constexpr (N >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The values of a lane pair {l, l ^ M}, lower lane first, in both lanes of the pair: row
// rotation by 8 inside 16-lane rows (M = 8), self-swap of odd and even 16-lane rows (M = 16)
// or of the two 32-lane halves (M = 32). VALU only (no LDS round trip); both lanes get the
// same ordered pair, so anything computed from it is identical in both.
struct FPair {
  float lo, hi;
};
template <int M>
__device__ __forceinline__ FPair lane_pair(float x) {
  static_assert(M == 8 || M == 16 || M == 32, "lane_pair supports M = 8, 16, 32");
  if constexpr (M == 8) {
    const float o = __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x128, 0xf, 0xf, false));
    const bool upper = (__lane_id() & 8) != 0;
    return FPair{upper ? o : x, upper ? x : o};
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return FPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return FPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
  }
}

}  // namespace sa

// Kernel launchers (defined in the .hip files; return hipSuccess or the launch error).
namespace sa {
hipError_t launch_index(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                        int32_t* scores, int64_t row_stride, hipStream_t stream);
hipError_t launch_topk(const KvView& kv, const int32_t* scores, int64_t row_stride, int q_len,
                       int q_tail, int top_k, int32_t* indices, void* ws, size_t ws_bytes,
                       hipStream_t stream);
size_t topk_workspace_bytes(const KvView& kv, int q_len, int top_k);
hipError_t launch_attn_gather(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                              int q_tail, const int32_t* indices, int index_width, float sm_scale,
                              int num_splits, float* ws, uint16_t* out, float* lse,
                              hipStream_t stream);
size_t gather_workspace_bytes(int64_t units, int group, int head_dim, int num_splits);
// Merge of split partials ([unit][split][G][D] accumulators, then [unit][split][G][2] (max in
// exp2 units, sum)) into out and lse; unit = (row, KV head), G = num_q_heads / num_kv_heads.
hipError_t launch_merge_splits(const float* ws, int64_t units, int num_splits, int num_q_heads,
                               int num_kv_heads, int head_dim, uint16_t* out, float* lse,
                               hipStream_t stream);
int auto_splits(int64_t units, int index_width, int head_dim, int group);
// Static split-partials buffer of sparse_attn_fwd_decode_noalloc: its size, and its device
// address on the current device (looked up once per device, no allocation).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(float** ptr);
bool fused_applies(const KvView& kv, int q_len);
size_t fused_workspace_bytes(const KvView& kv);
hipError_t launch_index_topk_fused(const KvView& kv, const int8_t* q_idx, int q_tail, int top_k,
                                   int32_t* indices, void* ws, hipStream_t stream);
hipError_t launch_attn_sparse_mfma(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                                   int q_tail, const int32_t* indices, int index_width,
                                   float sm_scale, uint16_t* out, float* lse, hipStream_t stream);
hipError_t launch_attn_dense(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                             int q_tail, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t stream);
// Fused prefill selection on 16-bit order-preserving indexer keys (exact: ties in a key are
// settled by recomputed int8 scores).
hipError_t launch_index_coarse(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                               uint16_t* keys, int64_t row_stride, hipStream_t stream);
bool topk_coarse_applies(const KvView& kv, int q_len);
hipError_t launch_topk_coarse(const KvView& kv, const uint16_t* keys, int64_t row_stride, int q_len,
                              int q_tail, int top_k, const int8_t* q_idx, int32_t* indices,
                              hipStream_t stream);
// Hybrid index lists (local window + global top-K): shortened lengths, then the window appended.
hipError_t launch_window_lens(const KvView& kv, int window, int32_t* short_lens, hipStream_t stream);
hipError_t launch_window_finish(const KvView& kv, const int32_t* short_lens, int q_len, int q_tail,
                                int top_k, int window, const int32_t* lists, int32_t* indices,
                                hipStream_t stream);
// KV-cache append: new tokens' rows written into the paged pools.
hipError_t launch_kv_append(const KvView& kv, const uint16_t* k_new, const uint16_t* v_new,
                            const int8_t* kidx_new, int n_new, hipStream_t stream);
// KV-cache block allocator: per-(layer, head) block maps, allocation and release.
constexpr int kAllocMaxBatch = 8192;  // sequences per allocation call (offsets held in LDS)
int map_words(int num_pages);
hipError_t launch_kv_alloc(int num_maps, int num_pages, uint32_t* maps, int batch, int page_size,
                           int max_pages, const int32_t* old_lens, const int32_t* new_lens,
                           int32_t* tables, int32_t* status, hipStream_t stream);
hipError_t launch_kv_release(int num_maps, int num_pages, uint32_t* maps, int batch, int page_size,
                             int max_pages, const int32_t* seq_lens, const int32_t* release,
                             int32_t* tables, hipStream_t stream);
// Masked-dense sparse prefill: selection masks built from index lists in the workspace, then
// the dense kernel with every unselected score set to -inf.
int sel_query_blocks(int q_len);
int sel_tiles(const KvView& kv);
size_t sel_workspace_bytes(const KvView& kv, int q_len);
hipError_t launch_attn_masked(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                              int q_tail, const int32_t* indices, int index_width, float sm_scale,
                              void* ws, uint16_t* out, float* lse, hipStream_t stream);
// The masked-dense attention on selection masks already in `sel` (sel_workspace_bytes), with
// its causal key tiles split among num_splits workgroups per query block when num_splits > 1
// (part: dense_split_bytes of split partials, merged by launch_merge_splits).
int dense_splits(const KvView& kv, int num_q_heads, int q_len, int q_tail);
size_t dense_split_bytes(const KvView& kv, int num_q_heads, int q_len, int num_splits);
hipError_t launch_attn_masked_records(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                                      int q_tail, float sm_scale, const uint64_t* sel, int num_splits,
                                      float* part, uint16_t* out, float* lse, hipStream_t stream);
// Per-row selection thresholds (tau, t_cut) from recomputed indexer scores, and optionally the
// masked-dense attention's selection masks written from them (sel: sel_workspace_bytes or NULL).
bool sel_thresh_applies(const KvView& kv);
hipError_t launch_sel_thresh(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail, int top_k,
                             int32_t* thresholds, uint64_t* sel, hipStream_t stream);
// Validation of device-side contents (sequence lengths, page-table entries, index lists) into
// an int32 [kReportWords] report; the SPARSE_ATTN_CHECK mode adds to a report of the library.
constexpr int kReportWords = 8;
hipError_t launch_check(const KvView& kv, const int32_t* indices, int index_width, int q_len, int q_tail,
                        int32_t* report, hipStream_t stream);
hipError_t launch_check_reset(int32_t* report, hipStream_t stream);
hipError_t launch_check_copy_reset(int32_t* report, int32_t* out, hipStream_t stream);
hipError_t check_report_ptr(int32_t** ptr, hipStream_t stream);
// Roofline micro-benchmarks (streaming read, random 256-byte row gather, MFMA loops).
hipError_t launch_calib_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                             hipStream_t stream);
hipError_t launch_calib_gather(const void* pool, size_t pool_bytes, const int32_t* rows, int64_t n_rows,
                               uint32_t* sink, int workgroups, hipStream_t stream);
hipError_t launch_calib_mfma(int kind, int iters, int workgroups, uint32_t* sink, hipStream_t stream);
}  // namespace sa
