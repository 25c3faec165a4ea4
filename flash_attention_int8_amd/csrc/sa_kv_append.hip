// KV-cache append: new tokens' K, V and indexer-key rows written into the paged pools.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析":
//   §2.2  the cache is kept in fixed blocks of contiguous tokens, found through a block table;
//   §2.3  each decode step adds the new token to the cache before selection and attention.
//
// One workgroup per (sequence, new token). Token i of sequence b sits at position
// seq_lens[b] - n_new + i (the lengths already count the new tokens) and lands in physical
// page page_table[b][pos >> page_shift] at slot pos & (page_size - 1). Every row is copied
// with 16-byte loads and stores: per KV head one K and one V row (d bf16 each), per indexer
// head one d_idx-byte row. Positions below 0, past max_seq_len, or whose page entry is outside
// [0, num_pages) are skipped.
#include "sa_common.h"

namespace sa {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void k_kv_append(KvView kv, uint16_t* __restrict__ k_pool,
                                                             uint16_t* __restrict__ v_pool,
                                                             int8_t* __restrict__ kidx_pool,
                                                             const uint16_t* __restrict__ k_new,
                                                             const uint16_t* __restrict__ v_new,
                                                             const int8_t* __restrict__ kidx_new,
                                                             int n_new) {
  const int64_t bi = blockIdx.x;  // b * n_new + i
  const int b = (int)(bi / n_new);
  const int i = (int)(bi - (int64_t)b * n_new);
  const int pos = min(kv.seq_lens[b], kv.max_seq_len) - n_new + i;
  if (pos < 0 || pos >= kv.max_seq_len) return;
  const int lp = pos >> kv.page_shift;
  if (lp >= kv.max_pages_per_seq) return;
  const int64_t ph = kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
  if (ph < 0 || ph >= kv.num_pages) return;
  const int slot = pos & (kv.page_size - 1);
  const int H = kv.num_kv_heads, D = kv.head_dim;
  const int cpr = D / 8;  // 16-byte chunks per K or V row
  if (k_pool != nullptr) {
    for (int c = threadIdx.x; c < 2 * H * cpr; c += kAppendThreads) {
      const int which = c / (H * cpr);  // 0: K, 1: V
      const int r = c - which * H * cpr;
      const int h = r / cpr, part = r - h * cpr;
      const uint16_t* src = (which ? v_new : k_new) + (bi * H + h) * (int64_t)D + part * 8;
      uint16_t* dst = (which ? v_pool : k_pool) +
                      ((ph * H + h) * kv.page_size + slot) * (int64_t)D + part * 8;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
  if (kidx_pool != nullptr) {
    const int Hi = kv.num_idx_heads, Di = kv.idx_dim, cpi = Di / 16;
    for (int c = threadIdx.x; c < Hi * cpi; c += kAppendThreads) {
      const int h = c / cpi, part = c - h * cpi;
      const int8_t* src = kidx_new + (bi * Hi + h) * (int64_t)Di + part * 16;
      int8_t* dst = kidx_pool + ((ph * Hi + h) * kv.page_size + slot) * (int64_t)Di + part * 16;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const KvView& kv, const uint16_t* k_new, const uint16_t* v_new,
                            const int8_t* kidx_new, int n_new, hipStream_t stream) {
  const int64_t wgs = (int64_t)kv.batch * n_new;
  if (wgs == 0) return hipSuccess;
  // the descriptor's pools are the caller's writable device memory; K/V are written when new
  // K/V rows are given, indexer keys when new indexer rows are given
  uint16_t* kp = k_new != nullptr ? const_cast<uint16_t*>(kv.k_pool) : nullptr;
  uint16_t* vp = k_new != nullptr ? const_cast<uint16_t*>(kv.v_pool) : nullptr;
  int8_t* ip = kidx_new != nullptr ? const_cast<int8_t*>(kv.kidx_pool) : nullptr;
  hipLaunchKernelGGL(k_kv_append, dim3((unsigned)wgs), dim3(kAppendThreads), 0, stream, kv, kp, vp, ip,
                     k_new, v_new, kidx_new, n_new);
  return hipGetLastError();
}

}  // namespace sa
