// Hybrid index lists: a local window of the most recent keys next to the global top-K.
//
// [MTT-page] = "…在摩尔线程MTT S5000上的原生推理优化实践" (blog.csdn.net) §2.3: hybrid attention
// combines global sparse attention with local sliding-window attention. [DSA-page] =
// "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.4: forced keys bypass the
// screening.
//
// A query at position pos always attends to the window pos - window + 1 .. pos (clipped at 0)
// and to the forced prefix; the top-K runs over the causal keys outside both. Since the window
// holds the highest positions, that selection is the ordinary one for a query at pos - window:
// the selection kernels run unchanged on a copy of the sequence lengths shortened by the window,
// and k_window_finish appends the window to each list (ascending order is kept: every window
// key lies above every selected key).
#include "sa_common.h"

namespace sa {
namespace {

__global__ void k_window_lens(const int32_t* __restrict__ seq_lens, int32_t* __restrict__ out, int batch,
                              int window, int max_seq_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) out[b] = max(min(seq_lens[b], max_seq_len) - window, 0);
}

// One workgroup per (sequence, query, indexer head) row: the row of the shortened selection
// (width P + K, its valid entries first) is copied, the window keys follow, -1 pads to P + K +
// window.
__global__ __launch_bounds__(256) void k_window_finish(KvView kv, const int32_t* __restrict__ short_lens,
                                                       int q_len, int q_tail, int top_k, int window,
                                                       const int32_t* __restrict__ lists,
                                                       int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const int64_t bi = row / kv.num_idx_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int P = kv.prefix_len;
  const int W1 = P + top_k, W2 = W1 + window;
  const int pos = min(kv.seq_lens[b], kv.max_seq_len) - q_tail + i;
  const int pos_s = short_lens[b] - q_tail + i;  // the position the selection ran at
  int nvalid = 0;
  if (pos_s >= 0) nvalid = min(P, pos_s + 1) + min(top_k, max(pos_s - P + 1, 0));
  const int lo = max(0, pos_s + 1);               // first window key
  const int nw = pos >= lo ? pos - lo + 1 : 0;
  const int32_t* src = lists + row * (int64_t)W1;
  int32_t* dst = out + row * (int64_t)W2;
  for (int j = threadIdx.x; j < W2; j += 256) {
    int v = -1;
    if (j < nvalid) v = src[j];
    else if (j < nvalid + nw) v = lo + (j - nvalid);
    dst[j] = v;
  }
}

}  // namespace

hipError_t launch_window_lens(const KvView& kv, int window, int32_t* short_lens, hipStream_t stream) {
  hipLaunchKernelGGL(k_window_lens, dim3((kv.batch + 255) / 256), dim3(256), 0, stream, kv.seq_lens,
                     short_lens, kv.batch, window, kv.max_seq_len);
  return hipGetLastError();
}

hipError_t launch_window_finish(const KvView& kv, const int32_t* short_lens, int q_len, int q_tail,
                                int top_k, int window, const int32_t* lists, int32_t* indices,
                                hipStream_t stream) {
  const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_window_finish, dim3((unsigned)rows), dim3(256), 0, stream, kv, short_lens, q_len,
                     q_tail, top_k, window, lists, indices);
  return hipGetLastError();
}

}  // namespace sa
