// Validation of the device-side contents the entry points take on trust: sequence lengths,
// the page-table entries a sequence uses, and index lists. The kernels never read out of bounds
// whatever these hold (bad page ids and list entries are skipped), but the results are then
// unspecified; this check reports such data instead of silently skipping it.
//
// Report (int32 [kReportWords], counts added with atomics, first positions kept with atomicMin):
//   [0] sequence lengths outside [1, max_seq_len]
//   [1] page-table entries, among the pages a sequence's tokens use, outside [0, num_pages)
//   [2] list entries that are neither -1 nor a token in [0, pos] of their query
//   [3] list entries not above the entry before them (lists are ascending, -1 at the end)
//   [4] flat index (b * max_pages_per_seq + p) of the first bad page-table entry, or INT32_MAX
//   [5] flat index of the first bad list entry (row * width + k), or INT32_MAX
//   [6] calls checked
#include <climits>
#include <mutex>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kChkNT = 256;

__device__ __forceinline__ int seq_len_of(const KvView& kv, int b) {
  return min(kv.seq_lens[b], kv.max_seq_len);
}

// grid.x = batch: the length and the page-table entries of sequence b.
__global__ __launch_bounds__(kChkNT) void k_check_pages(KvView kv, int32_t* __restrict__ report) {
  const int b = blockIdx.x;
  const int raw_len = kv.seq_lens[b];
  if (threadIdx.x == 0 && (raw_len < 1 || raw_len > kv.max_seq_len)) atomicAdd(&report[0], 1);
  const int len = max(0, min(raw_len, kv.max_seq_len));
  const int pages = min((len + kv.page_size - 1) >> kv.page_shift, kv.max_pages_per_seq);
  int bad = 0, first = INT_MAX;
  for (int p = threadIdx.x; p < pages; p += kChkNT) {
    const int64_t e = kv.page_table[(int64_t)b * kv.max_pages_per_seq + p];
    if (e < 0 || e >= kv.num_pages) {
      ++bad;
      first = min(first, b * kv.max_pages_per_seq + p);
    }
  }
  if (bad) {
    atomicAdd(&report[1], bad);
    atomicMin(&report[4], first);
  }
}

// grid = (ceil(width / kChkNT), rows): one list entry per thread.
__global__ __launch_bounds__(kChkNT) void k_check_lists(KvView kv, const int32_t* __restrict__ indices,
                                                       int width, int q_len, int q_tail,
                                                       int32_t* __restrict__ report) {
  const int64_t row = blockIdx.y;  // (b * q_len + i) * H_idx + gi
  const int k = blockIdx.x * kChkNT + threadIdx.x;
  if (k >= width) return;
  const int64_t bi = row / kv.num_idx_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int pos = seq_len_of(kv, b) - q_tail + i;
  const int32_t* list = indices + row * width;
  const int t = list[k];
  const int prev = k > 0 ? list[k - 1] : -2;
  const bool out_of_range = t != -1 && (t < 0 || t > pos);
  // ascending: after an entry of -1 only -1 may follow; otherwise each entry exceeds the last
  const bool disorder = k > 0 && ((prev == -1 && t != -1) || (prev != -1 && t != -1 && t <= prev));
  if (out_of_range) atomicAdd(&report[2], 1);
  if (disorder) atomicAdd(&report[3], 1);
  if (out_of_range || disorder) {
    const int64_t flat = row * width + k;
    atomicMin(&report[5], flat < INT_MAX ? (int)flat : INT_MAX);
  }
}

__global__ void k_check_count(int32_t* __restrict__ report) {
  if (threadIdx.x == 0) atomicAdd(&report[6], 1);
}

__global__ void k_check_reset(int32_t* __restrict__ report) {
  const int x = threadIdx.x;
  if (x < kReportWords) report[x] = (x == 4 || x == 5) ? INT_MAX : 0;
}

__global__ void k_check_copy_reset(int32_t* __restrict__ report, int32_t* __restrict__ out) {
  const int x = threadIdx.x;
  if (x < kReportWords) {
    out[x] = report[x];
    report[x] = (x == 4 || x == 5) ? INT_MAX : 0;
  }
}

}  // namespace

hipError_t launch_check(const KvView& kv, const int32_t* indices, int index_width, int q_len, int q_tail,
                        int32_t* report, hipStream_t stream) {
  hipLaunchKernelGGL(k_check_count, dim3(1), dim3(64), 0, stream, report);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv.page_table != nullptr && kv.seq_lens != nullptr) {
    hipLaunchKernelGGL(k_check_pages, dim3((unsigned)kv.batch), dim3(kChkNT), 0, stream, kv, report);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (indices != nullptr && index_width > 0) {
    const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
    hipLaunchKernelGGL(k_check_lists, dim3((unsigned)((index_width + kChkNT - 1) / kChkNT), (unsigned)rows),
                       dim3(kChkNT), 0, stream, kv, indices, index_width, q_len, q_tail, report);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_check_reset(int32_t* report, hipStream_t stream) {
  hipLaunchKernelGGL(k_check_reset, dim3(1), dim3(64), 0, stream, report);
  return hipGetLastError();
}

hipError_t launch_check_copy_reset(int32_t* report, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_check_copy_reset, dim3(1), dim3(64), 0, stream, report, out);
  return hipGetLastError();
}

// The report the SPARSE_ATTN_CHECK mode adds to: a device array of the library (each GPU has its
// own copy), found once per device and cleared by a kernel (no allocation, no memset node).
static __device__ __align__(256) int32_t check_report[kReportWords];

namespace {
constexpr int kMaxCheckDevices = 64;
int32_t* g_check_ptr[kMaxCheckDevices];
bool g_check_init[kMaxCheckDevices];
std::mutex g_check_mutex;
}  // namespace

hipError_t check_report_ptr(int32_t** ptr, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxCheckDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_check_mutex);
  if (!g_check_init[dev]) {
    void* addr = nullptr;
    if ((e = hipGetSymbolAddress(&addr, HIP_SYMBOL(check_report))) != hipSuccess) return e;
    g_check_ptr[dev] = static_cast<int32_t*>(addr);
    if ((e = launch_check_reset(g_check_ptr[dev], stream)) != hipSuccess) return e;
    g_check_init[dev] = true;
  }
  *ptr = g_check_ptr[dev];
  return hipSuccess;
}

}  // namespace sa
