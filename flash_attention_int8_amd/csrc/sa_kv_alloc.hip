// KV-cache block allocator: block maps per (layer, head), allocation and release on the GPU.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.4: a KV
// dynamic allocator hands out and takes back cache blocks; in sparse mode it tracks layer and
// head and keeps an independent block map per head, so heads never write into each other's
// blocks. Here each map is a bitmap over num_pages blocks (bit p % 32 of word p / 32 set =
// block p taken) with its own block table [batch][max_pages], and one launch serves every
// map of a step, so a decode loop grows its caches without a round trip to the host.
//
// Allocation, one 1024-thread workgroup per map (the maps are independent):
//   1. the need of sequence b is its logical blocks ceil(old/ps) .. ceil(new/ps) - 1; a
//      workgroup prefix sum over the batch gives each sequence its first request number;
//   2. a scan over the map, 1024 words per step (popcount of the free bits, prefix sum),
//      stops at the word holding the need-th free block, or reports the shortfall and
//      leaves the map and table untouched;
//   3. a second scan up to that word hands free block number r (in ascending block order)
//      to request r: a binary search over the request offsets names the sequence and its
//      logical block. Each thread owns one word, so the map is updated with plain stores.
// The result is the first-fit assignment in (sequence, logical block) order, so it is
// deterministic. Release clears the bits of the released sequences' blocks (atomic AND:
// several blocks share a word) and sets their table entries to -1.
#include "sa_select_dev.h"

namespace sa {
namespace {

constexpr int kAllocNT = 1024;
constexpr int kReleaseNT = 256;

__device__ __forceinline__ int blocks_for(int tokens, int page_size) {  // tokens >= 0
  return tokens / page_size + (tokens % page_size != 0);
}

__device__ __forceinline__ uint32_t usable_bits(int wi, int words, int num_pages) {
  const int rem = num_pages & 31;
  return (wi == words - 1 && rem != 0) ? ((1u << rem) - 1u) : 0xffffffffu;
}

__global__ __launch_bounds__(kAllocNT) void k_kv_alloc(int num_pages, int words,
                                                      uint32_t* __restrict__ maps, int batch,
                                                      int page_size, int max_pages,
                                                      const int32_t* __restrict__ old_lens,
                                                      const int32_t* __restrict__ new_lens,
                                                      int32_t* __restrict__ tables,
                                                      int32_t* __restrict__ status) {
  __shared__ int32_t s_off[kAllocMaxBatch];  // first request number of each sequence
  __shared__ int32_t s_wave[kAllocNT / 64];
  __shared__ int32_t s_bad;
  __shared__ int32_t s_last_word;
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t* map = maps + (int64_t)m * words;
  int32_t* table = tables + (int64_t)m * batch * max_pages;
  if (tid == 0) { s_bad = 0; s_last_word = -1; }
  __syncthreads();
  int need = 0;  // workgroup-uniform running total
  for (int b0 = 0; b0 < batch; b0 += kAllocNT) {
    const int b = b0 + tid;
    int n = 0;
    if (b < batch) {
      const int old = old_lens[b], nw = new_lens[b];
      if (old < 0 || nw < 0 || blocks_for(nw, page_size) > max_pages)
        s_bad = 1;  // every writer stores the same value
      else
        n = max(blocks_for(nw, page_size) - blocks_for(old, page_size), 0);
    }
    int tot;
    const int incl = sel::block_incl_scan<kAllocNT>(n, s_wave, &tot);
    if (b < batch) s_off[b] = need + incl - n;
    need += tot;
  }
  // block_incl_scan ends on a barrier, so s_bad and s_off are visible here
  if (s_bad) {
    if (tid == 0) status[m] = -1;
    return;
  }
  if (need == 0) {
    if (tid == 0) status[m] = 0;
    return;
  }
  // the word holding free block number need - 1
  int seen = 0, last_w0 = -1;
  for (int w0 = 0; w0 < words; w0 += kAllocNT) {
    const int wi = w0 + tid;
    const int f = wi < words ? __popc(~map[wi] & usable_bits(wi, words, num_pages)) : 0;
    int tot;
    const int incl = sel::block_incl_scan<kAllocNT>(f, s_wave, &tot);
    if (seen + tot >= need) {  // uniform: tot is the workgroup total
      if (f > 0 && seen + incl - f < need && seen + incl >= need) s_last_word = wi;
      last_w0 = w0;
      break;
    }
    seen += tot;
  }
  if (last_w0 < 0) {
    if (tid == 0) status[m] = need - seen;  // too few free blocks: nothing changes
    return;
  }
  __syncthreads();
  const int last_word = s_last_word;
  seen = 0;
  for (int w0 = 0; w0 <= last_w0; w0 += kAllocNT) {
    const int wi = w0 + tid;
    const uint32_t word = wi < words ? map[wi] : 0xffffffffu;
    uint32_t freeb = wi < words ? (~word & usable_bits(wi, words, num_pages)) : 0u;
    const int f = __popc(freeb);
    int tot;
    const int incl = sel::block_incl_scan<kAllocNT>(f, s_wave, &tot);
    if (wi <= last_word && f > 0) {
      int r = seen + incl - f;  // number of this word's first free block
      uint32_t taken = 0;
      while (freeb != 0 && r < need) {
        const int bit = __builtin_ctz(freeb);
        freeb &= freeb - 1;
        // request r belongs to the last sequence whose first request number is <= r
        int lo = 0, hi = batch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
        }
        const int lp = blocks_for(old_lens[lo], page_size) + (r - s_off[lo]);
        table[(int64_t)lo * max_pages + lp] = wi * 32 + bit;
        taken |= 1u << bit;
        ++r;
      }
      map[wi] = word | taken;
    }
    seen += tot;
  }
  if (tid == 0) status[m] = 0;
}

__global__ __launch_bounds__(kReleaseNT) void k_kv_release(int num_pages, int words,
                                                          uint32_t* __restrict__ maps, int batch,
                                                          int page_size, int max_pages,
                                                          const int32_t* __restrict__ seq_lens,
                                                          const int32_t* __restrict__ release,
                                                          int32_t* __restrict__ tables) {
  const int m = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * kReleaseNT + threadIdx.x;
  if (i >= (int64_t)batch * max_pages) return;
  const int b = (int)(i / max_pages);
  const int lp = (int)(i - (int64_t)b * max_pages);
  if (release[b] == 0) return;
  const int n = seq_lens[b];
  if (lp >= (n <= 0 ? 0 : min(blocks_for(n, page_size), max_pages))) return;
  int32_t* entry = tables + ((int64_t)m * batch + b) * max_pages + lp;
  const int p = *entry;
  if (p >= 0 && p < num_pages) atomicAnd(&maps[(int64_t)m * words + (p >> 5)], ~(1u << (p & 31)));
  *entry = -1;
}

}  // namespace

int map_words(int num_pages) { return num_pages / 32 + (num_pages % 32 != 0); }

hipError_t launch_kv_alloc(int num_maps, int num_pages, uint32_t* maps, int batch, int page_size,
                           int max_pages, const int32_t* old_lens, const int32_t* new_lens,
                           int32_t* tables, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(k_kv_alloc, dim3((unsigned)num_maps), dim3(kAllocNT), 0, stream, num_pages,
                     map_words(num_pages), maps, batch, page_size, max_pages, old_lens, new_lens,
                     tables, status);
  return hipGetLastError();
}

hipError_t launch_kv_release(int num_maps, int num_pages, uint32_t* maps, int batch, int page_size,
                             int max_pages, const int32_t* seq_lens, const int32_t* release,
                             int32_t* tables, hipStream_t stream) {
  const int64_t n = (int64_t)batch * max_pages;
  const unsigned gx = (unsigned)((n + kReleaseNT - 1) / kReleaseNT);
  hipLaunchKernelGGL(k_kv_release, dim3(gx, (unsigned)num_maps), dim3(kReleaseNT), 0, stream,
                     num_pages, map_words(num_pages), maps, batch, page_size, max_pages, seq_lens,
                     release, tables);
  return hipGetLastError();
}

}  // namespace sa
