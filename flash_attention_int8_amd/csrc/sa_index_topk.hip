// Fused indexer + exact top-K for decode-shaped calls: one query per sequence, long rows.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.1: the index
// is generated on the GPU before each layer's attention, scoring every cached key and keeping
// the top-K. This path produces the same index lists as scoring into memory and selecting
// afterwards, but never writes the full score rows: the indexer is HBM-bound, and writing a
// 4-byte score for every 64-byte key into the middle of that read stream costs about a fifth
// of its time on MI355X.
//
// Three launches over rows r = (sequence, indexer head):
//   sample  one workgroup per row scores an evenly spaced sample of the row's 64-token
//           blocks (about kSampleBlocks of them) and picks a provisional threshold bin
//           theta: the highest bin whose sampled tail holds well over the sampled share of
//           K (twice the expected count plus four standard deviations plus 16). It also
//           clears the row histogram used by the next pass.
//   main    per (row, 8192-token chunk): scores every key of the chunk, adds the exact
//           histogram of key >> 12 into the row histogram, and compacts the keys in bins
//           >= theta, in token order, into the chunk's candidate slots.
//   final   one workgroup per row: the exact histogram gives b1, the bin of the K-th largest
//           key. If b1 >= theta every selected key is a candidate, and the exact selection
//           runs on the candidates (a few thousand per row). Otherwise (the sample misjudged
//           the tail) the workgroup rescores the row and collects the keys in bins >= b1
//           first, so the result stays exact whatever the score distribution.
#include "sa_index_dev.h"
#include "sa_select_dev.h"

namespace sa {
namespace {

using namespace idx;
using namespace sel;

constexpr int kFChunk = 8192;             // tokens per main-pass workgroup
constexpr int kFBlocks = kFChunk / 64;    // 64-token blocks per chunk
constexpr int kSampleBlocks = 64;         // sampled blocks per row (about)
constexpr int kFinalNT = 1024;

struct FusedWs {
  uint32_t* hist1;  // [rows][4096]
  int32_t* state;   // [rows][4]: theta (a key value), -
  int32_t* ccount;  // [rows][chunks]
  int2* cand;       // [rows][chunks][kFChunk]: (key, token)
};

__device__ __forceinline__ FusedWs fused_ws(void* ws, int64_t rows, int chunks) {
  FusedWs w;
  w.hist1 = static_cast<uint32_t*>(ws);
  w.state = reinterpret_cast<int32_t*>(w.hist1 + rows * kBins);
  w.ccount = w.state + rows * 4;
  int64_t off = rows * (kBins + 4) + rows * chunks;
  off = (off + 3) & ~(int64_t)3;
  w.cand = reinterpret_cast<int2*>(static_cast<int32_t*>(ws) + off);
  return w;
}

struct FRow {
  int b, gi, pos, P, n, nf, W, blk_first, blk_last;
};

__device__ __forceinline__ FRow frow(const KvView& kv, int64_t row, int q_tail, int top_k) {
  FRow r;
  r.b = (int)(row / kv.num_idx_heads);
  r.gi = (int)(row - (int64_t)r.b * kv.num_idx_heads);
  r.P = kv.prefix_len;
  r.W = r.P + top_k;
  r.pos = min(kv.seq_lens[r.b], kv.max_seq_len) - q_tail;
  r.nf = r.pos < 0 ? 0 : min(r.P, r.pos + 1);
  r.n = r.pos - r.P + 1;
  r.blk_first = r.P >> 6;
  r.blk_last = r.pos >> 6;
  return r;
}

// Byte offset of 64-token block `blk` of row (b, gi) in the indexer pool, or -1.
template <int D>
__device__ __forceinline__ int64_t block_base(const KvView& kv, int b, int gi, int blk) {
  const int64_t phys = phys_page(kv, b, blk << 6);
  if (phys < 0) return -1;
  const int slot0 = (blk << 6) & (kv.page_size - 1);
  return ((phys * kv.num_idx_heads + gi) * kv.page_size + slot0) * (int64_t)D;
}

// ---------------------------------------------------------------------------------- sample
template <int D>
__global__ __launch_bounds__(kFinalNT) void k_fused_sample(KvView kv, const int8_t* __restrict__ q_idx,
                                                           int q_tail, int top_k, void* ws,
                                                           int chunks) {
  constexpr int NT = kFinalNT;
  __shared__ TopkShared<NT> sh;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const FusedWs w = fused_ws(ws, gridDim.x, chunks);
  const FRow r = frow(kv, row, q_tail, top_k);
  uint32_t* h1 = w.hist1 + row * kBins;
  for (int j = threadIdx.x; j < kBins; j += NT) {
    h1[j] = 0u;
    sh.hist[j] = 0u;
  }
  if (threadIdx.x == 0) { sh.found_bin = 0; sh.found_above = 0; }
  if (r.n <= top_k) return;  // uniform: the final pass lists every candidate
  __syncthreads();
  const v4i qf = *reinterpret_cast<const v4i*>(q_idx + (row * (int64_t)D) + lane_part<D>(lane) * 16);
  const int n_blk = r.blk_last - r.blk_first + 1;
  const int stride = max(1, n_blk / kSampleBlocks);
  constexpr int SU = kSampleBlocks / (NT / 64);  // sampled blocks per wave, loads issued together
  for (int j0 = wave * SU; j0 * stride < n_blk; j0 += (NT / 64) * SU) {
    int64_t base[SU];
    v4i kd[SU][Blk<D>::R];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j = j0 + u;
      base[u] = (j * stride < n_blk) ? block_base<D>(kv, r.b, r.gi, r.blk_first + j * stride) : -1;
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      if (base[u] >= 0) {
        load_block<D>(kv.kidx_pool + base[u], lane, kd[u]);
      } else {
#pragma unroll
        for (int q = 0; q < Blk<D>::R; ++q) kd[u][q] = v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int s = to_token_order<D>(score_block<D>(qf, kd[u], lane), lane);
      const int t = ((r.blk_first + (j0 + u) * stride) << 6) + lane;
      if (base[u] >= 0 && t >= r.P && t <= r.pos) atomicAdd(&sh.hist[score_key(s) >> 12], 1u);
    }
  }
  __syncthreads();
  // total sampled keys, and the share of K they should hold above the threshold
  int cnt = 0;
  for (int j = threadIdx.x; j < kBins; j += NT) cnt += sh.hist[j];
  int n_s;
  block_incl_scan<NT>(cnt, sh.wave_tot, &n_s);
  const float expect = (float)top_k * (float)n_s / (float)r.n;
  const int target = (int)(2.f * expect + 4.f * sqrtf(expect) + 16.f);
  int theta = 0;  // collect everything unless the sample supports a higher bin
  if (target < n_s) {
    find_bin<NT>(sh, target);
    theta = sh.found_bin << 12;
  }
  if (threadIdx.x == 0) w.state[row * 4 + 0] = theta;
}

// ------------------------------------------------------------------------------------ main
// Compacts, in token order, the keys of one 16-block slab with key >= theta. Wave w holds
// blocks u = 0..U-1 at slab positions w*U + u, with lane l holding token l of each block.
template <int NW, int U>
__device__ __forceinline__ int compact_slab(const uint32_t (&key)[U], const bool (&keep)[U],
                                            const int (&tok)[U], int32_t* wave_tot, int2* dst,
                                            int fill) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t mask[U];
  int wcount = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    mask[u] = __ballot(keep[u]);
    wcount += __popcll(mask[u]);
  }
  if (lane == 0) wave_tot[wave] = wcount;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int x = wave_tot[v];
    before += (v < wave) ? x : 0;
    total += x;
  }
  int off = fill + before;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (keep[u]) dst[off + __popcll(mask[u] & lt)] = make_int2((int)key[u], tok[u]);
    off += __popcll(mask[u]);
  }
  __syncthreads();  // wave_tot is rewritten by the next slab
  return fill + total;
}

template <int D>
__global__ __launch_bounds__(256) void k_fused_main(KvView kv, const int8_t* __restrict__ q_idx,
                                                    int q_tail, int top_k, void* ws, int chunks) {
  constexpr int NW = 4;
  constexpr int U = 4;  // blocks per wave per slab; a slab is NW * U = 16 blocks
  __shared__ uint32_t h[kBins];
  __shared__ int32_t wave_tot[NW];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const FusedWs w = fused_ws(ws, gridDim.y, chunks);
  const FRow r = frow(kv, row, q_tail, top_k);
  if (r.n <= top_k) return;
  if (c * kFChunk > r.pos) {
    if (threadIdx.x == 0) w.ccount[row * chunks + c] = 0;
    return;
  }
  const v4i qf = *reinterpret_cast<const v4i*>(q_idx + (row * (int64_t)D) + lane_part<D>(lane) * 16);
  const uint32_t theta = (uint32_t)w.state[row * 4 + 0];
  for (int j = threadIdx.x; j < kBins; j += 256) h[j] = 0u;
  __syncthreads();
  int2* dst = w.cand + (row * chunks + c) * (int64_t)kFChunk;
  int fill = 0;
  for (int slab = 0; slab < kFBlocks / (NW * U); ++slab) {
    const int blk0 = c * kFBlocks + slab * NW * U + wave * U;
    int64_t base[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = blk0 + u;
      base[u] = (blk >= r.blk_first && blk <= r.blk_last) ? block_base<D>(kv, r.b, r.gi, blk) : -1;
    }
    v4i kd[U][Blk<D>::R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base[u] >= 0) {
        load_block<D>(kv.kidx_pool + base[u], lane, kd[u]);
      } else {
#pragma unroll
        for (int q = 0; q < Blk<D>::R; ++q) kd[u][q] = v4i{0, 0, 0, 0};
      }
    }
    uint32_t key[U];
    bool keep[U];
    int tok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = to_token_order<D>(score_block<D>(qf, kd[u], lane), lane);
      tok[u] = ((blk0 + u) << 6) + lane;
      const bool in = base[u] >= 0 && tok[u] >= r.P && tok[u] <= r.pos;
      key[u] = score_key(s);
      if (in) atomicAdd(&h[key[u] >> 12], 1u);
      keep[u] = in && key[u] >= theta;
    }
    fill = compact_slab<NW, U>(key, keep, tok, wave_tot, dst, fill);
  }
  uint32_t* h1 = w.hist1 + row * kBins;
  for (int j = threadIdx.x; j < kBins; j += 256)
    if (h[j]) atomicAdd(&h1[j], h[j]);
  if (threadIdx.x == 0) w.ccount[row * chunks + c] = fill;
}

// ----------------------------------------------------------------------------------- final
template <int D>
__global__ __launch_bounds__(kFinalNT) void k_fused_final(KvView kv, const int8_t* __restrict__ q_idx,
                                                          int q_tail, int top_k, void* ws,
                                                          int chunks, int32_t* __restrict__ indices) {
  constexpr int NT = kFinalNT;
  constexpr int NW = NT / 64;
  __shared__ TopkShared<NT> sh;
  __shared__ int32_t s_off[1025];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const FusedWs w = fused_ws(ws, gridDim.x, chunks);
  const FRow r = frow(kv, row, q_tail, top_k);
  int32_t* out = indices + row * r.W;
  for (int j = tid; j < r.nf; j += NT) out[j] = j;
  if (r.n <= top_k) {
    const int m = r.n > 0 ? r.n : 0;
    for (int j = tid; j < m; j += NT) out[r.nf + j] = r.P + j;
    for (int j = r.nf + m + tid; j < r.W; j += NT) out[j] = -1;
    return;
  }
  const uint32_t* h1 = w.hist1 + row * kBins;
  const uint32_t theta = (uint32_t)w.state[row * 4 + 0];
  for (int j = tid; j < kBins; j += NT) sh.hist[j] = h1[j];
  if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
  __syncthreads();
  find_bin<NT>(sh, top_k);
  const uint32_t b1 = (uint32_t)sh.found_bin;
  const int above1 = sh.found_above;
  if ((b1 << 12) < theta) {
    // The provisional threshold excluded part of bin b1 or above: rescore the row and
    // collect every key in bins >= b1, chunk by chunk, into the same slots.
    const v4i qf = *reinterpret_cast<const v4i*>(q_idx + (row * (int64_t)D) + lane_part<D>(lane) * 16);
    for (int c = 0; c < chunks; ++c) {
      int2* dst = w.cand + (row * chunks + c) * (int64_t)kFChunk;
      int fill = 0;
      if (c * kFChunk <= r.pos) {
        for (int slab = 0; slab < kFBlocks / NW; ++slab) {
          const int blk = c * kFBlocks + slab * NW + wave;
          const int64_t base =
              (blk >= r.blk_first && blk <= r.blk_last) ? block_base<D>(kv, r.b, r.gi, blk) : -1;
          v4i kd[1][Blk<D>::R];
          if (base >= 0) {
            load_block<D>(kv.kidx_pool + base, lane, kd[0]);
          } else {
#pragma unroll
            for (int q = 0; q < Blk<D>::R; ++q) kd[0][q] = v4i{0, 0, 0, 0};
          }
          const int s = to_token_order<D>(score_block<D>(qf, kd[0], lane), lane);
          uint32_t key[1] = {score_key(s)};
          int tok[1] = {(blk << 6) + lane};
          bool keep[1] = {base >= 0 && tok[0] >= r.P && tok[0] <= r.pos && (key[0] >> 12) >= b1};
          fill = compact_slab<NW, 1>(key, keep, tok, sh.wave_tot2, dst, fill);
        }
      }
      if (tid == 0) w.ccount[row * chunks + c] = fill;
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
  }
  select_candidates<NT>(sh, s_off, w.cand + row * chunks * (int64_t)kFChunk, w.ccount + row * chunks,
                        chunks, kFChunk, b1, above1, top_k, out + r.nf);
}

template <int D>
hipError_t launch_d(const KvView& kv, const int8_t* q_idx, int q_tail, int top_k, int32_t* indices,
                    void* ws, hipStream_t stream) {
  const int64_t rows = (int64_t)kv.batch * kv.num_idx_heads;
  const int chunks = (kv.max_seq_len + kFChunk - 1) / kFChunk;
  if (chunks > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fused_sample<D>, dim3((unsigned)rows), dim3(kFinalNT), 0, stream, kv, q_idx,
                     q_tail, top_k, ws, chunks);
  hipLaunchKernelGGL(k_fused_main<D>, dim3(chunks, (unsigned)rows), dim3(256), 0, stream, kv, q_idx,
                     q_tail, top_k, ws, chunks);
  hipLaunchKernelGGL(k_fused_final<D>, dim3((unsigned)rows), dim3(kFinalNT), 0, stream, kv, q_idx,
                     q_tail, top_k, ws, chunks, indices);
  return hipGetLastError();
}

}  // namespace

bool fused_applies(const KvView& kv, int q_len) {
  const int64_t rows = (int64_t)kv.batch * kv.num_idx_heads;
  return q_len == 1 && rows <= 4096 && kv.max_seq_len - kv.prefix_len >= 16384 &&
         (kv.max_seq_len + kFChunk - 1) / kFChunk <= 1024;
}

size_t fused_workspace_bytes(const KvView& kv) {
  const int64_t rows = (int64_t)kv.batch * kv.num_idx_heads;
  const int64_t chunks = (kv.max_seq_len + kFChunk - 1) / kFChunk;
  const int64_t head = (rows * (kBins + 4) + rows * chunks + 3) & ~(int64_t)3;
  return (size_t)(head + rows * chunks * kFChunk * 2) * sizeof(int32_t);
}

hipError_t launch_index_topk_fused(const KvView& kv, const int8_t* q_idx, int q_tail, int top_k,
                                   int32_t* indices, void* ws, hipStream_t stream) {
  switch (kv.idx_dim) {
    case 32: return launch_d<32>(kv, q_idx, q_tail, top_k, indices, ws, stream);
    case 64: return launch_d<64>(kv, q_idx, q_tail, top_k, indices, ws, stream);
    case 128: return launch_d<128>(kv, q_idx, q_tail, top_k, indices, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
