// Fused indexer + exact top-K for decode-shaped calls: one query per sequence, long rows.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.1: the index
// is generated on the GPU before each layer's attention, scoring every cached key and keeping
// the top-K. This path produces the same index lists as scoring into memory and selecting
// afterwards, but never writes the full score rows: the indexer is HBM-bound, and writing a
// 4-byte score for every 64-byte key into the middle of that read stream costs about a fifth
// of its time on MI355X.
//
// Two launches over rows r = (sequence, indexer head):
//   main    per (row, 8192-token chunk): scores every key of the chunk; the histogram of key >> 12
//           over the chunk's first 4096 keys sets the chunk's threshold theta_c: the lower edge
//           of the highest bin whose tail holds well over those keys' share of K, refined to a
//           single key by a histogram of that bin's low digits when the bin alone holds many
//           more (scores packed into a few bins). The keys >= theta_c are compacted, in token
//           order, into the chunk's candidate slots, except that keys equal to theta_c stop
//           being kept once the chunk holds K candidates: each later one has K keys of its own
//           chunk ranked above it (larger, or equal and earlier), so it is not in the top K.
//           With every score equal this keeps about K keys per chunk instead of all of them.
//   final   one workgroup per row: tau_c, the K-th largest candidate key. If tau_c >= theta_c
//           for every chunk, every key of the row >= tau_c is a candidate, so tau_c is the
//           row's K-th largest key and the exact selection runs on the candidates (a few
//           thousand per row). Otherwise (a chunk holds far more than its share of the top)
//           the workgroup rescores the chunks whose threshold lies above tau_c: an exact
//           histogram (their keys plus the other chunks' candidates) first, then every key of
//           theirs in bins >= the exact b1 is collected, so the result stays exact whatever the
//           score distribution.
#include "sa_index_dev.h"
#include "sa_select_dev.h"

namespace sa {
namespace {

using namespace idx;
using namespace sel;

constexpr int kFChunk = 8192;             // tokens per main-pass workgroup
constexpr int kFBlocks = kFChunk / 64;    // 64-token blocks per chunk
constexpr int kSampleSlabs = 4;           // 1024-token slabs whose histogram sets the chunk threshold
constexpr int kFinalNT = 1024;

struct FusedWs {
  int32_t* ccount;  // [rows][chunks]: candidates kept by the chunk
  int32_t* cth;     // [rows][chunks]: the chunk's threshold bin theta_c
  int2* cand;       // [rows][chunks][kFChunk]: (key, token)
};

__device__ __forceinline__ int64_t fused_cand_offset(int64_t rows, int chunks) {
  return (2 * rows * chunks + 3) & ~(int64_t)3;  // int32 units; keeps cand 16-byte aligned
}

__device__ __forceinline__ FusedWs fused_ws(void* ws, int64_t rows, int chunks) {
  FusedWs w;
  w.ccount = static_cast<int32_t*>(ws);
  w.cth = w.ccount + rows * chunks;
  w.cand = reinterpret_cast<int2*>(static_cast<int32_t*>(ws) + fused_cand_offset(rows, chunks));
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

// Compacts, in token order, the keys of one 16-block slab that `keep` marks. Wave w holds
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

// ------------------------------------------------------------------------------------ main
template <int D>
__global__ __launch_bounds__(256, D == 128 ? 2 : 4) void k_fused_main(KvView kv, const int8_t* __restrict__ q_idx,
                                                    int q_tail, int top_k, void* ws, int chunks) {
  constexpr int NT = 256;
  constexpr int NW = NT / 64;
  constexpr int U = 4;  // blocks per wave per slab; a slab is NW * U = 16 blocks (1024 tokens)
  __shared__ TopkShared<NT> sh;
  __shared__ uint4 s_sample[kSampleSlabs][NT];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const FusedWs w = fused_ws(ws, gridDim.y, chunks);
  const FRow r = frow(kv, row, q_tail, top_k);
  if (r.n <= top_k) return;  // the final pass lists every candidate
  if (c * kFChunk > r.pos) {
    if (tid == 0) {
      w.ccount[row * chunks + c] = 0;
      w.cth[row * chunks + c] = 0;
    }
    return;
  }
  const v4i qf = *reinterpret_cast<const v4i*>(q_idx + (row * (int64_t)D) + lane_part<D>(lane) * 16);
  for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
  if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
  __syncthreads();
  int2* dst = w.cand + (row * chunks + c) * (int64_t)kFChunk;
  // Page-table entries of a slab's blocks, requested a slab ahead of their use. The loads are
  // unconditional (index clamped into the table) so that no wait lands next to them; the
  // entries are checked in score_slab.
  auto slab_pages = [&](int slab, int32_t (&raw)[U]) {
    const int blk0 = c * kFBlocks + slab * NW * U + wave * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int lp = min(((blk0 + u) << 6) >> kv.page_shift, kv.max_pages_per_seq - 1);
      raw[u] = kv.page_table[(int64_t)r.b * kv.max_pages_per_seq + lp];
    }
  };
  // Requests the keys of slab `slab` (its page-table entries in `raw`): unconditional loads, a
  // block without a page reading page 0 and flagged in `ok`, so that the loads can stay in
  // flight across the compaction of the previous slab.
  auto issue_slab = [&](int slab, const int32_t (&raw)[U], v4i (&kd)[U][Blk<D>::R], bool (&ok)[U]) {
    const int blk0 = c * kFBlocks + slab * NW * U + wave * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = blk0 + u;
      const int lp = (blk << 6) >> kv.page_shift;
      ok[u] = blk >= r.blk_first && blk <= r.blk_last && lp < kv.max_pages_per_seq &&
              raw[u] >= 0 && raw[u] < kv.num_pages;
      const int64_t base = (((int64_t)(ok[u] ? raw[u] : 0) * kv.num_idx_heads + r.gi) * kv.page_size +
                            ((blk << 6) & (kv.page_size - 1))) * (int64_t)D;
      load_block<D>(kv.kidx_pool + base, lane, kd[u]);
    }
  };
  // scores a loaded slab: key, whether the token is a candidate, token index
  auto score_slab = [&](int slab, const v4i (&kd)[U][Blk<D>::R], const bool (&ok)[U], uint32_t (&key)[U],
                        bool (&in)[U], int (&tok)[U]) {
    const int blk0 = c * kFBlocks + slab * NW * U + wave * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = to_token_order<D>(score_block<D>(qf, kd[u], lane), lane);
      tok[u] = ((blk0 + u) << 6) + lane;
      in[u] = ok[u] && tok[u] >= r.P && tok[u] <= r.pos;
      key[u] = score_key(s);
    }
  };
  constexpr int kSlabs = kFBlocks / (NW * U);
  static_assert(kSampleSlabs >= 1 && kSampleSlabs < kSlabs, "the sample is a proper prefix of the chunk");
  uint32_t key[U];
  bool in[U], keep[U], ok[U];
  int tok[U];
  int32_t raw_cur[U], raw_nxt[U];
  v4i kd[U][Blk<D>::R];
  slab_pages(0, raw_cur);
  slab_pages(1, raw_nxt);
  issue_slab(0, raw_cur, kd, ok);
  // After a slab is scored its registers take the next slab's loads, which stay in flight
  // while the slab is compacted (and, for the sample slabs, while the threshold is found).
  auto next_slab = [&](int slab) {
    if (slab + 1 < kSlabs) {
#pragma unroll
      for (int u = 0; u < U; ++u) raw_cur[u] = raw_nxt[u];
      slab_pages(slab + 2, raw_nxt);  // past the chunk: clamped, in bounds, never used
      issue_slab(slab + 1, raw_cur, kd, ok);
    }
  };
  // The chunk's threshold from its first kSampleSlabs slabs: the lower edge of the highest bin
  // whose tail holds well over the sample's share of K (twice the expected count plus three
  // standard deviations plus 8), refined to a single key when that bin holds most of the tail.
  // Any value is safe: the final pass checks it and rescores the chunks whose threshold was too
  // high. A larger sample gives a threshold closer to the sample's share, so fewer candidates
  // reach the final pass.
  // The sample keys wait in LDS (each lane reads back only its own), kNotIn marking the
  // tokens that are not candidates; keys are at most 24 bits, so the mark is unambiguous.
  static_assert(U == 4, "one 16-byte LDS entry per lane and slab");
  constexpr uint32_t kNotIn = 0xffffffffu;
#pragma unroll
  for (int sl = 0; sl < kSampleSlabs; ++sl) {
    score_slab(sl, kd, ok, key, in, tok);
    next_slab(sl);
    s_sample[sl][tid] = make_uint4(in[0] ? key[0] : kNotIn, in[1] ? key[1] : kNotIn,
                                   in[2] ? key[2] : kNotIn, in[3] ? key[3] : kNotIn);
#pragma unroll
    for (int u = 0; u < U; ++u) hist_add_wave(sh.hist, key[u] >> 12, in[u]);
  }
  __syncthreads();
  uint32_t th = 0;  // the chunk keeps its keys >= th
  {
    int cnt = 0;
    for (int j = tid; j < kBins; j += NT) cnt += sh.hist[j];
    int n_s;
    block_incl_scan<NT>(cnt, sh.wave_tot, &n_s);
    const float expect = (float)top_k * (float)n_s / (float)r.n;
    const int target = (int)(2.f * expect + 3.f * sqrtf(expect) + 8.f);
    if (n_s >= 256 && target < n_s) {  // short samples (row edges) keep everything
      find_bin<NT>(sh, target);
      const uint32_t tb = (uint32_t)sh.found_bin;
      const int above = sh.found_above;
      const int tail = above + (int)sh.hist[tb];
      th = tb << 12;
      if (tail > 2 * target) {
        // The bin is crowded (scores packed into few bins): refine the threshold to one key
        // with a histogram of the sample's keys in that bin.
        __syncthreads();
        for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
        if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < kSampleSlabs; ++sl) {
          const uint4 pk = s_sample[sl][tid];
          const uint32_t kk[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
            hist_add_wave(sh.hist, kk[u] & 0xfffu, kk[u] != kNotIn && (kk[u] >> 12) == tb);
        }
        __syncthreads();
        find_bin<NT>(sh, target - above);
        th |= (uint32_t)sh.found_bin;
      }
    }
  }
  int fill = 0;
#pragma unroll
  for (int sl = 0; sl < kSampleSlabs; ++sl) {
    const int blk0 = c * kFBlocks + sl * NW * U + wave * U;
    const uint4 pk = s_sample[sl][tid];
    key[0] = pk.x; key[1] = pk.y; key[2] = pk.z; key[3] = pk.w;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      tok[u] = ((blk0 + u) << 6) + lane;
      keep[u] = key[u] != kNotIn && (key[u] > th || (key[u] == th && fill < top_k));
    }
    fill = compact_slab<NW, U>(key, keep, tok, sh.wave_tot2, dst, fill);
  }
  for (int slab = kSampleSlabs; slab < kSlabs; ++slab) {
    score_slab(slab, kd, ok, key, in, tok);
    next_slab(slab);
#pragma unroll
    for (int u = 0; u < U; ++u) keep[u] = in[u] && (key[u] > th || (key[u] == th && fill < top_k));
    fill = compact_slab<NW, U>(key, keep, tok, sh.wave_tot2, dst, fill);
  }
  if (tid == 0) {
    w.ccount[row * chunks + c] = fill;
    w.cth[row * chunks + c] = (int32_t)th;
  }
}

// ----------------------------------------------------------------------------------- final
constexpr int kRegPer = 24;    // candidates per lane held in registers by the final pass
constexpr int kRegSpec = 8;    // of those, loaded before the counts are known (one chunk per wave)
constexpr int kFineBins = 1024;
constexpr int kFineShift = 8;  // fine bins are 256 key units; 1024 of them span 64 coarse bins

// Exact selection for one row from the candidates held in registers. Wave w owns chunks
// [w*cpw, (w+1)*cpw) and their candidates, in token order, as e[k] for index k*64 + lane.
// Every key of the row at or above theta_max, the highest chunk threshold, is a candidate; so
// if at least K candidates lie at or above theta_max, the K largest keys of the row are the K
// largest of those candidates. A 1024-bin histogram of
// 256-unit fine bins above that base locates the K-th largest to one fine bin and a 256-entry
// histogram of that bin gives it exactly. Returns false (uniformly, nothing written) when a
// wave holds more candidates than its registers, when fewer than K candidates lie above the
// base, or when the K-th largest lies beyond the fine range; the caller then takes the
// general path.
struct RegRow {
  int2 e[kRegPer];  // the wave's candidates, index k * 64 + lane
  int ccl, thl;     // lane i < number of the wave's chunks: count and threshold of chunk i
  int cpw, c0, nch;
  bool spec;        // e[0 .. kRegSpec) were loaded before the counts were known
};

// Issues the loads of the register path; they depend on nothing but the row, so they go out
// before the row's length is known. With one chunk per wave the chunk's first slots are loaded
// at once (they lie inside its region; entries past its count are ignored).
template <int NT>
__device__ __forceinline__ void reg_row_prefetch(const FusedWs& w, int64_t row, int chunks,
                                                 RegRow& q) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  q.cpw = (chunks + NW - 1) / NW;
  q.c0 = wave * q.cpw;
  q.nch = max(0, min(chunks, q.c0 + q.cpw) - q.c0);
  const int64_t crow = row * chunks;
  q.spec = (q.cpw == 1 && q.nch == 1);
  if (q.spec) {
    const int2* cw = w.cand + (crow + q.c0) * (int64_t)kFChunk;
#pragma unroll
    for (int k = 0; k < kRegSpec; ++k) q.e[k] = cw[k * 64 + lane];
  }
  q.ccl = lane < q.nch ? w.ccount[crow + q.c0 + lane] : 0;
  q.thl = lane < q.nch ? w.cth[crow + q.c0 + lane] : 0;
}

template <int NT>
__device__ __forceinline__ bool select_row_registers(TopkShared<NT>& sh, const FusedWs& w,
                                                     int64_t row, int chunks, int top_k,
                                                     int32_t* __restrict__ out, RegRow& q) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nch = q.nch;
  const int ccl = q.ccl, thl = q.thl;
  const bool spec = q.spec;
  int2 (&e)[kRegPer] = q.e;
  const int2* cw = w.cand + (row * chunks + q.c0) * (int64_t)kFChunk;  // the wave's first chunk
  for (int j = tid; j < kFineBins + 256; j += NT) sh.hist[j] = 0u;
  const int incl = wave_incl_sum(ccl);
  const int ex = incl - ccl;  // offset of chunk c0 + lane inside the wave's candidates
  const int wtot = __builtin_amdgcn_readlane(incl, 63);  // wave-uniform: loops below end on it
  const int thw = __builtin_amdgcn_readlane(wave_incl_max_nonneg(thl), 63);
  if (lane == 0) {
    sh.wave_tot[wave] = wtot;
    sh.wave_tot2[wave] = thw;
  }
  __syncthreads();
  uint32_t thmax = 0;
  bool over = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    thmax = max(thmax, (uint32_t)sh.wave_tot2[v]);
    over |= sh.wave_tot[v] > kRegPer * 64;
  }
  if (over) return false;
  const int kfirst = spec ? kRegSpec : 0;
  // Wave-local candidate j = k * 64 + lane belongs to the last chunk whose offset is <= j.
  // The offsets rise with the chunk number, so a wave-uniform cursor walks forward with k and
  // only the chunk boundaries that fall inside the current 64 candidates are compared per lane.
  const int nchu = __builtin_amdgcn_readfirstlane(nch);
  int cur = 0;
#pragma unroll
  for (int k = 0; k < kRegPer; ++k) {
    if (k * 64 >= wtot) break;
    if (k < kfirst) continue;
    while (cur + 1 < nchu && __builtin_amdgcn_readlane(ex, cur + 1) <= k * 64) ++cur;
    const int j = k * 64 + lane;
    int ci = cur, off = __builtin_amdgcn_readlane(ex, cur);
    for (int t = cur + 1; t < nchu; ++t) {
      const int o = __builtin_amdgcn_readlane(ex, t);
      if (o > k * 64 + 63) break;
      if (j >= o) { ci = t; off = o; }
    }
    if (j < wtot) e[k] = cw[ci * (int64_t)kFChunk + (j - off)];
  }
  const uint32_t base = thmax;
#pragma unroll
  for (int k = 0; k < kRegPer; ++k) {
    if (k * 64 >= wtot) break;
    const uint32_t key = (uint32_t)e[k].x;
    if (k * 64 + lane < wtot && key >= base)
      atomicAdd(&sh.hist[min((key - base) >> kFineShift, (uint32_t)kFineBins - 1)], 1u);
  }
  __syncthreads();
  static_assert(kFineBins == NW * 64, "one 64-bin segment per wave");
  int above_fb;
  const int fb = block_find_bin_segments<NW>(sh.hist, reinterpret_cast<int32_t*>(sh.hist + kFineBins + 256),
                                             top_k, &above_fb);
  if (fb < 0 || fb == kFineBins - 1) return false;
  const uint32_t fb_lo = base + ((uint32_t)fb << kFineShift);
#pragma unroll
  for (int k = 0; k < kRegPer; ++k) {
    if (k * 64 >= wtot) break;
    const uint32_t key = (uint32_t)e[k].x;
    // fb_lo need not be 256-aligned: the sub-bin is the offset from it
    if (k * 64 + lane < wtot && key >= fb_lo && key < fb_lo + (1u << kFineShift))
      atomicAdd(&sh.hist[kFineBins + (key - fb_lo)], 1u);
  }
  __syncthreads();
  int above_sb;
  const int sb = wave_find_bin<4>(sh.hist + kFineBins, top_k - above_fb, &above_sb);
  const uint32_t tau = fb_lo + (uint32_t)sb;
  const int need = top_k - above_fb - above_sb;  // keys == tau to take, in token order
  int gt_w = 0, eq_w = 0;
#pragma unroll
  for (int k = 0; k < kRegPer; ++k) {
    if (k * 64 >= wtot) break;
    const bool valid = k * 64 + lane < wtot;
    gt_w += __popcll(__ballot(valid && (uint32_t)e[k].x > tau));
    eq_w += __popcll(__ballot(valid && (uint32_t)e[k].x == tau));
  }
  if (lane == 0) {
    sh.wave_tot[wave] = gt_w;
    sh.wave_tot2[wave] = eq_w;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    gt_before += (v < wave) ? sh.wave_tot[v] : 0;
    eq_before += (v < wave) ? sh.wave_tot2[v] : 0;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int slot = gt_before + min(need, eq_before);
  int eq_seen = eq_before;
#pragma unroll
  for (int k = 0; k < kRegPer; ++k) {
    if (k * 64 >= wtot) break;
    const bool valid = k * 64 + lane < wtot;
    const bool gt = valid && (uint32_t)e[k].x > tau;
    const bool eq = valid && (uint32_t)e[k].x == tau;
    const uint64_t eq_mask = __ballot(eq);
    const bool take = gt || (eq && eq_seen + __popcll(eq_mask & lt) < need);
    const uint64_t take_mask = __ballot(take);
    const int o = slot + __popcll(take_mask & lt);
    if (take && o < top_k) out[o] = e[k].y;
    slot += __popcll(take_mask);
    eq_seen += __popcll(eq_mask);
  }
  return true;
}

template <int D>
__global__ __launch_bounds__(kFinalNT) void k_fused_final(KvView kv, const int8_t* __restrict__ q_idx,
                                                          int q_tail, int top_k, void* ws,
                                                          int chunks, int32_t* __restrict__ indices) {
  constexpr int NT = kFinalNT;
  constexpr int NW = NT / 64;
  __shared__ TopkShared<NT> sh;
  __shared__ int32_t s_off[1025];
  __shared__ int32_t s_thmax;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const FusedWs w = fused_ws(ws, gridDim.x, chunks);
  RegRow q;
  reg_row_prefetch<NT>(w, row, chunks, q);
  const FRow r = frow(kv, row, q_tail, top_k);
  int32_t* out = indices + row * r.W;
  for (int j = tid; j < r.nf; j += NT) out[j] = j;
  if (r.n <= top_k) {
    const int m = r.n > 0 ? r.n : 0;
    for (int j = tid; j < m; j += NT) out[r.nf + j] = r.P + j;
    for (int j = r.nf + m + tid; j < r.W; j += NT) out[j] = -1;
    return;
  }
  if (select_row_registers<NT>(sh, w, row, chunks, top_k, out + r.nf, q)) return;
  // General path: candidates streamed from the workspace.
  const int32_t* cc = w.ccount + row * chunks;
  const int32_t* cth = w.cth + row * chunks;
  const int2* cand = w.cand + row * chunks * (int64_t)kFChunk;
  __syncthreads();  // every wave is done with the shared arrays of the register path
  if (tid == 0) s_thmax = 0;
  __syncthreads();
  if (tid < chunks) atomicMax(&s_thmax, cth[tid]);  // the highest chunk threshold
  __syncthreads();
  // the selection from the candidates, valid when their K-th largest key is >= every chunk's
  // threshold
  uint32_t lb = 0;
  if (!select_candidates<NT>(sh, s_off, cand, cc, chunks, kFChunk, 0u, 0, top_k, out + r.nf,
                             s_thmax, &lb)) {
    // Some chunk's threshold lies above lb = tau_c, the candidates' K-th largest key: such a
    // chunk may miss part of the top, and only those chunks are rescored. Every other chunk's
    // threshold is <= tau_c, and it kept all its keys >= that threshold but ties dropped past
    // K candidates, which are never in the top K. Adding keys only raises the K-th largest, so
    // tau_c <= tau, the row's K-th largest key, and those chunks hold every key > tau and
    // enough ties at tau, in token order, for the top K. A histogram of their candidates plus
    // every key of the rescored chunks then counts every bin above tau's exactly and reaches K
    // at tau's bin b1, which gives the row's b1 and the count above it; the rescored chunks'
    // candidates are rewritten with every key in bins >= b1, and the final selection sees
    // every key of the top K.
    __syncthreads();
    const v4i qf = *reinterpret_cast<const v4i*>(q_idx + (row * (int64_t)D) + lane_part<D>(lane) * 16);
    for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
    if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
    __syncthreads();
    auto offending = [&](int ch) { return (uint32_t)cth[ch] > lb; };
    for (int ch = 0; ch < chunks; ++ch) {
      if (offending(ch)) {
        if (ch * kFChunk > r.pos) continue;
        const int blk0 = max(r.blk_first, ch * kFBlocks), blk1 = min(r.blk_last, ch * kFBlocks + kFBlocks - 1);
        for (int blk = blk0 + wave; blk <= blk1; blk += NW) {
          const int64_t base = block_base<D>(kv, r.b, r.gi, blk);
          if (base < 0) continue;  // wave-uniform
          v4i kd[Blk<D>::R];
          load_block<D>(kv.kidx_pool + base, lane, kd);
          const int s = to_token_order<D>(score_block<D>(qf, kd, lane), lane);
          const int tok = (blk << 6) + lane;
          if (tok >= r.P && tok <= r.pos) atomicAdd(&sh.hist[score_key(s) >> 12], 1u);
        }
      } else {
        const int2* cch = cand + (int64_t)ch * kFChunk;
        const int n = cc[ch];
        for (int j = tid; j < n; j += NT) atomicAdd(&sh.hist[(uint32_t)cch[j].x >> 12], 1u);
      }
    }
    __syncthreads();
    find_bin<NT>(sh, top_k);
    const uint32_t b1 = (uint32_t)sh.found_bin;
    const int above1 = sh.found_above;
    for (int ch = 0; ch < chunks; ++ch) {
      if (!offending(ch)) continue;  // uniform: every thread reads the same threshold
      int2* dst = w.cand + (row * chunks + ch) * (int64_t)kFChunk;
      int fill = 0;
      if (ch * kFChunk <= r.pos) {
        for (int slab = 0; slab < kFBlocks / NW; ++slab) {
          const int blk = ch * kFBlocks + slab * NW + wave;
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
      if (tid == 0) w.ccount[row * chunks + ch] = fill;
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    select_candidates<NT>(sh, s_off, cand, cc, chunks, kFChunk, b1, above1, top_k, out + r.nf);
  }
}

template <int D>
hipError_t launch_d(const KvView& kv, const int8_t* q_idx, int q_tail, int top_k, int32_t* indices,
                    void* ws, hipStream_t stream) {
  const int64_t rows = (int64_t)kv.batch * kv.num_idx_heads;
  const int chunks = (kv.max_seq_len + kFChunk - 1) / kFChunk;
  if (chunks > 1024) return hipErrorInvalidValue;
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
  const int64_t head = (2 * rows * chunks + 3) & ~(int64_t)3;  // ccount, cth
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
