// Exact top-K selection over int32 indexer scores, one workgroup per (sequence, query,
// indexer head) row.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析": §2.1 keeps
// the top-K key indices per query with a custom GPU reduction; §2.4 puts a forced prefix in
// front of every list without screening it.
//
// Order: score descending, token ascending. Scores are exact int32 with |s| < 2^23 (the
// indexer bounds them by d_idx * 2^14 <= 2^21), so key = s + 2^23 is a 24-bit unsigned
// order-preserving key, selected with a two-digit (12 + 12 bit) radix select in LDS:
//   pass 1  histogram of key >> 12 -> bin b1 holding the K-th largest key;
//   pass 2  histogram of the low 12 bits among keys in bin b1 -> the exact K-th key tau
//           and `need`, how many keys equal to tau are taken;
//   pass 3  one ordered sweep in token order: keys > tau are taken, and keys == tau while
//           fewer than `need` of them have been seen. Workgroup prefix sums (ballot +
//           popcount per wave, then across waves) give every taken token its slot, so the
//           list comes out ascending and no atomic decides any order.
// Histogram counts use LDS atomics, which are order-independent; the result is bit-exact
// and deterministic.
#include "sa_select_dev.h"

namespace sa {
namespace {

using namespace sel;


// Rows of up to 32768 candidates, streamed from the score row by one 256-thread workgroup
// per row: few registers and about 26 KB of LDS, so six rows are in flight per CU and their
// latencies overlap. Wave w streams the contiguous quarter [w * Q, (w + 1) * Q) of the row
// (Q a multiple of 64), so token order is wave-major.
//   sample    1024 keys (16 evenly spaced runs of 64) give a threshold bin theta (its tail
//             holds 1.25 times the sampled share of K plus three standard deviations plus 8);
//   stream    every key at or above T = theta << 12 is appended, in token order, to its wave's
//             list in LDS (ballots only, no barrier) as one word: its offset above T (clamped
//             to 65535) in the high half, its candidate index in the low half; the next batch
//             of loads is in flight while one is appended;
//   select    when the lists hold at least K keys and none overflowed, the K largest keys of the
//             row are the K largest on the lists (every key >= T is on one): a 256-bin histogram
//             of 256-unit bins above T and a 256-entry histogram of the bin holding the K-th
//             largest give it exactly (the top bin, which holds the clamped offsets, must not
//             be that bin), and the output is written from the lists in order;
//   fallback  otherwise the exact two-digit radix select streams the row again, its 4096-bin
//             histograms held in the list space.
constexpr int kStrNT = 256;
constexpr int kStrCap = 1536;  // list entries per wave
constexpr int kStrLd = 8;      // keys per lane per batch

//
// Coarse variant (COARSE = true, used by the fused prefill selection): the row holds the 16-bit
// order-preserving keys c(s) of the indexer (c(s1) > c(s2) implies s1 > s2; a key c holds
// exact scores in [c * 2^shift - B, c * 2^shift - B + 2^shift], B = d_idx * 2^14, shift =
// log2(d_idx) - 1). The lists and the fine histograms run on c as above. Every key with c above
// the K-th largest key tau_c is taken; when the keys equal to tau_c are more than are needed, their
// exact scores are recomputed from the int8 query and key rows (r = s - tau_c * 2^shift + B,
// at most 2^shift + 1 values) and a histogram of r picks them exactly, ties by token. When the
// lists cannot decide, the streamed exact radix select runs on exact scores computed from the
// int8 rows.
template <bool COARSE>
__global__ __launch_bounds__(kStrNT) void k_topk_row_stream(KvView kv, const void* __restrict__ scores_v,
                                                          int64_t row_stride, int q_len, int q_tail,
                                                          int top_k, int32_t* __restrict__ indices,
                                                          const int8_t* __restrict__ q_idx) {
  constexpr int NT = kStrNT;
  constexpr int NW = NT / 64;
  constexpr int kBatch = 64 * kStrLd;
  constexpr int kCap = kStrCap;
  static_assert(NW * kCap >= kBins, "the list space holds a 4096-bin histogram");
  // per-wave lists, entry = min(key - T, 65535) << 16 | candidate index (or a histogram)
  __shared__ __align__(16) uint32_t l_key[NW * kCap];
  __shared__ __align__(16) uint32_t s_hist[512];          // fine (256) and sub (256) bins
  __shared__ int32_t s_cnt[NW], s_cnt2[NW], s_seg[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t row = blockIdx.x;
  const int64_t bi = row / kv.num_idx_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int P = kv.prefix_len;
  const int W = P + top_k;
  const int pos = min(kv.seq_lens[b], kv.max_seq_len) - q_tail + i;
  const int32_t* srow = static_cast<const int32_t*>(scores_v) + row * row_stride;
  const uint16_t* crow = static_cast<const uint16_t*>(scores_v) + row * row_stride;
  int32_t* out = indices + row * W;
  // coarse rows: exact int8 score of token t (the row's query against the key's indexer row;
  // a page missing from the table reads page 0, like the indexer's unspecified case)
  const int D = kv.idx_dim;
  const int gi = (int)(row - bi * kv.num_idx_heads);
  auto exact_score = [&](int t) -> int32_t {
    const int lp = min(t >> kv.page_shift, kv.max_pages_per_seq - 1);
    int64_t ph = kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
    ph = (ph >= 0 && ph < kv.num_pages) ? ph : 0;
    const int8_t* kr = kv.kidx_pool + ((ph * kv.num_idx_heads + gi) * kv.page_size +
                                       (t & (kv.page_size - 1))) * (int64_t)D;
    const int8_t* qr = q_idx + row * (int64_t)D;
    int acc = 0;
    for (int c = 0; c < D; c += 16) {
      const int4 a = *reinterpret_cast<const int4*>(qr + c);
      const int4 k = *reinterpret_cast<const int4*>(kr + c);
      acc = __builtin_amdgcn_sdot4(a.x, k.x, acc, false);
      acc = __builtin_amdgcn_sdot4(a.y, k.y, acc, false);
      acc = __builtin_amdgcn_sdot4(a.z, k.z, acc, false);
      acc = __builtin_amdgcn_sdot4(a.w, k.w, acc, false);
    }
    return acc;
  };
  bool exact_mode = false;  // coarse rows: the fallback streams exact scores
  // selection key of a loaded value: 16-bit coarse key, or the 24-bit key of an exact score
  auto key_of = [&](uint32_t raw) -> uint32_t {
    return (COARSE && !exact_mode) ? raw : score_key((int32_t)raw);
  };
  constexpr int kShift1 = COARSE ? 4 : 12;  // sample histogram: key >> kShift1, 4096 bins

  const int nf = pos < 0 ? 0 : min(P, pos + 1);
  for (int j = tid; j < nf; j += NT) out[j] = j;
  const int n = pos - P + 1;
  if (n <= top_k) {
    const int m = n > 0 ? n : 0;
    for (int j = tid; j < m; j += NT) out[nf + j] = P + j;
    for (int j = nf + m + tid; j < W; j += NT) out[j] = -1;
    return;
  }
  out += nf;
  const int Q = ((n + NW * 64 - 1) / (NW * 64)) * 64;
  const int j_begin = wv * Q, j_end = min(n, j_begin + Q);  // this wave's candidates
  // kStrLd keys of the row per lane, requested together (index clamped into the row, so no
  // load is guarded and none is waited for where it is issued)
  auto load_batch = [&](int j0, uint32_t (&k)[kStrLd]) {
    if (COARSE && exact_mode) {
#pragma unroll
      for (int u = 0; u < kStrLd; ++u) k[u] = (uint32_t)exact_score(P + min(j0 + u * 64 + lane, n - 1));
    } else {
#pragma unroll
      for (int u = 0; u < kStrLd; ++u) {
        const int j = P + min(j0 + u * 64 + lane, n - 1);
        k[u] = COARSE ? (uint32_t)crow[j] : (uint32_t)srow[j];
      }
    }
  };
  // visits every key of this wave's range in order: f(j0, keys) per batch, loads one batch ahead
  auto stream = [&](auto&& f) {
    uint32_t ka[kStrLd], kb[kStrLd];
    int j0 = j_begin;
    if (j0 < j_end) load_batch(j0, ka);
    for (; j0 < j_end; j0 += 2 * kBatch) {
      const int j1 = j0 + kBatch;
      if (j1 < j_end) load_batch(j1, kb);
      f(j0, ka);
      if (j1 >= j_end) break;
      if (j1 + kBatch < j_end) load_batch(j1 + kBatch, ka);
      f(j1, kb);
    }
  };

  // sample: 1024 keys into a 4096-bin histogram (in the list space), taken as 16 runs of 64
  // consecutive keys at evenly spaced starts (2 cache lines each, so the sample reads about
  // 1/16 of a long row instead of every line of it), or evenly spaced keys in rows under 2048
  for (int j = tid; j < kBins; j += NT) l_key[j] = 0u;
  __syncthreads();
  const int ns = min(1024, n);
  {
    uint32_t sk[1024 / NT];
#pragma unroll
    for (int t = 0; t < 1024 / NT; ++t) {
      const int sidx = min(tid + t * NT, ns - 1);
      const int js = n >= 2048 ? (int)((int64_t)(sidx >> 6) * n / 16) + (sidx & 63)
                               : (int)((int64_t)sidx * n / ns);
      sk[t] = COARSE ? (uint32_t)crow[P + js] : (uint32_t)srow[P + js];
    }
#pragma unroll
    for (int t = 0; t < 1024 / NT; ++t)
      if (tid + t * NT < ns) atomicAdd(&l_key[key_of(sk[t]) >> kShift1], 1u);
  }
  __syncthreads();
  const float expect = (float)top_k * (float)ns / (float)n;
  const int target = (int)(1.25f * expect + 3.f * sqrtf(expect) + 8.f);
  uint32_t T = 0u;
  if (target < ns) {
    int ab = 0;
    T = (uint32_t)block_find_bin_segments<NW, 16>(l_key, s_seg, target, &ab) << kShift1;
  }
  for (int j = tid; j < 512; j += NT) s_hist[j] = 0u;
  __syncthreads();  // the sample histogram is no longer read

  // stream the row into the per-wave lists
  uint32_t* lk = l_key + wv * kCap;
  int cnt = 0;
  if constexpr (COARSE) {
    // Lane-major: each lane takes 8 consecutive 16-bit keys (one 16-byte load) per step, so a
    // step covers 512 consecutive keys with lane order = token order; one wave prefix sum of
    // the per-lane counts places a lane's kept keys, and it loops over those only. Four steps
    // of loads are kept in flight.
    if (j_begin < j_end) {  // uniform
      const int r_begin = P + j_begin, r_end = P + j_end;  // row indices of this wave's range
      const int a0 = r_begin & ~7;
      const int a_last = (r_end - 1) & ~7;  // last 8-key block holding range keys (in bounds)
      auto ld = [&](int a) {
        return *reinterpret_cast<const uint4*>(crow + min(a + lane * 8, a_last));
      };
      auto put = [&](int a, const uint4 v) {
        const int r0 = a + lane * 8;  // row index of this lane's first key (before clamping)
        const uint64_t lo = ((uint64_t)v.y << 32) | v.x, hi = ((uint64_t)v.w << 32) | v.z;
        uint32_t bits = 0;
        if (a >= r_begin && a + 512 <= r_end) {  // uniform: every key of the step is in range
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t key = (uint32_t)(((u < 4 ? lo : hi) >> ((u & 3) * 16)) & 0xffffu);
            bits |= (uint32_t)(key >= T) << u;
          }
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t key = (uint32_t)(((u < 4 ? lo : hi) >> ((u & 3) * 16)) & 0xffffu);
            const bool in = (unsigned)(r0 + u - r_begin) < (unsigned)(r_end - r_begin);
            bits |= (uint32_t)(in && key >= T) << u;
          }
        }
        const int c = __popc(bits);
        const int incl = wave_incl_sum(c);
        int o = cnt + incl - c;
        cnt += __builtin_amdgcn_readlane(incl, 63);
        if (cnt <= kCap) {  // uniform: the whole step fits in the list
          while (bits != 0u) {
            const int u = __builtin_ctz(bits);
            bits &= bits - 1u;
            const uint32_t key = (uint32_t)(((u < 4 ? lo : hi) >> ((u & 3) * 16)) & 0xffffu);
            lk[o++] = ((key - T) << 16) | (uint32_t)(r0 + u - P);
          }
        } else {
          while (bits != 0u) {
            const int u = __builtin_ctz(bits);
            bits &= bits - 1u;
            const uint32_t key = (uint32_t)(((u < 4 ? lo : hi) >> ((u & 3) * 16)) & 0xffffu);
            if (o < kCap) lk[o] = ((key - T) << 16) | (uint32_t)(r0 + u - P);
            ++o;
          }
        }
      };
      // kAhead steps of loads in flight per wave (a step is one 1 KiB load instruction; with
      // one step ahead the stream waited a round trip per step)
      constexpr int kAhead = 4;
      uint4 ring[kAhead];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) ring[k] = ld(a0 + k * 512);  // clamped: in bounds
      for (int a = a0; a <= a_last; a += 512 * kAhead) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
          const int ak = a + k * 512;
          if (ak > a_last) break;  // uniform
          const uint4 v = ring[k];
          ring[k] = ld(ak + kAhead * 512);
          put(ak, v);
        }
      }
    }
  } else {
    stream([&](int j0, const uint32_t (&k)[kStrLd]) {
#pragma unroll
      for (int u = 0; u < kStrLd; ++u) {
        const int j = j0 + u * 64 + lane;
        const uint32_t key = key_of(k[u]);
        const bool keep = j < j_end && key >= T;
        const uint64_t km = __ballot(keep);
        const int o = cnt + __popcll(km & lt_mask);
        if (keep && o < kCap) lk[o] = (min(key - T, 65535u) << 16) | (uint32_t)j;
        cnt += __popcll(km);
      }
    });
  }
  if (lane == 0) s_cnt[wv] = cnt;
  __syncthreads();
  int m = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    m += s_cnt[w];
    over = over || s_cnt[w] > kCap;
  }
  if (m >= top_k && !over) {
    for (int c = lane; c < cnt; c += 64) atomicAdd(&s_hist[lk[c] >> 24], 1u);
    __syncthreads();
    int above_fb = 0;
    const int fb = block_find_bin_segments<NW, 1>(s_hist, s_seg, top_k, &above_fb);
    // (coarse offsets are never clamped: every bin is exact)
    if (fb >= 0 && (COARSE || fb < 255)) {  // uniform
      // offsets (key - T) from here on; the clamped ones all lie in bin 255, above tau
      const uint32_t lo = (uint32_t)fb << 8;
      for (int c = lane; c < cnt; c += 64) {
        const uint32_t off = lk[c] >> 16;
        if (off >= lo && off < lo + 256u) atomicAdd(&s_hist[256 + (off - lo)], 1u);
      }
      __syncthreads();
      int above_sb = 0;
      const int sb = wave_find_bin<4>(s_hist + 256, top_k - above_fb, &above_sb);
      const uint32_t tau = lo + (uint32_t)sb;
      const int need = top_k - above_fb - above_sb;
      int gt_w = 0, eq_w = 0;
      for (int c0 = 0; c0 < cnt; c0 += 64) {
        const int c = c0 + lane;
        const uint32_t key = c < cnt ? lk[c] >> 16 : 0u;
        gt_w += __popcll(__ballot(c < cnt && key > tau));
        eq_w += __popcll(__ballot(c < cnt && key == tau));
      }
      if (lane == 0) {
        s_cnt[wv] = gt_w;
        s_cnt2[wv] = eq_w;
      }
      __syncthreads();
      if constexpr (COARSE) {
        int eq_total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) eq_total += s_cnt2[w];
        if (eq_total > need) {  // uniform: the keys equal to tau_c are decided by exact scores
          const int shift = D == 32 ? 4 : (D == 64 ? 5 : 6);
          const int64_t lo_s = ((int64_t)(T + tau) << shift) - ((int64_t)D << 14);
          uint32_t* rh = s_hist;  // free again: 256 bins of r
          for (int j = tid; j < 256; j += NT) rh[j] = 0u;
          __syncthreads();
          // one pass computes the exact scores: every entry's high half becomes its class,
          // 0xffff above tau, 0x100 | r at tau, 0 below
          for (int c = lane; c < cnt; c += 64) {
            const uint32_t e = lk[c];
            const uint32_t off = e >> 16;
            uint32_t cls = 0u;
            if (off > tau) {
              cls = 0xffffu;
            } else if (off == tau) {
              const int64_t rr = exact_score(P + (int)(e & 0xffffu)) - lo_s;
              const uint32_t r = (uint32_t)(rr < 0 ? 0 : (rr > 255 ? 255 : rr));
              atomicAdd(&rh[r], 1u);
              cls = 0x100u | r;
            }
            lk[c] = (cls << 16) | (e & 0xffffu);
          }
          __syncthreads();
          int above_r = 0;
          const uint32_t rstar = 0x100u | (uint32_t)wave_find_bin<4>(rh, need, &above_r);
          const int need_r = need - above_r;  // keys at r* to take, in token order
          // classes: gt 0xffff; above r* (0x100 | r, r > r*) taken; at r* the first need_r
          int tk_c = 0, er_c = 0;
          for (int c0 = 0; c0 < cnt; c0 += 64) {
            const int c = c0 + lane;
            const uint32_t cls = c < cnt ? lk[c] >> 16 : 0u;
            tk_c += __popcll(__ballot(cls > rstar));
            er_c += __popcll(__ballot(cls == rstar));
          }
          __syncthreads();  // every wave has read the first-pass counts
          if (lane == 0) {
            s_cnt[wv] = tk_c;
            s_cnt2[wv] = er_c;
          }
          __syncthreads();
          int taken = 0, er_run = 0;
          for (int w = 0; w < wv; ++w) {
            taken += s_cnt[w];
            er_run += s_cnt2[w];
          }
          taken += min(er_run, need_r);
          for (int c0 = 0; c0 < cnt; c0 += 64) {
            const int c = c0 + lane;
            const uint32_t e = c < cnt ? lk[c] : 0u;
            const uint32_t cls = e >> 16;
            const bool eqr = c < cnt && cls == rstar;
            const uint64_t rm = __ballot(eqr);
            const bool take = (c < cnt && cls > rstar) || (eqr && er_run + __popcll(rm & lt_mask) < need_r);
            const uint64_t tm = __ballot(take);
            if (take) out[taken + __popcll(tm & lt_mask)] = P + (int)(e & 0xffffu);
            taken += __popcll(tm);
            er_run += __popcll(rm);
          }
          return;
        }
      }
      int gt_run = 0, eq_run = 0;
      for (int w = 0; w < wv; ++w) {
        gt_run += s_cnt[w];
        eq_run += s_cnt2[w];
      }
      for (int c0 = 0; c0 < cnt && gt_run + min(eq_run, need) < top_k; c0 += 64) {
        const int c = c0 + lane;
        const uint32_t e = c < cnt ? lk[c] : 0u;
        const uint32_t key = e >> 16;
        const bool gt = c < cnt && key > tau;
        const bool eq = c < cnt && key == tau;
        const uint64_t gm = __ballot(gt), em = __ballot(eq);
        const int gt_before = gt_run + __popcll(gm & lt_mask);
        const int eq_before = eq_run + __popcll(em & lt_mask);
        if (gt || (eq && eq_before < need)) out[gt_before + min(eq_before, need)] = P + (int)(e & 0xffffu);
        gt_run += __popcll(gm);
        eq_run += __popcll(em);
      }
      return;
    }
  }
  // exact two-digit radix select, streamed; the histograms live in the list space (coarse
  // rows stream exact scores recomputed from the int8 rows)
  exact_mode = true;
  uint32_t* hist = l_key;
  __syncthreads();  // the lists are no longer read
  for (int j = tid; j < kBins; j += NT) hist[j] = 0u;
  __syncthreads();
  stream([&](int j0, const uint32_t (&k)[kStrLd]) {
#pragma unroll
    for (int u = 0; u < kStrLd; ++u)
      if (j0 + u * 64 + lane < j_end) atomicAdd(&hist[key_of(k[u]) >> 12], 1u);
  });
  __syncthreads();
  int above1 = 0;
  const uint32_t b1 = (uint32_t)block_find_bin_segments<NW, 16>(hist, s_seg, top_k, &above1);
  __syncthreads();
  for (int j = tid; j < kBins; j += NT) hist[j] = 0u;
  __syncthreads();
  stream([&](int j0, const uint32_t (&k)[kStrLd]) {
#pragma unroll
    for (int u = 0; u < kStrLd; ++u) {
      const uint32_t key = key_of(k[u]);
      if (j0 + u * 64 + lane < j_end && (key >> 12) == b1) atomicAdd(&hist[key & 0xfff], 1u);
    }
  });
  __syncthreads();
  int above2 = 0;
  const uint32_t b2 = (uint32_t)block_find_bin_segments<NW, 16>(hist, s_seg, top_k - above1, &above2);
  const uint32_t tau = (b1 << 12) | b2;
  const int need = top_k - above1 - above2;
  int gt_w = 0, eq_w = 0;
  stream([&](int j0, const uint32_t (&k)[kStrLd]) {
#pragma unroll
    for (int u = 0; u < kStrLd; ++u) {
      const bool valid = j0 + u * 64 + lane < j_end;
      const uint32_t key = key_of(k[u]);
      gt_w += __popcll(__ballot(valid && key > tau));
      eq_w += __popcll(__ballot(valid && key == tau));
    }
  });
  if (lane == 0) {
    s_cnt[wv] = gt_w;
    s_cnt2[wv] = eq_w;
  }
  __syncthreads();
  int gt_run = 0, eq_run = 0;
  for (int w = 0; w < wv; ++w) {
    gt_run += s_cnt[w];
    eq_run += s_cnt2[w];
  }
  stream([&](int j0, const uint32_t (&k)[kStrLd]) {
#pragma unroll
    for (int u = 0; u < kStrLd; ++u) {
      const int j = j0 + u * 64 + lane;
      const uint32_t key = key_of(k[u]);
      const bool gt = j < j_end && key > tau;
      const bool eq = j < j_end && key == tau;
      const uint64_t gm = __ballot(gt), em = __ballot(eq);
      const int gt_before = gt_run + __popcll(gm & lt_mask);
      const int eq_before = eq_run + __popcll(em & lt_mask);
      if (gt || (eq && eq_before < need)) out[gt_before + min(eq_before, need)] = P + j;
      gt_run += __popcll(gm);
      eq_run += __popcll(em);
    }
  });
}

// Rows longer than the register path holds: three passes over the scores in global memory
// (high digit, low digit within bin b1, ordered compaction by wave segments).
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_row(KvView kv, const int32_t* __restrict__ scores,
                                                 int64_t row_stride, int q_len, int q_tail,
                                                 int top_k, int32_t* __restrict__ indices) {
  constexpr int NW = NT / 64;
  __shared__ TopkShared<NT> sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t row = blockIdx.x;
  const int64_t bi = row / kv.num_idx_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int P = kv.prefix_len;
  const int W = P + top_k;
  const int pos = min(kv.seq_lens[b], kv.max_seq_len) - q_tail + i;
  const int32_t* srow = scores + row * row_stride;
  int32_t* out = indices + row * W;
  const int nf = pos < 0 ? 0 : min(P, pos + 1);
  for (int j = tid; j < nf; j += NT) out[j] = j;
  const int n = pos - P + 1;
  if (n <= top_k) {
    const int m = n > 0 ? n : 0;
    for (int j = tid; j < m; j += NT) out[nf + j] = P + j;
    for (int j = nf + m + tid; j < W; j += NT) out[j] = -1;
    return;
  }
  if (tid == 0) {
    sh.found_bin = 0;
    sh.found_above = 0;
  }
  for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0;
  __syncthreads();
  // kLd keys per thread are requested at once (indices clamped into the row, so no load is
  // guarded) before any is used.
  constexpr int kLd = 8;
  auto load_batch = [&](int j0, int step, uint32_t (&k)[kLd]) {
#pragma unroll
    for (int u = 0; u < kLd; ++u) k[u] = (uint32_t)srow[P + min(j0 + u * step, n - 1)];
#pragma unroll
    for (int u = 0; u < kLd; ++u) k[u] = score_key((int32_t)k[u]);
  };
  for (int j0 = tid; j0 < n; j0 += kLd * NT) {
    uint32_t k[kLd];
    load_batch(j0, NT, k);
#pragma unroll
    for (int u = 0; u < kLd; ++u)
      if (j0 + u * NT < n) atomicAdd(&sh.hist[k[u] >> 12], 1u);
  }
  __syncthreads();
  find_bin<NT>(sh, top_k);
  const uint32_t b1 = sh.found_bin;
  const int above1 = sh.found_above;
  for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0;
  __syncthreads();
  for (int j0 = tid; j0 < n; j0 += kLd * NT) {
    uint32_t k[kLd];
    load_batch(j0, NT, k);
#pragma unroll
    for (int u = 0; u < kLd; ++u)
      if (j0 + u * NT < n && (k[u] >> 12) == b1) atomicAdd(&sh.hist[k[u] & 0xfff], 1u);
  }
  __syncthreads();
  find_bin<NT>(sh, top_k - above1);
  const uint32_t tau = (b1 << 12) | (uint32_t)sh.found_bin;
  const int need = top_k - above1 - sh.found_above;
  const int seg = ((n + NW * 64 - 1) / (NW * 64)) * 64;
  const int s0 = wv * seg, s1 = min(n, s0 + seg);
  int gt_w = 0, eq_w = 0;
  for (int j0 = s0; j0 < s1; j0 += kLd * 64) {
    uint32_t k[kLd];
    load_batch(j0 + lane, 64, k);
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int j = j0 + u * 64 + lane;
      gt_w += __popcll(__ballot(j < s1 && k[u] > tau));
      eq_w += __popcll(__ballot(j < s1 && k[u] == tau));
    }
  }
  if (lane == 0) {
    sh.wave_tot[wv] = gt_w;
    sh.wave_tot2[wv] = eq_w;
  }
  __syncthreads();
  int gt_run = 0, eq_run = 0;
  for (int w = 0; w < wv; ++w) {
    gt_run += sh.wave_tot[w];
    eq_run += sh.wave_tot2[w];
  }
  for (int j0 = s0; j0 < s1 && gt_run + min(eq_run, need) < top_k; j0 += kLd * 64) {
    uint32_t k[kLd];
    load_batch(j0 + lane, 64, k);
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int j = j0 + u * 64 + lane;
      const bool gt = j < s1 && k[u] > tau;
      const bool eq = j < s1 && k[u] == tau;
      const uint64_t gm = __ballot(gt), em = __ballot(eq);
      const int gt_before = gt_run + __popcll(gm & lt_mask);
      const int eq_before = eq_run + __popcll(em & lt_mask);
      if (gt || (eq && eq_before < need)) out[nf + gt_before + min(eq_before, need)] = P + j;
      gt_run += __popcll(gm);
      eq_run += __popcll(em);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Long rows (decode: a handful of rows of 10^5..10^6 scores) are split over many workgroups
// of kChunk scores each, in four launches plus a clearing fill:
//   hist1    per chunk, an LDS histogram of key >> 12, added into the row histogram with
//            global atomics on non-empty bins (integer sums: the result does not depend on
//            their order);
//   find     one workgroup per row finds b1, the bin holding the K-th largest key, and
//            `above1`, the number of keys in higher bins;
//   collect  per chunk, the keys in bins >= b1 (every selected key, plus the rest of bin b1)
//            are compacted in token order into the chunk's own slot range, with their count;
//   final    one workgroup per row walks those candidates in chunk order: an LDS histogram of
//            the low digit of the bin-b1 keys gives tau and `need`, then an ordered pass keeps
//            keys > tau and the first `need` keys == tau, writing them ascending.
// Typical rows leave about K + |bin b1| candidates, so final touches a few thousand entries;
// with heavy ties it simply walks more of them. Workspace (int32 words):
//   hist1 [rows][4096] | state [rows][4] | ccount [rows][chunks] | cand [rows][chunks][kChunk][2]
constexpr int kChunk = 8192;
constexpr int kMT = 256;
constexpr int kLoads = kChunk / (kMT * 4);
constexpr int kFinalNT = 1024;

struct RowGeom {
  int pos, nf, n, P, W;
};

__device__ __forceinline__ RowGeom row_geom(const KvView& kv, int64_t row, int q_len, int q_tail,
                                            int top_k) {
  const int64_t bi = row / kv.num_idx_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  RowGeom g;
  g.P = kv.prefix_len;
  g.W = g.P + top_k;
  g.pos = min(kv.seq_lens[b], kv.max_seq_len) - q_tail + i;
  g.nf = g.pos < 0 ? 0 : min(g.P, g.pos + 1);
  g.n = g.pos - g.P + 1;
  return g;
}

struct MultiWs {
  uint32_t* hist1;
  int32_t* state;   // [rows][4]: b1, above1
  int32_t* ccount;  // [rows][chunks]
  int2* cand;       // [rows][chunks][kChunk]: (key, token)
  int chunks;
};

__device__ __forceinline__ MultiWs multi_ws(void* ws, int64_t rows, int chunks) {
  MultiWs w;
  w.hist1 = static_cast<uint32_t*>(ws);
  w.state = reinterpret_cast<int32_t*>(w.hist1 + rows * kBins);
  w.ccount = w.state + rows * 4;
  int64_t off = (int64_t)(rows * (kBins + 4) + rows * chunks);
  off = (off + 3) & ~(int64_t)3;  // 16-byte alignment for the candidate pairs
  w.cand = reinterpret_cast<int2*>(static_cast<int32_t*>(ws) + off);
  w.chunks = chunks;
  return w;
}

__global__ __launch_bounds__(256) void k_topk_zero(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256)
    p[j] = 0u;
}

__global__ __launch_bounds__(kMT) void k_topk_hist1(KvView kv, const int32_t* __restrict__ scores,
                                                    int64_t row_stride, int q_len, int q_tail,
                                                    int top_k, void* ws, int chunks) {
  __shared__ uint32_t h[kBins];
  const int64_t row = blockIdx.y;
  const RowGeom g = row_geom(kv, row, q_len, q_tail, top_k);
  const int t_begin = blockIdx.x * kChunk;
  if (g.n <= top_k || t_begin > g.pos) return;
  const MultiWs w = multi_ws(ws, gridDim.y, chunks);
  for (int j = threadIdx.x; j < kBins; j += kMT) h[j] = 0u;
  __syncthreads();
  const int32_t* srow = scores + row * row_stride;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int t = t_begin + j * kMT * 4 + threadIdx.x * 4;
    if (t <= g.pos) {
      const int4 v = *reinterpret_cast<const int4*>(srow + t);
      const int e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (t + u >= g.P && t + u <= g.pos) atomicAdd(&h[score_key(e[u]) >> 12], 1u);
    }
  }
  __syncthreads();
  uint32_t* dst = w.hist1 + row * kBins;
  for (int j = threadIdx.x; j < kBins; j += kMT)
    if (h[j]) atomicAdd(&dst[j], h[j]);
}

__global__ __launch_bounds__(kMT) void k_topk_find(KvView kv, int q_len, int q_tail, int top_k,
                                                   void* ws, int chunks) {
  __shared__ TopkShared<kMT> sh;
  const int64_t row = blockIdx.x;
  const RowGeom g = row_geom(kv, row, q_len, q_tail, top_k);
  if (g.n <= top_k) return;
  const MultiWs w = multi_ws(ws, gridDim.x, chunks);
  const uint32_t* h1 = w.hist1 + row * kBins;
  for (int j = threadIdx.x; j < kBins; j += kMT) sh.hist[j] = h1[j];
  if (threadIdx.x == 0) { sh.found_bin = 0; sh.found_above = 0; }
  __syncthreads();
  find_bin<kMT>(sh, top_k);
  if (threadIdx.x == 0) {
    w.state[row * 4 + 0] = sh.found_bin;
    w.state[row * 4 + 1] = sh.found_above;
  }
}

__global__ __launch_bounds__(kMT) void k_topk_collect(KvView kv, const int32_t* __restrict__ scores,
                                                      int64_t row_stride, int q_len, int q_tail,
                                                      int top_k, void* ws, int chunks) {
  __shared__ int32_t wave_tot[kMT / 64];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const RowGeom g = row_geom(kv, row, q_len, q_tail, top_k);
  if (g.n <= top_k) return;
  const MultiWs w = multi_ws(ws, gridDim.y, chunks);
  const int t_begin = c * kChunk;
  if (t_begin > g.pos) {
    if (threadIdx.x == 0) w.ccount[row * chunks + c] = 0;
    return;
  }
  const uint32_t b1 = (uint32_t)w.state[row * 4 + 0];
  int2* dst = w.cand + (row * chunks + c) * (int64_t)kChunk;
  const int32_t* srow = scores + row * row_stride;
  int fill = 0;
  for (int j = 0; j < kLoads; ++j) {
    const int t = t_begin + j * kMT * 4 + threadIdx.x * 4;
    int e[4] = {0, 0, 0, 0};
    if (t <= g.pos) {
      const int4 v = *reinterpret_cast<const int4*>(srow + t);
      e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
    }
    int n_keep = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = t + u >= g.P && t + u <= g.pos;
      n_keep += (in && (score_key(e[u]) >> 12) >= b1) ? 1 : 0;
    }
    int tile;
    int slot = fill + block_excl_scan<kMT>(n_keep, wave_tot, &tile);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t key = score_key(e[u]);
      const bool in = t + u >= g.P && t + u <= g.pos;
      if (in && (key >> 12) >= b1) dst[slot++] = make_int2((int)key, t + u);
    }
    fill += tile;
  }
  if (threadIdx.x == 0) w.ccount[row * chunks + c] = fill;
}

__global__ __launch_bounds__(kFinalNT) void k_topk_final(KvView kv, int q_len, int q_tail,
                                                         int top_k, void* ws, int chunks,
                                                         int32_t* __restrict__ indices) {
  constexpr int NT = kFinalNT;
  __shared__ TopkShared<NT> sh;
  __shared__ int32_t s_off[1025];  // exclusive candidate offsets of the chunks (<= 1024 chunks)
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const RowGeom g = row_geom(kv, row, q_len, q_tail, top_k);
  int32_t* out = indices + row * g.W;
  for (int j = tid; j < g.nf; j += NT) out[j] = j;
  if (g.n <= top_k) {
    const int m = g.n > 0 ? g.n : 0;
    for (int j = tid; j < m; j += NT) out[g.nf + j] = g.P + j;
    for (int j = g.nf + m + tid; j < g.W; j += NT) out[j] = -1;
    return;
  }
  const MultiWs w = multi_ws(ws, gridDim.x, chunks);
  const uint32_t b1 = (uint32_t)w.state[row * 4 + 0];
  const int above1 = w.state[row * 4 + 1];
  select_candidates<NT>(sh, s_off, w.cand + row * chunks * (int64_t)kChunk,
                        w.ccount + row * chunks, chunks, kChunk, b1, above1, top_k, out + g.nf);
}

bool use_multi(int64_t rows, int longest) { return longest >= 16384 && rows <= 2048; }

int64_t multi_chunks(const KvView& kv) { return (kv.max_seq_len + kChunk - 1) / kChunk; }

}  // namespace

size_t topk_workspace_bytes(const KvView& kv, int q_len, int) {
  const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
  if (!use_multi(rows, kv.max_seq_len - kv.prefix_len)) return 0;
  const int64_t chunks = multi_chunks(kv);
  const int64_t head = (rows * (kBins + 4) + rows * chunks + 3) & ~(int64_t)3;
  return (size_t)(head + rows * chunks * kChunk * 2) * sizeof(int32_t);
}

hipError_t launch_topk(const KvView& kv, const int32_t* scores, int64_t row_stride, int q_len,
                       int q_tail, int top_k, int32_t* indices, void* ws, size_t,
                       hipStream_t stream) {
  const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
  if (rows == 0) return hipSuccess;
  const int longest = kv.max_seq_len - kv.prefix_len;
  if (use_multi(rows, longest)) {
    const int chunks = (int)multi_chunks(kv);
    if (chunks > 1024) return hipErrorInvalidValue;
    const int64_t nz = rows * kBins;
    const int64_t zb = (nz + 255) / 256 < 4096 ? (nz + 255) / 256 : 4096;
    hipLaunchKernelGGL(k_topk_zero, dim3((unsigned)zb), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), nz);
    const dim3 grid(chunks, (unsigned)rows);
    hipLaunchKernelGGL(k_topk_hist1, grid, dim3(kMT), 0, stream, kv, scores, row_stride, q_len,
                       q_tail, top_k, ws, chunks);
    hipLaunchKernelGGL(k_topk_find, dim3((unsigned)rows), dim3(kMT), 0, stream, kv, q_len, q_tail,
                       top_k, ws, chunks);
    hipLaunchKernelGGL(k_topk_collect, grid, dim3(kMT), 0, stream, kv, scores, row_stride, q_len,
                       q_tail, top_k, ws, chunks);
    hipLaunchKernelGGL(k_topk_final, dim3((unsigned)rows), dim3(kFinalNT), 0, stream, kv, q_len,
                       q_tail, top_k, ws, chunks, indices);
    return hipGetLastError();
  }
  // rows that fit are held in registers (one read of the scores); longer ones take three passes
  if (longest <= 32768) {
    hipLaunchKernelGGL(k_topk_row_stream<false>, dim3((unsigned)rows), dim3(kStrNT), 0, stream,
                       kv, (const void*)scores, row_stride, q_len, q_tail, top_k, indices,
                       (const int8_t*)nullptr);
  } else {
    hipLaunchKernelGGL((k_topk_row<1024>), dim3((unsigned)rows), dim3(1024), 0, stream, kv, scores,
                       row_stride, q_len, q_tail, top_k, indices);
  }
  return hipGetLastError();
}

bool topk_coarse_applies(const KvView& kv, int q_len) {
  const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
  const int longest = kv.max_seq_len - kv.prefix_len;
  return q_len >= 16 && longest <= 32768 && !use_multi(rows, longest);
}

hipError_t launch_topk_coarse(const KvView& kv, const uint16_t* keys, int64_t row_stride, int q_len,
                              int q_tail, int top_k, const int8_t* q_idx, int32_t* indices,
                              hipStream_t stream) {
  const int64_t rows = (int64_t)kv.batch * q_len * kv.num_idx_heads;
  if (rows == 0) return hipSuccess;
  if (!topk_coarse_applies(kv, q_len)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_topk_row_stream<true>, dim3((unsigned)rows), dim3(kStrNT), 0, stream, kv,
                     (const void*)keys, row_stride, q_len, q_tail, top_k, indices, q_idx);
  return hipGetLastError();
}

}  // namespace sa
