// Device helpers for exact top-K selection over int32 indexer scores (shared by the
// stand-alone selection kernels and the fused index + selection kernels).
//
// Scores are exact int32 with |s| < 2^23 (an int8 indexer bounds them by d_idx * 2^14 <=
// 2^21), so key = s + 2^23 is a 24-bit unsigned key that preserves order; selection works
// on two 12-bit digits of it.
#pragma once

#include "sa_common.h"

namespace sa {
namespace sel {

constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t score_key(int32_t s) {
  int64_t k = (int64_t)s + (1 << 23);
  k = k < 0 ? 0 : (k > 0xffffff ? 0xffffff : k);
  return (uint32_t)k;
}

template <int NT>
struct TopkShared {
  alignas(16) uint32_t hist[kBins];
  int32_t wave_tot[NT / 64];
  int32_t wave_tot2[NT / 64];
  int32_t found_bin;
  int32_t found_above;
};

// Inclusive prefix sum / maximum over the 64 lanes of a wave, on DPP: row_shr 1, 2, 4, 8
// inside each 16-lane row, then row_bcast:15 (rows 1 and 3 add the last lane of the row
// before) and row_bcast:31 (rows 2 and 3 add lane 31). Lanes shifted in from outside a row
// read 0 (for the maximum, 0 is the identity on the non-negative values it is used on).
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ int wave_incl_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
  return v;
}

// Wave-uniform search over a histogram held in LDS, highest bin first: lane l owns the PER
// consecutive bins starting at l * PER. Returns the bin holding the k-th largest element and
// writes the number of elements in higher bins to *above; returns -1 if the histogram holds
// fewer than k elements. Every wave may run it at once on the same bins (read only).
template <int PER>
__device__ __forceinline__ int wave_find_bin(const uint32_t* hist, int k, int* above) {
  const int lane = threadIdx.x & 63;
  uint32_t h[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + lane * PER + i);
    h[i] = v.x; h[i + 1] = v.y; h[i + 2] = v.z; h[i + 3] = v.w;
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += (int)h[i];
  const int incl = wave_incl_sum(s);
  const int all = __builtin_amdgcn_readlane(incl, 63);
  const int mine_above = all - incl;  // elements in the bins of higher lanes
  const uint64_t hit = __ballot(mine_above < k && mine_above + s >= k);
  if (hit == 0) return -1;
  const int L = __builtin_ctzll(hit);
  int bin = -1, acc = mine_above, res_above = 0;
  if (lane == L) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (bin < 0 && acc + (int)h[i] >= k) { bin = lane * PER + i; res_above = acc; }
      acc += (int)h[i];
    }
  }
  *above = __builtin_amdgcn_readlane(res_above, L);
  return __builtin_amdgcn_readlane(bin, L);
}

// Bin holding the k-th largest element of a histogram of NW * 64 * BPL bins in LDS (wave w
// totals bins [w * 64 * BPL, (w + 1) * 64 * BPL) into seg[w], one barrier, then every wave
// finds the segment and the bin inside it on its own, so all waves leave with the same
// answer). Writes the number of elements in higher bins to *above; returns -1 if the
// histogram holds fewer than k. BPL is 1 or a multiple of 4.
template <int NW, int BPL = 1>
__device__ __forceinline__ int block_find_bin_segments(const uint32_t* hist, int32_t* seg, int k,
                                                       int* above) {
  static_assert(BPL == 1 || BPL % 4 == 0, "bins per lane: 1 or a multiple of 4");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  {
    int v = 0;
    if constexpr (BPL == 1) {
      v = (int)hist[wave * 64 + lane];
    } else {
#pragma unroll
      for (int i = 0; i < BPL; i += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(hist + (wave * 64 + lane) * BPL + i);
        v += (int)(q.x + q.y + q.z + q.w);
      }
    }
    const int t = wave_incl_sum(v);
    if (lane == 63) seg[wave] = t;
  }
  __syncthreads();
  const int sv = lane < NW ? seg[lane] : 0;
  const int incl_s = wave_incl_sum(sv);
  const int above_s = __builtin_amdgcn_readlane(incl_s, 63) - incl_s;  // in later segments
  const uint64_t hit = __ballot(lane < NW && above_s < k && above_s + sv >= k);
  if (hit == 0) return -1;
  const int S = __builtin_ctzll(hit);
  const int base_s = __builtin_amdgcn_readlane(above_s, S);
  if constexpr (BPL == 1) {
    const int hv = (int)hist[S * 64 + lane];
    const int incl_b = wave_incl_sum(hv);
    const int ab = base_s + __builtin_amdgcn_readlane(incl_b, 63) - incl_b;  // in higher bins
    const uint64_t hit2 = __ballot(ab < k && ab + hv >= k);
    const int L = __builtin_ctzll(hit2);
    *above = __builtin_amdgcn_readlane(ab, L);
    return S * 64 + L;
  } else {
    int ab = 0;
    const int bin = wave_find_bin<BPL>(hist + S * 64 * BPL, k - base_s, &ab);
    *above = base_s + ab;
    return S * 64 * BPL + bin;
  }
}

// Inclusive prefix sum over the workgroup (thread order); returns the inclusive value and
// writes the workgroup total to *total. Contains two barriers.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int32_t* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  v = wave_incl_sum(v);
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int x = wave_tot[w];
    before += (w < wave) ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Adds one to hist[bin] for every active lane of the wave. The lanes whose bin equals the
// first active lane's add together with one atomic, so a wave whose keys share a bin (packed
// or tied scores) costs one LDS atomic instead of 64 serialised on one address.
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, uint32_t bin, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int first = __builtin_ctzll(act);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  const uint64_t same = __ballot(active && bin == b0);
  if (active && bin != b0) atomicAdd(&hist[bin], 1u);
  if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], (uint32_t)__popcll(same));
}

// Largest bin b with sum(hist[b..]) >= k; stores b and sum(hist[b+1..]) in shared memory.
template <int NT>
__device__ __forceinline__ void find_bin(TopkShared<NT>& sh, int k) {
  constexpr int C = kBins / NT;
  const int base = threadIdx.x * C;
  int s = 0;
#pragma unroll
  for (int j = 0; j < C; ++j) s += sh.hist[base + j];
  int total;
  const int incl = block_incl_scan<NT>(s, sh.wave_tot, &total);
  int acc = total - incl;  // sum of bins above this thread's range
  if (acc < k && acc + s >= k) {
    for (int j = C - 1; j >= 0; --j) {
      const int h = sh.hist[base + j];
      if (acc + h >= k) {
        sh.found_bin = base + j;
        sh.found_above = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// Workgroup-exclusive prefix sum (thread order) and total; two barriers.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int32_t* wave_tot, int* total) {
  const int incl = block_incl_scan<NT>(v, wave_tot, total);
  return incl - v;
}

// Exact top-K among candidates that were compacted per chunk, in token order:
//   cand [chunks][chunk_cap] (key, token) with ccount[chunk] valid entries each.
// Every selected key must be among them; b1 is the bin (key >> 12) holding the K-th largest
// key and `above1` the number of keys in higher bins. Candidates below bin b1 may be
// present and are ignored. Writes the selected tokens, ascending, to out[0..top_k).
// s_off needs chunks + 1 <= NT + 1 entries.
//
// After the threshold (tau, need) is known, each wave owns one contiguous segment of the
// candidate list: it counts its keys > tau and == tau with ballots, one workgroup scan over
// the waves gives every segment its output offset and its number of earlier keys == tau,
// and each wave then writes its taken keys in order. Two barriers instead of two
// workgroup scans per 1024 candidates.
//
// With check_key >= 0, b1 and above1 are not given: they are taken from the candidates' own
// histogram, and the candidates must hold every key of the row >= check_key. If the K-th
// largest candidate key tau is below check_key, that is not enough to know the row's K-th
// largest key: nothing is written, *tau_lb receives tau and the call returns false
// (uniformly). Otherwise, and always with check_key < 0, it returns true.
template <int NT>
__device__ __forceinline__ bool select_candidates(TopkShared<NT>& sh, int32_t* s_off,
                                                  const int2* __restrict__ cand,
                                                  const int32_t* __restrict__ ccount, int chunks,
                                                  int chunk_cap, uint32_t b1, int above1,
                                                  int top_k, int32_t* __restrict__ out,
                                                  int check_key = -1, uint32_t* tau_lb = nullptr) {
  constexpr int NW = NT / 64;
  constexpr int kPer = 8;  // candidates per lane loaded together
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  {
    const int v = tid < chunks ? ccount[tid] : 0;
    int total;
    const int ex = block_excl_scan<NT>(v, sh.wave_tot, &total);
    if (tid < chunks) s_off[tid] = ex;
    if (tid == 0) s_off[chunks] = total;
    for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
    if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
    __syncthreads();
  }
  const int total = s_off[chunks];
  // candidate number j -> its chunk (binary search over the offsets) and slot
  auto fetch = [&](int j) -> int2 {
    int lo = 0, hi = chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return cand[(int64_t)lo * chunk_cap + (j - s_off[lo])];
  };
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (total <= NT * kPer) {
    // Fast path: each wave loads its segment once (kPer steps of 64) and keeps it in
    // registers through the histogram, the counts and the ordered write.
    const int seg_begin = wave * 64 * kPer;
    int2 e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = seg_begin + k * 64 + lane;
      e[k] = (j < total) ? fetch(j) : make_int2(0, 0);
    }
    if (check_key >= 0) {  // b1 from the candidates' high digits
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        hist_add_wave(sh.hist, (uint32_t)e[k].x >> 12, seg_begin + k * 64 + lane < total);
      __syncthreads();
      find_bin<NT>(sh, top_k);
      b1 = (uint32_t)sh.found_bin;
      above1 = sh.found_above;
      for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
      if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      hist_add_wave(sh.hist, (uint32_t)e[k].x & 0xfff,
                    seg_begin + k * 64 + lane < total && ((uint32_t)e[k].x >> 12) == b1);
    __syncthreads();
    find_bin<NT>(sh, top_k - above1);
    const uint32_t tau = (b1 << 12) | (uint32_t)sh.found_bin;
    if (check_key >= 0 && (int)tau < check_key) {
      *tau_lb = tau;
      return false;
    }
    const int need = top_k - above1 - sh.found_above;
    int gt_w = 0, eq_w = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool valid = seg_begin + k * 64 + lane < total;
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
    int slot = gt_before + min(need, eq_before);
    int eq_seen = eq_before;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool valid = seg_begin + k * 64 + lane < total;
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
  // General path (more candidates than the workgroup holds at once): streamed passes.
  if (check_key >= 0) {  // b1 from the candidates' high digits
    for (int base = 0; base < total; base += NT * kPer) {
      int2 e[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int j = base + k * NT + tid;
        e[k] = (j < total) ? fetch(j) : make_int2(0, 0);
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        hist_add_wave(sh.hist, (uint32_t)e[k].x >> 12, base + k * NT + tid < total);
    }
    __syncthreads();
    find_bin<NT>(sh, top_k);
    b1 = (uint32_t)sh.found_bin;
    above1 = sh.found_above;
    for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0u;
    if (tid == 0) { sh.found_bin = 0; sh.found_above = 0; }
    __syncthreads();
  }
  // exact threshold inside bin b1
  for (int base = 0; base < total; base += NT * kPer) {
    int2 e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = base + k * NT + tid;
      e[k] = (j < total) ? fetch(j) : make_int2(0, 0);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      hist_add_wave(sh.hist, (uint32_t)e[k].x & 0xfff,
                    base + k * NT + tid < total && ((uint32_t)e[k].x >> 12) == b1);
  }
  __syncthreads();
  find_bin<NT>(sh, top_k - above1);
  const uint32_t tau = (b1 << 12) | (uint32_t)sh.found_bin;
  if (check_key >= 0 && (int)tau < check_key) {
    *tau_lb = tau;
    return false;
  }
  const int need = top_k - above1 - sh.found_above;

  // wave segments of whole 64-entry steps
  const int steps = (total + 63) / 64;
  const int seg_steps = (steps + NW - 1) / NW;
  const int seg_begin = wave * seg_steps * 64;
  const int seg_end = min(total, seg_begin + seg_steps * 64);
  int gt_w = 0, eq_w = 0;
  for (int j0 = seg_begin; j0 < seg_end; j0 += 64 * kPer) {
    int2 e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = j0 + k * 64 + lane;
      e[k] = (j < seg_end) ? fetch(j) : make_int2(0, 0);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool valid = j0 + k * 64 + lane < seg_end;
      gt_w += __popcll(__ballot(valid && (uint32_t)e[k].x > tau));
      eq_w += __popcll(__ballot(valid && (uint32_t)e[k].x == tau));
    }
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
  // keys == tau are taken in token order: the segments before this one took min(need, eq_before)
  int slot = gt_before + min(need, eq_before);
  int eq_seen = eq_before;
  for (int j0 = seg_begin; j0 < seg_end; j0 += 64 * kPer) {
    int2 e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = j0 + k * 64 + lane;
      e[k] = (j < seg_end) ? fetch(j) : make_int2(0, 0);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool valid = j0 + k * 64 + lane < seg_end;
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
  }
  return true;
}

}  // namespace sel
}  // namespace sa
