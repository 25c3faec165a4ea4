// Prefill selection without index lists: per-row selection thresholds, and the attention's
// selection masks written straight from recomputed indexer scores.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析":
//   §2.1  every cached key is scored against the query and the top-K keys are kept;
//   §2.3  prefill fuses index selection with the attention over the selected keys.
//
// The top-K of a row (score descending, token ascending) is fixed by two numbers: tau, the
// K-th largest score among the row's candidates, and t_cut, the last token with score tau
// that is still taken (ties go to the lower token). Key t of the row is selected exactly when
//   s(t) > tau,  or  s(t) == tau and t <= t_cut
// (rows with at most K candidates take all of them: tau = INT32_MIN, t_cut = INT32_MAX). So a
// prefill block needs no index lists: k_sel_thresh finds (tau, t_cut) for 32 queries of one
// indexer head by streaming radix histograms over scores that it recomputes with
// v_mfma_i32_32x32x32_i8 on every pass (the int8 work is cheap next to the attention; the
// indexer keys of one head stay in L2), and then writes the masked-dense attention's per-tile
// lane masks from the same recomputed scores.
//
// Passes over the candidate tiles (64 keys each; each of the 16 waves takes every 16th tile):
//   1. histogram of the top 10 bits of acc = s + d_idx * 2^14 (in [0, 2^RB]: 1025 bins of
//      32-bit counters per query), then per query the bin holding the K-th largest;
//   2. the keys of that bin collected into per-query lists in LDS as (low bits, token) keys,
//      then per query an 8-bit radix select over its list gives tau and t_cut; when the lists
//      do not fit, histograms of the next <= 11 bits among the bin's keys (16-bit counters, two
//      per word) instead, repeated until the K-th largest is known exactly, and then
//   3. only when some query has more keys equal to tau than it takes: ties counted per 64-key
//      tile, the tile holding the last tie taken found by a prefix sum, and that tile rescored
//      key by key to find t_cut;
//   4. the selection masks (when asked for): for every tile, one ballot per accumulator
//      element is exactly one 64-bit mask word of the dense kernel's record.
// Keys on a page missing from the table are never candidates.
#include <climits>

#include "sa_common.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16;

// 16 waves (four per SIMD, within 128 VGPRs): against 8 waves the 32K prefill's threshold
// selection takes 2.46 instead of 3.43 ms, its passes being bound by latency and LDS atomics
// that more resident waves overlap.
constexpr int kThWaves = 16;
constexpr int kThNT = 64 * kThWaves;
constexpr int kQB = 32;           // queries per workgroup: one 32-query mask block
constexpr int kTile = 64;         // keys per tile (the dense kernel's key tile)
constexpr int kHStride = 1025;    // histogram words per query (odd: queries on distinct banks)
constexpr int kFineBits = 11;     // bits per refining pass: 2048 16-bit counters per query
// tie counts (uint16 [32][tiles]) reuse the histogram space
constexpr int kMaxTiles = (kHStride * 4 * kQB) / (2 * kQB) - 2;
constexpr int kListCap = kQB * kHStride;  // list keys the histogram space holds
constexpr int kTokBits = 17;              // tokens < 2^17 (max_seq_len <= 131072)
constexpr int kTokMask = (1 << kTokBits) - 1;
constexpr int kMode0 = 0;         // every candidate is selected (or no candidates)
constexpr int kMode1 = 1;         // searching / tau known

template <int DI>
struct Radix {
  static constexpr int kBias = DI << 14;  // >= |s|: acc = s + kBias is never negative
  static constexpr int kBits = (DI == 32 ? 5 : (DI == 64 ? 6 : 7)) + 15;  // acc <= 2^kBits
  static constexpr int kShift1 = kBits - 10;                               // coarse bins 0..1024
};

// Offset within its tile of the key that accumulator element r of block mb holds in a lane of
// half hi (the 32x32 MFMA result layout: rows 8 (r / 4) + 4 hi + r % 4 of each 32-row block).
__device__ __forceinline__ constexpr int key_off(int mb, int r, int hi) {
  return mb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), on DPP: row_shr 1, 2, 4, 8 inside each
// 16-lane row, then row_bcast:15 and row_bcast:31 carry the row totals forward (no LDS round
// trip per step, as a shuffle would take).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// For counts c[0..nb) read through get(x): the largest bin b with sum_{x >= b} c[x] >= need,
// the sum over x > b and the total (b = -1 when the total is below need). Whole wave.
template <typename Get>
__device__ void find_from_top(Get get, int nb, int need, int& bin, int& above, int& total) {
  const int lane = lane_id();
  const int C = (nb + 63) >> 6;
  const int hi_x = nb - lane * C;  // this lane's bins: [lo_x, hi_x), lane 0 the top ones
  const int lo_x = max(0, hi_x - C);
  int s = 0;
  for (int x = lo_x; x < hi_x; ++x) s += get(x);
  const int incl = wave_incl_scan(s);
  total = __builtin_amdgcn_readlane(incl, 63);
  const uint64_t m = __ballot(incl >= need);
  if (m == 0) {
    bin = -1;
    above = total;
    return;
  }
  const int L = __ffsll((unsigned long long)m) - 1;
  int b = -1, run = incl - s;
  if (lane == L) {
    for (int x = hi_x - 1; x >= lo_x; --x) {
      const int c = get(x);
      if (run + c >= need) {
        b = x;
        break;
      }
      run += c;
    }
  }
  bin = __builtin_amdgcn_readlane(b, L);
  above = __builtin_amdgcn_readlane(run, L);
}

// For counts c[0..nb) (tokens ascending): the first x with sum_{y <= x} c[y] >= need and the
// sum over y < x. Whole wave; the caller guarantees the total reaches need.
template <typename Get>
__device__ void find_from_bottom(Get get, int nb, int need, int& pos, int& below) {
  const int lane = lane_id();
  const int C = (nb + 63) >> 6;
  const int lo_x = lane * C;
  const int hi_x = min(nb, lo_x + C);
  int s = 0;
  for (int x = lo_x; x < hi_x; ++x) s += get(x);
  const int incl = wave_incl_scan(s);
  const uint64_t m = __ballot(incl >= need);
  const int L = m ? __ffsll((unsigned long long)m) - 1 : 63;
  int p = -1, run = incl - s;
  if (lane == L) {
    for (int x = lo_x; x < hi_x; ++x) {
      const int c = get(x);
      if (run + c >= need) {
        p = x;
        break;
      }
      run += c;
    }
  }
  pos = __builtin_amdgcn_readlane(p, L);
  below = __builtin_amdgcn_readlane(run, L);
}

template <int DI>
__global__ __launch_bounds__(kThNT, 1) void k_sel_thresh(KvView kv, const int8_t* __restrict__ q_idx,
                                                        int q_len, int q_tail, int top_k,
                                                        int32_t* __restrict__ thr,
                                                        uint64_t* __restrict__ sel, int sel_qblocks,
                                                        int sel_tiles) {
  constexpr int KS = DI / 32;  // k-steps of the 32x32x32 int8 MFMA
  using R = Radix<DI>;
  __shared__ uint32_t hist[kQB * kHStride];
  __shared__ uint32_t whist[kThWaves][256];
  __shared__ int32_t st_mode[kQB], st_prefix[kQB], st_need[kQB], st_eq[kQB], st_tcut[kQB];
  __shared__ int32_t st_cnt[kQB], st_off[kQB], st_fill[kQB];
  __shared__ int32_t st_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  // Workgroups are dealt round-robin to the 8 XCDs (one L2 each); the remap gives each XCD a
  // contiguous run of the (b, gi)-major order, so the indexer keys one XCD streams are those of
  // few heads and stay in its L2 across the passes.
  int wg;
  {
    const int total = (int)(gridDim.x * gridDim.y);
    const int bid = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int per = total / 8, extra = total % 8;
    const int xcd = bid % 8, r = bid / 8;
    wg = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + r;
  }
  const int qb = wg % (int)gridDim.x;
  const int bg = wg / (int)gridDim.x;  // b * H_idx + gi
  const int b = bg / kv.num_idx_heads;
  const int gi = bg - b * kv.num_idx_heads;
  const int P = kv.prefix_len;
  const int seq_len = __builtin_amdgcn_readfirstlane(min(kv.seq_lens[b], kv.max_seq_len));
  const int pos0 = seq_len - q_tail;
  const int i0 = qb * kQB;
  const int n_valid = max(0, min(kQB, q_len - i0));
  const bool want_thr = n_valid > 0;
  // last position of any query of this block (for padding blocks: of the call's last query,
  // which is how far the attention reads this block's masks)
  const int pos_last = pos0 + (want_thr ? i0 + n_valid - 1 : q_len - 1);
  const int pos_first = pos0 + i0;
  const int my_i = i0 + l32;
  const bool my_valid = my_i < q_len;
  const int my_pos = my_valid ? pos0 + my_i : -1;
  if (!want_thr && sel == nullptr) return;
  if (pos_last < 0) {  // no query of the block sees a key: nothing to select, no masks read
    if (tid < n_valid) {
      const int64_t row = ((int64_t)b * q_len + i0 + tid) * kv.num_idx_heads + gi;
      thr[row * 2 + 0] = INT_MIN;
      thr[row * 2 + 1] = INT_MAX;
    }
    return;
  }

  // B operand: query l32's indexer bytes ks*32 + hi*16 .. +16 (zero for padding queries)
  i32x4 qf[KS];
  {
    const int qi = my_valid ? my_i : 0;
    const int8_t* qp = q_idx + (((int64_t)b * q_len + qi) * kv.num_idx_heads + gi) * DI + hi * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const i32x4*>(qp + ks * 32);
      if (!my_valid) qf[ks] = i32x4{0, 0, 0, 0};
    }
  }

  // A operand of one tile: key mb*32 + l32, bytes ks*32 + hi*16 .. +16. Loads are
  // unconditional (a missing page reads page 0 and is reported through the return value; the
  // page-table index is clamped).
  const int64_t head_stride = (int64_t)kv.page_size * DI;
  auto raw_page = [&](int tile) -> int32_t {
    const int lp = min((tile * kTile) >> kv.page_shift, kv.max_pages_per_seq - 1);
    return kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
  };
  auto load_tile = [&](int tile, int32_t raw, i32x4 (&ka)[2][KS]) -> bool {
    const int lp = (tile * kTile) >> kv.page_shift;
    const bool ok = lp < kv.max_pages_per_seq && raw >= 0 && raw < kv.num_pages;
    const int64_t phys = ok ? raw : 0;
    const int8_t* base = kv.kidx_pool + (phys * kv.num_idx_heads + gi) * head_stride +
                         (int64_t)((tile * kTile) & (kv.page_size - 1)) * DI;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[mb][ks] = *reinterpret_cast<const i32x4*>(base + (mb * 32 + l32) * DI + ks * 32 + hi * 16);
    return ok;
  };
  // acc[mb][r] = s + kBias for key key_off(mb, r, hi) of the tile and query l32
  auto scores = [&](const i32x4 (&ka)[2][KS], i32x16 (&acc)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = R::kBias;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[mb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[mb][ks], qf[ks], acc[mb], 0, 0, 0);
    }
  };
  // Runs fn(tile, page_ok, acc) on the tiles j_first + wave, + 8, ... <= j_last, the next
  // tile's operands in flight while one is processed.
  auto for_tiles = [&](int j_first, int j_last, auto&& fn) {
    int j = j_first + wave;
    if (j > j_last) return;
    i32x4 ka0[2][KS], ka1[2][KS];
    int32_t raw_n = raw_page(j + kThWaves);
    bool ok0 = load_tile(j, raw_page(j), ka0), ok1 = false;
    for (;;) {
      int32_t raw_a = raw_page(j + 2 * kThWaves);
      if (j + kThWaves <= j_last) ok1 = load_tile(j + kThWaves, raw_n, ka1);
      {
        i32x16 acc[2];
        scores(ka0, acc);
        fn(j, ok0, acc);
      }
      j += kThWaves;
      if (j > j_last) break;
      raw_n = raw_page(j + 2 * kThWaves);
      if (j + kThWaves <= j_last) ok0 = load_tile(j + kThWaves, raw_a, ka0);
      {
        i32x16 acc[2];
        scores(ka1, acc);
        fn(j, ok1, acc);
      }
      j += kThWaves;
      if (j > j_last) break;
    }
  };
  // candidate test of element (mb, r) of tile t0 for this lane's query
  auto is_cand = [&](int t0, int mb, int r) {
    const int t = t0 + key_off(mb, r, hi);
    return t >= P && t <= my_pos;
  };
  // body(mb, r) on the elements of tile t0 that are candidates of this lane's query. A tile
  // past the prefix and at or below the block's first position is wholly candidate for every
  // query (the common case: it needs no per-element position test, which would cost as much
  // as the rest of a pass); only the tiles at the prefix edge and on the diagonal test each.
  auto for_cands = [&](int t0, auto&& body) {
    if (t0 >= P && t0 + kTile - 1 <= pos_first) {  // wave-uniform
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) body(mb, r);
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (is_cand(t0, mb, r)) body(mb, r);
    }
  };
  uint32_t* hq = hist + l32 * kHStride;

  const int j_cand0 = P / kTile;                       // first tile holding a candidate
  const int j_cand1 = pos_last >= P ? pos_last / kTile : -1;
  int tau_l = 0x40000000, tcut_l = INT_MAX;            // this lane's query: nothing selected

  if (want_thr) {
    // ---- pass 1: coarse histogram (top 10 bits of acc)
    for (int x = tid; x < kQB * kHStride; x += kThNT) hist[x] = 0;
    __syncthreads();
    for_tiles(j_cand0, j_cand1, [&](int j, bool ok, const i32x16 (&acc)[2]) {
      if (!ok) return;
      for_cands(j * kTile, [&](int mb, int r) { atomicAdd(&hq[acc[mb][r] >> R::kShift1], 1u); });
    });
    __syncthreads();
    // per query: the coarse bin of the K-th largest, the keys above it and the keys in it
    for (int qq = wave; qq < kQB; qq += kThWaves) {
      int bin, above, total;
      const uint32_t* h = hist + qq * kHStride;
      find_from_top([&](int x) { return (int)h[x]; }, 1025, top_k, bin, above, total);
      if (lane == 0) {
        const bool search = qq < n_valid && total > top_k;
        st_mode[qq] = search ? kMode1 : kMode0;
        st_prefix[qq] = search ? bin : -1;
        st_need[qq] = search ? top_k - above : 0;
        st_cnt[qq] = search ? (int)h[bin] : 0;
        st_eq[qq] = 0;
        st_tcut[qq] = INT_MAX;
      }
    }
    __syncthreads();
    // list offsets (exclusive prefix over the queries), whether every list fits in the LDS,
    // whether any query searches
    if (wave == 0) {
      const int c = lane < kQB ? st_cnt[lane] : 0;
      const int incl = wave_incl_scan(c);
      if (lane < kQB) {
        st_off[lane] = incl - c;
        st_fill[lane] = 0;
      }
      const bool srch = __any(lane < kQB && st_mode[lane] == kMode1);
      if (lane == 63) st_flag = (incl <= kListCap ? 1 : 0) | (srch ? 2 : 0);
    }
    __syncthreads();
    const int flags = st_flag;
    if ((flags & 3) == 3) {
      // ---- pass 2: the keys of each query's coarse bin collected into LDS lists as unique
      //      32-bit keys (fine bits << 17) | (131071 - token): a larger key is a higher score, or
      //      the same score at a lower token. A query's keys come from every wave (each takes
      //      every 16th tile), so its list is filled through one LDS counter per query.
      uint32_t* list = hist;
      const int my_bin = st_prefix[l32];  // -1 for queries not searching: never matches
      const int my_off = st_off[l32];
      int32_t* fill = &st_fill[l32];
      constexpr int fmask = (1 << R::kShift1) - 1;
      for_tiles(j_cand0, j_cand1, [&](int j, bool ok, const i32x16 (&acc)[2]) {
        if (!ok) return;
        const int t0 = j * kTile;
        const int tb = kTokMask - t0 - hi * 4;  // 131071 - token of element (mb, r) = tb - offset
        for_cands(t0, [&](int mb, int r) {
          const int a = acc[mb][r];
          if ((a >> R::kShift1) == my_bin)
            list[my_off + atomicAdd(fill, 1)] = ((uint32_t)(a & fmask) << kTokBits) |
                                                (uint32_t)(tb - (mb * 32 + (r >> 2) * 8 + (r & 3)));
        });
      });
      __syncthreads();
      // per query: the need-th largest list key, 8 bits at a time (histograms per wave)
      for (int qq = wave; qq < kQB; qq += kThWaves) {
        if (st_mode[qq] != kMode1) continue;  // wave-uniform
        const uint32_t* lq = list + st_off[qq];
        const int n = st_cnt[qq];
        uint32_t* wh = whist[wave];
        int rem = st_need[qq];
        uint32_t prefix = 0, pmask = 0;
        for (int sh = 24; sh >= 0; sh -= 8) {
          for (int x = lane; x < 256; x += 64) wh[x] = 0;
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
          for (int x = lane; x < n; x += 64) {
            const uint32_t k = lq[x];
            if ((k & pmask) == prefix) atomicAdd(&wh[(k >> sh) & 255u], 1u);
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
          int d, above, total;
          find_from_top([&](int x) { return (int)wh[x]; }, 256, rem, d, above, total);
          d = max(d, 0);  // (the list holds >= need keys, so a digit is always found)
          rem -= above;
          prefix |= (uint32_t)d << sh;
          pmask |= 255u << sh;
          __builtin_amdgcn_wave_barrier();
        }
        // prefix is the last key taken; a key with the same score at a higher token is not
        const uint32_t fine = prefix >> kTokBits, tokr = prefix & (uint32_t)kTokMask;
        bool after = false;
        for (int x = lane; x < n; x += 64) {
          const uint32_t k = lq[x];
          after |= (k >> kTokBits) == fine && (k & (uint32_t)kTokMask) < tokr;
        }
        const bool any_after = __any(after);
        if (lane == 0) {
          st_prefix[qq] = (st_prefix[qq] << R::kShift1) | (int)fine;
          st_tcut[qq] = any_after ? kTokMask - (int)tokr : INT_MAX;
        }
      }
      __syncthreads();
    } else if ((flags & 2) != 0) {
      // the lists would not fit (many keys share the boundary bin): histogram passes instead
      // ---- pass 2: refine the K-th largest to the exact value, <= 11 bits at a time
      int bits = R::kShift1;  // low bits of acc not yet fixed
      while (bits > 0) {
        const int dg = min(bits, kFineBits), lo = bits - dg;
        const int words = 1 << (dg - 1);
        for (int x = tid; x < kQB * words; x += kThNT) hist[(x / words) * kHStride + (x % words)] = 0;
        __syncthreads();
        const int my_prefix = st_prefix[l32];  // -1 for queries not searching: never matches
        const int fmask = (1 << dg) - 1;
        for_tiles(j_cand0, j_cand1, [&](int j, bool ok, const i32x16 (&acc)[2]) {
          if (!ok) return;
          for_cands(j * kTile, [&](int mb, int r) {
            const int a = acc[mb][r];
            if ((a >> bits) == my_prefix) {
              const int f = (a >> lo) & fmask;
              atomicAdd(&hq[f >> 1], 1u << ((f & 1) << 4));
            }
          });
        });
        __syncthreads();
        for (int qq = wave; qq < kQB; qq += kThWaves) {
          if (st_mode[qq] != kMode1) continue;  // wave-uniform
          const uint32_t* h = hist + qq * kHStride;
          int f1, above, total;
          find_from_top([&](int x) { return (int)((h[x >> 1] >> ((x & 1) << 4)) & 0xffffu); }, 1 << dg,
                        st_need[qq], f1, above, total);
          if (lane == 0) {
            st_prefix[qq] = (st_prefix[qq] << dg) | f1;
            st_need[qq] -= above;
            if (lo == 0) st_eq[qq] = (int)((h[f1 >> 1] >> ((f1 & 1) << 4)) & 0xffffu);
          }
        }
        __syncthreads();
        bits = lo;
      }

      // ---- pass 3: the last tie taken, when a query has more keys at tau than it takes
      if (tid == 0) st_flag = 0;
      __syncthreads();
      if (tid < kQB && st_mode[tid] == kMode1 && st_eq[tid] > st_need[tid]) st_flag = 1;
      __syncthreads();
      if (st_flag != 0 && j_cand1 >= 0) {
        const int nt = j_cand1 + 1;  // tie counts of tiles 0..j_cand1 (<= kMaxTiles)
        uint16_t* cnt = reinterpret_cast<uint16_t*>(hist);
        for (int x = tid; x < kQB * nt; x += kThNT) cnt[x] = 0;
        __syncthreads();
        const bool my_tie = my_valid && st_mode[l32] == kMode1 && st_eq[l32] > st_need[l32];
        const int my_tau = my_tie ? st_prefix[l32] : -1;
        for_tiles(j_cand0, j_cand1, [&](int j, bool ok, const i32x16 (&acc)[2]) {
          if (!ok) return;
          int c = 0;
          for_cands(j * kTile, [&](int mb, int r) { c += acc[mb][r] == my_tau ? 1 : 0; });
          c += __shfl_xor(c, 32, 64);
          if (hi == 0 && c != 0) cnt[l32 * nt + j] = (uint16_t)c;
        });
        __syncthreads();
        for (int qq = wave; qq < kQB; qq += kThWaves) {
          if (!(st_mode[qq] == kMode1 && st_eq[qq] > st_need[qq])) continue;  // wave-uniform
          const uint16_t* cq = cnt + qq * nt;
          int tile, below;
          find_from_bottom([&](int x) { return (int)cq[x]; }, nt, st_need[qq], tile, below);
          if (tile < 0) continue;  // (counts short of need: cannot happen; no cut is recorded)
          const int rank = st_need[qq] - below;  // the rank-th tie of that tile (1-based) is the last taken
          // rescore that tile key by key: lane = key
          const int t = tile * kTile + lane;
          const int32_t raw = raw_page(tile);
          const int lp = (tile * kTile) >> kv.page_shift;
          const bool ok = lp < kv.max_pages_per_seq && raw >= 0 && raw < kv.num_pages;
          const int8_t* kr = kv.kidx_pool + ((int64_t)(ok ? raw : 0) * kv.num_idx_heads + gi) * head_stride +
                             (int64_t)(t & (kv.page_size - 1)) * DI;
          const int8_t* qr = q_idx + (((int64_t)b * q_len + i0 + qq) * kv.num_idx_heads + gi) * DI;
          int s = 0;
#pragma unroll
          for (int w = 0; w < DI / 16; ++w) {
            const i32x4 kw = *reinterpret_cast<const i32x4*>(kr + w * 16);
            const i32x4 qw = *reinterpret_cast<const i32x4*>(qr + w * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_sdot4(kw[e], qw[e], s, false);
          }
          const int pos_q = pos0 + i0 + qq;
          uint64_t m = __ballot(ok && s + R::kBias == st_prefix[qq] && t >= P && t <= pos_q);
          for (int k = 1; k < rank; ++k) m &= m - 1;
          if (lane == 0) st_tcut[qq] = tile * kTile + (__ffsll((unsigned long long)m) - 1);
        }
        __syncthreads();
      }

    }

    // ---- thresholds out: (tau, t_cut) in score units
    if (tid < n_valid) {
      const int64_t row = ((int64_t)b * q_len + i0 + tid) * kv.num_idx_heads + gi;
      const bool all = st_mode[tid] == kMode0;
      thr[row * 2 + 0] = all ? INT_MIN : st_prefix[tid] - R::kBias;
      thr[row * 2 + 1] = all ? INT_MAX : st_tcut[tid];
    }
    if (my_valid) {
      const bool all = st_mode[l32] == kMode0;
      tau_l = all ? -1 : st_prefix[l32];
      tcut_l = all ? INT_MAX : st_tcut[l32];
    }
  }

  // ---- pass 4: the selection masks of the masked-dense attention, tiles 0 .. pos_last / 64
  if (sel == nullptr) return;
  uint64_t* rec = sel + (((int64_t)bg * sel_qblocks + qb) * sel_tiles) * 32;
  const int j_rec1 = pos_last / kTile;
  if (!want_thr) {  // padding block: zero masks
    for (int x = tid; x < (j_rec1 + 1) * 32; x += kThNT) rec[x] = 0;
    return;
  }
  for_tiles(0, j_rec1, [&](int j, bool ok, const i32x16 (&acc)[2]) {
    const int t0 = j * kTile;
    uint32_t w_lo = 0, w_hi = 0;  // lane k < 32 collects mask word k
    // fast path: every pair of the tile is a candidate and no query's tie cut lies inside it,
    // so selection is one comparison with a per-query threshold
    const bool inner = t0 >= P && t0 + kTile - 1 <= pos_first;
    const bool cut_inside = tcut_l >= t0 && tcut_l < t0 + kTile - 1;
    if (ok && inner && !__any(cut_inside)) {
      const int th = tau_l + (tcut_l < t0 ? 1 : 0);  // ties after the cut are not taken
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint64_t m = __ballot(acc[mb][r] >= th);
          const bool mine = __builtin_amdgcn_inverse_ballot_w64(1ull << (mb * 16 + r));
          w_lo = mine ? (uint32_t)m : w_lo;
          w_hi = mine ? (uint32_t)(m >> 32) : w_hi;
        }
    } else if (ok) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + key_off(mb, r, hi);
          const int a = acc[mb][r];
          const bool s_ok = t <= my_pos && (t < P || a > tau_l || (a == tau_l && t <= tcut_l));
          const uint64_t m = __ballot(s_ok);
          const bool mine = __builtin_amdgcn_inverse_ballot_w64(1ull << (mb * 16 + r));
          w_lo = mine ? (uint32_t)m : w_lo;
          w_hi = mine ? (uint32_t)(m >> 32) : w_hi;
        }
    }
    if (lane < 32) reinterpret_cast<uint2*>(rec + (int64_t)j * 32)[lane] = make_uint2(w_lo, w_hi);
  });
}

template <int DI>
hipError_t launch_sel_thresh_d(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                               int top_k, int32_t* thr, uint64_t* sel, hipStream_t stream) {
  const int n_qb = sel != nullptr ? sel_query_blocks(q_len) : (q_len + kQB - 1) / kQB;
  dim3 grid((unsigned)n_qb, (unsigned)(kv.batch * kv.num_idx_heads));
  hipLaunchKernelGGL((k_sel_thresh<DI>), grid, dim3(kThNT), 0, stream, kv, q_idx, q_len, q_tail, top_k,
                     thr, sel, sel_query_blocks(q_len), sel_tiles(kv));
  return hipGetLastError();
}

}  // namespace

bool sel_thresh_applies(const KvView& kv) {
  return (kv.max_seq_len + kTile - 1) / kTile <= kMaxTiles &&
         (kv.idx_dim == 32 || kv.idx_dim == 64 || kv.idx_dim == 128);
}

hipError_t launch_sel_thresh(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail, int top_k,
                             int32_t* thresholds, uint64_t* sel, hipStream_t stream) {
  if (!sel_thresh_applies(kv)) return hipErrorInvalidValue;
  switch (kv.idx_dim) {
    case 32: return launch_sel_thresh_d<32>(kv, q_idx, q_len, q_tail, top_k, thresholds, sel, stream);
    case 64: return launch_sel_thresh_d<64>(kv, q_idx, q_len, q_tail, top_k, thresholds, sel, stream);
    case 128: return launch_sel_thresh_d<128>(kv, q_idx, q_len, q_tail, top_k, thresholds, sel, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
