// Indexer kernels: exact int8 x int8 -> int32 scores of every candidate key.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析", §2.1: the
// indexer runs on the GPU and scores each cached key against the query before the top-K.
//
// Two kernels, chosen by how many queries share the keys:
//  * k_index_stream (few queries per sequence, i.e. decode): HBM-bound streaming of the
//    indexer keys. A wave reads one 64-token block of one indexer head (64*d_idx contiguous
//    bytes) with 16-byte loads, so every load instruction moves 1 KiB of consecutive bytes.
//    d_idx/16 neighbouring lanes hold one token's key; each does 4 v_dot4_i32_i8 against the
//    matching 16 query bytes, and a DPP butterfly sums the lane group. After the reduction
//    lane l keeps the token of load (l mod d_idx/16), so a wave stores 64 consecutive scores
//    with one instruction.
//  * k_index_mfma (many queries, i.e. prefill): scores are a causal int8 GEMM
//    S^T = K_idx * Q_idx^T on v_mfma_i32_16x16x32_i8. Keys are the M side so each lane's four
//    accumulator rows are four consecutive tokens of one query; a 16-query x 64-key tile goes
//    through LDS and out as whole 256-byte row segments.
#include "sa_index_dev.h"

namespace sa {
namespace {

using namespace idx;

constexpr int kStreamBlocksPerWave = 4;

// grid: x = ceil(token blocks / (4 waves * kStreamBlocksPerWave)), y = batch * H_idx.
// Each wave scores kStreamBlocksPerWave consecutive 64-token blocks of one row. The first
// query's fragment and the page-table entries are requested before the key loads, and all
// key loads of the wave are in flight before any is used.
template <int D>
__global__ __launch_bounds__(256) void k_index_stream(KvView kv, const int8_t* __restrict__ q_idx,
                                                      int q_len, int q_tail,
                                                      int32_t* __restrict__ scores,
                                                      int64_t row_stride) {
  constexpr int LPT = D / 16;   // lanes holding one token's key
  constexpr int TPL = 64 / LPT; // tokens covered by one 1 KiB load instruction
  constexpr int R = LPT;        // load instructions per 64-token block
  constexpr int U = kStreamBlocksPerWave;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.y;
  const int b = row / kv.num_idx_heads;
  const int gi = row - b * kv.num_idx_heads;
  const int part = lane % LPT;                // which 16-byte chunk of a key row
  const int my_tok = part * TPL + lane / LPT; // token (within the block) this lane stores
  const int8_t* qrow = q_idx + ((int64_t)b * q_len * kv.num_idx_heads + gi) * D + part * 16;
  const v4i q0 = *reinterpret_cast<const v4i*>(qrow);  // query 0, requested first
  const int T = min(kv.seq_lens[b], kv.max_seq_len);
  const int P = kv.prefix_len;
  const int pos0 = T - q_tail;               // position of query 0
  const int pmax = pos0 + q_len - 1;
  if (pmax < P || pmax < 0) return;
  const int blk_first = P >> 6;
  const int blk_last = pmax >> 6;
  const int blk0 = blk_first + (blockIdx.x * 4 + wave) * U;
  if (blk0 > blk_last) return;

  int64_t phys[U];
#pragma unroll
  for (int u = 0; u < U; ++u) phys[u] = (blk0 + u <= blk_last) ? phys_page(kv, b, (blk0 + u) << 6) : -1;
  v4i kd[U][R];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (phys[u] >= 0) {
      const int slot0 = ((blk0 + u) << 6) & (kv.page_size - 1);
      const int8_t* base = kv.kidx_pool +
          ((phys[u] * kv.num_idx_heads + gi) * kv.page_size + slot0) * (int64_t)D;
#pragma unroll
      for (int r = 0; r < R; ++r)
        kd[u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + r * 1024 + lane * 16));
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) kd[u][r] = v4i{0, 0, 0, 0};
    }
  }

  for (int i = 0; i < q_len; ++i) {
    const int pos = pos0 + i;
    if (pos < P) continue;
    const v4i qf = (i == 0) ? q0 : *reinterpret_cast<const v4i*>(qrow + (int64_t)i * kv.num_idx_heads * D);
    int32_t* srow = scores + (((int64_t)b * q_len + i) * kv.num_idx_heads + gi) * row_stride;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (phys[u] < 0) continue;
      int mine = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int s = group_sum_i<LPT>(dot16(qf, kd[u][r]));
        if (part == r) mine = s;
      }
      const int t = ((blk0 + u) << 6) + my_tok;
      if (t >= P && t <= pos) srow[t] = mine;
    }
  }
}

// ---------------------------------------------------------------------------------------
// MFMA indexer. Wave tile: 64 keys (one 64-token block) x 64 queries. grid.x enumerates
// (query tile, key chunk) pairs, 4 per workgroup (one per wave); grid.y = batch * H_idx.
typedef long i64x1;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kMfmaKeyBlocksPerWave = 8;  // 512 keys per wave item
constexpr int kStageStride = 68;          // ints per staged score row (64 + 4 of padding)

// Coarse 16-bit keys (used by the fused prefill selection): c(s) = min((s + B) >> shift, 65535)
// with B = D * 2^14 >= |s| and shift = log2(D) - 1, so c is order-preserving (s1 > s2 whenever
// c(s1) > c(s2)) and a key of c carries the exact score in [c * 2^shift - B, (c + 1) * 2^shift - B].
template <int D>
struct Coarse {
  static constexpr int kShift = D == 32 ? 4 : (D == 64 ? 5 : 6);
  static constexpr int kBias = D << 14;
};
template <int D>
__device__ __forceinline__ uint16_t coarse_key(int s) {
  return (uint16_t)min((s + Coarse<D>::kBias) >> Coarse<D>::kShift, 65535);
}

template <int D, bool COARSE>
__global__ __launch_bounds__(256) void k_index_mfma(KvView kv, const int8_t* __restrict__ q_idx,
                                                    int q_len, int q_tail,
                                                    void* __restrict__ scores_out,
                                                    int64_t row_stride, int n_qtiles,
                                                    int n_kchunks) {
  int32_t* __restrict__ scores = static_cast<int32_t*>(scores_out);
  uint16_t* __restrict__ ckeys = static_cast<uint16_t*>(scores_out);
  constexpr int KS = D / 32;   // k-steps of the 16x16x32 MFMA
  constexpr int CH = D / 4;    // bytes of a row held by one lane group (l / 16)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= n_qtiles * n_kchunks) return;
  const int qt = item / n_kchunks;
  const int kc = item - qt * n_kchunks;
  const int row = blockIdx.y;
  const int b = row / kv.num_idx_heads;
  const int gi = row - b * kv.num_idx_heads;
  const int T = min(kv.seq_lens[b], kv.max_seq_len);
  const int P = kv.prefix_len;
  const int pos0 = T - q_tail;
  const int i0 = qt * 64;
  const int i_end = min(q_len, i0 + 64);
  const int pmax = pos0 + i_end - 1;
  const int pmin = pos0 + i0;
  if (pmax < P) return;
  const int blk_first = (P >> 6) + kc * kMfmaKeyBlocksPerWave;
  const int blk_last = min(pmax >> 6, blk_first + kMfmaKeyBlocksPerWave - 1);
  if (blk_first > blk_last) return;

  const int l16 = lane & 15;
  const int lg = lane >> 4;
  __shared__ __align__(16) int32_t s_stage[4][16][kStageStride];  // (coarse: 16-bit rows of 72)

  // B operand: 4 query blocks of 16, lane holds query (n*16 + l16), bytes lg*CH .. +CH.
  i64x1 qb[4][KS];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i = i0 + n * 16 + l16;
    if (i < q_len) {
      const int8_t* qp = q_idx + (((int64_t)b * q_len + i) * kv.num_idx_heads + gi) * D + lg * CH;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[n][ks] = *reinterpret_cast<const i64x1*>(qp + ks * 8);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[n][ks] = 0;
    }
  }

  // Block k of the item is loaded one step before it is multiplied, and its page-table entry
  // one step before that. All of these loads are unconditional (a missing page reads page 0;
  // the page-table index is clamped) so that none is waited for where it is issued; a block
  // without a page is skipped at compute time.
  auto raw_page = [&](int blk) -> int32_t {
    const int lp = min((blk << 6) >> kv.page_shift, kv.max_pages_per_seq - 1);
    return kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
  };
  // A operand: 4 key blocks of 16, lane holds key (m*16 + l16), bytes lg*CH .. +CH.
  auto load_k = [&](int blk, int32_t raw, i64x1 (&ka)[4][KS]) -> bool {
    const int lp = (blk << 6) >> kv.page_shift;
    const bool ok = lp < kv.max_pages_per_seq && raw >= 0 && raw < kv.num_pages;
    const int64_t phys = ok ? raw : 0;
    const int8_t* kbase = kv.kidx_pool +
        ((phys * kv.num_idx_heads + gi) * kv.page_size + ((blk << 6) & (kv.page_size - 1))) * (int64_t)D;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int8_t* kp = kbase + (m * 16 + l16) * D + lg * CH;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[m][ks] = *reinterpret_cast<const i64x1*>(kp + ks * 8);
    }
    return ok;
  };
  // Score rows of a full block leave through the wave's LDS tile so that every store
  // instruction writes whole 256-byte row segments (4 rows of 64 keys) instead of 64-byte
  // pieces of 16 rows.
  int32_t (&stg)[16][kStageStride] = s_stage[wave];
  auto compute = [&](int blk, const i64x1 (&ka)[4][KS]) {
    const int t0 = blk << 6;
    const bool full = (t0 >= P) && (t0 + 63 <= pmin);  // every (key, query) pair is a candidate
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      i32x4 acc[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[m] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ka[m][ks], qb[n][ks], acc[m], 0, 0, 0);
      }
      // acc[m][j] = score(key m*16 + lg*4 + j, query n*16 + l16)
      if (full && COARSE) {
        // 16-bit keys: a 64-key row segment is 128 bytes, 8 lanes of 16 bytes; 8 rows per store
        uint16_t (*stg16)[72] = reinterpret_cast<uint16_t (*)[72]>(&stg[0][0]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint2 w;
          w.x = (uint32_t)coarse_key<D>(acc[m][0]) | ((uint32_t)coarse_key<D>(acc[m][1]) << 16);
          w.y = (uint32_t)coarse_key<D>(acc[m][2]) | ((uint32_t)coarse_key<D>(acc[m][3]) << 16);
          *reinterpret_cast<uint2*>(&stg16[l16][m * 16 + lg * 4]) = w;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int qr = rr * 8 + (lane >> 3);
          const int c = lane & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(&stg16[qr][c * 8]);
          const int iq = i0 + n * 16 + qr;
          if (iq < q_len)
            *reinterpret_cast<uint4*>(ckeys + (((int64_t)b * q_len + iq) * kv.num_idx_heads + gi) *
                                                  row_stride + t0 + c * 8) = v;
        }
        __builtin_amdgcn_wave_barrier();
      } else if (full) {
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<i32x4*>(&stg[l16][m * 16 + lg * 4]) = acc[m];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int qr = rr * 4 + (lane >> 4);  // query of the n-block; lanes 16k..16k+15 cover its 64 keys
          const int c = lane & 15;
          const i32x4 v = *reinterpret_cast<const i32x4*>(&stg[qr][c * 4]);
          const int iq = i0 + n * 16 + qr;
          if (iq < q_len)
            *reinterpret_cast<i32x4*>(scores + (((int64_t)b * q_len + iq) * kv.num_idx_heads + gi) *
                                                   row_stride + t0 + c * 4) = v;
        }
        __builtin_amdgcn_wave_barrier();  // the tile is read before the next n-block writes it
      } else {
        const int i = i0 + n * 16 + l16;
        if (i >= q_len) continue;
        const int pos = pos0 + i;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int t = t0 + m * 16 + lg * 4;
          const int64_t o = (((int64_t)b * q_len + i) * kv.num_idx_heads + gi) * row_stride + t;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (t + j >= P && t + j <= pos) {
              if constexpr (COARSE) ckeys[o + j] = coarse_key<D>(acc[m][j]);
              else scores[o + j] = acc[m][j];
            }
          }
        }
      }
    }
  };
  i64x1 ka0[4][KS], ka1[4][KS];
  int32_t r_next = raw_page(blk_first + 1);
  bool ok0 = load_k(blk_first, raw_page(blk_first), ka0), ok1 = false;
  for (int blk = blk_first; blk <= blk_last; blk += 2) {
    int32_t r_after = raw_page(blk + 2);
    if (blk + 1 <= blk_last) ok1 = load_k(blk + 1, r_next, ka1);
    if (ok0) compute(blk, ka0);
    if (blk + 1 > blk_last) break;
    r_next = raw_page(blk + 3);
    if (blk + 2 <= blk_last) ok0 = load_k(blk + 2, r_after, ka0);
    if (ok1) compute(blk + 1, ka1);
  }
}

template <int D>
hipError_t launch_index_d(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                          int32_t* scores, int64_t row_stride, hipStream_t stream) {
  const int rows = kv.batch * kv.num_idx_heads;
  const int pmax = kv.max_seq_len - q_tail + q_len - 1;  // largest position any query can have
  if (pmax < kv.prefix_len) return hipSuccess;
  const int blocks = (pmax >> 6) - (kv.prefix_len >> 6) + 1;
  if (q_len < 16) {
    const int per_wg = 4 * kStreamBlocksPerWave;
    dim3 grid((blocks + per_wg - 1) / per_wg, rows);
    hipLaunchKernelGGL(k_index_stream<D>, grid, dim3(256), 0, stream, kv, q_idx, q_len, q_tail,
                       scores, row_stride);
  } else {
    const int n_qtiles = (q_len + 63) / 64;
    const int n_kchunks = (blocks + kMfmaKeyBlocksPerWave - 1) / kMfmaKeyBlocksPerWave;
    const int64_t items = (int64_t)n_qtiles * n_kchunks;
    dim3 grid((unsigned)((items + 3) / 4), rows);
    hipLaunchKernelGGL((k_index_mfma<D, false>), grid, dim3(256), 0, stream, kv, q_idx, q_len, q_tail,
                       (void*)scores, row_stride, n_qtiles, n_kchunks);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_index_coarse_d(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                                 uint16_t* keys, int64_t row_stride, hipStream_t stream) {
  const int rows = kv.batch * kv.num_idx_heads;
  const int pmax = kv.max_seq_len - q_tail + q_len - 1;
  if (pmax < kv.prefix_len) return hipSuccess;
  const int blocks = (pmax >> 6) - (kv.prefix_len >> 6) + 1;
  const int n_qtiles = (q_len + 63) / 64;
  const int n_kchunks = (blocks + kMfmaKeyBlocksPerWave - 1) / kMfmaKeyBlocksPerWave;
  const int64_t items = (int64_t)n_qtiles * n_kchunks;
  dim3 grid((unsigned)((items + 3) / 4), rows);
  hipLaunchKernelGGL((k_index_mfma<D, true>), grid, dim3(256), 0, stream, kv, q_idx, q_len, q_tail,
                     (void*)keys, row_stride, n_qtiles, n_kchunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_coarse(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                               uint16_t* keys, int64_t row_stride, hipStream_t stream) {
  if (q_len < 16) return hipErrorInvalidValue;  // the many-query (MFMA) indexer only
  switch (kv.idx_dim) {
    case 32: return launch_index_coarse_d<32>(kv, q_idx, q_len, q_tail, keys, row_stride, stream);
    case 64: return launch_index_coarse_d<64>(kv, q_idx, q_len, q_tail, keys, row_stride, stream);
    case 128: return launch_index_coarse_d<128>(kv, q_idx, q_len, q_tail, keys, row_stride, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_index(const KvView& kv, const int8_t* q_idx, int q_len, int q_tail,
                        int32_t* scores, int64_t row_stride, hipStream_t stream) {
  switch (kv.idx_dim) {
    case 32: return launch_index_d<32>(kv, q_idx, q_len, q_tail, scores, row_stride, stream);
    case 64: return launch_index_d<64>(kv, q_idx, q_len, q_tail, scores, row_stride, stream);
    case 128: return launch_index_d<128>(kv, q_idx, q_len, q_tail, scores, row_stride, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sa
