// Dense causal FlashAttention forward on bf16 MFMA: the special case of the sparse path in
// which every causal key is selected.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.3: prefill
// is the compute-heavy phase and runs on the matrix units.
//
// Workgroup: 8 waves, 256 queries of one query head (32 per wave, two waves per SIMD),
// streaming 64-key tiles of the KV head through LDS. K runs one tile ahead of V: each
// iteration computes the scores of the next tile and the softmax and P V product of the current
// one (see the loop). Waves 0-3 stage K tiles, waves 4-7 stage V tiles; global loads stay in
// flight across the compute and land in LDS at its end.
// Per wave and tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K * Q^T   (A = K tile rows from LDS, B = the wave's Q^T held in registers).
//                   The accumulator layout gives each lane 32 of the 64 scores of ONE query
//                   (the other 32 sit in lane ^ 32), so the softmax row max is a local max
//                   plus one cross-half exchange, and row sums stay per lane until the end.
//   O^T += V^T * P^T  (A = V^T fragments read from the row-major V tile with ds_read_b64_tr_b16,
//                   B = P^T taken straight from the S^T accumulators: the 8 scores a lane holds
//                   for one 16-key step become its B operand, and the transposed reads fetch
//                   the same key permutation, so no shuffle is needed).
// K and V tiles are copied into LDS as they are. Softmax is base 2 with sm_scale*log2(e) applied to
// the fp32 scores; Q, K and V stay exact bf16, accumulation is fp32, P is rounded to bf16 and
// the row sum adds the rounded P. Workgroups are ordered for L2 reuse across the 8 XCDs.
// Key splits (masked attention of blocks too short to fill the chip): each workgroup streams
// its split's share of the block's causal tiles and writes the unnormalised O, the maximum and
// the row sum of its queries, which the split merge combines.
#include "sa_common.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int BN = 64;    // keys per tile
constexpr int kNumXcd = 8;
constexpr int kDenseWaves = 8;                    // waves per workgroup (2 per SIMD)
constexpr int kDenseThreads = 64 * kDenseWaves;  // MI355X: 8 accelerator dies, 32 CUs and one L2 each
// The running maximum used in the exponent is only moved when a row's maximum grows by more
// than 2^kRescaleLog2 (in exp2 units); until then P stays below 2^kRescaleLog2, far inside
// the bf16 and fp32 ranges, and the result is unchanged because O and the row sum use the
// same stale maximum.
constexpr float kRescaleLog2 = 8.f;
constexpr int KPAD = 8;   // bf16 padding of a K row in LDS
constexpr int VPAD = 32;  // bf16 padding of a V row in LDS (row stride 2D + 64 B: the 4-row groups of
                          // a transposed read land on distinct banks)

// max(x[l], x[l ^ 32]) in every lane l: a self-swap of the two 32-lane halves gives both
// values whichever half moves.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D>
struct DenseShared {
  uint16_t k[2][BN][D + KPAD];
  uint16_t v[2][BN][D + VPAD];  // row-major V tiles, read transposed
};

union Frag8 {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
};

// One workgroup: 4 waves, 128 queries of one query head; each wave owns 32 queries.
// Software pipeline over 64-key tiles, K one tile ahead of V:
//   iteration j:  [QK(j+1) on MFMA, softmax(j) on VALU]  ->  [P V(j) on MFMA, mask + row max of
//                 S(j+1)]  ->  stage tiles j+2 (K) and j+1 (V) into LDS  ->  barrier
// The source places the exponentials of tile j between the QK^T instructions of tile j+1; the
// masked kernel keeps that order, while in the causal kernel the compiler moves them after the
// QK^T instructions, ahead of the P V product (forcing them back in place measured 5% slower,
// and moving the masked kernel's exponentials after QK^T 7% slower). LDS holds two K tiles and
// two V^T tiles.
template <int D, bool MASKED>
__global__ __launch_bounds__(kDenseThreads, 1) void k_attn_dense(
    KvView kv, const uint16_t* __restrict__ q, int num_q_heads, int q_len, int q_tail, float qscale,
    uint16_t* __restrict__ out, float* __restrict__ lse, int n_qblocks,
    const uint64_t* __restrict__ sel, int sel_qblocks, int sel_tiles, int num_splits,
    int tiles_per_split, float* __restrict__ part) {
  constexpr int KS = D / 16;     // k-steps of QK^T
  constexpr int DB = D / 32;     // 32-dim blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int KPT = D / 32;    // key rows per thread in the tile loader (half the workgroup)
  constexpr int QW = 32;         // queries per wave
  constexpr int BMQ = kDenseWaves * QW;  // queries per workgroup
  __shared__ DenseShared<D> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work order. Workgroups are dealt round-robin to the 8 XCDs, each with its own L2; the
  // remap gives every XCD a contiguous run of the logical order, which is (b, KV head) major,
  // then query blocks heaviest first (causal work grows with the block index), then key
  // splits, then the G query heads of the group. The workgroups resident on one XCD then
  // stream the same KV range and share it in L2.
  const int G = num_q_heads / kv.num_kv_heads;
  int wg;
  {
    const int total = (int)gridDim.x, bid = (int)blockIdx.x;
    const int per = total / kNumXcd, extra = total % kNumXcd;
    const int xcd = bid % kNumXcd, r = bid / kNumXcd;
    wg = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + r;
  }
  const int per_qblk = num_splits * G;
  const int per_pair = n_qblocks * per_qblk;
  const int pair = wg / per_pair;
  const int rem = wg - pair * per_pair;
  const int qblk = n_qblocks - 1 - rem / per_qblk;
  const int split = (rem % per_qblk) / G;
  const int b = pair / kv.num_kv_heads;
  const int g = pair - b * kv.num_kv_heads;
  const int h = g * G + rem % G;
  const int seq_len = __builtin_amdgcn_readfirstlane(min(kv.seq_lens[b], kv.max_seq_len));
  const int pos0 = seq_len - q_tail;              // position of query 0
  const int i_blk = qblk * BMQ;
  const int i_w = i_blk + wave * QW;              // first query of this wave
  const int i_last_blk = min(q_len, i_blk + BMQ) - 1;
  const int wave_pos_max = pos0 + min(q_len - 1, i_w + QW - 1);
  const int blk_pos_max = pos0 + i_last_blk;
  if (blk_pos_max < 0 && part == nullptr) return;
  // Key tiles of this workgroup: [t_lo, t_hi) of the block's causal tiles (all of them without
  // key splits; with splits, the split's share, possibly none). A split that holds no tile of
  // a query still writes that query's partial result (empty).
  const int n_tiles = blk_pos_max >= 0 ? blk_pos_max / BN + 1 : 0;
  const int t_lo = split * tiles_per_split;
  const int t_hi = min(n_tiles, t_lo + tiles_per_split);
  const int n_own = max(0, t_hi - t_lo);  // tiles this workgroup streams (workgroup-uniform)
  // last tile this wave attends, within the workgroup's range (below t_lo: none)
  const int last_w = wave_pos_max >= 0 ? min(wave_pos_max / BN, t_hi - 1) : -1;

  const int my_i = i_w + l32;
  const int my_pos = pos0 + my_i;
  const bool my_valid = my_i < q_len;
  // Selection masks of this wave's 32 queries (masked mode): one 256-byte record per 64-key
  // tile, 32 lane masks in the order of the S^T accumulator elements.
  const uint64_t* selw = nullptr;
  if constexpr (MASKED) {
    const int gi = kv.num_idx_heads == 1 ? 0 : g;
    const int qb = qblk * kDenseWaves + wave;
    selw = sel + (((int64_t)b * kv.num_idx_heads + gi) * sel_qblocks + qb) * (int64_t)sel_tiles * 32;
  }

  // Q^T fragments (B operand): lane holds query l32, dims ks*16 + hi*8 .. +8.
  Frag8 qf[KS];
  {
    const int qi = my_valid ? my_i : i_blk;  // any valid row; never stored
    const uint16_t* qp = q + (((int64_t)b * q_len + qi) * num_q_heads + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks].u = *reinterpret_cast<const uint4*>(qp + ks * 16);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Tile loaders: waves 0-3 stage K, waves 4-7 stage V (each SIMD runs one of each). K: dims
  // chunk ld_c (8 dims) of key rows ld_kq*KPT .. +KPT, so 16 neighbouring lanes load and store
  // 256 contiguous bytes of a row. V (stored transposed): 4 neighbouring lanes cover 64
  // contiguous bytes of a row (dims chunks 4*c_hi .. +3) and the next lanes walk the key
  // groups, so one load touches 16 row segments of 64 B, and a transposed store of one dim by
  // a half-wave hits 32 distinct 8-byte bank pairs (V^T row stride 136 B).
  const bool k_loader = wave < kDenseWaves / 2;  // wave-uniform
  const int ltid = tid & (kDenseThreads / 2 - 1);
  const int ld_c = ltid % CPR;
  const int ld_kq = ltid / CPR;
  const int64_t head_stride = (int64_t)kv.page_size * D;
  const int64_t page_stride = head_stride * kv.num_kv_heads;

  // Global -> registers for one tile of K or V. The loads are unconditional and always in
  // bounds: a tile never crosses a page, and a page missing from the table reads page 0. Rows
  // that must not be attended (past the end of the sequence, or of a missing page) are zeroed
  // when the tile is stored to LDS, so the loads stay in flight until then; the scores of a
  // missing page's keys are masked like those of keys past the query. The tile base is
  // wave-uniform; each lane adds one 32-bit offset (its first row and dims chunk).
  const uint32_t k_off = (uint32_t)(ld_kq * KPT * D + ld_c * 8);
  auto load_rows = [&](const uint16_t* pool, int tile, int64_t ph, uint32_t lane_off, uint4 (&dst)[KPT]) {
    const int t0 = tile * BN;
    const uint16_t* tp = pool + ((ph < 0 ? 0 : ph) * page_stride + g * head_stride +
                                 (int64_t)(t0 & (kv.page_size - 1)) * D);
#pragma unroll
    for (int r = 0; r < KPT; ++r) dst[r] = *reinterpret_cast<const uint4*>(tp + lane_off + r * D);
  };
  // rows of tile `tile` that hold attendable keys (wave-uniform)
  auto valid_rows = [&](int tile, int64_t ph) { return ph < 0 ? 0 : seq_len - tile * BN; };
  // Page-table entry of a tile, loaded one iteration before it is needed and checked only
  // where it is used: the load is unconditional (index clamped into the table) so that no
  // wait for it is placed next to the load.
  auto raw_page = [&](int tile) -> int32_t {
    const int lp = min((tile * BN) >> kv.page_shift, kv.max_pages_per_seq - 1);
    return kv.page_table[(int64_t)b * kv.max_pages_per_seq + lp];
  };
  auto checked_page = [&](int tile, int32_t raw) -> int64_t {
    const int lp = (tile * BN) >> kv.page_shift;
    return (lp < kv.max_pages_per_seq && raw >= 0 && raw < kv.num_pages) ? (int64_t)raw : -1;
  };
  auto mask_rows = [&](uint4 (&v)[KPT], int row0, int lim) {
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      if (row0 + r >= lim) v[r] = make_uint4(0, 0, 0, 0);
  };
  auto store_k = [&](int buf, const uint4 (&src)[KPT]) {
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      *reinterpret_cast<uint4*>(&sh.k[buf][ld_kq * KPT + r][ld_c * 8]) = src[r];
  };
  auto store_v = [&](int buf, const uint4 (&src)[KPT]) {  // row-major, like K
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      *reinterpret_cast<uint4*>(&sh.v[buf][ld_kq * KPT + r][ld_c * 8]) = src[r];
  };

  // S^T = K Q^T for the K tile in buffer buf. s[mb][j*4+i] is key mb*32 + j*8 + hi*4 + i of the
  // tile, query column l32.
  auto qk = [&](int buf, f32x16 (&s)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        Frag8 a;
        a.u = *reinterpret_cast<const uint4*>(&sh.k[buf][mb * 32 + l32][ks * 16 + hi * 8]);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, qf[ks].v, s[mb], 0, 0, 0);
      }
  };
  // Causal mask (only tiles that reach past the wave's first query need it). The row maximum
  // of the masked tile is taken a few elements per step inside the P V product of the tile
  // before (so its VALU work sits between matrix instructions); finish_max combines the two
  // halves of the row and moves the running maximum, rescaling O and the row sum (the scale
  // is positive, so it is applied in the exponent).
  // Masked mode: every key outside the query's selection (a subset of 0..pos) gets -inf, one
  // v_cndmask per score with the tile record's lane masks (scalar loads) as the condition.
  // A tile on a page missing from the table (page_ok false, wave-uniform) is masked whole, as
  // the gathered kernels skip such keys: its masks are cleared (scalar work) or its causal
  // limit is put below the tile.
  auto apply_sel = [&](const uint64_t (&mw)[32], f32x16 (&s)[2], bool page_ok) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[mb][r] = __builtin_amdgcn_inverse_ballot_w64(page_ok ? mw[mb * 16 + r] : 0ull) ? s[mb][r]
                                                                                          : -INFINITY;
  };
  auto mask_tile = [&](int tile, f32x16 (&s)[2], bool page_ok) {
    if constexpr (MASKED) {  // the prologue's tile; the loop uses apply_sel
      uint64_t mw[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) mw[k] = selw[(int64_t)tile * 32 + k];
      apply_sel(mw, s, page_ok);
      return;
    }
    const int t0 = tile * BN;
    if (!page_ok || t0 + BN - 1 > pos0 + i_w) {
      const int lim = page_ok ? my_pos - t0 - hi * 4 : -BN;  // key offsets above lim are masked
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mb * 32 + (r >> 2) * 8 + (r & 3) > lim) s[mb][r] = -INFINITY;
    }
  };
  auto finish_max = [&](float mx) {
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    // wave-uniform test; -inf - -inf is NaN and compares false
    if (__any((m_new - m_run) * qscale > kRescaleLog2)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * qscale);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;
    }
  };
  // QK(next tile) and softmax(current tile) in lock step: k-step ks issues the two MFMAs of
  // S_next (K fragments read one step ahead) and then exponentiates 32/KS of the current
  // scores; a scheduling barrier closes every step, so each step's VALU work sits between
  // matrix instructions instead of after all of them. P^T is packed into the B operands of
  // the P V product (step (mb, kk) takes elements 8kk .. 8kk+7 of block mb), and the row sum
  // adds the bf16-rounded P, the values that product sees.
  auto qk_softmax = [&](int buf, f32x16 (&sn)[2], const f32x16 (&sc)[2], Frag8 (&pf)[4]) {
    constexpr int EPS = 32 / KS;  // score elements per step (4 for d = 128, 8 for d = 64)
    const float mq = (m_run == -INFINITY) ? 0.f : m_run * qscale;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[mb][r] = 0.f;
    Frag8 ka[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      ka[0][mb].u = *reinterpret_cast<const uint4*>(&sh.k[buf][mb * 32 + l32][hi * 8]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          ka[(ks + 1) & 1][mb].u =
              *reinterpret_cast<const uint4*>(&sh.k[buf][mb * 32 + l32][(ks + 1) * 16 + hi * 8]);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        sn[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1][mb].v, qf[ks].v, sn[mb], 0, 0, 0);
      // elements u = ks*EPS .. +EPS of the current tile; u -> (mb, kk, e) = (u/16, (u/8)%2, u%8)
#pragma unroll
      for (int u2 = 0; u2 < EPS; u2 += 2) {
        const int u = ks * EPS + u2;
        const int mb = u >> 4, kk = (u >> 3) & 1, e = u & 7;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[mb][kk * 8 + e], qscale, -mq));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[mb][kk * 8 + e + 1], qscale, -mq));
        const uint32_t w = pack_bf16x2(p0, p1);
        uint32_t* fw = reinterpret_cast<uint32_t*>(&pf[mb * 2 + kk].u);
        fw[e >> 1] = w;
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, psum, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum;
  };
  // O^T += V^T P^T. Step st = (mb, kk) covers keys mb*32 + kk*16 + {hi*4 + 0..3, 8 + hi*4 + 0..3},
  // the key permutation of the P^T fragments.
  auto pv = [&](int buf, const Frag8 (&pf)[4], const f32x16 (&sm)[2], float& mx) {
    auto vfrag = [&](int i) {  // i = st * DB + db; st outer: step st needs the first 8(st+1) exps
      const int st = i / DB, db = i % DB;
      const int kb = (st >> 1) * 32 + (st & 1) * 16 + hi * 4;
      // transposed reads: in each 16-lane group, lane c supplies key row kb + c/4, dims
      // db*32 + 16*(group & 1) + 4*(c % 4) .. +4, and receives its own dim (db*32 + l32) of the
      // four rows; the second read takes keys kb + 8 .. kb + 11
      const int c = lane & 15;
      const uint16_t* vp = &sh.v[buf][kb + (c >> 2)][db * 32 + 16 * ((lane >> 4) & 1) + 4 * (c & 3)];
      Frag8 a;
      a.h[0] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (__attribute__((address_space(3))) v4s*)(vp)));
      a.h[1] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (__attribute__((address_space(3))) v4s*)(vp + 8 * (D + VPAD))));
      return a;
    };
    // V^T fragments are read kVPre steps ahead into a rolling buffer; a scheduling barrier
    // after each step keeps the reads ahead of the matrix instructions that consume them.
    constexpr int kVPre = 4;
    Frag8 va[kVPre];
#pragma unroll
    for (int i = 0; i < kVPre; ++i) va[i] = vfrag(i);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % kVPre].v, pf[i / DB].v, o[i % DB], 0, 0, 0);
      if (i + kVPre < 4 * DB) va[i % kVPre] = vfrag(i + kVPre);
      // (taken on every tile: the maximum of the one extra tile past the wave's end is never
      // used, and a conditional maximum costs a select per step)
#pragma unroll
      for (int e = i * (32 / (4 * DB)); e < (i + 1) * (32 / (4 * DB)); ++e) mx = fmaxf(mx, sm[e >> 4][e & 15]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: K(t_lo), V(t_lo) and K(t_lo+1) in LDS, S(t_lo) computed, masked and its maximum
  // taken. Each loader role looks its page up one iteration ahead of the load that needs it.
  // Buffers are indexed by the tile's offset from t_lo.
  uint4 st[KPT];
  int32_t raw_next = 0;  // page-table entry of the next tile this wave loads
  // Whether the page of the tile whose scores the wave masks next is in the table: V loaders
  // look up tile j+1 in iteration j (the tile masked there), K loaders one iteration earlier.
  bool ok_tile0 = true, ok_ahead = true;
  f32x16 sa[2], sb[2];
  if (n_own > 0) {  // workgroup-uniform
    if (k_loader) {
      int64_t ph = phys_page(kv, b, t_lo * BN);
      ok_tile0 = ph >= 0;
      load_rows(kv.k_pool, t_lo, ph, k_off, st);
      int lim = valid_rows(t_lo, ph);
      if (lim < BN) mask_rows(st, ld_kq * KPT, lim);
      store_k(0, st);
      if (n_own > 1) {
        ph = phys_page(kv, b, (t_lo + 1) * BN);
        ok_ahead = ph >= 0;
        load_rows(kv.k_pool, t_lo + 1, ph, k_off, st);
        lim = valid_rows(t_lo + 1, ph);
        if (lim < BN) mask_rows(st, ld_kq * KPT, lim);
        store_k(1, st);
      }
      raw_next = raw_page(t_lo + 2);
    } else {
      const int64_t ph = phys_page(kv, b, t_lo * BN);
      ok_tile0 = ph >= 0;
      load_rows(kv.v_pool, t_lo, ph, k_off, st);
      const int lim = valid_rows(t_lo, ph);
      if (lim < BN) mask_rows(st, ld_kq * KPT, lim);
      store_v(0, st);
      raw_next = raw_page(t_lo + 1);
    }
    __syncthreads();
  }
  if (last_w >= t_lo) {
    qk(0, sa);
    mask_tile(t_lo, sa, ok_tile0);
    float mx0 = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx0 = fmaxf(mx0, sa[e >> 4][e & 15]);
    finish_max(mx0);
  }

  // Iteration j (r = j - t_lo): on entry K buffer (r+1)&1 holds K(j+1), V buffer r&1 holds
  // V(j), sc holds the masked S(j) and m_run its running maximum. K loaders fetch K(j+2) into
  // registers while the tile is computed and store it to K buffer r&1; V loaders do the same
  // with V(j+1) and V buffer (r+1)&1. Neither buffer is read during iteration j.
  auto iter = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int r = j - t_lo;
    // the load past the last tile reads the last tile's slots of page 0 (in bounds) and is
    // never stored
    const int ltile = k_loader ? j + 2 : j + 1;
    const bool more = ltile < t_hi;
    const int lt = more ? ltile : t_hi - 1;
    const int64_t ph = more ? checked_page(ltile, raw_next) : 0;
    raw_next = raw_page(ltile + 1);
    bool ok_next;  // page status of tile j+1, whose scores this iteration masks
    if (k_loader) {
      ok_next = ok_ahead;
      ok_ahead = ph >= 0;
    } else {
      ok_next = ph >= 0;
    }
    load_rows(k_loader ? kv.k_pool : kv.v_pool, lt, ph, k_off, st);
    const int lim = __builtin_amdgcn_readfirstlane(valid_rows(lt, ph));
    float mx = -INFINITY;
    if (j <= last_w) {
      // S(j+1) is computed unconditionally (one extra tile at the wave's end, never used) so
      // that its matrix instructions share a basic block with the exponentials of S(j).
      Frag8 pf[4];
      // masked mode: the record of tile j+1 is requested before the QK^T of that tile so that
      // the scalar loads are back when its scores are masked (clamped: in bounds, unused)
      uint64_t mw[32];
      if constexpr (MASKED) {
        const uint64_t* w = selw + (int64_t)min(j + 1, last_w) * 32;
#pragma unroll
        for (int k = 0; k < 32; ++k) mw[k] = w[k];
      }
      qk_softmax((r + 1) & 1, sn, sc, pf);
      // (masked mode applies the record unconditionally: S(j+1) is not used past last_w, and
      // a conditional use would let the compiler sink the loads to it)
      if constexpr (MASKED) apply_sel(mw, sn, ok_next);
      else if (j + 1 <= last_w) mask_tile(j + 1, sn, ok_next);
      pv(r & 1, pf, sn, mx);
    }
    if (more) {
      if (lim < BN) mask_rows(st, ld_kq * KPT, lim);
      if (k_loader) store_k(r & 1, st);
      else store_v((r + 1) & 1, st);
    }
    if (j + 1 <= last_w) finish_max(mx);
    __syncthreads();
  };
  for (int j = t_lo; j < t_hi; j += 2) {
    iter(j, sa, sb);
    if (j + 1 < t_hi) iter(j + 1, sb, sa);
  }

  // finalize: O^T[db*32 + j*8 + hi*4 + i][query l32]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!my_valid) return;
  if (part != nullptr) {
    // Key splits: this split's unnormalised O, its maximum in exp2 units and its row sum, in
    // the split-merge layout: [unit][split][head of group][D] accumulators, then
    // [unit][split][head of group][2] (max, sum), unit = (b, query, KV head).
    const int64_t units = (int64_t)kv.batch * q_len * kv.num_kv_heads;
    const int64_t slot = ((((int64_t)b * q_len + my_i) * kv.num_kv_heads + g) * num_splits + split) * G +
                         (h - g * G);
    float* acc = part + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(acc + db * 32 + j * 8 + hi * 4) =
            make_float4(o[db][j * 4 + 0], o[db][j * 4 + 1], o[db][j * 4 + 2], o[db][j * 4 + 3]);
    if (hi == 0) {
      float* ml = part + units * num_splits * G * D + slot * 2;
      ml[0] = (m_run == -INFINITY) ? -INFINITY : m_run * qscale;
      ml[1] = l_tot;
    }
    return;
  }
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const int64_t orow = (((int64_t)b * q_len + my_i) * num_q_heads + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 w;
      w.x = pack_bf16x2(o[db][j * 4 + 0] * inv, o[db][j * 4 + 1] * inv);
      w.y = pack_bf16x2(o[db][j * 4 + 2] * inv, o[db][j * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(out + orow + db * 32 + j * 8 + hi * 4) = w;
    }
  if (lse != nullptr && hi == 0)
    lse[((int64_t)b * q_len + my_i) * num_q_heads + h] =
        (l_tot > 0.f) ? (m_run * qscale + log2f(l_tot)) * kLn2 : -INFINITY;
}

// Causal key tiles of the block's last query (host bound from max_seq_len).
int64_t block_tiles(const KvView& kv, int q_len, int q_tail) {
  const int64_t last_pos = (int64_t)kv.max_seq_len - q_tail + q_len - 1;
  return last_pos < 0 ? 0 : last_pos / BN + 1;
}

template <int D>
hipError_t launch_dense_d(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                          int q_tail, float sm_scale, uint16_t* out, float* lse,
                          const uint64_t* sel, int num_splits, float* part, hipStream_t stream) {
  constexpr int BMQ = kDenseWaves * 32;
  const int nqb = (q_len + BMQ - 1) / BMQ;
  const int split = num_splits > 1 ? num_splits : 1;
  const int64_t wgs = (int64_t)nqb * kv.batch * num_q_heads * split;
  const int tps = split > 1 ? (int)((block_tiles(kv, q_len, q_tail) + split - 1) / split) : (1 << 30);
  float* p = split > 1 ? part : nullptr;
  if (sel == nullptr) {
    hipLaunchKernelGGL((k_attn_dense<D, false>), dim3((unsigned)wgs), dim3(kDenseThreads), 0, stream,
                       kv, q, num_q_heads, q_len, q_tail, sm_scale * kLog2e, out, lse, nqb,
                       (const uint64_t*)nullptr, 0, 0, split, tps, p);
  } else {
    hipLaunchKernelGGL((k_attn_dense<D, true>), dim3((unsigned)wgs), dim3(kDenseThreads), 0, stream,
                       kv, q, num_q_heads, q_len, q_tail, sm_scale * kLog2e, out, lse, nqb, sel,
                       sel_query_blocks(q_len), sel_tiles(kv), split, tps, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  const int64_t units = (int64_t)kv.batch * q_len * kv.num_kv_heads;
  return launch_merge_splits(part, units, split, num_q_heads, kv.num_kv_heads, D, out, lse, stream);
}

// Selection masks from index lists. One workgroup per (sequence, indexer head, block of 32
// queries) builds the block's records for a range of up to kSelRange tiles in LDS (bits set
// with LDS atomics, which commute) and writes them out whole, so every record of the
// workspace is written, zeros included (queries past q_len, keys never selected).
constexpr int kSelRange = 512;   // tiles per LDS pass: 512 x 256 B = 128 KiB
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void k_sel_masks(KvView kv, int q_len, int q_tail,
                                                           const int32_t* __restrict__ indices, int W,
                                                           uint64_t* __restrict__ sel, int n_qb,
                                                           int n_tiles) {
  __shared__ uint32_t bits[kSelRange * 64];  // [tile - j0][element w][lane half]
  const int qb = blockIdx.x;
  const int bg = blockIdx.y;  // b * H_idx + gi
  const int b = bg / kv.num_idx_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int NW = kSelThreads / 64;
  const int seq_len = min(kv.seq_lens[b], kv.max_seq_len);
  uint64_t* dst = sel + ((int64_t)bg * n_qb + qb) * (int64_t)n_tiles * 32;
  for (int j0 = 0; j0 < n_tiles; j0 += kSelRange) {
    const int nt = min(kSelRange, n_tiles - j0);
    for (int k = tid; k < nt * 16; k += kSelThreads)
      reinterpret_cast<uint4*>(bits)[k] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    const int key_lo = j0 * BN, key_hi = (j0 + nt) * BN;  // keys of this range: [key_lo, key_hi)
    for (int ql = wave; ql < 32; ql += NW) {
      const int i = qb * 32 + ql;
      if (i >= q_len) continue;  // wave-uniform
      const int pos = seq_len - q_tail + i;
      const int lim = min(pos + 1, min(seq_len, key_hi));  // keys >= lim are never attended
      const int32_t* list = indices + (((int64_t)b * q_len + i) * kv.num_idx_heads +
                                       (bg - b * kv.num_idx_heads)) * (int64_t)W;
      auto set = [&](int t) {
        if (t >= key_lo && t < lim) {
          const int o = t & (BN - 1);
          const int o2 = o & 31;
          const int w = (o >> 5) * 16 + (o2 >> 3) * 4 + (o2 & 3);
          atomicOr(&bits[((t >> 6) - j0) * 64 + w * 2 + ((o2 >> 2) & 1)], 1u << ql);
        }
      };
      if ((W & 3) == 0) {  // rows start 16-byte aligned: four entries per load
        const int4* l4 = reinterpret_cast<const int4*>(list);
#pragma unroll 8
        for (int e = lane; e < (W >> 2); e += 64) {
          const int4 v = l4[e];
          set(v.x);
          set(v.y);
          set(v.z);
          set(v.w);
        }
      } else {
#pragma unroll 8
        for (int e = lane; e < W; e += 64) set(list[e]);
      }
    }
    __syncthreads();
    uint4* d4 = reinterpret_cast<uint4*>(dst + (int64_t)j0 * 32);
    for (int k = tid; k < nt * 16; k += kSelThreads) d4[k] = reinterpret_cast<const uint4*>(bits)[k];
    __syncthreads();
  }
}

}  // namespace

// Key splits of the masked dense attention: a block whose workgroups would leave CUs idle (a
// short block: one 8-wave workgroup per 256 queries and query head fills a CU) splits its
// causal key tiles among up to that many workgroups, at least kMinSplitTiles tiles each, and
// the split results are merged like the decode splits.
constexpr int kNumCus = 256;  // MI355X
constexpr int kMinSplitTiles = 8;
constexpr int kMaxDenseSplits = 64;

int dense_splits(const KvView& kv, int num_q_heads, int q_len, int q_tail) {
  const int G = num_q_heads / kv.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return 1;  // group sizes the merge is built for
  constexpr int BMQ = kDenseWaves * 32;
  const int64_t wgs = (int64_t)((q_len + BMQ - 1) / BMQ) * kv.batch * num_q_heads;
  int64_t s = kNumCus / wgs;
  s = std::min<int64_t>(s, block_tiles(kv, q_len, q_tail) / kMinSplitTiles);
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxDenseSplits));
}

size_t dense_split_bytes(const KvView& kv, int num_q_heads, int q_len, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)kv.batch * q_len * num_q_heads * num_splits * (kv.head_dim + 2) * sizeof(float);
}

int sel_query_blocks(int q_len) {
  constexpr int BMQ = kDenseWaves * 32;
  return (q_len + BMQ - 1) / BMQ * kDenseWaves;
}

int sel_tiles(const KvView& kv) { return (kv.max_seq_len + BN - 1) / BN; }

size_t sel_workspace_bytes(const KvView& kv, int q_len) {
  return (size_t)kv.batch * kv.num_idx_heads * sel_query_blocks(q_len) * sel_tiles(kv) * 256;
}

hipError_t launch_attn_dense(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                             int q_tail, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t stream) {
  if (kv.head_dim == 128)
    return launch_dense_d<128>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, nullptr, 1, nullptr, stream);
  if (kv.head_dim == 64)
    return launch_dense_d<64>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, nullptr, 1, nullptr, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_masked(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                              int q_tail, const int32_t* indices, int index_width, float sm_scale,
                              void* ws, uint16_t* out, float* lse, hipStream_t stream) {
  uint64_t* sel = static_cast<uint64_t*>(ws);
  const int n_qb = sel_query_blocks(q_len), n_tiles = sel_tiles(kv);
  hipLaunchKernelGGL(k_sel_masks, dim3((unsigned)n_qb, (unsigned)(kv.batch * kv.num_idx_heads)),
                     dim3(kSelThreads), 0, stream, kv, q_len, q_tail, indices, index_width, sel, n_qb,
                     n_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv.head_dim == 128)
    return launch_dense_d<128>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, sel, 1, nullptr, stream);
  if (kv.head_dim == 64)
    return launch_dense_d<64>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, sel, 1, nullptr, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_masked_records(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                                      int q_tail, float sm_scale, const uint64_t* sel, int num_splits,
                                      float* part, uint16_t* out, float* lse, hipStream_t stream) {
  if (kv.head_dim == 128)
    return launch_dense_d<128>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, sel, num_splits, part, stream);
  if (kv.head_dim == 64)
    return launch_dense_d<64>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, sel, num_splits, part, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
