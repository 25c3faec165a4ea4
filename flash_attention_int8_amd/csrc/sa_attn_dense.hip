// Dense causal FlashAttention forward on bf16 MFMA: the special case of the sparse path in
// which every causal key is selected.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" §2.3: prefill
// is the compute-heavy phase and runs on the matrix units.
//
// Workgroup: 4 waves, 128 queries of one query head (32 per wave), streaming 64-key tiles
// of the KV head through LDS with a two-stage buffer (the next tile's global loads are in
// flight while the current tile is computed).
// Per wave and tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K * Q^T   (A = K tile rows from LDS, B = the wave's Q^T held in registers).
//                   The accumulator layout gives each lane 32 of the 64 scores of ONE query
//                   (the other 32 sit in lane ^ 32), so the softmax row max is a local max
//                   plus one cross-half exchange, and row sums stay per lane until the end.
//   O^T += V^T * P^T  (A = V^T from LDS, B = P^T taken straight from the S^T accumulators:
//                   the 8 scores a lane holds for one 16-key step become its B operand, and
//                   the V^T reads use the same key permutation, so no shuffle is needed).
// V is transposed into LDS on the way in: each thread loads D/32 key rows x 8 dims and
// writes D/32-key runs of each dim. Softmax is base 2 with sm_scale*log2(e) applied to the
// fp32 scores; Q, K and V stay exact bf16, accumulation is fp32, P is rounded to bf16.
#include "sa_common.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int BN = 64;    // keys per tile
constexpr int KPAD = 8;   // bf16 padding of a K row in LDS
constexpr int VPAD = 4;   // bf16 padding of a V^T row in LDS (row stride 136 B: 16 consecutive rows
                          // hit 16 distinct 8-byte bank pairs)

template <int D>
struct DenseShared {
  uint16_t k[2][BN][D + KPAD];
  uint16_t vt[2][D][BN + VPAD];
};

union Frag8 {
  bf16x8 v;
  uint4 u;
  uint2 h[2];
};

// NQB = 32-query column blocks per wave. With NQB = 2 a wave owns 64 queries, so every K and
// V^T fragment read from LDS feeds two MFMAs: half the LDS traffic per flop of NQB = 1.
template <int D, int NQB>
__global__ __launch_bounds__(256, (NQB == 1 ? 2 : 1)) void k_attn_dense(
    KvView kv, const uint16_t* __restrict__ q, int num_q_heads, int q_len, int q_tail, float qscale,
    uint16_t* __restrict__ out, float* __restrict__ lse, int n_qblocks) {
  constexpr int KS = D / 16;     // k-steps of QK^T
  constexpr int DB = D / 32;     // 32-dim blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int KPT = D / 32;    // key rows per thread in the tile loader
  constexpr int QW = 32 * NQB;   // queries per wave
  constexpr int BMQ = 4 * QW;    // queries per workgroup
  __shared__ DenseShared<D> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // heaviest query blocks first (causal work grows with the block index)
  const int bh_count = kv.batch * num_q_heads;
  const int qblk = n_qblocks - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / num_q_heads;
  const int h = bh - b * num_q_heads;
  const int g = h / (num_q_heads / kv.num_kv_heads);
  const int seq_len = min(kv.seq_lens[b], kv.max_seq_len);
  const int pos0 = seq_len - q_tail;              // position of query 0
  const int i_blk = qblk * BMQ;
  const int i_w = i_blk + wave * QW;              // first query of this wave
  const int i_last_blk = min(q_len, i_blk + BMQ) - 1;
  const int wave_pos_max = pos0 + min(q_len - 1, i_w + QW - 1);
  const int blk_pos_max = pos0 + i_last_blk;
  if (blk_pos_max < 0) return;
  const int n_tiles = blk_pos_max / BN + 1;

  // per column block nb: this lane's query, its position and validity
  int my_i[NQB], my_pos[NQB];
  bool my_valid[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    my_i[nb] = i_w + nb * 32 + l32;
    my_pos[nb] = pos0 + my_i[nb];
    my_valid[nb] = my_i[nb] < q_len;
  }

  // Q^T fragments (B operand): lane holds query l32 of block nb, dims ks*16 + hi*8 .. +8.
  Frag8 qf[NQB][KS];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int qi = my_valid[nb] ? my_i[nb] : i_blk;  // any valid row; never stored
    const uint16_t* qp = q + (((int64_t)b * q_len + qi) * num_q_heads + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nb][ks].u = *reinterpret_cast<const uint4*>(qp + ks * 16);
  }

  f32x16 o[DB][NQB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][nb][r] = 0.f;
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }

  // Tile loader mappings. K: dims chunk ld_c (8 dims) of key rows ld_kq*KPT .. +KPT, so 16
  // neighbouring lanes store 256 contiguous bytes of a row. V (stored transposed): each group
  // of 16 lanes shares one dims chunk and walks the 16 key groups, so a transposed store of
  // one dim writes 16 contiguous KPT-key runs instead of 16 rows that share a bank.
  const int ld_c = tid % CPR;
  const int ld_kq = tid / CPR;
  constexpr int KQ = BN / KPT;                       // key groups per tile (16)
  const int lv_c = (tid / KQ) % CPR;                 // V dims chunk
  const int lv_kq = tid % KQ;                        // V key group
  const int64_t head_stride = (int64_t)kv.page_size * D;
  const int64_t page_stride = head_stride * kv.num_kv_heads;

  uint4 pk[KPT], pv[KPT];
  auto load_tile = [&](int tile) {
    const int t0 = tile * BN;
    const int64_t ph = phys_page(kv, b, t0);
    if (ph < 0) {
#pragma unroll
      for (int r = 0; r < KPT; ++r) { pk[r] = make_uint4(0, 0, 0, 0); pv[r] = make_uint4(0, 0, 0, 0); }
      return;
    }
    const int64_t base = ph * page_stride + g * head_stride + (int64_t)(t0 & (kv.page_size - 1)) * D;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int krow = ld_kq * KPT + r;
      const int vrow = lv_kq * KPT + r;
      // rows past the end of the sequence are never attended; they are kept finite
      pk[r] = (t0 + krow < seq_len) ? *reinterpret_cast<const uint4*>(kv.k_pool + base + (int64_t)krow * D + ld_c * 8)
                                    : make_uint4(0, 0, 0, 0);
      pv[r] = (t0 + vrow < seq_len) ? *reinterpret_cast<const uint4*>(kv.v_pool + base + (int64_t)vrow * D + lv_c * 8)
                                    : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      *reinterpret_cast<uint4*>(&sh.k[buf][ld_kq * KPT + r][ld_c * 8]) = pk[r];
    // transpose V: for each of the 8 dims, write the KPT keys as one run
    const uint32_t* w[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) w[r] = reinterpret_cast<const uint32_t*>(&pv[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t vals[KPT];
#pragma unroll
      for (int r = 0; r < KPT; ++r) vals[r] = (uint16_t)((w[r][e >> 1] >> ((e & 1) * 16)) & 0xffff);
      uint16_t* dst = &sh.vt[buf][lv_c * 8 + e][lv_kq * KPT];
      if constexpr (KPT == 4) {
        uint2 pkd;
        pkd.x = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
        pkd.y = (uint32_t)vals[2] | ((uint32_t)vals[3] << 16);
        *reinterpret_cast<uint2*>(dst) = pkd;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) load_tile(tile + 1);
    const int t0 = tile * BN;
    if (t0 <= wave_pos_max) {
      // S^T = K Q^T: 32-key blocks mb x 32-query blocks nb; each K fragment feeds NQB MFMAs
      f32x16 s[2][NQB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[mb][nb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          Frag8 a;
          a.u = *reinterpret_cast<const uint4*>(&sh.k[buf][mb * 32 + l32][ks * 16 + hi * 8]);
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb)
            s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, qf[nb][ks].v, s[mb][nb], 0, 0, 0);
        }
      // causal mask and row max on the raw scores (the scale is positive, so it is applied in
      // the exponent). s[mb][nb][j*4+i] is key t0 + mb*32 + j*8 + hi*4 + i, query column l32.
      const bool diag = (t0 + BN - 1) > (pos0 + i_w);
      Frag8 pf[NQB][4];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (diag) {
              const int key = t0 + mb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
              if (key > my_pos[nb]) s[mb][nb][r] = -INFINITY;
            }
            mx = fmaxf(mx, s[mb][nb][r]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[nb], mx);
        // Rescale the running sum and O only when some lane's maximum grew (wave-uniform test).
        if (__any(m_new > m_run[nb])) {
          const float alpha =
              (m_run[nb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run[nb] - m_new) * qscale);
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][nb][r] *= alpha;
          m_run[nb] = m_new;
        }
        const float mq = (m_run[nb] == -INFINITY) ? 0.f : m_run[nb] * qscale;
        float psum = 0.f;
        // P^T as B operands: step (mb, kk) takes j = 2kk, 2kk+1 of block mb (8 values)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][kk * 8 + e], qscale, -mq));
              psum += p[e];
            }
            Frag8& f = pf[nb][mb * 2 + kk];
            f.u.x = pack_bf16x2(p[0], p[1]);
            f.u.y = pack_bf16x2(p[2], p[3]);
            f.u.z = pack_bf16x2(p[4], p[5]);
            f.u.w = pack_bf16x2(p[6], p[7]);
          }
        l_run[nb] += psum;
      }
      // O^T += V^T P^T. Step st = (mb, kk) covers keys mb*32 + kk*16 + {hi*4 + 0..3, 8 + hi*4 + 0..3};
      // each V^T fragment feeds NQB MFMAs.
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kb = (st >> 1) * 32 + (st & 1) * 16 + hi * 4;
          const uint16_t* vrow = &sh.vt[buf][db * 32 + l32][0];
          Frag8 a;
          a.h[0] = *reinterpret_cast<const uint2*>(vrow + kb);
          a.h[1] = *reinterpret_cast<const uint2*>(vrow + kb + 8);
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb)
            o[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, pf[nb][st].v, o[db][nb], 0, 0, 0);
        }
    }
    if (tile + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // finalize: O^T[db*32 + j*8 + hi*4 + i][query l32 of block nb]
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 32, 64);
    if (!my_valid[nb]) continue;
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int64_t orow = (((int64_t)b * q_len + my_i[nb]) * num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w;
        w.x = pack_bf16x2(o[db][nb][j * 4 + 0] * inv, o[db][nb][j * 4 + 1] * inv);
        w.y = pack_bf16x2(o[db][nb][j * 4 + 2] * inv, o[db][nb][j * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(out + orow + db * 32 + j * 8 + hi * 4) = w;
      }
    if (lse != nullptr && hi == 0)
      lse[((int64_t)b * q_len + my_i[nb]) * num_q_heads + h] =
          (l_tot > 0.f) ? (m_run[nb] * qscale + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int NQB>
hipError_t launch_dense_d(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                          int q_tail, float sm_scale, uint16_t* out, float* lse,
                          hipStream_t stream) {
  constexpr int BMQ = 4 * 32 * NQB;
  const int nqb = (q_len + BMQ - 1) / BMQ;
  const int64_t wgs = (int64_t)nqb * kv.batch * num_q_heads;
  hipLaunchKernelGGL((k_attn_dense<D, NQB>), dim3((unsigned)wgs), dim3(256), 0, stream, kv, q,
                     num_q_heads, q_len, q_tail, sm_scale * kLog2e, out, lse, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_dense(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                             int q_tail, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t stream) {
  // 64 queries per wave halves LDS traffic per flop but leaves one wave per SIMD, which loses
  // more (no overlap of one wave's softmax with another's MFMAs) than it gains on MI355X.
  const bool wide = false;
  if (kv.head_dim == 128)
    return wide ? launch_dense_d<128, 2>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream)
                : launch_dense_d<128, 1>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream);
  if (kv.head_dim == 64)
    return wide ? launch_dense_d<64, 2>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream)
                : launch_dense_d<64, 1>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
