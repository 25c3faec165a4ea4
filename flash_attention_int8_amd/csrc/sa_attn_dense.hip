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
constexpr int BM = 128;   // queries per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int KPAD = 8;   // bf16 padding of a K row in LDS
constexpr int VPAD = 8;   // bf16 padding of a V^T row in LDS

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

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_dense(KvView kv, const uint16_t* __restrict__ q,
                                                       int num_q_heads, int q_len, int q_tail,
                                                       float qscale, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int n_qblocks) {
  constexpr int KS = D / 16;     // k-steps of QK^T
  constexpr int DB = D / 32;     // 32-dim blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int KPT = D / 32;    // key rows per thread in the tile loader
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
  const int i_blk = qblk * BM;
  const int i_w = i_blk + wave * 32;              // first query of this wave
  const int i_last_blk = min(q_len, i_blk + BM) - 1;
  const int my_i = i_w + l32;                     // query this lane's column belongs to
  const int my_pos = pos0 + my_i;
  const bool my_valid = my_i < q_len;
  const int wave_pos_max = pos0 + min(q_len - 1, i_w + 31);
  const int blk_pos_max = pos0 + i_last_blk;
  if (blk_pos_max < 0) return;
  const int n_tiles = blk_pos_max / BN + 1;

  // Q^T fragments (B operand): lane holds query l32, dims ks*16 + hi*8 .. +8.
  Frag8 qf[KS];
  {
    const int qi = my_valid ? my_i : i_blk;  // any valid row; its results are never stored
    const uint16_t* qp = q + (((int64_t)b * q_len + qi) * num_q_heads + h) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks].u = *reinterpret_cast<const uint4*>(qp + ks * 16);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // tile loader mapping: dims chunk c (8 dims), keys kq*KPT .. +KPT
  const int ld_c = tid % CPR;
  const int ld_kq = tid / CPR;
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
    const int64_t base = ph * page_stride + g * head_stride +
                         (int64_t)(t0 & (kv.page_size - 1)) * D + ld_c * 8;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int row = ld_kq * KPT + r;
      if (t0 + row < seq_len) {
        const int64_t o2 = base + (int64_t)row * D;
        pk[r] = *reinterpret_cast<const uint4*>(kv.k_pool + o2);
        pv[r] = *reinterpret_cast<const uint4*>(kv.v_pool + o2);
      } else {  // past the end of the sequence: never attended, kept finite
        pk[r] = make_uint4(0, 0, 0, 0);
        pv[r] = make_uint4(0, 0, 0, 0);
      }
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
      uint16_t* dst = &sh.vt[buf][ld_c * 8 + e][ld_kq * KPT];
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
      // S^T = K Q^T : two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag8 a;
          a.u = *reinterpret_cast<const uint4*>(&sh.k[buf][mb * 32 + l32][ks * 16 + hi * 8]);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, qf[ks].v, s[mb], 0, 0, 0);
        }
      }
      // scale, causal mask, row max. s[mb][j*4+i] is key t0 + mb*32 + j*8 + hi*4 + i.
      const bool diag = (t0 + BN - 1) > (pos0 + i_w);
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[mb][r] * qscale;
          if (diag) {
            const int key = t0 + mb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            if (key > my_pos) v = -INFINITY;
          }
          s[mb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      // P^T as B operands: step kk of block mb takes j = 2kk', 2kk'+1 (8 values)
      Frag8 pf[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = exp2f(s[mb][kk * 8 + e] - m_use);
            psum += p[e];
          }
          Frag8& f = pf[mb * 2 + kk];
          f.u.x = pack_bf16x2(p[0], p[1]);
          f.u.y = pack_bf16x2(p[2], p[3]);
          f.u.z = pack_bf16x2(p[4], p[5]);
          f.u.w = pack_bf16x2(p[6], p[7]);
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      // O^T += V^T P^T. Step (mb, kk) covers keys mb*32 + kk*16 + {hi*4 + 0..3, 8 + hi*4 + 0..3}.
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kb = (st >> 1) * 32 + (st & 1) * 16 + hi * 4;
          const uint16_t* vrow = &sh.vt[buf][db * 32 + l32][0];
          Frag8 a;
          a.h[0] = *reinterpret_cast<const uint2*>(vrow + kb);
          a.h[1] = *reinterpret_cast<const uint2*>(vrow + kb + 8);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, pf[st].v, o[db], 0, 0, 0);
        }
    }
    if (tile + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // finalize: O^T[db*32 + j*8 + hi*4 + i][query l32]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_valid) {
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
          (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_dense_d(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                          int q_tail, float sm_scale, uint16_t* out, float* lse,
                          hipStream_t stream) {
  const int nqb = (q_len + BM - 1) / BM;
  const int64_t wgs = (int64_t)nqb * kv.batch * num_q_heads;
  hipLaunchKernelGGL(k_attn_dense<D>, dim3((unsigned)wgs), dim3(256), 0, stream, kv, q, num_q_heads,
                     q_len, q_tail, sm_scale * kLog2e, out, lse, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_dense(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                             int q_tail, float sm_scale, uint16_t* out, float* lse,
                             hipStream_t stream) {
  if (kv.head_dim == 128) return launch_dense_d<128>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream);
  if (kv.head_dim == 64) return launch_dense_d<64>(kv, q, num_q_heads, q_len, q_tail, sm_scale, out, lse, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
