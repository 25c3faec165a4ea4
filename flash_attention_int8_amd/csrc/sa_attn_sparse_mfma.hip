// Sparse prefill attention on bf16 MFMA: online-softmax attention of each query token over its
// own index list (forced prefix + top-K), gathered from the paged KV pool.
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析":
//   §2.2  the selected rows are gathered out of fixed-size KV pages into a contiguous tile;
//   §2.3  prefill is the compute-heavy phase and runs on the matrix units, with the gather of
//         the next tile overlapping the compute of the current one.
//
// A unit is one (sequence, query token, KV group); its G = H_q / H_kv query heads share the index
// list, so one gathered K/V row serves G heads. One wave takes one unit and walks its list in
// tiles of 32 keys, with v_mfma_f32_16x16x32_bf16 (16 rows x 16 columns x 32-deep):
//   S^T = K Q^T   A = 16 gathered K rows, loaded from the pool straight into the operand
//                 registers (lane l: 16 bytes of key l%16), B = Q^T with the G heads as columns
//                 (the other 16 - G columns are zero), C: lane l holds keys 4(l/16)+i of head
//                 l%16. Only V goes through LDS (for the transposed reads), which keeps LDS and
//                 registers low enough for three waves per SIMD.
//   O^T += V^T P^T  A = V^T: 16 dims x 32 keys, read from the row-major V tile with two
//                 ds_read_b64_tr_b16 (lane l gets dim l%16 of keys {4g..4g+3} and
//                 {16+4g..16+4g+3}, g = l/16); B = P^T straight from the two S^T accumulators
//                 of the tile, whose key order is the same {4g+i, 16+4g+i}.
// The heads fill only G of the 16 MFMA columns, so at most G/16 of the matrix work is useful;
// the matrix units still do the 4*G*d flop per key in a fraction of the time the VALU needs,
// and the kernel is bound by the gather of the selected rows through L2 and the Infinity Cache.
// Softmax is base 2 with sm_scale*log2(e) applied in the exponent; P is rounded to bf16 for P V.
// Two row sums are kept: the rounded P normalises O (an exact convex combination of the weights
// P V saw, as in the dense kernel) and the fp32 P gives the LSE (only fp32 rounding); the kernel
// is bound by its row gathers, so the extra adds are free. The running maximum moves only when
// a score exceeds it by more than 2^8 (exp2 units), which leaves the result unchanged.
#include "sa_common.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;
constexpr int TK = 32;  // keys per tile

union Frag8 {
  bf16x8 v;
  uint4 u;
  v4s h[2];
};

template <int D>
struct SparseShared {
  uint16_t v[TK][D + 16];   // gathered V rows; row stride 288 B: the 4 rows of one transposed
                            // read hit 4 distinct 8-bank groups
  int32_t rid[2][TK];       // resolved pool rows of the current and the next tile (-1: none)
};

template <int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_attn_sparse_mfma(
    KvView kv, const uint16_t* __restrict__ q, int num_q_heads, int q_len, int q_tail,
    const int32_t* __restrict__ indices, int W, int top_k, float qscale,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(G <= 16, "the heads of a group are the 16 MFMA columns");
  constexpr int KS = D / 32;  // 32-deep k-steps of QK^T
  constexpr int NB = D / 16;  // 16-dim blocks of O^T
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int RPL = TK * CPR / 64;  // V row chunks each lane loads per tile
  __shared__ SparseShared<D> sh;

  const int lane = threadIdx.x;
  const int col = lane & 15;   // MFMA column: head (S^T, O^T) / row of A
  const int grp = lane >> 4;   // k-group of the MFMA operands, row group of C
  const int64_t unit = blockIdx.x;  // (b * q_len + i) * H_kv + g
  const int g = (int)(unit % kv.num_kv_heads);
  const int64_t bi = unit / kv.num_kv_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int seq_len = __builtin_amdgcn_readfirstlane(min(kv.seq_lens[b], kv.max_seq_len));
  const int pos = seq_len - q_tail + i;
  const int gi = (kv.num_idx_heads == 1) ? 0 : g;
  const int32_t* ilist = indices + (bi * kv.num_idx_heads + gi) * (int64_t)W;
  // entries of the list that can hold keys: the forced prefix, then at most top_k selected
  const int P = kv.prefix_len;
  const int nf = pos < 0 ? 0 : min(P, pos + 1);
  const int ncand = pos - P + 1;
  const int w_valid = min(W, nf + (ncand > 0 ? min(top_k, ncand) : 0));
  const int n_tiles = (w_valid + TK - 1) / TK;

  const int64_t head_stride = (int64_t)kv.page_size * D;
  const int64_t page_stride = head_stride * kv.num_kv_heads;
  const uint16_t* kbase = kv.k_pool + g * head_stride;
  const uint16_t* vbase = kv.v_pool + g * head_stride;

  // Q^T fragments (B operand of S^T): column col = head, dims ks*32 + grp*8 .. +8
  Frag8 qf[KS];
  {
    const int h = col < G ? col : 0;
    const uint16_t* qp = q + (bi * num_q_heads + (int64_t)g * G + h) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks].u = *reinterpret_cast<const uint4*>(qp + ks * 32);
      if (col >= G) qf[ks].u = make_uint4(0, 0, 0, 0);
    }
  }
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f, l_exact = 0.f;
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};

  // List entry -> pool row in three steps, each issued an iteration before its result is used
  // (lanes 0..31 hold the tile's 32 entries): the entry (token), its page-table entry, and the
  // row id written to LDS with the tile's valid-key mask.
  const int32_t* ptab = kv.page_table + (int64_t)b * kv.max_pages_per_seq;
  auto fetch_tok = [&](int t) -> int {
    const int e = t * TK + lane;
    return (lane < TK && e < w_valid) ? ilist[e] : -1;
  };
  auto tok_ok = [&](int tok) {
    return tok >= 0 && tok <= pos && (tok >> kv.page_shift) < kv.max_pages_per_seq;
  };
  auto fetch_page = [&](int tok) -> int { return tok_ok(tok) ? ptab[tok >> kv.page_shift] : -1; };
  auto finish = [&](int tok, int pt, int slot) -> uint32_t {
    const bool ok = tok_ok(tok) && pt >= 0 && pt < kv.num_pages;
    const int rid = ok ? pt * kv.page_size + (tok & (kv.page_size - 1)) : -1;
    if (lane < TK) sh.rid[slot][lane] = rid;
    return (uint32_t)__ballot(lane < TK && rid >= 0);
  };
  auto row_off = [&](int rid) -> int64_t {
    return (int64_t)(rid >> kv.page_shift) * page_stride + (int64_t)(rid & (kv.page_size - 1)) * D;
  };
  // The tile's K rows -> the S^T A operands: kf[hh][ks] is 16 bytes of key hh*16 + col at dims
  // ks*32 + grp*8. V rows -> registers, lane loads chunk (lane % CPR) of rows r*64/CPR + lane/CPR.
  Frag8 kf[2][KS];
  uint4 vr[RPL];
  auto load_tile = [&](int slot) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int rid = sh.rid[slot][hh * 16 + col];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[hh][ks].u = rid >= 0 ? *reinterpret_cast<const uint4*>(kbase + row_off(rid) + ks * 32 + grp * 8)
                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int rid = sh.rid[slot][r * (64 / CPR) + lane / CPR];
      vr[r] = rid >= 0 ? *reinterpret_cast<const uint4*>(vbase + row_off(rid) + (lane % CPR) * 8)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      *reinterpret_cast<uint4*>(&sh.v[r * (64 / CPR) + lane / CPR][(lane % CPR) * 8]) = vr[r];
  };

  uint32_t vmask = 0, vmask_next = 0;
  int tok_n2 = -1;  // list entries of tile t+2
  if (n_tiles > 0) {
    int tk = fetch_tok(0);
    vmask = finish(tk, fetch_page(tk), 0);
    tk = fetch_tok(1);
    vmask_next = finish(tk, fetch_page(tk), 1);
    tok_n2 = fetch_tok(2);
    __syncthreads();
    load_tile(0);
    store_v();
    __syncthreads();
  }
  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1, nxt = cur ^ 1;
    // S^T for the two 16-key halves of the tile (its K operands were loaded an iteration ago)
    f32x4 s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[hh][ks].v, qf[ks].v, s[hh], 0, 0, 0);
    }
    // rows of tile t+1, page entries of tile t+2 and list entries of tile t+3 in flight while
    // the rest of tile t is computed (the K operand registers are free once S^T is issued)
    if (t + 1 < n_tiles) load_tile(nxt);
    const int tok_n3 = fetch_tok(t + 3);
    const int pt_n2 = fetch_page(tok_n2);
    // keys without a row (padding, past the causal end, missing page) are masked
    float mx = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = hh * 16 + grp * 4 + r;
        if (!((vmask >> key) & 1u)) s[hh][r] = -INFINITY;
        mx = fmaxf(mx, s[hh][r]);
      }
    {
      const FPair p16 = lane_pair<16>(mx);
      const FPair p32 = lane_pair<32>(fmaxf(p16.lo, p16.hi));
      mx = fmaxf(p32.lo, p32.hi);
    }
    const float m_new = fmaxf(m_run, mx);
    if (__any((m_new - m_run) * qscale > kRescaleLog2)) {  // wave-uniform, rare
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * qscale);
      l_part *= alpha;
      l_exact *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nb][r] *= alpha;
      m_run = m_new;
    }
    const float mq = (m_run == -INFINITY) ? 0.f : m_run * qscale;
    // P^T fragment: keys {4g+0..3} then {16+4g+0..3}, the k order of the V^T fragment
    Frag8 pf;
    {
      float p[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[hh * 4 + r] = __builtin_amdgcn_exp2f(fmaf(s[hh][r], qscale, -mq));
      pf.u.x = pack_bf16x2(p[0], p[1]);
      pf.u.y = pack_bf16x2(p[2], p[3]);
      pf.u.z = pack_bf16x2(p[4], p[5]);
      pf.u.w = pack_bf16x2(p[6], p[7]);
      l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pf.u.x), ones, l_part, false);
      l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pf.u.y), ones, l_part, false);
      l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pf.u.z), ones, l_part, false);
      l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pf.u.w), ones, l_part, false);
      l_exact += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    // O^T += V^T P^T. Transposed reads: source lane s of group g supplies row 4g + s/4 (and
    // 16 + 4g + s/4), dims nb*16 + 4(s%4) .. +4; lane l receives dim nb*16 + l%16 of the 4 rows.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      Frag8 a;
      const int vrow = grp * 4 + (col >> 2);
      const int vcol = nb * 16 + (col & 3) * 4;
      a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(&sh.v[vrow][vcol]));
      a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(&sh.v[16 + vrow][vcol]));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, pf.v, o[nb], 0, 0, 0);
    }
    // tile t+2's rows go to the slot tile t used (its rows were loaded an iteration ago)
    const uint32_t vmask_after = finish(tok_n2, pt_n2, cur);
    tok_n2 = tok_n3;
    if (t + 1 < n_tiles) {
      __syncthreads();  // the tile's LDS reads are done
      store_v();
    }
    __syncthreads();
    vmask = vmask_next;
    vmask_next = vmask_after;
  }

  // l over the 4 lanes of each head; O^T[dim nb*16 + 4g + r][head col] sits in o[nb][r]
  const FPair l16 = lane_pair<16>(l_part);
  const FPair l32 = lane_pair<32>(l16.lo + l16.hi);
  const float l_tot = l32.lo + l32.hi;
  const FPair e16 = lane_pair<16>(l_exact);
  const FPair e32 = lane_pair<32>(e16.lo + e16.hi);
  const float l_ex = e32.lo + e32.hi;
  if (col >= G) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t qh = bi * num_q_heads + (int64_t)g * G + col;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint2 w;
    w.x = pack_bf16x2(o[nb][0] * inv, o[nb][1] * inv);
    w.y = pack_bf16x2(o[nb][2] * inv, o[nb][3] * inv);
    *reinterpret_cast<uint2*>(out + qh * D + nb * 16 + grp * 4) = w;
  }
  if (lse != nullptr && grp == 0)
    lse[qh] = l_ex > 0.f ? (m_run * qscale + log2f(l_ex)) * kLn2 : -INFINITY;
}

template <int D, int G>
hipError_t launch_dg(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len, int q_tail,
                     const int32_t* indices, int W, int top_k, float sm_scale, uint16_t* out,
                     float* lse, hipStream_t stream) {
  const int64_t units = (int64_t)kv.batch * q_len * kv.num_kv_heads;
  hipLaunchKernelGGL((k_attn_sparse_mfma<D, G>), dim3((unsigned)units), dim3(64), 0, stream, kv, q,
                     num_q_heads, q_len, q_tail, indices, W, top_k, sm_scale * kLog2e, out, lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len, int q_tail,
                    const int32_t* indices, int W, int top_k, float sm_scale, uint16_t* out,
                    float* lse, hipStream_t stream) {
  switch (num_q_heads / kv.num_kv_heads) {
    case 1: return launch_dg<D, 1>(kv, q, num_q_heads, q_len, q_tail, indices, W, top_k, sm_scale, out, lse, stream);
    case 2: return launch_dg<D, 2>(kv, q, num_q_heads, q_len, q_tail, indices, W, top_k, sm_scale, out, lse, stream);
    case 4: return launch_dg<D, 4>(kv, q, num_q_heads, q_len, q_tail, indices, W, top_k, sm_scale, out, lse, stream);
    case 8: return launch_dg<D, 8>(kv, q, num_q_heads, q_len, q_tail, indices, W, top_k, sm_scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_sparse_mfma(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                                   int q_tail, const int32_t* indices, int index_width,
                                   float sm_scale, uint16_t* out, float* lse, hipStream_t stream) {
  // lists hold the prefix, then at most top_k selected keys, then -1 entries
  const int top_k = index_width > kv.prefix_len ? index_width - kv.prefix_len : 0;
  if (kv.head_dim == 128)
    return launch_d<128>(kv, q, num_q_heads, q_len, q_tail, indices, index_width, top_k, sm_scale, out, lse, stream);
  if (kv.head_dim == 64)
    return launch_d<64>(kv, q, num_q_heads, q_len, q_tail, indices, index_width, top_k, sm_scale, out, lse, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
