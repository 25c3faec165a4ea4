// Attention over per-query index lists: the decode path (split-K + exact merge) and the
// sparse prefill path (one unit per query token and KV group).
//
// [DSA-page] = "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析":
//   §2.2  the selected rows are gathered out of fixed-size KV pages;
//   §2.3  decode is memory-bound, so only the active rows are loaded, straight into
//         registers; prefill overlaps the gather of the next rows with compute.
//
// A unit is one (sequence, query token, KV group); its G = H_q/H_kv query heads share the
// index list, so every gathered K/V row is used by G heads. A workgroup of 4 waves takes a
// contiguous chunk of the list (a "split"). In a wave, d/8 lanes cover one key row (16 bytes
// of bf16 each), so a wave holds 64/(d/8) keys at once ("lane groups"). Each wave works in
// batches: it loads NB list entries per lane group, resolves their pages, issues all K and
// V row loads of the batch, then computes: G dot products per key (8 FMAs per lane + a DPP
// butterfly over the lane group), one running-max update per batch and G x 8 FMAs per key
// for the V accumulation. Every lane group keeps its own online-softmax state (max m, sum
// l, weighted V sum in fp32, base-2 exponent with log2(e) folded into the query); states
// are merged across lane groups and waves at the end, then either normalised and stored
// (one split) or written as partials for k_merge_splits (several splits). All merges run in
// a fixed order, so results are deterministic.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "sa_common.h"

namespace sa {
namespace {

// A K or V row piece read with the nontemporal hint: a decode step reads each selected row once,
// so the rows need not displace cached lines (measured: the 128K step's attention 25.8 -> 24.8
// us, cold caches).
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
__device__ __forceinline__ uint4 load_nt(const uint16_t* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSeg = 2048;  // list entries resolved into LDS at a time

// Keys each lane group loads at once: as many as the registers allow with 2 waves per SIMD.
template <int G>
struct KeysPerLaneGroup {
  static constexpr int value = G <= 2 ? 16 : (G == 4 ? 8 : 4);
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// a.lo * b.lo + a.hi * b.hi + c for two bf16 pairs packed in 32-bit words (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}
// (lo half of a, lo half of b) and (hi half of a, hi half of b) as packed pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float safe_scale(float m_old, float m_new) {
  return (m_old == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
}

// The running maximum used in the exponent moves only when a key's score exceeds it by more
// than 2^kRescaleLog2 (exp2 units): P stays below 2^kRescaleLog2, far inside bf16 and fp32
// range, and the result is unchanged because the sum and the V accumulator use the same
// maximum. Rescaling the accumulator then happens on a few keys per list instead of every
// sub-batch.
constexpr float kRescaleLog2 = 8.f;

template <int D, int G>
__global__ __launch_bounds__(256, 2) void k_attn_gather(KvView kv, const uint16_t* __restrict__ q,
                                                     int num_q_heads, int q_len, int q_tail,
                                                     const int32_t* __restrict__ indices, int W,
                                                     float qscale, int num_splits,
                                                     int keys_per_split, float* __restrict__ ws,
                                                     uint16_t* __restrict__ out,
                                                     float* __restrict__ lse) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPW = 64 / LPK;     // keys a wave holds at once (lane groups)
  constexpr int NW = 4;
  constexpr int STRIDE = NW * KPW;  // list entries covered by one load round of the workgroup
  constexpr int kNB = KeysPerLaneGroup<G>::value;  // keys per lane group per batch
  constexpr int kSB = 4;                           // keys per online-softmax update
  __shared__ int32_t sh_rid[kSeg];  // resolved rows (phys_page * page_size + slot) or -1
  __shared__ float sh_m[NW][G];
  __shared__ float sh_l[NW][G];
  __shared__ float sh_acc[NW][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPK;       // lane group = key slot
  const int part = lane % LPK;      // dims part*8 .. part*8+7
  const int64_t unit = blockIdx.x / num_splits;  // (b * q_len + i) * H_kv + g
  const int split = (int)(blockIdx.x - unit * num_splits);
  const int g = (int)(unit % kv.num_kv_heads);
  const int64_t bi = unit / kv.num_kv_heads;
  const int b = (int)(bi / q_len);
  const int i = (int)(bi - (int64_t)b * q_len);
  const int pos = min(kv.seq_lens[b], kv.max_seq_len) - q_tail + i;
  const int gi = (kv.num_idx_heads == 1) ? 0 : g;
  const int32_t* ilist = indices + (bi * kv.num_idx_heads + gi) * (int64_t)W;
  const int64_t head_stride = (int64_t)kv.page_size * D;  // one head of one page
  const int64_t page_stride = head_stride * kv.num_kv_heads;
  const uint16_t* kbase = kv.k_pool + g * head_stride + part * 8;
  const uint16_t* vbase = kv.v_pool + g * head_stride + part * 8;

  // Query fragments stay packed bf16 (converted per use); the softmax scale sm_scale*log2(e)
  // is applied to the reduced dot products.
  uint4 qw[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qw[h] = *reinterpret_cast<const uint4*>(q + (bi * num_q_heads + (int64_t)g * G + h) * D + part * 8);

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int k_begin = split * keys_per_split;
  const int k_end = min(W, k_begin + keys_per_split);

  auto row_off = [&](int rid) -> int64_t {
    return (int64_t)(rid >> kv.page_shift) * page_stride + (int64_t)(rid & (kv.page_size - 1)) * D;
  };

  for (int seg = k_begin; seg < k_end; seg += kSeg) {
    const int n_seg = min(kSeg, k_end - seg);
    // Resolve list entries -> pool rows, cooperatively (one entry per thread per pass).
    __syncthreads();  // the previous segment's rows are no longer read
    for (int j = threadIdx.x; j < n_seg; j += 256) {
      const int t = ilist[seg + j];
      int rid = -1;
      if (t >= 0 && t <= pos) {
        const int64_t ph = phys_page(kv, b, t);
        if (ph >= 0) rid = (int)(ph * kv.page_size + (t & (kv.page_size - 1)));
      }
      sh_rid[j] = rid;
    }
    __syncthreads();

    const int n_batches = (n_seg + STRIDE * kNB - 1) / (STRIDE * kNB);
    for (int bt = 0; bt < n_batches; ++bt) {
      // every K and V row of the batch is requested before any is used
      uint4 ck[kNB], cv[kNB];
      bool cok[kNB];
#pragma unroll
      for (int u = 0; u < kNB; ++u) {
        const int j = (bt * kNB + u) * STRIDE + wave * KPW + grp;
        const int rid = (j < n_seg) ? sh_rid[j] : -1;
        cok[u] = rid >= 0;
        if (cok[u]) {
          const int64_t o = row_off(rid);
          ck[u] = load_nt(kbase + o);
          cv[u] = load_nt(vbase + o);
        } else {
          ck[u] = make_uint4(0, 0, 0, 0);
          cv[u] = make_uint4(0, 0, 0, 0);
        }
      }
      // consume the batch in sub-batches of kSB keys: scores, one running-max update, V
#pragma unroll
      for (int u0 = 0; u0 < kNB; u0 += kSB) {
        float s[kSB][G];
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
          const uint4 kr = ck[u0 + u];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float d = dot2_bf16(qw[h].x, kr.x, 0.f);
            d = dot2_bf16(qw[h].y, kr.y, d);
            d = dot2_bf16(qw[h].z, kr.z, d);
            d = dot2_bf16(qw[h].w, kr.w, d);
            s[u][h] = group_sum_f<LPK>(d) * qscale;
          }
        }
        float mb[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          mb[h] = m[h];
#pragma unroll
          for (int u = 0; u < kSB; ++u) mb[h] = cok[u0 + u] ? fmaxf(mb[h], s[u][h]) : mb[h];
          grow = grow || (mb[h] > m[h] + kRescaleLog2);  // false while both are -inf
        }
        if (__any(grow)) {  // wave-uniform; rare after the first keys of a list
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float mn = (mb[h] > m[h] + kRescaleLog2) ? mb[h] : m[h];
            const float sc = safe_scale(m[h], mn);
            l[h] *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= sc;
            m[h] = mn;
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int u = 0; u < kSB; ++u) {
            s[u][h] = cok[u0 + u] ? __builtin_amdgcn_exp2f(s[u][h] - m[h]) : 0.f;
            l[h] += s[u][h];
          }
        }
        // P.V over key pairs: (p_u, p_u+1) . (v_u[e], v_u+1[e]) with one dot2 per dim
#pragma unroll
        for (int u = 0; u < kSB; u += 2) {
          const uint4 va = cv[u0 + u], vb = cv[u0 + u + 1];
          const uint32_t vv[8] = {pair_lo(va.x, vb.x), pair_hi(va.x, vb.x), pair_lo(va.y, vb.y),
                                  pair_hi(va.y, vb.y), pair_lo(va.z, vb.z), pair_hi(va.z, vb.z),
                                  pair_lo(va.w, vb.w), pair_hi(va.w, vb.w)};
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint32_t pp = pack_bf16x2(s[u][h], s[u + 1][h]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = dot2_bf16(pp, vv[e], acc[h][e]);
          }
        }
      }
    }
  }

  // merge the lane groups of this wave (groups differ in lane bits >= log2(LPK))
  auto merge_pairs = [&](auto mask_c) {
    constexpr int M = decltype(mask_c)::value;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const FPair mp = lane_pair<M>(m[h]);
      const FPair lp = lane_pair<M>(l[h]);
      const float mn = fmaxf(mp.lo, mp.hi);
      const float s_lo = safe_scale(mp.lo, mn);
      const float s_hi = safe_scale(mp.hi, mn);
      l[h] = lp.lo * s_lo + lp.hi * s_hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const FPair ap = lane_pair<M>(acc[h][e]);
        acc[h][e] = ap.lo * s_lo + ap.hi * s_hi;
      }
      m[h] = mn;
    }
  };
  if constexpr (LPK <= 8) merge_pairs(std::integral_constant<int, 8>{});
  merge_pairs(std::integral_constant<int, 16>{});
  merge_pairs(std::integral_constant<int, 32>{});
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (part == 0) {
        sh_m[wave][h] = m[h];
        sh_l[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_acc[wave][h][part * 8 + e] = acc[h][e];
    }
  }
  __syncthreads();

  // merge the waves: thread -> (head, dim) pairs
  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int h = x / D;
    const int dd = x - h * D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sh_m[w][h]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = safe_scale(sh_m[w][h], mm);
      ll += sh_l[w][h] * sc;
      aa += sh_acc[w][h][dd] * sc;
    }
    const int64_t qh = bi * num_q_heads + (int64_t)g * G + h;  // output row (b, i, head)
    if (num_splits == 1) {
      const float o = (ll > 0.f) ? aa / ll : 0.f;
      out[qh * D + dd] = (uint16_t)f32_to_bf16(o);
      if (lse != nullptr && dd == 0) lse[qh] = (ll > 0.f) ? (mm + log2f(ll)) * kLn2 : -INFINITY;
    } else {
      // partials: ws_acc [units][splits][G][D], then ws_ml [units][splits][G][2]
      const int64_t slot = unit * num_splits + split;
      ws[(slot * G + h) * D + dd] = aa;
      if (dd == 0) {
        float* ml = ws + (int64_t)gridDim.x * G * D;  // gridDim.x = units * num_splits
        ml[(slot * G + h) * 2 + 0] = mm;
        ml[(slot * G + h) * 2 + 1] = ll;
      }
    }
  }
}

// Exact merge of split partials, one workgroup per unit. The (max, sum) pairs of all splits
// are staged in LDS with one parallel load; each thread then reads its (head, dim) column of
// every split with independent loads and combines them in split order.
constexpr int kMaxSplits = 256;

template <int D, int G>
__global__ __launch_bounds__(256) void k_merge_splits(const float* __restrict__ ws, int64_t units,
                                                      int num_splits, int num_q_heads,
                                                      int num_kv_heads, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  __shared__ float s_w[kMaxSplits][G];  // m_s, then exp2(m_s - M)
  __shared__ float s_l[kMaxSplits][G];
  __shared__ float s_M[G], s_L[G];
  constexpr int NPER = (G * D + 255) / 256;  // output columns per thread
  constexpr int kPre = 8;                    // splits whose columns are loaded at entry
  const int64_t unit = blockIdx.x;
  const float* ml = ws + units * num_splits * G * D + unit * num_splits * G * 2;
  const float* acc = ws + unit * num_splits * G * D;
  // Every load is issued before the first wait: the (max, sum) pairs into LDS and, for the
  // first kPre splits, this thread's accumulator columns into registers (split index clamped,
  // so the loads are unconditional; the extra ones get weight 0).
  float pre[NPER][kPre];
#pragma unroll
  for (int k = 0; k < NPER; ++k) {
    const int x = min((int)threadIdx.x + k * 256, G * D - 1);
#pragma unroll
    for (int u = 0; u < kPre; ++u) pre[k][u] = acc[(int64_t)min(u, num_splits - 1) * G * D + x];
  }
  for (int x = threadIdx.x; x < num_splits * G; x += 256) {
    s_w[x / G][x % G] = ml[x * 2];
    s_l[x / G][x % G] = ml[x * 2 + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < num_splits; ++s) M = fmaxf(M, s_w[s][h]);
    float L = 0.f;
    for (int s = 0; s < num_splits; ++s) {
      const float w = safe_scale(s_w[s][h], M);
      L += s_l[s][h] * w;
      s_w[s][h] = w;
    }
    s_M[h] = M;
    s_L[h] = L;
  }
  __syncthreads();
  const int g = (int)(unit % num_kv_heads);
  const int64_t bi = unit / num_kv_heads;
#pragma unroll
  for (int k = 0; k < NPER; ++k) {
    const int x = threadIdx.x + k * 256;
    if (x >= G * D) break;
    const int h = x / D;
    float aa = 0.f;
#pragma unroll
    for (int u = 0; u < kPre; ++u)
      if (u < num_splits) aa += pre[k][u] * s_w[u][h];
    for (int s = kPre; s < num_splits; ++s) aa += acc[(int64_t)s * G * D + x] * s_w[s][h];
    const float L = s_L[h];
    const int64_t qh = bi * num_q_heads + (int64_t)g * G + h;
    out[qh * D + (x - h * D)] = (uint16_t)f32_to_bf16((L > 0.f) ? aa / L : 0.f);
    if (lse != nullptr && x - h * D == 0) lse[qh] = (L > 0.f) ? (s_M[h] + log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int D, int G>
hipError_t launch_dg(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len, int q_tail,
                     const int32_t* indices, int W, float sm_scale, int num_splits, float* ws,
                     uint16_t* out, float* lse, hipStream_t stream) {
  const int64_t units = (int64_t)kv.batch * q_len * kv.num_kv_heads;
  const int kps = (W + num_splits - 1) / num_splits;
  dim3 grid((unsigned)(units * num_splits));
  hipLaunchKernelGGL((k_attn_gather<D, G>), grid, dim3(256), 0, stream, kv, q, num_q_heads, q_len,
                     q_tail, indices, W, sm_scale * kLog2e, num_splits, kps, ws, out, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || num_splits == 1) return e;
  hipLaunchKernelGGL((k_merge_splits<D, G>), dim3((unsigned)units), dim3(256), 0, stream, ws, units,
                     num_splits, num_q_heads, kv.num_kv_heads, out, lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len, int q_tail,
                    const int32_t* indices, int W, float sm_scale, int num_splits, float* ws,
                    uint16_t* out, float* lse, hipStream_t stream) {
  switch (num_q_heads / kv.num_kv_heads) {
    case 1: return launch_dg<D, 1>(kv, q, num_q_heads, q_len, q_tail, indices, W, sm_scale, num_splits, ws, out, lse, stream);
    case 2: return launch_dg<D, 2>(kv, q, num_q_heads, q_len, q_tail, indices, W, sm_scale, num_splits, ws, out, lse, stream);
    case 4: return launch_dg<D, 4>(kv, q, num_q_heads, q_len, q_tail, indices, W, sm_scale, num_splits, ws, out, lse, stream);
    case 8: return launch_dg<D, 8>(kv, q, num_q_heads, q_len, q_tail, indices, W, sm_scale, num_splits, ws, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gather_workspace_bytes(int64_t units, int group, int head_dim, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)units * num_splits * group * (head_dim + 2) * sizeof(float);
}

int auto_splits(int64_t units, int index_width, int head_dim, int group) {
  // A load batch of a workgroup is 4 waves x (64 / (d/8)) lane groups x keys per lane group.
  // Two batches per workgroup measured faster than one (fewer partials to merge, every
  // workgroup resident at once) as long as that still gives every CU a workgroup.
  const int batch = 4 * (64 / (head_dim / 8)) * (group <= 2 ? 16 : (group == 4 ? 8 : 4));
  int s = (index_width + 2 * batch - 1) / (2 * batch);
  if (units * s < 256) s = (index_width + batch - 1) / batch;
  return s < 1 ? 1 : (s > 256 ? 256 : s);
}

// Split partials of the decode entry point that allocates nothing: a file-scope device array
// (each GPU holds its own copy for the life of the process). Host code never passes the
// array's name to a kernel; it looks up each device's address once and passes that.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (addr == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_merge_splits(const float* ws, int64_t units, int num_splits, int num_q_heads,
                               int num_kv_heads, int head_dim, uint16_t* out, float* lse,
                               hipStream_t stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid((unsigned)units);
#define SA_MERGE(D, G)                                                                              \
  hipLaunchKernelGGL((k_merge_splits<D, G>), grid, dim3(256), 0, stream, ws, units, num_splits,    \
                     num_q_heads, num_kv_heads, out, lse)
  const int group = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  switch (group) {
    case 1: if (head_dim == 128) SA_MERGE(128, 1); else SA_MERGE(64, 1); break;
    case 2: if (head_dim == 128) SA_MERGE(128, 2); else SA_MERGE(64, 2); break;
    case 4: if (head_dim == 128) SA_MERGE(128, 4); else SA_MERGE(64, 4); break;
    case 8: if (head_dim == 128) SA_MERGE(128, 8); else SA_MERGE(64, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_MERGE
  return hipGetLastError();
}

hipError_t launch_attn_gather(const KvView& kv, const uint16_t* q, int num_q_heads, int q_len,
                              int q_tail, const int32_t* indices, int index_width, float sm_scale,
                              int num_splits, float* ws, uint16_t* out, float* lse,
                              hipStream_t stream) {
  if (kv.head_dim == 128)
    return launch_d<128>(kv, q, num_q_heads, q_len, q_tail, indices, index_width, sm_scale, num_splits, ws, out, lse, stream);
  if (kv.head_dim == 64)
    return launch_d<64>(kv, q, num_q_heads, q_len, q_tail, indices, index_width, sm_scale, num_splits, ws, out, lse, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
