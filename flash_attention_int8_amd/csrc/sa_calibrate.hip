// Roofline micro-benchmarks: what one MI355X reaches on the operations the attention path is
// bound by, measured with the same load and matrix instructions the kernels use. They set the
// measured denominators of the roofline fractions next to the vendor peaks:
//   k_calib_read    streaming read of a buffer (16-byte loads with the nontemporal hint, eight
//                   in flight per lane; the hint is worth about 13% here, 6.2 -> 7.0 TB/s)
//   k_calib_gather  random 256-byte rows of a pool (the K or V row of one token at d = 128:
//                   the decode and sparse-prefill gather unit), 16 lanes per row, eight rows
//                   in flight per lane group, nontemporal loads as in the decode gather
//   k_calib_mfma    back-to-back v_mfma_f32_32x32x16_bf16 or v_mfma_i32_32x32x32_i8 on
//                   register operands, four independent accumulators per wave
// Each kernel folds what it read or computed into one word per workgroup of `sink`, so the
// work cannot be dropped by the compiler.
#include "sa_common.h"

namespace sa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

constexpr int kCalNT = 256;

constexpr int kCalU = 8;  // 16-byte loads (read) or rows (gather) in flight per lane

__device__ __forceinline__ void fold_to_sink(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t red[kCalNT];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < kCalNT; ++k) r ^= red[k];
    sink[blockIdx.x] = r;
  }
}

// Each workgroup streams whole chunks of kCalNT * kCalU 16-byte words (32 KiB), chunk c
// going to workgroup c % gridDim.x, with every load of a chunk issued before any is used.
__global__ __launch_bounds__(kCalNT) void k_calib_read(const uint4* __restrict__ p, int64_t n16,
                                                      uint32_t* __restrict__ sink) {
  constexpr int64_t kChunk = (int64_t)kCalNT * kCalU;
  uint32_t acc = 0;
  const int64_t full = n16 / kChunk;
  for (int64_t c = blockIdx.x; c < full; c += gridDim.x) {
    const uint4* q = p + c * kChunk + threadIdx.x;
    uint4 v[kCalU];
#pragma unroll
    for (int u = 0; u < kCalU; ++u) v[u] = load_nt(q + u * kCalNT);
#pragma unroll
    for (int u = 0; u < kCalU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = full * kChunk + (int64_t)blockIdx.x * kCalNT + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kCalNT) {
    const uint4 a = load_nt(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  fold_to_sink(acc, sink);
}

// rows[] are 256-byte row numbers of the pool; a row outside [0, n_pool_rows) reads row 0.
// Each group of 16 lanes loads one row; a lane group keeps kCalU rows in flight.
__global__ __launch_bounds__(kCalNT) void k_calib_gather(const uint4* __restrict__ pool, int64_t n_pool_rows,
                                                        const int32_t* __restrict__ rows, int64_t n_rows,
                                                        uint32_t* __restrict__ sink) {
  const int lane16 = threadIdx.x & 15;
  const int64_t grp = ((int64_t)blockIdx.x * kCalNT + threadIdx.x) >> 4;
  const int64_t ngrp = ((int64_t)gridDim.x * kCalNT) >> 4;
  auto row_of = [&](int64_t k) -> int64_t {
    const int64_t r = rows[k];
    return (r >= 0 && r < n_pool_rows) ? r : 0;
  };
  uint32_t acc = 0;
  int64_t k = grp;
  for (; k + (kCalU - 1) * ngrp < n_rows; k += kCalU * ngrp) {
    int64_t r[kCalU];
#pragma unroll
    for (int u = 0; u < kCalU; ++u) r[u] = row_of(k + u * ngrp);
    uint4 v[kCalU];
#pragma unroll
    for (int u = 0; u < kCalU; ++u) v[u] = load_nt(pool + r[u] * 16 + lane16);
#pragma unroll
    for (int u = 0; u < kCalU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; k < n_rows; k += ngrp) {
    const uint4 a = load_nt(pool + row_of(k) * 16 + lane16);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  fold_to_sink(acc, sink);
}

template <bool I8>
__global__ __launch_bounds__(kCalNT) void k_calib_mfma(int iters, uint32_t* __restrict__ sink) {
  const int t = threadIdx.x;
  if constexpr (I8) {
    const i32x4 a = {t, t + 1, t + 2, t + 3}, b = {t * 3, t ^ 5, t + 7, t * 11};
    i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) r ^= (uint32_t)(c0[k] ^ c1[k] ^ c2[k] ^ c3[k]);
    if (r == 0x9e3779b9u) sink[blockIdx.x] = r;  // never true in practice; keeps the work
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = (__bf16)(float)((t + k) & 7);
      b[k] = (__bf16)(float)((t * 3 + k) & 7);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) r += c0[k] + c1[k] + c2[k] + c3[k];
    if (r == -1.f) sink[blockIdx.x] = 1u;  // never true (sums of products of non-negatives)
  }
}

}  // namespace

hipError_t launch_calib_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_calib_read, dim3((unsigned)workgroups), dim3(kCalNT), 0, stream,
                     static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_calib_gather(const void* pool, size_t pool_bytes, const int32_t* rows, int64_t n_rows,
                               uint32_t* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(k_calib_gather, dim3((unsigned)workgroups), dim3(kCalNT), 0, stream,
                     static_cast<const uint4*>(pool), (int64_t)(pool_bytes / 256), rows, n_rows, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int kind, int iters, int workgroups, uint32_t* sink, hipStream_t stream) {
  if (kind == 1)
    hipLaunchKernelGGL(k_calib_mfma<true>, dim3((unsigned)workgroups), dim3(kCalNT), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(k_calib_mfma<false>, dim3((unsigned)workgroups), dim3(kCalNT), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace sa
