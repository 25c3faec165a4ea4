// Device helpers for scoring int8 indexer keys, shared by the stand-alone indexer and the
// fused index + selection kernels.
//
// One wave scores one 64-token block of one indexer head: the block is 64 * D contiguous
// bytes (D = d_idx), read with 16-byte loads so each load instruction moves 1 KiB. D/16
// neighbouring lanes hold one token's key; each does four v_dot4_i32_i8 against the matching
// 16 query bytes and a DPP butterfly sums the lane group, exactly, in int32.
#pragma once

#include "sa_common.h"

namespace sa {
namespace idx {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot16(const v4i a, const v4i b) {
  int acc = 0;
  acc = __builtin_amdgcn_sdot4(a.x, b.x, acc, false);
  acc = __builtin_amdgcn_sdot4(a.y, b.y, acc, false);
  acc = __builtin_amdgcn_sdot4(a.z, b.z, acc, false);
  acc = __builtin_amdgcn_sdot4(a.w, b.w, acc, false);
  return acc;
}

template <int D>
struct Blk {
  static constexpr int LPT = D / 16;    // lanes holding one token's key
  static constexpr int TPL = 64 / LPT;  // tokens covered by one 1 KiB load
  static constexpr int R = LPT;         // loads per 64-token block
};

// Which 16 query bytes a lane multiplies (its part of a key row).
template <int D>
__device__ __forceinline__ int lane_part(int lane) { return lane % Blk<D>::LPT; }

// Token (0..63 within the block) whose score a lane holds after score_block.
template <int D>
__device__ __forceinline__ int lane_token(int lane) {
  return (lane % Blk<D>::LPT) * Blk<D>::TPL + lane / Blk<D>::LPT;
}

template <int D>
__device__ __forceinline__ void load_block(const int8_t* base, int lane, v4i (&kd)[Blk<D>::R]) {
#pragma unroll
  for (int r = 0; r < Blk<D>::R; ++r)
    kd[r] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + r * 1024 + lane * 16));
}

// Score of token lane_token(lane): after the reduction every lane of a group has the sum of
// load r's token; lane l keeps load (l mod LPT).
template <int D>
__device__ __forceinline__ int score_block(const v4i qf, const v4i (&kd)[Blk<D>::R], int lane) {
  int mine = 0;
#pragma unroll
  for (int r = 0; r < Blk<D>::R; ++r) {
    const int s = group_sum_i<Blk<D>::LPT>(dot16(qf, kd[r]));
    if (lane_part<D>(lane) == r) mine = s;
  }
  return mine;
}

// Moves scores from lane_token order to natural order: lane l receives token l's score.
template <int D>
__device__ __forceinline__ int to_token_order(int mine, int lane) {
  const int src = (lane % Blk<D>::TPL) * Blk<D>::LPT + lane / Blk<D>::TPL;
  return __shfl(mine, src, 64);
}

}  // namespace idx
}  // namespace sa
