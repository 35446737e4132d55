// Token counting, expert-contiguous order and activation quantisation
// ("DeepSeek-V3.2-Exp · MoE update", moe-forward excerpt: a count of the
// selected experts, then for each expert the tokens that chose it in
// ascending token order; "DeepSeek-V3.2-Exp · Gate projection", the FP8
// Linear's activation quantisation), as device functions shared by the
// permutation kernels and the single-launch layer kernel.
#pragma once
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

namespace {

constexpr int MASK_WORDS = PERM_CHUNK / 32;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// mask[e][w] bit b: token chunk * PERM_CHUNK + 32 w + b chose expert e.
// Threads past PERM_CHUNK only clear and join the barriers.
template <bool COH = false>
__device__ __forceinline__ void build_masks(uint32_t* mask, const int32_t* idx, int T, int K, int E, int chunk) {
  for (int i = threadIdx.x; i < E * MASK_WORDS; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  const int t = chunk * PERM_CHUNK + threadIdx.x;
  if (threadIdx.x < PERM_CHUNK && t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = clamp_expert(ld<COH>(idx + (size_t)t * K + k), E);
      atomicOr(&mask[e * MASK_WORDS + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
    }
  }
  __syncthreads();
}

// Per-128-block e4m3 quantisation of bf16 rows: 8 lanes per block, 16
// elements per lane.  scale = amax / 448 (correctly rounded fp32 division),
// code = e4m3_rne(v / scale); an all-zero block gets scale 1.  The 8 lanes
// of a block are consecutive lanes of one wave and call this together.
template <bool COH = false>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t blk, int sub,
                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
  const uint4* p = (const uint4*)(x + blk * BLK + sub * 16);
  const uint4 u0 = p[0], u1 = p[1];
  const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const float sc = amax == 0.f ? 1.f : amax / E4M3_MAX;
  uint4 o;
  o.x = pack4_e4m3(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
  o.y = pack4_e4m3(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  o.z = pack4_e4m3(v[8] / sc, v[9] / sc, v[10] / sc, v[11] / sc);
  o.w = pack4_e4m3(v[12] / sc, v[13] / sc, v[14] / sc, v[15] / sc);
  st16<COH>(q + blk * BLK + sub * 16, o);
  if (sub == 0) st<COH>(scale + blk, sc);
}

// LDS of the one-workgroup permutation.
struct PermLds {
  uint32_t mask[256 * MASK_WORDS];
  int s[256];
  int s_off[256];
};

// T <= PERM_CHUNK tokens, E <= 256 experts, one workgroup of >= 256 threads
// (threads from 256 on only join the barriers): counts, offsets (E + 1),
// row_token (T*K + T: the shared expert's rows are the identity) and
// pair_row, and, when plan.tiles is set, the FFN tile list from the same
// offsets.  COH: idx is read and everything is written with agent-coherent
// accesses (common.h, ld / st).
template <bool COH = false>
__device__ __forceinline__ void permute_block(const int32_t* __restrict__ idx, int T, int K, int E,
                                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row,
                                              const PlanArgs& plan, PermLds& L) {
  build_masks<COH>(L.mask, idx, T, K, E, 0);
  const int e = threadIdx.x;
  const bool act = e < 256;
  int cnt = 0;
  if (e < E) {
#pragma unroll
    for (int j = 0; j < MASK_WORDS; ++j) cnt += __popc(L.mask[e * MASK_WORDS + j]);
  }
  if (act) L.s[e] = cnt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = act && e >= o ? L.s[e - o] : 0;
    __syncthreads();
    if (act) L.s[e] += v;
    __syncthreads();
  }
  if (act) L.s_off[e] = L.s[e] - cnt;
  if (e < E) {
    st<COH>(counts + e, (int32_t)cnt);
    st<COH>(offsets + e, (int32_t)(L.s[e] - cnt));
  }
  if (e == 255) st<COH>(offsets + E, (int32_t)L.s[255]);
  __syncthreads();
  const int t = threadIdx.x;
  if (t < T) {
    const int w = t >> 5;
    const uint32_t below = (1u << (t & 31)) - 1u;
    for (int k = 0; k < K; ++k) {
      const int ek = clamp_expert(ld<COH>(idx + (size_t)t * K + k), E);
      const uint32_t* m = L.mask + ek * MASK_WORDS;
      int rank = __popc(m[w] & below);
      for (int j = 0; j < w; ++j) rank += __popc(m[j]);
      const int pos = L.s_off[ek] + rank;
      st<COH>(row_token + pos, (int32_t)t);
      st<COH>(pair_row + (size_t)t * K + k, (int32_t)pos);
    }
    st<COH>(row_token + (size_t)T * K + t, (int32_t)t);
  }
  if (plan.tiles) {  // the FFN tile list from the same offsets
    __syncthreads();  // s is reused as the plan's scan buffer
    plan_tiles_block<COH>(e < E ? L.s_off[e] : 0, e < E ? cnt : 0, T, K, plan.tile_rows, plan.has_shared, plan.cap,
                          0, E, L.s, plan.tiles, plan.n_tiles);
  }
}

}  // namespace

}  // namespace moe
