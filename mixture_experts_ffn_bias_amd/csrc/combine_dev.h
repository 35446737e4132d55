// Router-weighted combine and shared-expert add ("DeepSeek-V3.2-Exp · MoE
// update", moe-forward excerpt: each expert's output rows, times their
// routing weights, accumulate into fp32 expert by expert in ascending id, the
// shared expert's output is added, and the sum is cast back to the input
// dtype; "DeepSeek-V3.2-Exp · Add shared output", formula).
//
// One workgroup per token and share of the row (small batches split each row
// over several workgroups to occupy the chip); the token's K rows are visited
// in ascending expert id, so the fp32 sum has the same order as the pages'
// loop and the result is deterministic (no atomics).
//
// The partial form serves one rank of an expert-parallel layer: it sums only
// the experts [e_lo, e_hi) a rank holds (its slice of the experts in the
// pages' expert-parallel loop) and leaves y in fp32 for the cross-rank sum.
//
// Device function shared by the combine kernels and the single-launch layer
// kernel.
#pragma once
#include "common.h"

namespace moe {

namespace {

// 16 bytes of an expert output row, read with the non-temporal hint: each
// row is read once, by one workgroup, in whole 128-byte lines per wave.
__device__ __forceinline__ uint4 ld_nt16(const uint16_t* p) {
  const v4i v = __builtin_nontemporal_load((const v4i*)p);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// PARTIAL: y (fp32) = the sum over choices with expert in [e_lo, e_hi), plus
// the shared row when has_shared; otherwise delta (bf16) = bf16(full sum).
// Token t, share `part` of `nparts` of the row (8-element chunks); called by
// every thread of the workgroup (K <= 32 <= blockDim.x).
struct CombineLds {
  int row[32];
  float w[32];
  int e[32];
  int n;
};

template <bool PARTIAL>
__device__ __forceinline__ void combine_token(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                              const int32_t* __restrict__ pair_row,
                                              const uint16_t* __restrict__ rows, int has_shared, int T, int K,
                                              int e_lo, int e_hi, int d, void* __restrict__ out, int t, int part,
                                              int nparts, CombineLds& L) {
  int* s_row = L.row;
  float* s_w = L.w;
  int* s_e = L.e;
  int& s_n = L.n;
  const int64_t TK = (int64_t)T * K;
  // the token's choices in the range, loaded in parallel and placed by rank in
  // ascending expert id (equal ids keep their order); others are left out
  const int me = threadIdx.x;
  int e = 0, row = 0;
  float wk = 0.f;
  bool in = false;
  if (me < K) {
    e = idx[(size_t)t * K + me];
    in = e >= e_lo && e < e_hi;
    row = pair_row[(size_t)t * K + me];
    row = row < 0 ? 0 : (row >= TK ? (int)(TK - 1) : row);
    wk = w[(size_t)t * K + me];
    s_e[me] = in ? e : 0x7fffffff;
  }
  __syncthreads();
  if (me < K && in) {
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int o = s_e[j];
      rank += (o < e || (o == e && j < me)) ? 1 : 0;
    }
    s_row[rank] = row;
    s_w[rank] = wk;
  }
  if (me == 0) {
    int n = 0;
    for (int j = 0; j < K; ++j) n += s_e[j] != 0x7fffffff ? 1 : 0;
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  // this workgroup's share of the row: 8-element chunks [c0, c1)
  const int nch = d / 8;
  const int per = (nch + nparts - 1) / nparts;
  const int c0 = part * per, c1 = min(nch, c0 + per);
  for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.f;
    // up to 8 rows loaded together (all in flight), then added in order
    for (int k0 = 0; k0 < n; k0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < n) v[j] = ld_nt16(rows + (size_t)s_row[k0 + j] * d + c * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j < n) {
          const float wk = s_w[k0 + j];
          const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[2 * i] = fmaf(wk, bf16_to_f32(u[i] & 0xFFFFu), y[2 * i]);
            y[2 * i + 1] = fmaf(wk, bf16_to_f32(u[i] >> 16), y[2 * i + 1]);
          }
        }
      }
    }
    if (has_shared) {
      const uint4 v = ld_nt16(rows + (size_t)(TK + t) * d + c * 8);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] += bf16_to_f32(u[i] & 0xFFFFu);
        y[2 * i + 1] += bf16_to_f32(u[i] >> 16);
      }
    }
    if constexpr (PARTIAL) {
      float4* dst = (float4*)((float*)out + (size_t)t * d + c * 8);
      dst[0] = make_float4(y[0], y[1], y[2], y[3]);
      dst[1] = make_float4(y[4], y[5], y[6], y[7]);
    } else {
      uint4 o;
      o.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
      o.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
      o.z = (uint32_t)f32_to_bf16(y[4]) | ((uint32_t)f32_to_bf16(y[5]) << 16);
      o.w = (uint32_t)f32_to_bf16(y[6]) | ((uint32_t)f32_to_bf16(y[7]) << 16);
      *(uint4*)((uint16_t*)out + (size_t)t * d + c * 8) = o;
    }
  }
}

}  // namespace

}  // namespace moe
