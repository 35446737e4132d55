// Router-weighted combine and shared-expert add ("DeepSeek-V3.2-Exp · MoE
// update", moe-forward excerpt: ``y[idx] += expert(x[idx]) * weights[idx, top]``
// over experts in ascending id into an fp32 accumulator, ``y +=
// shared_experts(x)``, then the cast back to the input dtype;
// "DeepSeek-V3.2-Exp · Add shared output", formula).
//
// One workgroup per token; the token's K rows are visited in ascending
// expert id, so the fp32 sum has the same order as the pages' loop and the
// result is deterministic (no atomics).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_row,
                                                      const uint16_t* __restrict__ rows, int has_shared, int T,
                                                      int K, int d, uint16_t* __restrict__ delta) {
  __shared__ int s_row[32];
  __shared__ float s_w[32];
  __shared__ int s_e[32];
  const int t = blockIdx.x;
  const int64_t TK = (int64_t)T * K;
  // the token's K choices, loaded in parallel and placed by rank in ascending expert id
  // (equal ids keep their order)
  const int me = threadIdx.x;
  int e = 0, row = 0;
  float wk = 0.f;
  if (me < K) {
    e = idx[(size_t)t * K + me];
    row = pair_row[(size_t)t * K + me];
    row = row < 0 ? 0 : (row >= TK ? (int)(TK - 1) : row);
    wk = w[(size_t)t * K + me];
    s_e[me] = e;
  }
  __syncthreads();
  if (me < K) {
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int o = s_e[j];
      rank += (o < e || (o == e && j < me)) ? 1 : 0;
    }
    s_row[rank] = row;
    s_w[rank] = wk;
  }
  __syncthreads();
  const int nch = d / 8;
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const uint4 v = *(const uint4*)(rows + (size_t)s_row[k] * d + c * 8);
      const float wk = s_w[k];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = fmaf(wk, bf16_to_f32(u[i] & 0xFFFFu), y[2 * i]);
        y[2 * i + 1] = fmaf(wk, bf16_to_f32(u[i] >> 16), y[2 * i + 1]);
      }
    }
    if (has_shared) {
      const uint4 v = *(const uint4*)(rows + (size_t)(TK + t) * d + c * 8);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] += bf16_to_f32(u[i] & 0xFFFFu);
        y[2 * i + 1] += bf16_to_f32(u[i] >> 16);
      }
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(y[4]) | ((uint32_t)f32_to_bf16(y[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(y[6]) | ((uint32_t)f32_to_bf16(y[7]) << 16);
    *(uint4*)(delta + (size_t)t * d + c * 8) = o;
  }
}

}  // namespace

hipError_t launch_combine(const int32_t* idx, const float* w, const int32_t* pair_row, const uint16_t* rows,
                          int has_shared, int T, int K, int E, int d, uint16_t* delta, hipStream_t s) {
  (void)E;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, s, idx, w, pair_row, rows, has_shared, T, K, d, delta);
  return hipGetLastError();
}

}  // namespace moe
