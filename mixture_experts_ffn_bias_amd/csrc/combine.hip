// Router-weighted combine and shared-expert add ("DeepSeek-V3.2-Exp · MoE
// update", moe-forward excerpt: ``y[idx] += expert(x[idx]) * weights[idx, top]``
// over experts in ascending id into an fp32 accumulator, ``y +=
// shared_experts(x)``, then the cast back to the input dtype;
// "DeepSeek-V3.2-Exp · Add shared output", formula).
//
// One workgroup per token and share of the row (small batches split each row
// over several workgroups to occupy the chip); the token's K rows are visited
// in ascending expert id, so the fp32 sum has the same order as the pages'
// loop and the result is deterministic (no atomics).
//
// The partial form serves one rank of an expert-parallel layer: it sums only
// the experts [e_lo, e_hi) a rank holds (the pages' experts_start_idx ..
// experts_end_idx slice) and leaves y in fp32 for the cross-rank sum.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// PARTIAL: y (fp32) = the sum over choices with expert in [e_lo, e_hi), plus
// the shared row when has_shared; otherwise delta (bf16) = bf16(full sum).
template <bool PARTIAL>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_row,
                                                      const uint16_t* __restrict__ rows, int has_shared, int T,
                                                      int K, int e_lo, int e_hi, int d, void* __restrict__ out) {
  __shared__ int s_row[32];
  __shared__ float s_w[32];
  __shared__ int s_e[32];
  __shared__ int s_n;
  const int t = blockIdx.x;
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
  const int per = (nch + gridDim.y - 1) / gridDim.y;
  const int c0 = blockIdx.y * per, c1 = min(nch, c0 + per);
  for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.f;
    for (int k = 0; k < n; ++k) {
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

namespace {

// workgroups per token: enough to cover the chip's 256 CUs at small T, with
// at least 64 eight-element chunks each
unsigned combine_split(int T, int d) {
  int sp = 1;
  while (T * sp < 512 && sp < 8 && d / 8 / (2 * sp) >= 64) sp *= 2;
  return (unsigned)sp;
}

}  // namespace

hipError_t launch_combine(const int32_t* idx, const float* w, const int32_t* pair_row, const uint16_t* rows,
                          int has_shared, int T, int K, int E, int d, uint16_t* delta, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel<false>, dim3(T, combine_split(T, d)), dim3(256), 0, s, idx, w, pair_row, rows,
                     has_shared, T, K, 0, E, d, (void*)delta);
  return hipGetLastError();
}

hipError_t launch_combine_partial(const int32_t* idx, const float* w, const int32_t* pair_row,
                                  const uint16_t* rows, int has_shared, int T, int K, int e_lo, int e_hi, int d,
                                  float* y, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel<true>, dim3(T, combine_split(T, d)), dim3(256), 0, s, idx, w, pair_row, rows,
                     has_shared, T, K, e_lo, e_hi, d, (void*)y);
  return hipGetLastError();
}

}  // namespace moe
