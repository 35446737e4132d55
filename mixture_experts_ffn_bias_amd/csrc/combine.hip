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
#include "combine_dev.h"
#include "kernels.h"

namespace moe {

namespace {

// grid (T, parts), 256 threads
template <bool PARTIAL>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_row,
                                                      const uint16_t* __restrict__ rows, int has_shared, int T,
                                                      int K, int e_lo, int e_hi, int d, void* __restrict__ out) {
  __shared__ CombineLds L;
  combine_token<PARTIAL>(idx, w, pair_row, rows, has_shared, T, K, e_lo, e_hi, d, out, blockIdx.x, blockIdx.y,
                         gridDim.y, L);
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
