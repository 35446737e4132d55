// Fused residual add + RMSNorm ("DeepSeek-V3.2-Exp · MoE update", rmsnorm
// excerpt, residual branch): r = float(x) + float(residual); the residual
// becomes bf16(r); the output is bf16(gain * (r * rsqrt(mean(r^2) + eps))),
// all arithmetic in fp32.  One workgroup per token; each thread keeps its
// share of r in registers, so `out` may alias `x`.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int NORM_THREADS = 256;
constexpr int NORM_CHUNKS = 8;  // 8-element chunks per thread: d <= 256 * 8 * 8 = 16384

__global__ __launch_bounds__(NORM_THREADS) void add_rmsnorm_kernel(const uint16_t* x,
                                                                    uint16_t* __restrict__ res,
                                                                    const float* __restrict__ gain, float eps,
                                                                    int d, uint16_t* out) {
  __shared__ float s_part[NORM_THREADS / 64];
  const size_t t = blockIdx.x;
  const int nch = d / 8;
  float r[NORM_CHUNKS][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NORM_CHUNKS; ++i) {
    const int c = threadIdx.x + NORM_THREADS * i;
    if (c < nch) {
      const uint4 xv = *(const uint4*)(x + t * d + c * 8);
      const uint4 rv = *(const uint4*)(res + t * d + c * 8);
      const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t ru[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[i][2 * j] = bf16_to_f32(xu[j] & 0xFFFFu) + bf16_to_f32(ru[j] & 0xFFFFu);
        r[i][2 * j + 1] = bf16_to_f32(xu[j] >> 16) + bf16_to_f32(ru[j] >> 16);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(r[i][j], r[i][j], ss);
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NORM_THREADS / 64; ++i) tot += s_part[i];
  const float rs = 1.f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int i = 0; i < NORM_CHUNKS; ++i) {
    const int c = threadIdx.x + NORM_THREADS * i;
    if (c < nch) {
      const float4 g0 = *(const float4*)(gain + c * 8);
      const float4 g1 = *(const float4*)(gain + c * 8 + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      uint32_t ro[4], oo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ro[j] = (uint32_t)f32_to_bf16(r[i][2 * j]) | ((uint32_t)f32_to_bf16(r[i][2 * j + 1]) << 16);
        oo[j] = (uint32_t)f32_to_bf16(gg[2 * j] * (r[i][2 * j] * rs)) |
                ((uint32_t)f32_to_bf16(gg[2 * j + 1] * (r[i][2 * j + 1] * rs)) << 16);
      }
      *(uint4*)(res + t * d + c * 8) = make_uint4(ro[0], ro[1], ro[2], ro[3]);
      *(uint4*)(out + t * d + c * 8) = make_uint4(oo[0], oo[1], oo[2], oo[3]);
    }
  }
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t* x, uint16_t* residual, const float* gain, float eps, int d,
                              int64_t T, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)T), dim3(NORM_THREADS), 0, s, x, residual, gain, eps, d,
                     out);
  return hipGetLastError();
}

}  // namespace moe
