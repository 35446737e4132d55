// Fused residual add + RMSNorm ("DeepSeek-V3.2-Exp · MoE update", rmsnorm
// excerpt, residual branch): r = float(x) + float(residual); the residual
// becomes bf16(r); the output is bf16(gain * r * rsqrt(mean(r^2) + eps)).
// The pages evaluate the normalisation in fp32 with an unspecified reduction
// order; here it is evaluated exactly enough to be order-independent: the
// sum of squares, the scale and the products in fp64, then one correct
// rounding to bf16.  (The e4m3 quantisation of the normalised rows downstream
// turns a one-ulp difference of a block maximum into a rescaled block, so the
// normalised values are worth getting exactly right.)  The residual add is
// the pages' fp32 add (exact for two bf16 values).  One workgroup per token;
// each thread keeps its share of r in registers, so `out` may alias `x`.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int NORM_THREADS = 256;

// NCH 8-element chunks per thread (d <= 256 * 8 * NCH).  Every load of the
// row is issued first, so that a thread's loads are in flight together; a
// chunk index past the row's end reads the row's last chunk instead and is
// not used.
template <int NCH>
__global__ __launch_bounds__(NORM_THREADS) void add_rmsnorm_kernel(const uint16_t* x,
                                                                    uint16_t* __restrict__ res,
                                                                    const float* __restrict__ gain, float eps,
                                                                    int d, uint16_t* out) {
  __shared__ double s_part[NORM_THREADS / 64];
  const size_t t = blockIdx.x;
  const int nch = d / 8;
  uint32_t xw[NCH][4], rw[NCH][4];  // the raw bf16 pairs of x and the residual
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = min((int)threadIdx.x + NORM_THREADS * i, nch - 1);
    const uint4 xv = *(const uint4*)(x + t * d + c * 8);
    const uint4 rv = *(const uint4*)(res + t * d + c * 8);
    xw[i][0] = xv.x; xw[i][1] = xv.y; xw[i][2] = xv.z; xw[i][3] = xv.w;
    rw[i][0] = rv.x; rw[i][1] = rv.y; rw[i][2] = rv.z; rw[i][3] = rv.w;
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NORM_THREADS * i;
    if (c < nch) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the sum of two bf16 values is exact in fp64
        const double lo = (double)bf16_to_f32(xw[i][j] & 0xFFFFu) + (double)bf16_to_f32(rw[i][j] & 0xFFFFu);
        const double hi = (double)bf16_to_f32(xw[i][j] >> 16) + (double)bf16_to_f32(rw[i][j] >> 16);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < NORM_THREADS / 64; ++i) tot += s_part[i];
  const double rs = 1.0 / sqrt(tot / (double)d + (double)eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NORM_THREADS * i;
    if (c < nch) {
      const float4 g0 = *(const float4*)(gain + c * 8);
      const float4 g1 = *(const float4*)(gain + c * 8 + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      uint32_t ro[4], oo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xl = bf16_to_f32(xw[i][j] & 0xFFFFu), xh = bf16_to_f32(xw[i][j] >> 16);
        const float rl = bf16_to_f32(rw[i][j] & 0xFFFFu), rh = bf16_to_f32(rw[i][j] >> 16);
        // new residual: the fp32 sum cast to bf16, as the pages write it
        ro[j] = (uint32_t)f32_to_bf16(xl + rl) | ((uint32_t)f32_to_bf16(xh + rh) << 16);
        const double sl = (double)xl + (double)rl, sh = (double)xh + (double)rh;
        oo[j] = (uint32_t)f64_to_bf16((double)gg[2 * j] * (sl * rs)) |
                ((uint32_t)f64_to_bf16((double)gg[2 * j + 1] * (sh * rs)) << 16);
      }
      *(uint4*)(res + t * d + c * 8) = make_uint4(ro[0], ro[1], ro[2], ro[3]);
      *(uint4*)(out + t * d + c * 8) = make_uint4(oo[0], oo[1], oo[2], oo[3]);
    }
  }
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t* x, uint16_t* residual, const float* gain, float eps, int d,
                              int64_t T, uint16_t* out, hipStream_t s) {
  const int per = (d / 8 + NORM_THREADS - 1) / NORM_THREADS;  // chunks per thread (d <= 16384: at most 8)
  const dim3 g((unsigned)T), b(NORM_THREADS);
  if (per <= 1)
    hipLaunchKernelGGL(add_rmsnorm_kernel<1>, g, b, 0, s, x, residual, gain, eps, d, out);
  else if (per <= 2)
    hipLaunchKernelGGL(add_rmsnorm_kernel<2>, g, b, 0, s, x, residual, gain, eps, d, out);
  else if (per <= 4)
    hipLaunchKernelGGL(add_rmsnorm_kernel<4>, g, b, 0, s, x, residual, gain, eps, d, out);
  else if (per <= 8)
    hipLaunchKernelGGL(add_rmsnorm_kernel<8>, g, b, 0, s, x, residual, gain, eps, d, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
