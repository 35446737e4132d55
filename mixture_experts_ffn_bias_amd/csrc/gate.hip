// Router kernels of the MoE layer ("DeepSeek-V3.2-Exp · MoE update",
// moe-forward excerpt: the gate call): K-split partial logits, then the
// selection per token.  The arithmetic is in gate_dev.h.
#include "gate_dev.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int GATE_KSPLIT_MAX = 16;  // K splits of the logits (partials the selection adds)

// Grid (ceil(T/64), E/16, ksplit), 256 threads; for small batches, where
// spreading the router weight over many workgroups matters more than
// sharing it.  Wave w owns tokens [t0, t0+16) and one 16-expert tile;
// blockIdx.z a K range.  zpart[z][t][e] receives the partial logits of that
// K range.
__global__ __launch_bounds__(256) void gate_logits_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ gw,
                                                          float* __restrict__ zpart, int T, int d, int E,
                                                          int kchunk) {
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 16;
  const int k0 = blockIdx.z * kchunk;
  if (t0 >= T) return;  // no barriers in this kernel
  gate_logits_wave<1>(x, gw, zpart + (size_t)blockIdx.z * T * E, T, d, E, t0, e0, 1, k0, min(d, k0 + kchunk));
}

// Grid (ceil(T/64), ceil(E/64), ksplit), 256 threads; for large batches.
// Wave w: tokens [t0, t0 + 16) and four 16-expert tiles; the workgroup's 64
// router-weight rows of each 32-wide K step
// are loaded once, split into bf16 hi/mid/lo once and kept in LDS in the
// MFMA operand layout for all four waves, instead of each wave loading and
// splitting them itself.  Two LDS buffers: a step's split weights go into one
// while the other is still being read, so one barrier per step suffices.
// The products are accumulated in the same order as gate_logits_wave.
__global__ __launch_bounds__(256) void gate_logits_lds_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ gw,
                                                              float* __restrict__ zpart, int T, int d, int E,
                                                              int kchunk) {
  __shared__ v8bf s_w[2][4][3][64];  // [buffer][expert tile][lo, mid, hi][lane]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 64;
  const int nt = min(4, (E - e0) >> 4);
  const int k0 = blockIdx.z * kchunk, k1 = min(d, k0 + kchunk);
  const bool live = t0 < T;  // wave-uniform; every wave joins the barriers
  // this thread's share of a step: 8 values of expert row e0 + we at K offset 8 wk,
  // which are lane (we % 16) + 16 wk of expert tile we / 16 in the operand layout
  const int we = threadIdx.x >> 2, wk = threadIdx.x & 3;
  const bool wvalid = we < 16 * nt;
  const float* wrow = gw + (size_t)(e0 + min(we, 16 * nt - 1)) * d + 8 * wk;
  const int wn = we >> 4, wl = (we & 15) + 16 * wk;
  const uint16_t* xr = x + (size_t)min(t0 + r, T - 1) * d + 8 * g;

  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  float4 f0 = {0.f, 0.f, 0.f, 0.f}, f1 = f0;
  v8bf a = {};
  if (k0 < k1) {
    f0 = *(const float4*)(wrow + k0);
    f1 = *(const float4*)(wrow + k0 + 4);
    a = *(const v8bf*)(xr + k0);
  }
  int buf = 0;
  for (int k = k0; k < k1; k += 32) {
    if (wvalid) {
      const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      v8bf hi, mid, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 h, m, l;
        split3(f[j], h, m, l);
        hi[j] = h;
        mid[j] = m;
        lo[j] = l;
      }
      s_w[buf][wn][0][wl] = lo;
      s_w[buf][wn][1][wl] = mid;
      s_w[buf][wn][2][wl] = hi;
    }
    __syncthreads();
    const v8bf cur = a;
    if (k + 32 < k1) {  // the next step's loads, in flight during this step's products
      f0 = *(const float4*)(wrow + k + 32);
      f1 = *(const float4*)(wrow + k + 36);
      a = *(const v8bf*)(xr + k + 32);
    }
    if (live) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (n < nt) {
          acc[n] = mfma_bf16(cur, s_w[buf][n][0][lane], acc[n]);
          acc[n] = mfma_bf16(cur, s_w[buf][n][1][lane], acc[n]);
          acc[n] = mfma_bf16(cur, s_w[buf][n][2][lane], acc[n]);
        }
      }
    }
    buf ^= 1;
  }
  if (!live) return;
  float* zp = zpart + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if (n < nt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 4 * g + j;
        if (t < T) zp[(size_t)t * E + e0 + 16 * n + r] = acc[n][j];
      }
    }
  }
}

// WIDE = false: one wave per token, 4 tokens per 256-thread block; lane l
// adds the K-split partial logits of experts l, l+64, l+128, l+192.
// WIDE = true (many K splits, few tokens): one token per block; thread e adds
// the partials of expert e (eight loads in flight), then wave 0 runs the
// selection.
template <bool WIDE>
__global__ __launch_bounds__(256) void gate_select_kernel(const float* __restrict__ zpart, int ksplit,
                                                          const float* __restrict__ bias, int T, int E, int G,
                                                          int TG, int K, float route_scale,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out) {
  __shared__ GateSlot slots[WIDE ? 1 : 4];
  const int wave = threadIdx.x >> 6;
  const int t = WIDE ? (int)blockIdx.x : (int)blockIdx.x * 4 + wave;
  const int tt = t < T ? t : T - 1;
  if constexpr (WIDE) {
    const int e = threadIdx.x;
    if (e < E) {
      const size_t split_stride = (size_t)T * E;
      const float* zp = zpart + (size_t)tt * E + e;
      float z = 0.f;
      int ks = 0;
      for (; ks + 8 <= ksplit; ks += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = zp[(ks + j) * split_stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) z += v[j];
      }
      for (; ks < ksplit; ++ks) z += zp[ks * split_stride];
      gate_score(slots[0], bias, e, z);
    }
    __syncthreads();
    if (wave == 0) gate_choose_wave(slots[0], E, G, TG, K, route_scale, t, t < T, idx_out, w_out);
  } else {
    gate_scores_wave(zpart, ksplit, bias, T, E, tt, slots[wave]);
    gate_choose_wave(slots[wave], E, G, TG, K, route_scale, t, t < T, idx_out, w_out);
  }
}

}  // namespace

namespace {

// 16-expert tiles per wave of the logits kernels: small batches spread the
// router weight over more workgroups (experts) instead of more K splits, which
// keeps the partial logits the selection has to add small; large batches
// share each workgroup's 64 weight rows in LDS (gate_logits_lds_kernel).
int gate_tiles_per_wave(int64_t T) { return T <= 256 ? 1 : 4; }

}  // namespace

int gate_ksplit(int64_t T, int d, int E) {
  const int ntw = gate_tiles_per_wave(T);
  int64_t base = ((T + 63) / 64) * ((E + 16 * ntw - 1) / (16 * ntw));
  if (base < 1) base = 1;
  const int64_t target = ntw == 4 ? 2048 : 512;
  int64_t ks = (target + base - 1) / base;
  const int ksteps = d / 32;
  if (ks > ksteps) ks = ksteps;
  if (ks > GATE_KSPLIT_MAX) ks = GATE_KSPLIT_MAX;
  if (ks < 1) ks = 1;
  return (int)ks;
}

hipError_t launch_gate(const uint16_t* x, const float* gate_w, const float* gate_b, int T, int d, int E, int G,
                       int TG, int K, float route_scale, float* zpart, int ksplit, int32_t* idx, float* w,
                       hipStream_t s) {
  const int ksteps = d / 32;
  const int kchunk = ((ksteps + ksplit - 1) / ksplit) * 32;
  const int kz = (d + kchunk - 1) / kchunk;
  const int ntw = gate_tiles_per_wave(T);
  dim3 grid((T + 63) / 64, (E + 16 * ntw - 1) / (16 * ntw), kz);
  if (ntw == 1)
    hipLaunchKernelGGL(gate_logits_kernel, grid, dim3(256), 0, s, x, gate_w, zpart, T, d, E, kchunk);
  else
    hipLaunchKernelGGL(gate_logits_lds_kernel, grid, dim3(256), 0, s, x, gate_w, zpart, T, d, E, kchunk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (kz >= 8 && T <= 1024)
    hipLaunchKernelGGL(gate_select_kernel<true>, dim3(T), dim3(256), 0, s, zpart, kz, gate_b, T, E, G, TG, K,
                       route_scale, idx, w);
  else
    hipLaunchKernelGGL(gate_select_kernel<false>, dim3((T + 3) / 4), dim3(256), 0, s, zpart, kz, gate_b, T, E, G,
                       TG, K, route_scale, idx, w);
  return hipGetLastError();
}

}  // namespace moe
