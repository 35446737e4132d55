// Router kernels of the MoE layer ("DeepSeek-V3.2-Exp · MoE update",
// moe-forward excerpt: the gate call): K-split partial logits, then the
// selection per token.  The arithmetic is in gate_dev.h.
#include "gate_dev.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int GATE_KSPLIT_MAX = 16;  // K splits of the logits (partials the selection adds)

// Grid (ceil(T/64), ceil(E/(16 NTW)), ksplit), 256 threads.  Wave w owns
// tokens [t0, t0+16) and up to NTW (1 or 4) 16-expert tiles; blockIdx.z a K
// range.  zpart[z][t][e] receives the partial logits of that K range.
template <int NTW>
__global__ __launch_bounds__(256) void gate_logits_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ gw,
                                                          float* __restrict__ zpart, int T, int d, int E,
                                                          int kchunk) {
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 16 * NTW;
  const int k0 = blockIdx.z * kchunk;
  if (t0 >= T) return;  // no barriers in this kernel
  gate_logits_wave<NTW>(x, gw, zpart + (size_t)blockIdx.z * T * E, T, d, E, t0, e0, min(NTW, (E - e0) >> 4), k0,
                        min(d, k0 + kchunk));
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

// 16-expert tiles per wave of the logits kernel: small batches spread the
// router weight over more workgroups (experts) instead of more K splits, which
// keeps the partial logits the selection has to add small.
int gate_tiles_per_wave(int64_t T) { return T <= 256 ? 1 : 4; }

}  // namespace

int gate_ksplit(int64_t T, int d, int E) {
  const int ntw = gate_tiles_per_wave(T);
  int64_t base = ((T + 63) / 64) * ((E + 16 * ntw - 1) / (16 * ntw));
  if (base < 1) base = 1;
  int64_t ks = (512 + base - 1) / base;
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
    hipLaunchKernelGGL(gate_logits_kernel<1>, grid, dim3(256), 0, s, x, gate_w, zpart, T, d, E, kchunk);
  else
    hipLaunchKernelGGL(gate_logits_kernel<4>, grid, dim3(256), 0, s, x, gate_w, zpart, T, d, E, kchunk);
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
