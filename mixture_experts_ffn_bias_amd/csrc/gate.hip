// Router of the MoE layer: logits x . Wg^T, sigmoid scores, bias for
// selection, group-limited top-k, normalised and scaled weights
// ("DeepSeek-V3.2-Exp · MoE update", moe-forward excerpt: the gate call; the
// router bias is implied by the MoE parameter count on "MoE transformer
// block", parameter accounting table).
//
// Logits: x is bf16, Wg is fp32.  Each fp32 weight is split into three bf16
// parts hi + mid + lo that sum to it exactly, so three bf16 MFMAs per K step
// give the fp32-weight product with fp32 accumulation on the matrix cores.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int GATE_KSPLIT_MAX = 16;  // K splits of the logits (partials the selection adds)

__device__ __forceinline__ void split3(float w, __bf16& hi, __bf16& mid, __bf16& lo) {
  const uint32_t u = __float_as_uint(w);
  const float h = __uint_as_float(u & 0xFFFF0000u);     // top 8 significant bits
  const float r1 = w - h;                                // exact
  const uint32_t u1 = __float_as_uint(r1);
  const float m = __uint_as_float(u1 & 0xFFFF0000u);
  const float r2 = r1 - m;                               // exact, fits in bf16
  hi = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
  mid = __builtin_bit_cast(__bf16, (uint16_t)(u1 >> 16));
  lo = (__bf16)r2;
}

// Grid (ceil(T/64), ceil(E/(16 ntw)), ksplit), 256 threads.  Wave w owns
// tokens [t0, t0+16) and up to ntw (1..4) 16-expert tiles; blockIdx.z a K
// range.  zpart[z][t][e] receives the partial logits of that K range.
__global__ __launch_bounds__(256) void gate_logits_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ gw,
                                                          float* __restrict__ zpart, int T, int d, int E,
                                                          int kchunk, int ntw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 16 * ntw;
  const int k0 = blockIdx.z * kchunk;
  const int k1 = min(d, k0 + kchunk);
  if (t0 >= T) return;  // no barriers in this kernel
  const int nt = min(ntw, (E - e0) >> 4);
  const uint16_t* xr = x + (size_t)min(t0 + r, T - 1) * d;
  const float* wr[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) wr[n] = gw + (size_t)(e0 + 16 * min(n, nt - 1) + r) * d;

  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int k = k0; k < k1; k += 32) {
    const v8bf a = *(const v8bf*)(xr + k + 8 * g);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n < nt) {
        const float4 f0 = *(const float4*)(wr[n] + k + 8 * g);
        const float4 f1 = *(const float4*)(wr[n] + k + 8 * g + 4);
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
        acc[n] = mfma_bf16(a, lo, acc[n]);
        acc[n] = mfma_bf16(a, mid, acc[n]);
        acc[n] = mfma_bf16(a, hi, acc[n]);
      }
    }
  }
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

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// WIDE = false: one wave per token, 4 tokens per 256-thread block; lane l
// adds the K-split partial logits of experts l, l+64, l+128, l+192.
// WIDE = true (many K splits, few tokens): one token per block; thread e adds
// the partials of expert e, then all four waves run the selection on that
// token and wave 0 writes it.
template <bool WIDE>
__global__ __launch_bounds__(256) void gate_select_kernel(const float* __restrict__ zpart, int ksplit,
                                                          const float* __restrict__ bias, int T, int E, int G,
                                                          int TG, int K, float route_scale,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out) {
  __shared__ float s_score[4][256];
  __shared__ float s_biased[4][256];
  __shared__ float s_gs[4][64];
  __shared__ int s_keep[4][64];
  __shared__ float s_sel[4][32];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = WIDE ? (int)blockIdx.x : (int)blockIdx.x * 4 + wave;
  const bool live = t < T && (!WIDE || wave == 0);
  const int tt = t < T ? t : T - 1;
  const int epg = E / G;
  const int slot = WIDE ? 0 : wave;  // LDS row of the token's scores
  const size_t split_stride = (size_t)T * E;

  if (WIDE) {
    // logits: the K-split partial sums, added in split order, eight loads in flight
    const int e = threadIdx.x;
    if (e < E) {
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
      const float s = 1.f / (1.f + expf(-z));
      float v = s + bias[e];
      if (v != v) v = -INFINITY;  // NaN never wins a comparison below
      s_score[0][e] = s;
      s_biased[0][e] = v;
    }
  } else {
    // logits: the K-split partial sums, added in split order; eight splits of
    // all four experts are loaded before they are added
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    const float* zp = zpart + (size_t)tt * E + lane;
    int ks = 0;
    for (; ks + 8 <= ksplit; ks += 8) {
      float v[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[j][i] = (lane + 64 * i < E) ? zp[(ks + j) * split_stride + 64 * i] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] += v[j][i];
    }
    for (; ks < ksplit; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E) z[i] += zp[ks * split_stride + 64 * i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const float s = 1.f / (1.f + expf(-z[i]));
        float v = s + bias[e];
        if (v != v) v = -INFINITY;
        s_score[wave][e] = s;
        s_biased[wave][e] = v;
      }
    }
  }
  __syncthreads();
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    b[i] = e < E ? s_biased[slot][e] : -INFINITY;
  }
  if (lane < G) {  // group score: sum of the two largest biased scores
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int j = 0; j < epg; ++j) {
      const float v = s_biased[slot][lane * epg + j];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    float gs = m1 + m2;
    if (gs != gs) gs = -INFINITY;
    s_gs[wave][lane] = gs;
  }
  __syncthreads();
  if (lane < G) {  // keep the topk_groups best groups, ties to the lower index
    const float gs = s_gs[wave][lane];
    int rank = 0;
    for (int h = 0; h < G; ++h) {
      const float o = s_gs[wave][h];
      rank += (o > gs || (o == gs && h < lane)) ? 1 : 0;
    }
    s_keep[wave][lane] = rank < TG;
  }
  __syncthreads();

  bool avail[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    avail[i] = e < E;
    if (avail[i] && !s_keep[wave][e / epg]) b[i] = -INFINITY;  // excluded group
  }
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (avail[i] && better(b[i], e, bv, bi)) {
        bv = b[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // bi < E always: at least K >= 1 available experts remain (K <= E)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == lane + 64 * i) avail[i] = false;
    if (lane == 0) {
      s_sel[wave][k] = s_score[slot][bi];
      if (live) idx_out[(size_t)t * K + k] = bi;
    }
  }
  __syncthreads();
  if (lane < K && live) {
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += s_sel[wave][k];
    w_out[(size_t)t * K + lane] = s_sel[wave][lane] / sum * route_scale;
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
  hipLaunchKernelGGL(gate_logits_kernel, grid, dim3(256), 0, s, x, gate_w, zpart, T, d, E, kchunk, ntw);
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
