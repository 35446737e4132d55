// Router device functions ("DeepSeek-V3.2-Exp · MoE update", moe-forward
// excerpt: the gate call; the router bias is implied by the MoE parameter
// count on "MoE transformer block", parameter accounting table): partial
// logits x . Wg^T on the matrix cores, sigmoid scores, bias for selection,
// group-limited top-k and the normalised, scaled weights.  Shared by the
// router kernels and the single-launch layer kernel.
//
// Logits: x is bf16, Wg is fp32.  Each fp32 weight is split into three bf16
// parts hi + mid + lo that sum to it exactly, so three bf16 MFMAs per K step
// give the fp32-weight product with fp32 accumulation.
#pragma once
#include "common.h"

namespace moe {

namespace {

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

// One wave: partial logits of tokens [t0, t0 + 16) (t0 < T; rows past T
// repeat row T - 1 and are not stored) and nt (1..NTW) 16-expert tiles from
// e0, over K range [k0, k1) (multiples of 32).  zp[t][e] (E columns)
// receives the partial sums of this K range (COH: agent-coherent stores).
// The loads of 4 / NTW K steps are issued before any of them is multiplied
// (the loop is latency-bound otherwise); the products are accumulated in K
// order all the same.
template <int NTW, bool COH = false>
__device__ __forceinline__ void gate_logits_wave(const uint16_t* __restrict__ x, const float* __restrict__ gw,
                                                 float* __restrict__ zp, int T, int d, int E, int t0, int e0,
                                                 int nt, int k0, int k1) {
  static_assert(NTW == 1 || NTW == 2 || NTW == 4, "expert tiles per wave");
  constexpr int U = 4 / NTW;  // K steps in flight
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const uint16_t* xr = x + (size_t)min(t0 + r, T - 1) * d;
  const float* wr[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) wr[n] = gw + (size_t)(e0 + 16 * min(n, nt - 1) + r) * d;

  v4f acc[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int k = k0; k < k1; k += 32 * U) {
    v8bf a[U];
    float4 f0[U][NTW], f1[U][NTW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 32 * u < k1) {
        const int kk = k + 32 * u + 8 * g;
        a[u] = *(const v8bf*)(xr + kk);
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          if (n < nt) {
            f0[u][n] = *(const float4*)(wr[n] + kk);
            f1[u][n] = *(const float4*)(wr[n] + kk + 4);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 32 * u < k1) {
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          if (n < nt) {
            const float f[8] = {f0[u][n].x, f0[u][n].y, f0[u][n].z, f0[u][n].w,
                                f1[u][n].x, f1[u][n].y, f1[u][n].z, f1[u][n].w};
            v8bf hi, mid, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              __bf16 h, m, l;
              split3(f[j], h, m, l);
              hi[j] = h;
              mid[j] = m;
              lo[j] = l;
            }
            acc[n] = mfma_bf16(a[u], lo, acc[n]);
            acc[n] = mfma_bf16(a[u], mid, acc[n]);
            acc[n] = mfma_bf16(a[u], hi, acc[n]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    if (n < nt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 4 * g + j;
        if (t < T) st<COH>(zp + (size_t)t * E + e0 + 16 * n + r, acc[n][j]);
      }
    }
  }
}

// LDS of one token's selection (E <= 256, G <= 64, K <= 32).
struct GateSlot {
  float score[256];   // sigmoid scores
  float biased[256];  // scores + bias (NaN -> -inf), the selection key
  float gs[64];       // group scores
  int keep[64];       // group kept
  float sel[32];      // scores of the chosen experts
};

// This wave's LDS writes are visible to all its lanes (the wave runs its LDS
// operations in order; the fences keep the compiler from moving accesses).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Score of expert e from its logit z into the slot.
__device__ __forceinline__ void gate_score(GateSlot& sl, const float* __restrict__ bias, int e, float z) {
  const float s = 1.f / (1.f + expf(-z));
  float v = s + bias[e];
  if (v != v) v = -INFINITY;  // NaN never wins a comparison below
  sl.score[e] = s;
  sl.biased[e] = v;
}

// One wave: the logits of token tt from ksplit partial planes (plane stride
// T*E), added in split order with eight splits of the lane's four experts
// (lane, lane + 64, lane + 128, lane + 192) loaded before they are added,
// then the scores into the slot.
__device__ __forceinline__ void gate_scores_wave(const float* __restrict__ zpart, int ksplit,
                                                 const float* __restrict__ bias, int T, int E, int tt,
                                                 GateSlot& sl) {
  const int lane = threadIdx.x & 63;
  const size_t split_stride = (size_t)T * E;
  float z[4] = {0.f, 0.f, 0.f, 0.f};
  const float* zp = zpart + (size_t)tt * E + lane;
  int ks = 0;
  for (; ks + 8 <= ksplit; ks += 8) {
    float v[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[j][i] = (lane + 64 * i < E) ? zp[(ks + j) * split_stride + 64 * i] : 0.f;
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
    if (e < E) gate_score(sl, bias, e, z[i]);
  }
}

// Largest v over the 64 lanes of the wave, in every lane.  Data-parallel
// (DPP) moves of the GFX9 family: max with the lane 1, 2, 4 and 8 places
// lower in the same 16-lane row (lane 15 of a row then holds the row's
// maximum), row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and
// 3 (lane 63 then holds the wave's maximum), and lane 63 read out.  Lanes a
// move has no source for take -inf.
__device__ __forceinline__ float wave_max_dpp(float v) {
  const int ninf = __float_as_int(-INFINITY);
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x111, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x112, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x114, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x118, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x142, 0xa, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x143, 0xc, 0xf, false))));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// One wave, scores of token t in the slot: group score = sum of the two
// largest biased scores of the group; the TG best groups are kept (ties to
// the lower group); then K times the best remaining biased score among kept
// experts (ties to the lower expert).  Weights = chosen sigmoid scores
// normalised to sum 1, times route_scale.  live: store idx and w of token t
// (COH: with agent-coherent stores).
//
// Lane l holds experts l, l + 64, l + 128, l + 192 (E <= 256).  When the
// group size divides 64 and is a power of two, a group is a segment of lanes
// in one of those four sets, and its top two come from a butterfly over the
// segment; otherwise lanes < G scan their group in LDS.  Each of the K picks
// is a DPP wave maximum of the lanes' best available scores, and the lowest
// expert index holding it comes from a ballot.
template <bool COH = false>
__device__ __forceinline__ void gate_choose_wave(GateSlot& sl, int E, int G, int TG, int K, float route_scale,
                                                 int t, bool live, int32_t* __restrict__ idx_out,
                                                 float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int epg = E / G;
  wave_lds_sync();
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    b[i] = e < E ? sl.biased[e] : -INFINITY;
  }
  if (epg <= 64 && (epg & (epg - 1)) == 0) {
    float m1[4], m2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m1[i] = b[i];
      m2[i] = -INFINITY;
    }
    for (int o = 1; o < epg; o <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a1 = __shfl_xor(m1[i], o), a2 = __shfl_xor(m2[i], o);
        m2[i] = fmaxf(fminf(m1[i], a1), fmaxf(m2[i], a2));
        m1[i] = fmaxf(m1[i], a1);
      }
    }
    if ((lane & (epg - 1)) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = (lane + 64 * i) / epg;
        if (g < G) {
          float gs = m1[i] + m2[i];
          if (gs != gs) gs = -INFINITY;
          sl.gs[g] = gs;
        }
      }
    }
  } else if (lane < G) {
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int j = 0; j < epg; ++j) {
      const float v = sl.biased[lane * epg + j];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    float gs = m1 + m2;
    if (gs != gs) gs = -INFINITY;
    sl.gs[lane] = gs;
  }
  wave_lds_sync();
  if (lane < G) {
    const float gs = sl.gs[lane];
    int rank = 0;
    for (int h = 0; h < G; ++h) {
      const float o = sl.gs[h];
      rank += (o > gs || (o == gs && h < lane)) ? 1 : 0;
    }
    sl.keep[lane] = rank < TG;
  }
  wave_lds_sync();

  bool avail[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    avail[i] = e < E;
    if (avail[i] && !sl.keep[e / epg]) b[i] = -INFINITY;  // excluded group
  }
  for (int k = 0; k < K; ++k) {
    float lv = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (avail[i]) lv = fmaxf(lv, b[i]);
    const float mx = wave_max_dpp(lv);
    // the lowest available expert holding mx (one exists: K <= E)
    int bi = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const uint64_t m = __ballot(avail[i] && b[i] == mx);
      if (m) bi = 64 * i + __builtin_ctzll(m);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bi == lane + 64 * i) avail[i] = false;
    if (lane == 0) {
      sl.sel[k] = sl.score[bi];
      if (live) st<COH>(idx_out + (size_t)t * K + k, (int32_t)bi);
    }
  }
  wave_lds_sync();
  if (lane < K && live) {
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += sl.sel[k];
    st<COH>(w_out + (size_t)t * K + lane, sl.sel[lane] / sum * route_scale);
  }
}

}  // namespace

}  // namespace moe
