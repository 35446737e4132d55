// Grouped SwiGLU expert FFN with FP8 (e4m3) weights and activations
// ("DeepSeek-V3.2-Exp · Gate projection": expert excerpt
// ``w2((silu(w1(x).float()) * w3(x).float()).type_as(x))`` and Linear excerpt:
// FP8 weights [out, in] with one fp32 scale per 128x128 block).
//
// Work unit ("tile"): up to 16*MT consecutive permuted rows of one expert.
// Up-projection workgroups own (tile, 128-column block of h): the 8 waves
// each compute 16 h columns from the matching 16 rows of w1 and of w3, so
// the workgroup holds the whole 128-wide block and quantises h to e4m3 in its
// epilogue.  Down-projection workgroups own (tile, 128 output features).
//
// Each 128-deep scale block is one block_dot (four bf16 MFMAs on exactly
// decoded e4m3 operands), so each block sum is scaled once:
// acc += P * (s_weight[block] * s_act[row, block]).
// Weights are the A operand (16 output features), activations the B operand
// (16 rows); lane l ends with features 4*(l/16)+j of row l%16.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// One block of 256 threads.  tiles[i] = {expert, first row, rows, 0}; the
// shared expert is expert E with rows [T*K, T*K + T).
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* __restrict__ offsets, int E, int T, int K,
                                                         int NT, int has_shared, int cap,
                                                         int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int s[256];
  const int e = threadIdx.x;
  const int TK = T * K;
  int lo = 0, cnt = 0, n = 0;
  if (e < E) {
    lo = clampi(offsets[e], 0, TK);
    const int hi = clampi(offsets[e + 1], lo, TK);
    cnt = hi - lo;
    n = (cnt + NT - 1) / NT;
  }
  s[e] = n;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  const int base = s[e] - n;
  const int routed = min(s[255], cap);
  for (int j = 0; j < n && base + j < cap; ++j)
    tiles[base + j] = make_int4(e, lo + j * NT, min(NT, cnt - j * NT), 0);
  int total = routed;
  if (has_shared) {
    const int nsh = (T + NT - 1) / NT;
    for (int j = threadIdx.x; j < nsh; j += blockDim.x)
      tiles[routed + j] = make_int4(E, TK + j * NT, min(NT, T - j * NT), 0);
    total += nsh;
  }
  if (threadIdx.x == 0) *n_tiles = total;
}

struct FfnArgs {
  ExpertPtrs routed;
  ExpertPtrs shared;
  int E, d, I, T, K;
  const int4* tiles;
  const int32_t* n_tiles;
  const int32_t* row_token;
  const uint8_t* xq;
  const float* xs;
  uint8_t* hq;
  float* hs;
  uint16_t* out;
};

// grid = max_tiles * (I/128), block = 512 (8 waves)
template <int MT>
__global__ __launch_bounds__(512) void ffn_up_kernel(FfnArgs a) {
  const int nib = a.I / BLK, nkb = a.d / BLK;
  const int tile = blockIdx.x / nib, ib = blockIdx.x - tile * nib;
  if (tile >= *a.n_tiles) return;  // uniform for the whole block, before any barrier
  const int4 td = a.tiles[tile];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const bool sh = e >= a.E;
  const ExpertPtrs& P = sh ? a.shared : a.routed;
  const size_t eo = sh ? 0 : (size_t)e;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int o = ib * BLK + 16 * wave + r;  // w1 / w3 row (h column) this lane loads
  const uint8_t* a1 = P.w1 + (eo * a.I + o) * (size_t)a.d;
  const uint8_t* a3 = P.w3 + (eo * a.I + o) * (size_t)a.d;
  const float* s1 = P.s1 + (eo * nib + ib) * nkb;
  const float* s3 = P.s3 + (eo * nib + ib) * nkb;
  const int mvalid = (nrows + 15) >> 4;

  const uint8_t* bq[MT];
  const float* bs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = row0 + min(16 * m + r, nrows - 1);
    const int tok = clampi(a.row_token[row], 0, a.T - 1);
    bq[m] = a.xq + (size_t)tok * a.d;
    bs[m] = a.xs + (size_t)tok * nkb;
  }
  v4f acc1[MT], acc3[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc1[m] = v4f{0.f, 0.f, 0.f, 0.f};
    acc3[m] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  for (int kb = 0; kb < nkb; ++kb) {
    const Frag A1 = decode_e4m3(load_frag_e4m3(a1 + kb * BLK, g));
    const Frag A3 = decode_e4m3(load_frag_e4m3(a3 + kb * BLK, g));
    const float sw1 = s1[kb], sw3 = s3[kb];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < mvalid) {
        const Frag B = decode_e4m3(load_frag_e4m3(bq[m] + kb * BLK, g));
        const float sx = bs[m][kb];
        const v4f p1 = block_dot(A1, B);
        const v4f p3 = block_dot(A3, B);
        const float f1 = sw1 * sx, f3 = sw3 * sx;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc1[m][j] = fmaf(p1[j], f1, acc1[m][j]);
          acc3[m][j] = fmaf(p3[j], f3, acc3[m][j]);
        }
      }
    }
  }

  // epilogue: h = bf16(silu(bf16 g) * bf16 u); per-row amax over the 128 columns
  __shared__ float red[8][MT * 16];
  float hv[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float gv = round_bf16(acc1[m][j]);
      const float uv = round_bf16(acc3[m][j]);
      const float h = round_bf16(gv / (1.f + expf(-gv)) * uv);
      hv[m][j] = h;
      amax = fmaxf(amax, fabsf(h));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (g == 0) red[wave][m * 16 + r] = amax;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < mvalid && 16 * m + r < nrows) {
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) amax = fmaxf(amax, red[w][m * 16 + r]);
      const float sc = amax == 0.f ? 1.f : amax / E4M3_MAX;
      const size_t row = (size_t)(row0 + 16 * m + r);
      const uint32_t q = pack4_e4m3(hv[m][0] / sc, hv[m][1] / sc, hv[m][2] / sc, hv[m][3] / sc);
      *(uint32_t*)(a.hq + row * a.I + ib * BLK + 16 * wave + 4 * g) = q;
      if (wave == 0 && g == 0) a.hs[row * nib + ib] = sc;
    }
  }
}

// grid = max_tiles * (d/128), block = 512 (8 waves)
template <int MT>
__global__ __launch_bounds__(512) void ffn_down_kernel(FfnArgs a) {
  const int nob = a.d / BLK, nkb = a.I / BLK;
  const int tile = blockIdx.x / nob, ob = blockIdx.x - tile * nob;
  if (tile >= *a.n_tiles) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, row0 = td.y, nrows = td.z;
  const bool sh = e >= a.E;
  const ExpertPtrs& P = sh ? a.shared : a.routed;
  const size_t eo = sh ? 0 : (size_t)e;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int o = ob * BLK + 16 * wave + r;
  const uint8_t* aw = P.w2 + (eo * a.d + o) * (size_t)a.I;
  const float* s2 = P.s2 + (eo * nob + ob) * nkb;
  const int mvalid = (nrows + 15) >> 4;

  const uint8_t* bq[MT];
  const float* bs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const size_t row = (size_t)(row0 + min(16 * m + r, nrows - 1));
    bq[m] = a.hq + row * a.I;
    bs[m] = a.hs + row * nkb;
  }
  v4f acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < nkb; ++kb) {
    const Frag A = decode_e4m3(load_frag_e4m3(aw + kb * BLK, g));
    const float sw = s2[kb];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < mvalid) {
        const Frag B = decode_e4m3(load_frag_e4m3(bq[m] + kb * BLK, g));
        const float f = sw * bs[m][kb];
        const v4f p = block_dot(A, B);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = fmaf(p[j], f, acc[m][j]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < mvalid && 16 * m + r < nrows) {
      const size_t row = (size_t)(row0 + 16 * m + r);
      uint2 v;
      v.x = (uint32_t)f32_to_bf16(acc[m][0]) | ((uint32_t)f32_to_bf16(acc[m][1]) << 16);
      v.y = (uint32_t)f32_to_bf16(acc[m][2]) | ((uint32_t)f32_to_bf16(acc[m][3]) << 16);
      *(uint2*)(a.out + row * a.d + ob * BLK + 16 * wave + 4 * g) = v;
    }
  }
}

template <int MT>
hipError_t launch_gemms(const FfnArgs& a, int64_t max_tiles, hipStream_t s, hipEvent_t* ev) {
  const int64_t g1 = max_tiles * (a.I / BLK), g2 = max_tiles * (a.d / BLK);
  if (ev) (void)hipEventRecord(ev[0], s);
  hipLaunchKernelGGL(ffn_up_kernel<MT>, dim3((unsigned)g1), dim3(512), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) (void)hipEventRecord(ev[1], s);
  hipLaunchKernelGGL(ffn_down_kernel<MT>, dim3((unsigned)g2), dim3(512), 0, s, a);
  err = hipGetLastError();
  if (ev) (void)hipEventRecord(ev[2], s);
  return err;
}

}  // namespace

int ffn_tile_rows(int64_t T) {
  if (T <= 16) return 16;
  if (T <= 32) return 32;
  if (T <= 64) return 64;
  return 128;
}

int64_t ffn_max_tiles(int64_t T, int K, int E, int tile_rows) {
  return (T * K) / tile_rows + E + (T + tile_rows - 1) / tile_rows + 1;
}

hipError_t launch_ffn(const ExpertPtrs& routed, const ExpertPtrs* shared, int T, int d, int I, int E, int K,
                      const int32_t* offsets, const int32_t* row_token, const uint8_t* xq, const float* xs,
                      int4* tiles, int32_t* n_tiles, uint8_t* hq, float* hs, uint16_t* out, hipStream_t s,
                      hipEvent_t* ev) {
  const int NT = ffn_tile_rows(T);
  const int64_t max_tiles = ffn_max_tiles(T, K, E, NT);
  const int nsh = shared ? (T + NT - 1) / NT : 0;
  hipLaunchKernelGGL(plan_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, T, K, NT, shared ? 1 : 0,
                     (int)(max_tiles - nsh), tiles, n_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FfnArgs a;
  a.routed = routed;
  a.shared = shared ? *shared : routed;
  a.E = E;
  a.d = d;
  a.I = I;
  a.T = T;
  a.K = K;
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.row_token = row_token;
  a.xq = xq;
  a.xs = xs;
  a.hq = hq;
  a.hs = hs;
  a.out = out;
  switch (NT) {
    case 16: return launch_gemms<1>(a, max_tiles, s, ev);
    case 32: return launch_gemms<2>(a, max_tiles, s, ev);
    case 64: return launch_gemms<4>(a, max_tiles, s, ev);
    default: return launch_gemms<8>(a, max_tiles, s, ev);
  }
}

}  // namespace moe
